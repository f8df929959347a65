// Exact Top-k of one query row's pool slots from their scores, by one
// workgroup of NT threads: the pool Top-K's selection step.
//
// "DeepSeek-V4.1-Flash 架构详解", §3.2: the Top-512 of a Full or Reindex layer
// is taken among the positions of the pool of blocks.
//
// Slot s of the row is position pool[s / 8] * 8 + s % 8 (pool = the row's
// block ids, slots of a block id outside [0, nb_cap) or past the visible
// length hold nothing).  Thread t holds the scores of slots [PER t, PER t +
// PER) in registers with a validity mask.  The threshold: 2048 bins linear in
// the score value between the row's minimum and maximum (bin order is key
// order), the bin holding the need-th largest slot, and the exact (key, slot)
// threshold inside it from LDS copies of that bin's items, or over every slot
// when that bin is too large.  The selection is VALU-bound on one compute
// unit, so each slot costs as few instructions as possible: the bins are
// computed once from the float scores and kept in registers, invalid slots
// go to a spare bin (no branch around the LDS atomic), and exact keys are
// formed only for the threshold bin.  Selected slots are reported in slot
// order, the k-th with output offset k.
#pragma once
#include "csa2_device.h"
#include "select_common.h"

namespace csa2 {

constexpr int kPoolSlots = kMaxPoolBlocks * kBlock;
constexpr int kPfBins = 2048;
constexpr int kPfCap = 2048;
constexpr int kRankMax = 256;   // threshold bins up to this size are resolved by counting ranks

template <int NT>
struct PoolSel {
  static constexpr int kPer = kPoolSlots / NT;      // slots per thread
  static constexpr int kBlocks = kPer / kBlock;     // pool blocks per thread
  static_assert(kPer * NT == kPoolSlots && kBlocks * kBlock == kPer, "whole blocks per thread");
  static_assert(kPer <= 32, "one validity bit per slot in a 32-bit mask");

  // LDS of one selection.
  struct Scratch {
    uint32_t keys[kPoolSlots];       // every slot's key (threshold bin too large)
    uint32_t hist[kPfBins + 1];      // + a spare bin for invalid slots
    uint32_t ckey[kPfCap];
    int32_t cid[kPfCap];
    uint32_t hist256[256];
    uint32_t wb[Wg<NT>::kScratch];
    uint32_t ccount;
  };

  // A thread's slots: their block ids and scores.
  struct Row {
    int blk[kBlocks];
    float sv[kPer];
  };

  // Slot PER t + e of thread t is kept at keys[e * NT + t] (the accesses of
  // a wave fall in distinct banks); empty slots hold key 0, which no finite
  // score has.
  struct LdsKeys {
    const uint32_t* k;
    __device__ uint32_t key(uint32_t c) const { return k[c]; }
    __device__ int32_t id(uint32_t c) const {
      return static_cast<int32_t>((c % NT) * kPer + c / NT);
    }
    static constexpr uint32_t n = kPoolSlots;
  };

  // Issues the loads of thread t's slots: block ids from prow[kb] and the
  // scores, stored per position (srow, non-null) or re-scored per slot
  // (ps[kb * 8]).  Clamped loads (no branch per load), then a select.
  __device__ __forceinline__ static void load(Row& row, const int32_t* prow, int kb, const float* srow,
                              const float* ps, int vis) {
    const int t = threadIdx.x;
    const int nslots = kb * kBlock;
    const int s0 = t * kPer;
    const bool mine = s0 < nslots;
#pragma unroll
    for (int u = 0; u < kBlocks; ++u) {
      const int bi = min((s0 >> 3) + u, kb - 1);
      const int v = prow[bi];
      row.blk[u] = (mine && (s0 >> 3) + u < kb) ? v : -1;
    }
    if (srow) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int pos = row.blk[e >> 3] * kBlock + (e & 7);
        row.sv[e] = srow[min(max(pos, 0), vis > 0 ? vis - 1 : 0)];
      }
    } else if (s0 + kPer <= nslots) {
      const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(ps + s0);
#pragma unroll
      for (int e4 = 0; e4 < kPer / 4; ++e4) {
        const f32x4_t v = p4[e4];
        row.sv[4 * e4] = v[0];
        row.sv[4 * e4 + 1] = v[1];
        row.sv[4 * e4 + 2] = v[2];
        row.sv[4 * e4 + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < kPer; ++e) row.sv[e] = ps[min(s0 + e, nslots - 1)];
    }
  }

  // The selection of min(top_k, valid slots) slots.  emit(off, pos, score)
  // is called once per selected slot with its output offset off < need
  // (kScore: the slot's score is passed; otherwise 0); returns need.  The
  // scratch must be free on entry (no barrier guards it); after the return
  // it is free once a barrier has passed.
  template <bool kScore, class Emit>
  __device__ __forceinline__ static uint32_t select(const Row& row, int nb_cap, int vis, int top_k,
                                    Scratch& sm, Emit emit) {
    using W = Wg<NT>;
    const int tid = threadIdx.x;
    const int s0 = tid * kPer;
    uint32_t vm = 0;   // bit e: slot s0 + e holds a visible position
#pragma unroll
    for (int u = 0; u < kBlocks; ++u) {
      const int bk = row.blk[u];
      if (bk >= 0 && bk < nb_cap) {
        const int m = min(max(vis - bk * kBlock, 0), kBlock);   // visible positions of the block
        vm |= ((1u << m) - 1u) << (kBlock * u);
      }
    }
    float vmax = -__builtin_inff(), vmin = __builtin_inff();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const bool v = (vm >> e) & 1u;
      vmax = fmaxf(vmax, v ? row.sv[e] : -__builtin_inff());
      vmin = fminf(vmin, v ? row.sv[e] : __builtin_inff());
    }
    uint32_t nv = static_cast<uint32_t>(__popc(vm));
    uint32_t mx = vm ? float_to_key(vmax) : 0u, mn_inv = vm ? ~float_to_key(vmin) : 0u;
    for (int i = tid; i <= kPfBins; i += NT) sm.hist[i] = 0;
    W::reduce_sum_max_max(nv, mx, mn_inv, sm.wb);   // includes the barrier after the clear
    const uint32_t n_valid = nv;
    const uint32_t need = min(static_cast<uint32_t>(max(top_k, 0)), n_valid);
    // Selection among the valid slots, by mode: 0 every one (need ==
    // n_valid); 1 bin > b1, or bin == b1 and (key, id) selected by K*, I*;
    // 2 (threshold bin too large) (key, id) selected by K*, I*.  Bin order
    // is key order, so every key of a higher bin exceeds every key of bin b1.
    int mode = 0, b1 = 0;
    uint32_t kstar = 0;
    int32_t istar = 0x7fffffff;
    int bin[kPer];
    if (need > 0 && need < n_valid) {
      mode = 1;
      const float vhi = key_to_float(mx);
      const float vlo = key_to_float(~mn_inv);
      // Bins linear in the value; subtraction, scaling and truncation never
      // reverse an order, so bin order is key order.
      const float range = vhi - vlo;
      const float scale = (range > 0.0f && range < __builtin_inff())
                              ? static_cast<float>(kPfBins) * 0.99999f / range : 0.0f;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int bv = min(kPfBins - 1, max(0, static_cast<int>((row.sv[e] - vlo) * scale)));
        bin[e] = ((vm >> e) & 1u) ? bv : kPfBins;
      }
      // A wave without a valid slot (a pool of fewer blocks than the
      // maximum leaves whole waves empty) adds nothing: its atomics would all
      // hit the spare bin one after another.
      if (__ballot(vm != 0u) != 0) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) atomicAdd(&sm.hist[bin[e]], 1u);
      }
      __syncthreads();
      uint32_t above;
      b1 = W::find_rank_bin(sm.hist, kPfBins, need, true, sm.wb, &above);
      const uint32_t ncand = sm.hist[b1];
      if (ncand <= static_cast<uint32_t>(kPfCap)) {
        if (tid == 0) sm.ccount = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const bool c = bin[e] == b1;
          if (__ballot(c) == 0) continue;   // wave-uniform
          const uint32_t slot = wave_append(c, &sm.ccount);
          if (c) {
            sm.ckey[slot] = float_to_key(row.sv[e]);
            sm.cid[slot] = s0 + e;
          }
        }
        __syncthreads();
        if (ncand <= static_cast<uint32_t>(kRankMax))
          resolve_by_rank<NT>(sm.ckey, sm.cid, ncand, need - above, sm.wb, &kstar, &istar);
        else
          W::resolve(ArrayCand{sm.ckey, sm.cid, ncand}, 0u, 32, need - above, sm.hist256, sm.wb,
                     &kstar, &istar);
      } else {
        // A huge threshold bin (scores barely spread): resolve over every slot.
#pragma unroll
        for (int e = 0; e < kPer; ++e)
          sm.keys[e * NT + tid] = ((vm >> e) & 1u) ? float_to_key(row.sv[e]) : 0u;
        __syncthreads();
        W::resolve(LdsKeys{sm.keys}, 0u, 32, need, sm.hist256, sm.wb, &kstar, &istar);
        mode = 2;
      }
    }
    // Selected slots: every valid one (mode 0); bin above b1, or the exact
    // (key, id) test inside bin b1 (mode 1); the exact test (mode 2).  The
    // exact test runs only where a wave holds a slot of bin b1.
    uint32_t selmask = 0;
    if (need > 0) {
      if (mode == 0) {
        selmask = vm;
      } else if (mode == 1) {
        uint32_t eq = 0;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          selmask |= bin[e] > b1 && bin[e] < kPfBins ? (1u << e) : 0u;
          eq |= bin[e] == b1 ? (1u << e) : 0u;
        }
        if (__ballot(eq != 0) != 0) {
#pragma unroll
          for (int e = 0; e < kPer; ++e)
            if (((eq >> e) & 1u) && selected(float_to_key(row.sv[e]), s0 + e, kstar, istar))
              selmask |= 1u << e;
        }
      } else {
#pragma unroll
        for (int e = 0; e < kPer; ++e)
          if (((vm >> e) & 1u) && selected(float_to_key(row.sv[e]), s0 + e, kstar, istar))
            selmask |= 1u << e;
      }
    }
    const uint32_t cnt = static_cast<uint32_t>(__popc(selmask));
    uint32_t total;
    uint32_t off = W::excl_scan_last(cnt, sm.wb, &total);
    if constexpr (kScore) {
      // Unrolled over the slots, so that each score stays in its register.
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if ((selmask >> e) & 1u) {
          if (off < need) emit(off, row.blk[e >> 3] * kBlock + (e & 7), row.sv[e]);
          ++off;
        }
      }
    } else {
      // Positions only: walk the set bits (slot e of block blk[e / 8]).
      uint32_t m = selmask;
      while (m != 0u) {
        const int e = __builtin_ctz(m);
        m &= m - 1u;
        int bk = row.blk[0];
#pragma unroll
        for (int u = 1; u < kBlocks; ++u) bk = (e >> 3) == u ? row.blk[u] : bk;
        if (off < need) emit(off, bk * kBlock + (e & 7), 0.0f);
        ++off;
      }
    }
    return need;
  }
};

}  // namespace csa2
