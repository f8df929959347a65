// Workgroup primitives of the exact Top-K selection (NT threads, wave64).
//
// Keys are order-preserving uint32 images of fp32 scores; a selection takes
// the first k items in (key descending, id ascending) order.  Radix selection
// finds the k-th key K* and, among items whose key equals K*, the largest id
// I* still taken; an item is selected iff
//     key > K*  or  (key == K* and id <= I*).
#pragma once
#include "csa2_device.h"

namespace csa2 {

constexpr int kHistBits = 12;                 // first-level bins: key bits [31:20]
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts
// (within rows of 16 lanes) and row broadcasts (across rows).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Maximum over the 64 lanes of a wave with DPP (quad swaps, mirrors, row
// broadcasts); lane 63 ends with the result, which is then read out.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, __builtin_amdgcn_update_dpp(v, v, 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = mx(v, __builtin_amdgcn_update_dpp(v, v, 0x4e, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = mx(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = mx(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));  // row_mirror
  v = mx(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = mx(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Appends `pred` lanes of the wave to a list through one atomic per wave;
// returns each predicated lane's slot.  Call with the whole wave.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return 0;
  const int lane = lane_id();
  const int leader = __ffsll(static_cast<long long>(m)) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, static_cast<uint32_t>(__popcll(m)));
  base = __shfl(base, leader, 64);
  return base + static_cast<uint32_t>(__popcll(m & ((1ull << lane) - 1ull)));
}

template <int NT>
struct Wg {
  static constexpr int kWaves = NT / 64;
  static constexpr int kScratch = 3 * kWaves + 4;   // uint32 words of scratch

  // Exclusive prefix sum in thread order; *total receives the sum.  Every
  // wave reads all wave totals and forms its own prefix (one barrier); the
  // second barrier leaves wb free for the next writer.
  __device__ static uint32_t excl_scan(uint32_t v, uint32_t* wb, uint32_t* total) {
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const uint32_t inc = wave_incl_scan_u32(v);
    if (lane == 63) wb[wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = wb[w];
      before += w < wave ? t : 0u;
      tot += t;
    }
    *total = tot;
    __syncthreads();
    return before + inc - v;
  }

  // As excl_scan with one barrier: every wave reads all wave totals and
  // forms its own prefix.  wb must not be written again before another
  // barrier (use it for the last scan of a kernel).
  __device__ static uint32_t excl_scan_last(uint32_t v, uint32_t* wb, uint32_t* total) {
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const uint32_t inc = wave_incl_scan_u32(v);
    if (lane == 63) wb[wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = wb[w];
      before += w < wave ? t : 0u;
      tot += t;
    }
    *total = tot;
    return before + inc - v;
  }

  __device__ static uint32_t sum(uint32_t v, uint32_t* wb) {
    uint32_t t;
    excl_scan(v, wb, &t);
    return t;
  }

  // Sum of a and maxima of b and c over the workgroup in one barrier
  // (wb needs 3 * kWaves words).
  __device__ static void reduce_sum_max_max(uint32_t& a, uint32_t& b, uint32_t& c,
                                            uint32_t* wb) {
    const int wave = threadIdx.x >> 6;
    const uint32_t sa = static_cast<uint32_t>(__builtin_amdgcn_readlane(
        static_cast<int>(wave_incl_scan_u32(a)), 63));
    const uint32_t mb = wave_max_u32(b), mc = wave_max_u32(c);
    if (lane_id() == 0) {
      wb[wave] = sa;
      wb[kWaves + wave] = mb;
      wb[2 * kWaves + wave] = mc;
    }
    __syncthreads();
    a = 0;
    b = 0;
    c = 0;
    for (int w = 0; w < kWaves; ++w) {
      a += wb[w];
      b = b > wb[kWaves + w] ? b : wb[kWaves + w];
      c = c > wb[2 * kWaves + w] ? c : wb[2 * kWaves + w];
    }
    __syncthreads();
  }

  __device__ static uint32_t reduce_max(uint32_t v, uint32_t* wb) {
    const int wave = threadIdx.x >> 6;
    v = wave_max_u32(v);
    if (lane_id() == 0) wb[wave] = v;
    __syncthreads();
    uint32_t m = 0;
    for (int w = 0; w < kWaves; ++w) m = m > wb[w] ? m : wb[w];
    __syncthreads();
    return m;
  }

  // Bin holding the item of 1-based rank `rank`, counting from the top bin
  // down (descending) or from bin 0 up; *before = items in bins passed first.
  // `hist` may be in LDS or global memory.  Needs 1 <= rank <= total.
  __device__ static int find_rank_bin(const uint32_t* hist, int nbins, uint32_t rank,
                                      bool descending, uint32_t* wb, uint32_t* before) {
    const int per = (nbins + NT - 1) / NT;
    const int t = threadIdx.x;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i) {
      const int idx = t * per + i;
      if (idx < nbins) s += hist[descending ? nbins - 1 - idx : idx];
    }
    uint32_t tot;
    uint32_t p = excl_scan(s, wb, &tot);
    if (p < rank && rank <= p + s) {
      for (int i = 0; i < per; ++i) {
        const int idx = t * per + i;
        const int bin = descending ? nbins - 1 - idx : idx;
        const uint32_t c = hist[bin];
        if (rank <= p + c) {
          wb[2 * kWaves + 1] = static_cast<uint32_t>(bin);
          wb[2 * kWaves + 2] = p;
          break;
        }
        p += c;
      }
    }
    __syncthreads();
    const int bin = static_cast<int>(wb[2 * kWaves + 1]);
    *before = wb[2 * kWaves + 2];
    __syncthreads();
    return bin;
  }

  // As find_rank_bin, with each thread's PER bins already in registers: v[i]
  // holds bin nbins - 1 - (t PER + i) (descending) or t PER + i.  Also
  // returns the found bin's count, so no bin is read from memory again, and
  // (if `total` is given) the sum of all bins modulo 2^32.  When rank exceeds
  // that sum the returned bin and counts are meaningless.
  template <int PER>
  __device__ static int find_rank_bin_regs(const uint32_t (&v)[PER], int nbins, uint32_t rank,
                                           bool descending, uint32_t* wb, uint32_t* before,
                                           uint32_t* count, uint32_t* total = nullptr) {
    const int t = threadIdx.x;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += v[i];
    uint32_t tot;
    uint32_t p = excl_scan(s, wb, &tot);
    if (total != nullptr) *total = tot;
    if (p < rank && rank <= p + s) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int idx = t * PER + i;
        if (rank <= p + v[i]) {
          wb[2 * kWaves + 1] = static_cast<uint32_t>(descending ? nbins - 1 - idx : idx);
          wb[2 * kWaves + 2] = p;
          wb[2 * kWaves + 3] = v[i];
          break;
        }
        p += v[i];
      }
    }
    __syncthreads();
    const int bin = static_cast<int>(wb[2 * kWaves + 1]);
    *before = wb[2 * kWaves + 2];
    *count = wb[2 * kWaves + 3];
    __syncthreads();
    return bin;
  }

  // Resolves the selection threshold among the items whose key bits above
  // `shift` equal `prefix` (prefix has zeros below `shift`): `rem` (>= 1) of
  // them are taken.  `cand` exposes n, key(i) and id(i) for i < n; other
  // items may be present and are ignored.  hist256 is 256 words of LDS.
  // Returns K* and I*.
  template <class Cand>
  __device__ static void resolve(const Cand& cand, uint32_t prefix, int shift, uint32_t rem,
                                 uint32_t* hist256, uint32_t* wb, uint32_t* kstar, int32_t* istar) {
    const uint32_t n = cand.n;
    uint32_t pmask = shift >= 32 ? 0u : (0xffffffffu << shift);
    uint32_t eq_count = 0xffffffffu;
    int lo = shift;
    while (lo > 0) {
      const int bits = lo >= 8 ? 8 : lo;
      lo -= bits;
      const uint32_t dmask = (1u << bits) - 1u;
      for (int i = threadIdx.x; i < 256; i += NT) hist256[i] = 0;
      __syncthreads();
      for (uint32_t c = threadIdx.x; c < n; c += NT) {
        const uint32_t k = cand.key(c);
        if ((k & pmask) == prefix) atomicAdd(&hist256[(k >> lo) & dmask], 1u);
      }
      __syncthreads();
      uint32_t before;
      const int d = find_rank_bin(hist256, 1 << bits, rem, true, wb, &before);
      eq_count = hist256[d];
      rem -= before;
      prefix |= static_cast<uint32_t>(d) << lo;
      pmask |= dmask << lo;
      __syncthreads();
    }
    *kstar = prefix;
    *istar = 0x7fffffff;
    if (eq_count == 0xffffffffu) {   // shift == 0: count the items equal to prefix
      uint32_t c = 0;
      for (uint32_t i = threadIdx.x; i < n; i += NT) c += cand.key(i) == prefix ? 1u : 0u;
      eq_count = sum(c, wb);
    }
    if (rem < eq_count) {
      uint32_t iprefix = 0, imask = 0;
      for (int lo2 = 24; lo2 > 0;) {
        lo2 -= 8;
        for (int i = threadIdx.x; i < 256; i += NT) hist256[i] = 0;
        __syncthreads();
        for (uint32_t c = threadIdx.x; c < n; c += NT) {
          const uint32_t id = static_cast<uint32_t>(cand.id(c));
          if (cand.key(c) == prefix && (id & imask) == iprefix)
            atomicAdd(&hist256[(id >> lo2) & 255u], 1u);
        }
        __syncthreads();
        uint32_t below;
        const int d = find_rank_bin(hist256, 256, rem, false, wb, &below);
        rem -= below;
        iprefix |= static_cast<uint32_t>(d) << lo2;
        imask |= 255u << lo2;
        __syncthreads();
      }
      *istar = static_cast<int32_t>(iprefix);
    }
  }
};

// Threshold among n <= NT candidates (LDS arrays) of which the first `rem`
// (>= 1) in (key descending, id ascending) order are taken: every candidate
// counts the candidates ordered before it; the one with rank rem - 1 gives
// K* and I*.  One pass and one barrier instead of radix passes.
template <int NT>
__device__ __forceinline__ void resolve_by_rank(const uint32_t* ckey, const int32_t* cid,
                                                uint32_t n, uint32_t rem, uint32_t* wb,
                                                uint32_t* kstar, int32_t* istar) {
  const int t = threadIdx.x;
  if (t < static_cast<int>(n)) {
    const uint32_t kc = ckey[t];
    const int32_t ic = cid[t];
    uint32_t rank = 0;
    for (uint32_t d = 0; d < n; ++d) {
      const uint32_t kd = ckey[d];
      rank += (kd > kc || (kd == kc && cid[d] < ic)) ? 1u : 0u;
    }
    if (rank == rem - 1) {
      wb[0] = kc;
      wb[1] = static_cast<uint32_t>(ic);
    }
  }
  __syncthreads();
  *kstar = wb[0];
  *istar = static_cast<int32_t>(wb[1]);
  __syncthreads();
}

// Candidate lists held as two arrays (LDS or global memory).
struct ArrayCand {
  const uint32_t* keys;
  const int32_t* ids;
  uint32_t n;
  __device__ uint32_t key(uint32_t i) const { return keys[i]; }
  __device__ int32_t id(uint32_t i) const { return ids[i]; }
};

__device__ __forceinline__ bool selected(uint32_t key, int32_t id, uint32_t kstar, int32_t istar) {
  return key > kstar || (key == kstar && id <= istar);
}

}  // namespace csa2
