// Two-level Top-K of the hierarchical sparse indexer.
//
// "DeepSeek-V4.1-Flash 架构详解", §3.2: the Full layer keeps at most 2,048
// blocks of 8 positions (a pool of at most 16,384 candidate positions) and
// its own Top-512; a Reindex layer re-scores only the pool with its own
// indexer query and takes a new Top-512.
//
// Every selection is exact (see select_common.h) and reports ascending ids.
// The selections of a decode step touch few query rows but many items per
// row, so they are spread over many workgroups:
//   block Top-K  (k_bt_hist, k_bt_filter, k_bt_final): a histogram of key
//     bits [31:20] built by all workgroups of a row; each workgroup then
//     writes the items above the threshold bin ("sure") and inside it
//     (candidates) to its own segment and adds the candidates to a second
//     histogram of bits [19:8]; one workgroup per row resolves the exact
//     threshold, marks the selection in an LDS bitmap over block ids and
//     compacts it in id order.
//   pool Top-K   (k_pool_score, k_pool_final): the pool positions are
//     re-scored on matrix cores (or stored scores are read); one workgroup
//     per row holds every slot's score in registers (16 per thread), finds
//     the threshold bin of a value-linear histogram, resolves it exactly,
//     and compacts the selection in slot order (= position order).
//   flat Top-K   (k_flat_select_reg, k_flat_select; prefill rows): one
//     workgroup per row; rows of up to 73,728 items are held in registers.
// Workgroups never wait on each other inside a kernel: kernel boundaries
// order the phases (a device-wide fence per workgroup would write back a
// whole L2).  The block Top-K histograms are accumulated with atomics, so
// they must start at zero: the final kernel clears them after reading, which
// leaves a workspace ready for the next call without a clearing kernel.  It
// also checks their totals (the visible block count, the candidate count);
// a workspace that did not start at zero fails that check, and the row is
// then selected exactly by radix passes over all its blocks.
#include <atomic>
#include <mutex>

#include "csa2_launch.h"
#include "index_core.h"
#include "pool_select.h"
#include "select_common.h"

namespace csa2 {
namespace {

// ---------------------------------------------------------------------------
// Block Top-K: k_bt_hist -> k_bt_filter -> k_bt_final.  Workgroups never
// wait on each other inside a kernel; the kernel boundaries order the phases.
constexpr int kBtThreads = 1024;
constexpr int kBtItems = 4096;          // block maxima per filter workgroup
constexpr int kBtMaxWgs = 128;          // filter workgroups per row (kBtMaxBlocks / kBtItems)
constexpr int kBtFinalCap = 8192;       // final-bucket candidates held in LDS
constexpr int kBtMaxBlocks = 1 << 19;   // LDS bitmap capacity (block ids)
constexpr int kBtWaves = kBtThreads / 64;
constexpr int kBtRankMax = 256;         // final buckets up to this size are resolved by ranks

struct BtWs {
  uint32_t* hist;    // [rows][kHistBins] bins of key bits [31:20]
  uint32_t* hist2;   // [rows][kHistBins] bins of key bits [19:8] inside the threshold bin
  uint32_t* wgcnt;   // [rows][kBtMaxWgs][2]: sure and candidate counts per filter workgroup
  int32_t* sure;     // [rows][nb_cap]: segment of workgroup w at [w * kBtItems, ...)
  uint32_t* ckey;    // [rows][nb_cap]
  int32_t* cid;      // [rows][nb_cap]
};

__device__ __forceinline__ uint32_t mid_bits(uint32_t key) { return (key >> 8) & 0xfffu; }

// Loads of row items i < n are written as row[min(i, n - 1)] followed by a
// select, not as a conditional load: a conditional load becomes a branch
// with its own wait, and a thread's loads would then run one at a time.

__global__ __launch_bounds__(kBtThreads) void k_bt_hist(const float* __restrict__ bm,
                                                        const int32_t* __restrict__ vis_len,
                                                        int N_cap, int k, BtWs ws) {
  __shared__ uint32_t h[kHistBins];
  const int r = blockIdx.y;
  const int nb_cap = (N_cap + 7) >> 3;
  const int i0 = blockIdx.x * kBtItems;
  // The row items are loaded (clamped to the row's capacity) together with
  // the visible length, not after it.
  const float* row = bm + static_cast<size_t>(r) * nb_cap;
  float v[kBtItems / kBtThreads];
#pragma unroll
  for (int j = 0; j < kBtItems / kBtThreads; ++j)
    v[j] = row[min(i0 + static_cast<int>(threadIdx.x) + j * kBtThreads, nb_cap - 1)];
  const int n = (min(max(vis_len[r], 0), N_cap) + 7) >> 3;
  if (n <= k || i0 >= n) return;
  for (int i = threadIdx.x; i < kHistBins; i += kBtThreads) h[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBtItems / kBtThreads; ++j) {
    const int i = i0 + threadIdx.x + j * kBtThreads;
    if (i < n) atomicAdd(&h[float_to_key(v[j]) >> kHistShift], 1u);
  }
  __syncthreads();
  uint32_t* gh = ws.hist + static_cast<size_t>(r) * kHistBins;
  for (int b = threadIdx.x; b < kHistBins; b += kBtThreads)
    if (h[b]) atomicAdd(&gh[b], h[b]);
}

__global__ __launch_bounds__(kBtThreads) void k_bt_filter(const float* __restrict__ bm,
                                                          const int32_t* __restrict__ vis_len,
                                                          int N_cap, int k, BtWs ws) {
  __shared__ uint32_t h2[kHistBins];
  __shared__ uint32_t wb[Wg<kBtThreads>::kScratch];
  __shared__ uint32_t cnt[2];
  using W = Wg<kBtThreads>;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int nb_cap = (N_cap + 7) >> 3;
  const int i0 = blockIdx.x * kBtItems;
  // The row items (clamped to the row's capacity), the histogram and the
  // visible length are loaded in one batch.
  const float* row = bm + static_cast<size_t>(r) * nb_cap;
  float v[kBtItems / kBtThreads];
#pragma unroll
  for (int j = 0; j < kBtItems / kBtThreads; ++j)
    v[j] = row[min(i0 + tid + j * kBtThreads, nb_cap - 1)];
  const uint32_t* gh = ws.hist + static_cast<size_t>(r) * kHistBins;
  constexpr int kPerBin = kHistBins / kBtThreads;
  uint32_t h1[kPerBin];
#pragma unroll
  for (int i = 0; i < kPerBin; ++i) h1[i] = gh[kHistBins - 1 - (tid * kPerBin + i)];
  const int n = (min(max(vis_len[r], 0), N_cap) + 7) >> 3;
  if (n <= k || i0 >= n) return;
  uint32_t above, n1;
  const int b1 =
      W::find_rank_bin_regs(h1, kHistBins, static_cast<uint32_t>(k), true, wb, &above, &n1);
  for (int i = tid; i < kHistBins; i += kBtThreads) h2[i] = 0;
  if (tid < 2) cnt[tid] = 0;
  __syncthreads();
  const size_t seg = static_cast<size_t>(r) * nb_cap + i0;
#pragma unroll
  for (int j = 0; j < kBtItems / kBtThreads; ++j) {
    const int i = i0 + tid + j * kBtThreads;
    const uint32_t key = float_to_key(v[j]);
    const int bin = static_cast<int>(key >> kHistShift);
    const bool is_sure = i < n && bin > b1;
    const bool is_cand = i < n && bin == b1;
    const uint32_t s = wave_append(is_sure, &cnt[0]);
    if (is_sure) ws.sure[seg + s] = i;
    const uint32_t c = wave_append(is_cand, &cnt[1]);
    if (is_cand) {
      ws.ckey[seg + c] = key;
      ws.cid[seg + c] = i;
      atomicAdd(&h2[mid_bits(key)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh2 = ws.hist2 + static_cast<size_t>(r) * kHistBins;
  for (int b = tid; b < kHistBins; b += kBtThreads)
    if (h2[b]) atomicAdd(&gh2[b], h2[b]);
  if (tid < 2) ws.wgcnt[(static_cast<size_t>(r) * kBtMaxWgs + blockIdx.x) * 2 + tid] = cnt[tid];
}

// One workgroup per row: second-level bin b2 of bits [19:8] inside b1, the
// exact threshold inside bucket (b1, b2), an LDS bitmap of the selection and
// its compaction in block-id order.
__global__ __launch_bounds__(kBtThreads) void k_bt_final(const float* __restrict__ bm,
                                                         const int32_t* __restrict__ vis_len,
                                                         int N_cap, int k, BtWs ws,
                                                         int32_t* __restrict__ out) {
  __shared__ uint32_t fkey[kBtFinalCap];
  __shared__ int32_t fid[kBtFinalCap];
  __shared__ uint32_t bitmap[kBtMaxBlocks / 32];
  __shared__ uint32_t off_c[kBtMaxWgs + 1];
  __shared__ uint32_t hist256[256];
  __shared__ uint32_t wb[Wg<kBtThreads>::kScratch];
  __shared__ uint32_t fcount;
  __shared__ uint32_t res[8];   // b1, above, n1, b2, above2, n2, totals of h1 and h2
  using W = Wg<kBtThreads>;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int nb_cap = (N_cap + 7) >> 3;
  // Both histograms, the filter workgroups' counts and the visible length
  // are loaded in one batch (one memory latency); the histograms are
  // searched in registers.
  uint32_t* gh = ws.hist + static_cast<size_t>(r) * kHistBins;
  uint32_t* gh2 = ws.hist2 + static_cast<size_t>(r) * kHistBins;
  constexpr int kPerBin = kHistBins / kBtThreads;
  static_assert(kHistBins % kBtThreads == 0, "whole bins per thread");
  static_assert(kBtMaxWgs == 128, "two filter workgroups per lane of the first wave");
  uint32_t h1[kPerBin], h2[kPerBin];
#pragma unroll
  for (int i = 0; i < kPerBin; ++i) {
    h1[i] = gh[kHistBins - 1 - (tid * kPerBin + i)];
    h2[i] = gh2[kHistBins - 1 - (tid * kPerBin + i)];
  }
  const uint32_t* wc = ws.wgcnt + static_cast<size_t>(r) * kBtMaxWgs * 2;
  const int wl = tid & 63;
  const u32x2 wca = *reinterpret_cast<const u32x2*>(wc + 2 * wl);
  const u32x2 wcb = *reinterpret_cast<const u32x2*>(wc + 2 * (wl + 64));
  const int n = (min(max(vis_len[r], 0), N_cap) + 7) >> 3;
  int32_t* orow = out + static_cast<size_t>(r) * k;
  if (n <= k) {  // every visible block is kept
    for (int i = tid; i < k; i += kBtThreads) orow[i] = i < n ? i : -1;
    return;
  }
  const uint32_t need = static_cast<uint32_t>(k);
  // Threshold bins b1 (rank need in h1) and b2 (rank need - above(b1) in
  // h2), counting from the top bin down, with one prefix sum of both
  // histograms' per-thread totals: three barriers.
  uint32_t s1 = 0, s2 = 0;
#pragma unroll
  for (int i = 0; i < kPerBin; ++i) {
    s1 += h1[i];
    s2 += h2[i];
  }
  const int wave = tid >> 6;
  {
    const uint32_t i1 = wave_incl_scan_u32(s1), i2 = wave_incl_scan_u32(s2);
    if (wl == 63) {
      wb[wave] = i1;
      wb[kBtWaves + wave] = i2;
    }
    __syncthreads();
    uint32_t p1 = i1 - s1, p2 = i2 - s2, t1 = 0, t2 = 0;
#pragma unroll
    for (int w = 0; w < kBtWaves; ++w) {
      const uint32_t a = wb[w], b = wb[kBtWaves + w];
      p1 += w < wave ? a : 0u;
      p2 += w < wave ? b : 0u;
      t1 += a;
      t2 += b;
    }
    if (p1 < need && need <= p1 + s1) {
      uint32_t q = p1;
#pragma unroll
      for (int i = 0; i < kPerBin; ++i) {
        if (need <= q + h1[i]) {
          res[0] = static_cast<uint32_t>(kHistBins - 1 - (tid * kPerBin + i));
          res[1] = q;
          res[2] = h1[i];
          break;
        }
        q += h1[i];
      }
    }
    if (tid == 0) {
      res[6] = t1;
      res[7] = t2;
    }
    __syncthreads();
    const uint32_t rem = need - res[1];
    if (p2 < rem && rem <= p2 + s2) {
      uint32_t q = p2;
#pragma unroll
      for (int i = 0; i < kPerBin; ++i) {
        if (rem <= q + h2[i]) {
          res[3] = static_cast<uint32_t>(kHistBins - 1 - (tid * kPerBin + i));
          res[4] = q;
          res[5] = h2[i];
          break;
        }
        q += h2[i];
      }
    }
    __syncthreads();
  }
  // With a dirty workspace the totals differ from the counts (checked below)
  // and these values are not used.
  const int b1 = static_cast<int>(res[0]);
  const uint32_t above = res[1], tot1 = res[6], tot2 = res[7];
  const uint32_t rem1 = need - above;
  const int b2 = static_cast<int>(res[3]);
  const uint32_t above2 = res[4], n2 = res[5];
  const uint32_t rem2 = rem1 - above2;
  const int nwg = (n + kBtItems - 1) / kBtItems;
  if (tid == 0) fcount = 0;
  const int nwords = (n + 31) >> 5;
  for (int w = tid; w < nwords; w += kBtThreads) bitmap[w] = 0u;
  // Candidate total over the segments: every wave holds every segment's
  // counts (lane l: segments l and l + 64) and sums them itself.
  uint32_t cc = (wl < nwg ? wca.y : 0u) + (wl + 64 < nwg ? wcb.y : 0u);
  const uint32_t n_cand = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan_u32(cc)), 63));
  __syncthreads();
  // The histograms were complete and started from zero exactly when their
  // totals are the visible block count and the candidate count.  Otherwise
  // (a workspace not left zeroed by a previous call) the threshold is
  // resolved exactly over the whole row instead.
  const bool clean = tot1 == static_cast<uint32_t>(n) && tot2 == n_cand;
  if (clean) {
    // The segments' items are cut into chunks of 64 (a segment has
    // ceil(max(sure, candidates) / 64) chunks); wave w takes chunks w, w + 16,
    // ... and, per chunk, marks its sure items and sorts its candidates by
    // bits [19:8] against b2 (above: marked; equal: kept in LDS for the exact
    // resolution).  A chunk's segment is found from the chunk counts' prefix
    // sums, which every wave forms itself (lane l: segments l and l + 64), by
    // one ballot.  Two chunks are loaded before either is worked on; loads
    // past a segment's count read its first item and are ignored.
    struct Chunk {
      int sid;
      uint32_t ck;
      int ci;
    };
    auto load = [&](int sg, uint32_t i0, uint32_t ns, uint32_t nc) {
      const size_t base = static_cast<size_t>(r) * nb_cap + static_cast<size_t>(sg) * kBtItems;
      const uint32_t i = i0 + static_cast<uint32_t>(wl);
      Chunk c;
      c.sid = ws.sure[base + (i < ns ? i : 0u)];
      c.ck = ws.ckey[base + (i < nc ? i : 0u)];
      c.ci = ws.cid[base + (i < nc ? i : 0u)];
      return c;
    };
    auto work = [&](const Chunk& c, uint32_t i0, uint32_t ns, uint32_t nc) {
      const uint32_t i = i0 + static_cast<uint32_t>(wl);
      if (i < ns) atomicOr(&bitmap[c.sid >> 5], 1u << (c.sid & 31));
      const bool in = i < nc;
      const int mb = static_cast<int>(mid_bits(c.ck));
      if (in && mb > b2) atomicOr(&bitmap[c.ci >> 5], 1u << (c.ci & 31));
      const bool fin = in && mb == b2;
      const uint32_t slot = wave_append(fin, &fcount);
      if (fin && slot < static_cast<uint32_t>(kBtFinalCap)) {
        fkey[slot] = c.ck;
        fid[slot] = c.ci;
      }
    };
    auto chunks = [](u32x2 c) { return (max(c.x, c.y) + 63u) >> 6; };
    const uint32_t cha = wl < nwg ? chunks(wca) : 0u, chb = wl + 64 < nwg ? chunks(wcb) : 0u;
    const uint32_t pa = wave_incl_scan_u32(cha);
    const uint32_t tot_a = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pa), 63));
    const uint32_t pb = wave_incl_scan_u32(chb) + tot_a;
    const uint32_t n_chunks =
        static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pb), 63));
    // Chunk c (wave-uniform) -> its segment, first item and the segment's counts.
    auto locate = [&](uint32_t c, int* sg, uint32_t* i0, uint32_t* ns, uint32_t* nc) {
      const uint64_t ma = __ballot(pa > c);
      uint32_t before;
      u32x2 cnt;
      if (ma != 0) {
        const int s0 = __ffsll(static_cast<long long>(ma)) - 1;
        before = s0 ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pa), s0 - 1))
                    : 0u;
        *sg = s0;
        cnt = wca;
      } else {
        const int s0 = __ffsll(static_cast<long long>(__ballot(pb > c))) - 1;
        before = s0 ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pb), s0 - 1))
                    : tot_a;
        *sg = 64 + s0;
        cnt = wcb;
      }
      const int ln = *sg & 63;
      *ns = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cnt.x), ln));
      *nc = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(cnt.y), ln));
      *i0 = (c - before) * 64u;
    };
    for (uint32_t c0 = static_cast<uint32_t>(wave); c0 < n_chunks; c0 += 2 * kBtWaves) {
      const uint32_t c1 = c0 + kBtWaves;
      int sg0, sg1 = 0;
      uint32_t i00, ns0, nc0, i01 = 0, ns1 = 0, nc1 = 0;
      locate(c0, &sg0, &i00, &ns0, &nc0);
      if (c1 < n_chunks) locate(c1, &sg1, &i01, &ns1, &nc1);
      const Chunk a = load(sg0, i00, ns0, nc0);
      const Chunk b = load(c1 < n_chunks ? sg1 : sg0, i01, ns1, nc1);
      work(a, i00, ns0, nc0);
      work(b, i01, ns1, nc1);
    }
    __syncthreads();
    const uint32_t prefix =
        (static_cast<uint32_t>(b1) << kHistShift) | (static_cast<uint32_t>(b2) << 8);
    uint32_t kstar;
    int32_t istar;
    if (n2 <= static_cast<uint32_t>(kBtFinalCap)) {
      if (n2 <= static_cast<uint32_t>(kBtRankMax))
        resolve_by_rank<kBtThreads>(fkey, fid, n2, rem2, wb, &kstar, &istar);
      else
        W::resolve(ArrayCand{fkey, fid, n2}, prefix, 8, rem2, hist256, wb, &kstar, &istar);
      for (uint32_t c = tid; c < n2; c += kBtThreads)
        if (selected(fkey[c], fid[c], kstar, istar))
          atomicOr(&bitmap[fid[c] >> 5], 1u << (fid[c] & 31));
    } else {
      // Degenerate input (a huge bucket of equal high bits): resolve by
      // re-reading the candidate segments, located through their prefix
      // offsets.
      if (tid < 64) {
        uint32_t pc = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int w = 64 * half + tid;
          const uint32_t c1 = w < nwg ? (half ? wcb.y : wca.y) : 0u;
          const uint32_t ic = wave_incl_scan_u32(c1);
          off_c[w + 1] = pc + ic;
          pc += __shfl(ic, 63, 64);
        }
        if (tid == 0) off_c[0] = 0;
      }
      __syncthreads();
      struct SegCand {
        const uint32_t* ckey;
        const int32_t* cid;
        const uint32_t* off;
        int nwg;
        size_t base;
        uint32_t n;
        __device__ size_t at(uint32_t g) const {
          int lo = 0, hi = nwg;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= g) lo = mid; else hi = mid;
          }
          return base + static_cast<size_t>(lo) * kBtItems + (g - off[lo]);
        }
        __device__ uint32_t key(uint32_t g) const { return ckey[at(g)]; }
        __device__ int32_t id(uint32_t g) const { return cid[at(g)]; }
      } sc{ws.ckey, ws.cid, off_c, nwg, static_cast<size_t>(r) * nb_cap, n_cand};
      W::resolve(sc, prefix, 8, rem2, hist256, wb, &kstar, &istar);
      for (uint32_t g = tid; g < n_cand; g += kBtThreads) {
        const uint32_t key = sc.key(g);
        const int id = sc.id(g);
        if ((key & 0xffffff00u) == prefix && selected(key, id, kstar, istar))
          atomicOr(&bitmap[id >> 5], 1u << (id & 31));
      }
    }
  } else {
    struct RowCand {
      const float* row;
      uint32_t n;
      __device__ uint32_t key(uint32_t i) const { return float_to_key(row[i]); }
      __device__ int32_t id(uint32_t i) const { return static_cast<int32_t>(i); }
    } rc{bm + static_cast<size_t>(r) * nb_cap, static_cast<uint32_t>(n)};
    uint32_t kstar;
    int32_t istar;
    W::resolve(rc, 0u, 32, need, hist256, wb, &kstar, &istar);
    for (uint32_t i = tid; i < rc.n; i += kBtThreads)
      if (selected(rc.key(i), static_cast<int32_t>(i), kstar, istar))
        atomicOr(&bitmap[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  // Compaction in block-id order.  In each pass of 4 x 1024 bitmap words,
  // thread t takes words t, t + 1024, t + 2048 and t + 3072, so a run of
  // selected blocks is spread over many threads; the four columns' per-thread
  // counts are prefix-summed together (two 16-bit counts per word).
  uint32_t written = 0;
  for (int base = 0; base < nwords; base += 4 * kBtThreads) {
    uint32_t wv[4], c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = base + tid + j * kBtThreads;
      wv[j] = w < nwords ? bitmap[w] : 0u;
      c[j] = static_cast<uint32_t>(__popc(wv[j]));
    }
    const uint32_t a = c[0] | (c[1] << 16), b = c[2] | (c[3] << 16);
    const uint32_t ia = wave_incl_scan_u32(a), ib = wave_incl_scan_u32(b);
    if (wl == 63) {
      wb[wave] = ia;
      wb[kBtWaves + wave] = ib;
    }
    __syncthreads();
    uint32_t pa = ia - a, pb = ib - b, ta = 0, tb = 0;
#pragma unroll
    for (int w = 0; w < kBtWaves; ++w) {
      const uint32_t x = wb[w], y = wb[kBtWaves + w];
      pa += w < wave ? x : 0u;
      pb += w < wave ? y : 0u;
      ta += x;
      tb += y;
    }
    if (base + 4 * kBtThreads < nwords) __syncthreads();   // wb is written again
    const uint32_t col[4] = {ta & 0xffffu, ta >> 16, tb & 0xffffu, tb >> 16};
    uint32_t off = written;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t o = off + ((j & 1) ? ((j < 2 ? pa : pb) >> 16) : ((j < 2 ? pa : pb) & 0xffffu));
      uint32_t bits = wv[j];
      const int w32 = (base + tid + j * kBtThreads) * 32;
      while (bits) {
        const int bb = __ffs(static_cast<int>(bits)) - 1;
        bits &= bits - 1u;
        if (o < need) orow[o] = w32 + bb;
        ++o;
      }
      off += col[j];
    }
    written = off;
  }
  for (int i = static_cast<int>(min(written, need)) + tid; i < k; i += kBtThreads) orow[i] = -1;
  // Both histograms are left zeroed for the next call: each thread clears
  // the four bins of each that it read, with one 16-byte store, after the
  // output (stores issued earlier would delay the loads behind them).
  static_assert(kPerBin == 4, "one 16-byte store per histogram");
  *reinterpret_cast<u32x4*>(gh + kHistBins - kPerBin * (tid + 1)) = u32x4{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4*>(gh2 + kHistBins - kPerBin * (tid + 1)) = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Pool Top-K: k_pool_score re-scores the pool positions (Reindex, or Full
// without stored scores) into a pool-score array; k_pool_final (one
// workgroup per row) holds every slot's score in registers and selects.
constexpr int kPsThreads = 1024;                // selection workgroup
constexpr int kPscThreads = 256;                // scoring workgroup: 4 waves x 2 tiles
constexpr int kPscWaves = kPscThreads / 64;
constexpr int kPsSlots = 2 * 32 * kPscWaves;    // slots per scoring workgroup
constexpr int kPsBlocks = kPsSlots / kBlock;

struct PoolArgs {
  const float* scores;       // stored scores [rows, N_cap], or null when re-scored
  const uint16_t* q_idx;
  const float* w_idx;
  const uint8_t* k_idx;
  Pages pg;                  // indexer-K page table (pg.bt == nullptr: contiguous)
  const int32_t* pool;       // [rows, kb]
  const int32_t* vis_len;
  int kb, n_q, N_cap, top_k;
  float* ps;                 // [rows][kb * 8] re-scored pool scores
  int32_t* out;              // [rows, top_k]
  float* out_key;            // [rows, top_k] or null
};

__device__ __forceinline__ bool pool_slot_valid(const int32_t* prow, int i, int nb_cap, int vis) {
  const int blk = prow[i >> 3];
  return blk >= 0 && blk < nb_cap && blk * kBlock + (i & 7) < vis;
}

template <int KD>
__global__ __launch_bounds__(kPscThreads) void k_pool_score(PoolArgs a) {
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int vis = min(max(a.vis_len[r], 0), a.N_cap);
  const int nb_cap = (a.N_cap + 7) >> 3;
  const int nslots = a.kb * kBlock;
  const int32_t* prow = a.pool + static_cast<size_t>(r) * a.kb;
  float* ps = a.ps + static_cast<size_t>(r) * nslots;
  // The query: for a bf16 query its loads go first; an FP4 query is loaded
  // and quantised after the key loads are issued, so that the quantisation
  // overlaps the dependent id -> key loads.
  QueryOp<KD> qa;
  float wr[16];
  auto query = [&]() {
    load_query<KD>(qa, a.q_idx + static_cast<size_t>(r) * kIdxHeads * kIdxDim, col, half);
    load_weights(wr, a.w_idx + static_cast<size_t>(r) * kIdxHeads, half);
  };
  if constexpr (KD != kKdFp4Q) query();
  const int b = r / a.n_q;
  // Tiles of 32 slots (4 pool blocks each); wave w takes tiles w and w + 4.
  const int slot0 = blockIdx.x * kPsSlots;
  KeyTile<KD> kt[2];
  constexpr int kRow = KeyFmt<KD>::kRowBytes;
  // MXFP4: the scales of all rows follow the rows of E2M1 in the buffer.
  const size_t total_rows = a.pg.bt != nullptr
                                ? (static_cast<size_t>(a.pg.num_pages) << a.pg.log2p)
                                : static_cast<size_t>(gridDim.y / a.n_q) * a.N_cap;
  const uint8_t* scales = a.k_idx + total_rows * kRow;
  bool valid[2];
  int slot[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    slot[u] = slot0 + 32 * (wave + kPscWaves * u) + col;
    valid[u] = slot[u] < nslots && pool_slot_valid(prow, slot[u], nb_cap, vis);
    const int pos = valid[u] ? prow[slot[u] >> 3] * kBlock + (col & 7) : 0;
    bool mapped;
    const size_t row = pool_row(a.pg, b, a.N_cap, pos, mapped);
    load_key_half<KD>(kt[u], a.k_idx + row * kRow, half, scales + row * 4);
  }
  if constexpr (KD == kKdFp4Q) query();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float s = head_sum(key_tile_dot<KD>(qa, kt[u]), wr);
    if (half == 0 && slot[u] < nslots) ps[slot[u]] = s;
  }
}

// One workgroup per row: the selection of pool_select.h over the row's
// slots (16 per thread), writing the positions (and scores) in slot order.
__global__ __launch_bounds__(kPsThreads) void k_pool_final(PoolArgs a) {
  using PS = PoolSel<kPsThreads>;
  __shared__ typename PS::Scratch sm;
  const int r = blockIdx.x;
  const int vis = min(max(a.vis_len[r], 0), a.N_cap);
  const int nb_cap = (a.N_cap + 7) >> 3;
  const int nslots = a.kb * kBlock;
  typename PS::Row row;
  PS::load(row, a.pool + static_cast<size_t>(r) * a.kb, a.kb,
           a.scores ? a.scores + static_cast<size_t>(r) * a.N_cap : nullptr,
           a.ps + static_cast<size_t>(r) * nslots, vis);
  int32_t* orow = a.out + static_cast<size_t>(r) * a.top_k;
  float* krow = a.out_key ? a.out_key + static_cast<size_t>(r) * a.top_k : nullptr;
  uint32_t need;
  if (krow == nullptr) {
    need = PS::template select<false>(row, nb_cap, vis, a.top_k, sm,
                                      [&](uint32_t off, int pos, float) { orow[off] = pos; });
  } else {
    need = PS::template select<true>(row, nb_cap, vis, a.top_k, sm,
                                     [&](uint32_t off, int pos, float v) {
                                       orow[off] = pos;
                                       krow[off] = v;
                                     });
  }
  for (int i = static_cast<int>(need) + threadIdx.x; i < a.top_k; i += kPsThreads) {
    orow[i] = -1;
    if (krow) krow[i] = -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// Flat Top-K of prefill rows: one workgroup per row over [0, vis).
constexpr int kFsThreads = 1024;
constexpr int kFsCandCap = 8192;
constexpr int kFsPer = 8;

// One row of scores, fp32 or bf16 bit patterns (BF16); at(i) is the score
// as a float (a bf16 value converts exactly).
template <bool BF16>
struct ScoreRow {
  const void* p;
  __device__ float at(int i) const {
    if constexpr (BF16)
      return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
    else
      return static_cast<const float*>(p)[i];
  }
};
template <bool BF16>
__device__ __forceinline__ ScoreRow<BF16> score_row(const void* scores, int r, int N_cap) {
  const size_t off = static_cast<size_t>(r) * N_cap * (BF16 ? 2 : 4);
  return ScoreRow<BF16>{static_cast<const uint8_t*>(scores) + off};
}

template <bool BF16>
struct FlatCand {
  ScoreRow<BF16> s;
  uint32_t n;
  __device__ uint32_t key(uint32_t i) const { return float_to_key(s.at(static_cast<int>(i))); }
  __device__ int32_t id(uint32_t i) const { return static_cast<int32_t>(i); }
};

// Gathers the items of the row whose key has `prefix` above `shift` into LDS.
template <bool BF16>
__device__ void flat_gather(ScoreRow<BF16> row, int n, uint32_t prefix, int shift, uint32_t* ckey,
                            int32_t* cid, uint32_t* counter) {
  const uint32_t pmask = 0xffffffffu << shift;
  for (int base = 0; base < n; base += kFsThreads * kFsPer) {
    float v[kFsPer];
#pragma unroll
    for (int e = 0; e < kFsPer; ++e) {
      const int i = base + e * kFsThreads + threadIdx.x;
      v[e] = row.at(min(i, n - 1));
      if (i >= n) v[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < kFsPer; ++e) {
      const int i = base + e * kFsThreads + threadIdx.x;
      const uint32_t key = float_to_key(v[e]);
      const bool c = i < n && (key & pmask) == prefix;
      const uint32_t s = wave_append(c, counter);
      if (c && s < static_cast<uint32_t>(kFsCandCap)) {
        ckey[s] = key;
        cid[s] = i;
      }
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kFsThreads) void k_flat_select(const void* __restrict__ scores,
                                                            const int32_t* __restrict__ vis_len,
                                                            int N_cap, int k,
                                                            int32_t* __restrict__ out,
                                                            float* __restrict__ out_key) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t ckey_l[kFsCandCap];
  __shared__ int32_t cid_l[kFsCandCap];
  __shared__ uint32_t hist256[256];
  __shared__ uint32_t wb[Wg<kFsThreads>::kScratch];
  __shared__ uint32_t ccount;
  using W = Wg<kFsThreads>;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = min(max(vis_len[r], 0), N_cap);
  const ScoreRow<BF16> row = score_row<BF16>(scores, r, N_cap);
  const uint32_t need = min(static_cast<uint32_t>(k), static_cast<uint32_t>(n));
  uint32_t kstar = 0;
  int32_t istar = 0x7fffffff;
  if (need > 0 && need < static_cast<uint32_t>(n)) {
    // Level 1: bins of key bits [31:20].
    for (int i = tid; i < kHistBins; i += kFsThreads) h[i] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += kFsThreads * kFsPer) {
      float v[kFsPer];
#pragma unroll
      for (int e = 0; e < kFsPer; ++e) {
        const int i = base + e * kFsThreads + tid;
        v[e] = row.at(min(i, n - 1));
        if (i >= n) v[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < kFsPer; ++e)
        if (base + e * kFsThreads + tid < n) atomicAdd(&h[float_to_key(v[e]) >> kHistShift], 1u);
    }
    __syncthreads();
    uint32_t above;
    const int b1 = W::find_rank_bin(h, kHistBins, need, true, wb, &above);
    uint32_t rem = need - above;
    uint32_t prefix = static_cast<uint32_t>(b1) << kHistShift;
    int shift = kHistShift;
    uint32_t ncand = h[b1];
    if (ncand > static_cast<uint32_t>(kFsCandCap)) {
      // Level 2: bins of key bits [19:8] inside b1.
      __syncthreads();
      for (int i = tid; i < kHistBins; i += kFsThreads) h[i] = 0;
      __syncthreads();
      for (int base = 0; base < n; base += kFsThreads * kFsPer) {
        float v[kFsPer];
#pragma unroll
        for (int e = 0; e < kFsPer; ++e) {
          const int i = base + e * kFsThreads + tid;
          v[e] = row.at(min(i, n - 1));
          if (i >= n) v[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < kFsPer; ++e) {
          const uint32_t key = float_to_key(v[e]);
          if (base + e * kFsThreads + tid < n && (key >> kHistShift) == static_cast<uint32_t>(b1))
            atomicAdd(&h[mid_bits(key)], 1u);
        }
      }
      __syncthreads();
      uint32_t above2;
      const int b2 = W::find_rank_bin(h, kHistBins, rem, true, wb, &above2);
      rem -= above2;
      prefix |= static_cast<uint32_t>(b2) << 8;
      shift = 8;
      ncand = h[b2];
    }
    if (tid == 0) ccount = 0;
    __syncthreads();
    if (ncand <= static_cast<uint32_t>(kFsCandCap)) {
      flat_gather(row, n, prefix, shift, ckey_l, cid_l, &ccount);
      __syncthreads();
      W::resolve(ArrayCand{ckey_l, cid_l, ncand}, prefix, shift, rem, hist256, wb, &kstar, &istar);
    } else {
      W::resolve(FlatCand<BF16>{row, static_cast<uint32_t>(n)}, prefix, shift, rem, hist256, wb,
                 &kstar, &istar);
    }
  }
  // Ordered compaction: rounds of kFsThreads * kFsPer items, thread-contiguous.
  int32_t* orow = out + static_cast<size_t>(r) * k;
  float* krow = out_key ? out_key + static_cast<size_t>(r) * k : nullptr;
  uint32_t written = 0;
  for (int base = 0; base < n && need > 0; base += kFsThreads * kFsPer) {
    float v[kFsPer];
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < kFsPer; ++e) {
      const int i = base + tid * kFsPer + e;
      v[e] = row.at(min(i, n - 1));
      if (i >= n) v[e] = -__builtin_inff();
      c += (i < n && selected(float_to_key(v[e]), i, kstar, istar)) ? 1u : 0u;
    }
    uint32_t round_total;
    uint32_t off = written + W::excl_scan(c, wb, &round_total);
#pragma unroll
    for (int e = 0; e < kFsPer; ++e) {
      const int i = base + tid * kFsPer + e;
      if (i < n && selected(float_to_key(v[e]), i, kstar, istar)) {
        if (off < need) {
          orow[off] = i;
          if (krow) krow[off] = v[e];
        }
        ++off;
      }
    }
    written += round_total;
  }
  for (int i = static_cast<int>(min(written, need)) + tid; i < k; i += kFsThreads) {
    orow[i] = -1;
    if (krow) krow[i] = -__builtin_inff();
  }
}

// Flat Top-K of rows that fit in registers (n <= kFrItems = 73,728): the
// row is read from memory once into registers, then
//   1. the row's value range [vmin, vmax] is found and the items are
//      counted into 2048 bins spread evenly over it (bin order is key order,
//      and the bins spread the scores, so the LDS atomics rarely collide);
//   2. the bin holding the k-th item is located; its items (usually a
//      handful) are copied to LDS and resolved exactly (key radix, then id);
//   3. the selected items are marked in an LDS bitmap over ids and written
//      in id order after one prefix sum over the bitmap words.
// A threshold bin too large for LDS is resolved over the whole row instead.
// fp32 scores: 1024 threads, item e * 1024 + t is thread t's key e (72
// keys).  bf16 scores: the keys need only 16 bits, so two share a register
// and a workgroup of 512 threads holds 144 per thread in half the registers
// of the fp32 form, which lets two workgroups (two rows) share a compute
// unit; thread t's keys 2 u and 2 u + 1 are items 2 (512 u + t) and
// 2 (512 u + t) + 1, read with one 4-byte load.
constexpr int kFrItems = 73728;
constexpr int kRawBufferFlags = 0x00020000;   // dword 3 of a raw (untyped) buffer descriptor
constexpr int kFrBins = 2048;
constexpr int kFrCap = 4096;
constexpr int kFrWords = kFrItems / 32;

template <bool BF16>
struct FrShape {
  static constexpr int kThreads = BF16 ? 512 : 1024;
  static constexpr int kPer = kFrItems / kThreads;     // keys per thread
  static constexpr int kRegs = BF16 ? kPer / 2 : kPer; // registers holding them
  static constexpr int kWordsPerThread = (kFrWords + kThreads - 1) / kThreads;
  // Item held as key e by thread t.
  __device__ static int item(int e, int t) {
    return BF16 ? 2 * (kThreads * (e >> 1) + t) + (e & 1) : e * kThreads + t;
  }
};

template <bool BF16>
__global__ __launch_bounds__(FrShape<BF16>::kThreads, 4) void k_flat_select_reg(
    const void* __restrict__ scores, const int32_t* __restrict__ vis_len, int N_cap, int k,
    int32_t* __restrict__ out, float* __restrict__ out_key) {
  using S = FrShape<BF16>;
  constexpr int NT = S::kThreads;
  constexpr int PER = S::kPer;
  __shared__ uint32_t hist[kFrBins];
  __shared__ uint32_t ckey_l[kFrCap];
  __shared__ int32_t cid_l[kFrCap];
  __shared__ uint32_t bitmap[kFrWords];
  __shared__ uint32_t hist256[256];
  __shared__ uint32_t wb[Wg<NT>::kScratch];
  __shared__ uint32_t ccount;
  using W = Wg<NT>;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = min(max(vis_len[r], 0), N_cap);
  const ScoreRow<BF16> row = score_row<BF16>(scores, r, N_cap);
  const uint32_t need = min(static_cast<uint32_t>(k), static_cast<uint32_t>(n));

  // Raw buffer loads through one descriptor sized to the row's visible
  // bytes (bf16: whole 4-byte words only; an odd last item is read on its
  // own below): lanes past the end read 0 without a branch, every load
  // shares the lane's offset register (load u adds a constant offset) and
  // all are in flight together.  Keys are the order-preserving images of
  // the scores (bf16: of the 16-bit pattern, in the register's high or low
  // half).
  uint32_t kr[S::kRegs];
  {
    const int bytes = BF16 ? (n >> 1) * 4 : n * 4;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(row.p), static_cast<short>(0), bytes, kRawBufferFlags);
#pragma unroll
    for (int u = 0; u < S::kRegs; ++u)
      kr[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * tid, 4 * NT * u, 0);
  }
  if constexpr (BF16) {
    if (n & 1) {
      // Item n - 1 is the low half of word (n - 1) / 2, which the
      // descriptor left out: its thread reads it alone (a select per
      // register keeps the index constant).
      const int w = (n - 1) >> 1;
      if (tid == w % NT) {
        const uint32_t v = static_cast<const uint16_t*>(row.p)[n - 1];
#pragma unroll
        for (int u = 0; u < S::kRegs; ++u) kr[u] = (u == w / NT) ? v : kr[u];
      }
    }
  }
  // Item e's score (e: a compile-time constant after unrolling); the bins
  // and the range work on the scores, and order keys are formed only where
  // items are compared.  Items past the row (read as 0) are never counted
  // or selected.
  auto val = [&](int e) -> float {
    if constexpr (BF16)
      return __builtin_bit_cast(float, (e & 1) ? (kr[e >> 1] & 0xffff0000u) : (kr[e >> 1] << 16));
    else
      return __builtin_bit_cast(float, kr[e]);
  };
  auto key = [&](int e) -> uint32_t { return float_to_key(val(e)); };
  auto valid = [&](int e) { return S::item(e, tid) < n; };

  // Every item is taken when need == n: K* = 0, I* = max.
  uint32_t kstar = 0;
  int32_t istar = 0x7fffffff;
  // The output is ordered through a bitmap over ids.  The candidate pass
  // marks the sure items (bins above the threshold bin) and the resolved
  // threshold bin is marked from its LDS list, so no second pass over the
  // registers is needed; `marked` says that happened.
  bool marked = false;
  for (int w = tid; w < kFrWords; w += NT) bitmap[w] = 0;
  if (need > 0 && need < static_cast<uint32_t>(n)) {
    float fmx = -__builtin_inff(), fmn = __builtin_inff();
    bool any = false;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (valid(e)) {
        const float v = val(e);
        fmx = fmaxf(fmx, v);
        fmn = fminf(fmn, v);
        any = true;
      }
    }
    uint32_t mx = any ? float_to_key(fmx) : 0u, mn_inv = any ? ~float_to_key(fmn) : 0u, unused = 0;
    for (int i = tid; i < kFrBins; i += NT) hist[i] = 0;
    W::reduce_sum_max_max(unused, mx, mn_inv, wb);
    const float vmax = key_to_float(mx);
    const float vmin = key_to_float(~mn_inv);
    // Bins linear in the score value between the row's min and max (scores
    // cluster in a few binades, so bins linear in the key bits would not
    // spread them).  Subtraction, scaling and truncation never reverse an
    // order, so bin order is key order; a row whose range is not finite
    // puts everything in bin 0 and is resolved over the whole row.
    const float range = vmax - vmin;
    const float scale = (range > 0.0f && range < __builtin_inff())
                            ? static_cast<float>(kFrBins) * 0.99999f / range : 0.0f;
    auto bin_of = [&](float v) {
      const float x = (v - vmin) * scale;
      return min(kFrBins - 1, max(0, static_cast<int>(x)));
    };
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (valid(e)) atomicAdd(&hist[bin_of(val(e))], 1u);
    __syncthreads();
    uint32_t above;
    const int b1 = W::find_rank_bin(hist, kFrBins, need, true, wb, &above);
    const uint32_t ncand = hist[b1];
    if (ncand <= static_cast<uint32_t>(kFrCap)) {
      if (tid == 0) ccount = 0;
      __syncthreads();
      // Items of bin b1 and above score at least flo, one bin width below
      // the bin's lower edge (a margin against rounding); only waves holding
      // such scores evaluate the exact bin.  Items of a higher bin are
      // selected whatever the threshold inside b1 (bin order is key order).
      // fp32: a wave's 64 items at index e are the ids of two bitmap words,
      // which its lanes 0 and 1 store from the wave's ballot of those items.
      // bf16: item e of thread t is 2 (NT (e / 2) + t) + e % 2, i.e. bit
      // 2 (t % 16) + e % 2 of word t / 16 + 32 (e / 2): one base word and two
      // bit masks per thread, and a constant offset per e.
      const float flo = scale > 0.0f ? vmin + (static_cast<float>(b1) - 1.0f) / scale
                                     : -__builtin_inff();
      const int mword = tid >> 4;
      const uint32_t mbit0 = 1u << (2 * (tid & 15)), mbit1 = mbit0 << 1;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float v = val(e);
        if (__ballot(v >= flo) == 0) continue;   // wave-uniform
        const int i = S::item(e, tid);
        const int bk = i < n ? bin_of(v) : -1;
        const bool c = bk == b1;
        const uint32_t slot = wave_append(c, &ccount);
        if (c) {
          ckey_l[slot] = float_to_key(v);
          cid_l[slot] = i;
        }
        if constexpr (BF16) {
          if (bk > b1) atomicOr(&bitmap[mword + 32 * (e >> 1)], (e & 1) ? mbit1 : mbit0);
        } else {
          static_assert(NT % 64 == 0, "a wave's items at one index start a bitmap word");
          const uint64_t sure = __ballot(bk > b1);
          const int lane = tid & 63;
          if (lane < 2)
            bitmap[(S::item(e, tid - lane) >> 5) + lane] =
                static_cast<uint32_t>(lane ? sure >> 32 : sure);
        }
      }
      __syncthreads();
      if (ncand <= static_cast<uint32_t>(kRankMax))
        resolve_by_rank<NT>(ckey_l, cid_l, ncand, need - above, wb, &kstar, &istar);
      else
        W::resolve(ArrayCand{ckey_l, cid_l, ncand}, 0u, 32, need - above, hist256, wb, &kstar,
                   &istar);
      for (uint32_t c = tid; c < ncand; c += NT) {
        const int32_t i = cid_l[c];
        if (selected(ckey_l[c], i, kstar, istar)) atomicOr(&bitmap[i >> 5], 1u << (i & 31));
      }
      marked = true;
    } else {
      W::resolve(FlatCand<BF16>{row, static_cast<uint32_t>(n)}, 0u, 32, need, hist256, wb, &kstar,
                 &istar);
    }
  }

  // Ordered output: thread t owns bitmap words kWordsPerThread t .. +
  // kWordsPerThread - 1.  Every item (need == n), or a threshold resolved
  // over the whole row, is marked by a pass over the registers.
  __syncthreads();
  if (!marked) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const uint32_t kk = key(e);
      if (__ballot(kk >= kstar) == 0) continue;   // selected items have key >= K*
      const int i = S::item(e, tid);
      if (i < n && selected(kk, i, kstar, istar)) atomicOr(&bitmap[i >> 5], 1u << (i & 31));
    }
    __syncthreads();
  }
  constexpr int WPT = S::kWordsPerThread;
  uint32_t words[WPT];
  uint32_t cnt = 0;
#pragma unroll
  for (int u = 0; u < WPT; ++u) {
    const int w = WPT * tid + u;
    words[u] = w < kFrWords ? bitmap[w] : 0u;
    cnt += __popc(words[u]);
  }
  uint32_t total;
  uint32_t off = W::excl_scan_last(cnt, wb, &total);
  int32_t* orow = out + static_cast<size_t>(r) * k;
  float* krow = out_key ? out_key + static_cast<size_t>(r) * k : nullptr;
#pragma unroll
  for (int u = 0; u < WPT; ++u) {
    uint32_t m = words[u];
    while (m != 0) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      const int id = 32 * (WPT * tid + u) + bit;
      if (off < need) {
        orow[off] = id;
        if (krow) krow[off] = row.at(id);
      }
      ++off;
    }
  }
  for (int i = static_cast<int>(min(total, need)) + tid; i < k; i += NT) {
    orow[i] = -1;
    if (krow) krow[i] = -__builtin_inff();
  }
}

}  // namespace

size_t block_topk_workspace_bytes(int rows, int N_cap) {
  const size_t nb_cap = (static_cast<size_t>(N_cap) + 7) / 8;
  return static_cast<size_t>(rows) * (2 * kHistBins + 2 * kBtMaxWgs + 3 * nb_cap) * 4;
}

size_t pool_topk_workspace_bytes(int rows, int k_blocks) {
  return static_cast<size_t>(rows) * static_cast<size_t>(k_blocks) * kBlock * 4;
}

int block_topk_max_blocks() { return kBtMaxBlocks; }

namespace {

hipError_t run_block_topk(const float* block_max, const int32_t* vis_len, int rows, int N_cap,
                          int k, int32_t* out, const BtWs& w, hipStream_t stream) {
  const size_t nb_cap = (static_cast<size_t>(N_cap) + 7) / 8;
  hipError_t e;
  dim3 grid(static_cast<unsigned>((nb_cap + kBtItems - 1) / kBtItems), rows);
  hipLaunchKernelGGL(k_bt_hist, grid, dim3(kBtThreads), 0, stream, block_max, vis_len, N_cap, k, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_bt_filter, grid, dim3(kBtThreads), 0, stream, block_max, vis_len, N_cap, k,
                     w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_bt_final, dim3(rows), dim3(kBtThreads), 0, stream, block_max, vis_len, N_cap,
                     k, w, out);
  return hipGetLastError();
}

// Workspace layout of a caller's buffer: histograms of the call's rows, then
// the per-workgroup counts and the segments.
BtWs caller_layout(void* ws, int rows, size_t nb_cap) {
  BtWs w;
  w.hist = static_cast<uint32_t*>(ws);
  w.hist2 = w.hist + static_cast<size_t>(rows) * kHistBins;
  w.wgcnt = w.hist2 + static_cast<size_t>(rows) * kHistBins;
  w.sure = reinterpret_cast<int32_t*>(w.wgcnt + static_cast<size_t>(rows) * kBtMaxWgs * 2);
  w.ckey = reinterpret_cast<uint32_t*>(w.sure + static_cast<size_t>(rows) * nb_cap);
  w.cid = reinterpret_cast<int32_t*>(w.ckey + static_cast<size_t>(rows) * nb_cap);
  return w;
}

// ---------------------------------------------------------------------------
// Allocation-free block Top-K: the workspace is a file-scope device array of
// fixed size, one copy per GPU, resolved once per device with
// hipGetSymbolAddress (in host code `scratch` names a host-side stand-in,
// never the device memory).  Its layout does not depend on the call: the
// histograms of all kNoAllocRows rows come first, so they are zero when the
// code object is loaded and every call leaves them zeroed again, whatever
// its row count; the counts and segments follow.  Calls that overlap on one
// GPU share the array and race.
constexpr int kNoAllocRows = 64;
constexpr size_t kNoAllocBytes = size_t{16} << 20;
constexpr size_t kNoAllocFixed = static_cast<size_t>(kNoAllocRows) * (2 * kHistBins + 2 * kBtMaxWgs) * 4;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

hipError_t launch_block_topk(const float* block_max, const int32_t* vis_len, int rows, int N_cap,
                             int k, int32_t* out, void* ws, hipStream_t stream) {
  const size_t nb_cap = (static_cast<size_t>(N_cap) + 7) / 8;
  return run_block_topk(block_max, vis_len, rows, N_cap, k, out, caller_layout(ws, rows, nb_cap),
                        stream);
}

bool block_topk_noalloc_fits(int rows, int N_cap) {
  const size_t nb_cap = (static_cast<size_t>(N_cap) + 7) / 8;
  return rows >= 1 && rows <= kNoAllocRows &&
         static_cast<size_t>(rows) * nb_cap * 3 * 4 <= kNoAllocBytes - kNoAllocFixed;
}

hipError_t launch_block_topk_noalloc(const float* block_max, const int32_t* vis_len, int rows,
                                     int N_cap, int k, int32_t* out, hipStream_t stream) {
  if (!block_topk_noalloc_fits(rows, N_cap)) return hipErrorInvalidValue;
  void* base = nullptr;
  hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return e;
  const size_t nb_cap = (static_cast<size_t>(N_cap) + 7) / 8;
  BtWs w;
  w.hist = static_cast<uint32_t*>(base);
  w.hist2 = w.hist + static_cast<size_t>(kNoAllocRows) * kHistBins;
  w.wgcnt = w.hist2 + static_cast<size_t>(kNoAllocRows) * kHistBins;
  w.sure = reinterpret_cast<int32_t*>(w.wgcnt + static_cast<size_t>(kNoAllocRows) * kBtMaxWgs * 2);
  w.ckey = reinterpret_cast<uint32_t*>(w.sure + static_cast<size_t>(rows) * nb_cap);
  w.cid = reinterpret_cast<int32_t*>(w.ckey + static_cast<size_t>(rows) * nb_cap);
  return run_block_topk(block_max, vis_len, rows, N_cap, k, out, w, stream);
}

hipError_t launch_pool_topk(int mode, const float* scores, const uint16_t* q_idx,
                            const float* w_idx, const void* k_idx, const Pages& pg,
                            const int32_t* pool_blocks,
                            int k_blocks, const int32_t* vis_len, int rows, int n_q, int N_cap,
                            int top_k, int32_t* out, float* out_key, void* ws,
                            hipStream_t stream) {
  PoolArgs a;
  a.scores = mode == 0 ? scores : nullptr;
  a.q_idx = q_idx;
  a.w_idx = w_idx;
  a.k_idx = static_cast<const uint8_t*>(k_idx);
  a.pg = pg;
  a.pool = pool_blocks;
  a.vis_len = vis_len;
  a.kb = k_blocks;
  a.n_q = n_q;
  a.N_cap = N_cap;
  a.top_k = top_k;
  a.ps = static_cast<float*>(ws);
  a.out = out;
  a.out_key = out_key;
  hipError_t e;
  if (mode != 0) {
    dim3 grid((k_blocks + kPsBlocks - 1) / kPsBlocks, rows);
    if (mode == 1)
      hipLaunchKernelGGL(k_pool_score<kKdFp8>, grid, dim3(kPscThreads), 0, stream, a);
    else if (mode == 2)
      hipLaunchKernelGGL(k_pool_score<kKdBf16>, grid, dim3(kPscThreads), 0, stream, a);
    else if (mode == 3)
      hipLaunchKernelGGL(k_pool_score<kKdFp4>, grid, dim3(kPscThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(k_pool_score<kKdFp4Q>, grid, dim3(kPscThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_pool_final, dim3(rows), dim3(kPsThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_flat_topk(const void* scores, const int32_t* vis_len, int rows, int N_cap,
                            int k, int32_t* out, float* out_key, hipStream_t stream, bool bf16) {
  const bool reg = N_cap <= kFrItems;
  const dim3 grid(rows), block(kFsThreads);
  if (reg && bf16)
    hipLaunchKernelGGL(k_flat_select_reg<true>, grid, dim3(FrShape<true>::kThreads), 0, stream,
                       scores, vis_len, N_cap, k, out, out_key);
  else if (reg)
    hipLaunchKernelGGL(k_flat_select_reg<false>, grid, dim3(FrShape<false>::kThreads), 0, stream,
                       scores, vis_len, N_cap, k, out, out_key);
  else if (bf16)
    hipLaunchKernelGGL(k_flat_select<true>, grid, block, 0, stream, scores, vis_len, N_cap, k, out,
                       out_key);
  else
    hipLaunchKernelGGL(k_flat_select<false>, grid, block, 0, stream, scores, vis_len, N_cap, k, out,
                       out_key);
  return hipGetLastError();
}

}  // namespace csa2
