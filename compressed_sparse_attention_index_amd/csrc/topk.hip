// Two-level Top-K of the hierarchical sparse indexer, and the pool re-scoring
// of Reindex layers.
//
// "DeepSeek-V4.1-Flash 架构详解", §3.2: the Full layer keeps at most 2,048
// blocks of 8 positions (a pool of at most 16,384 candidates) and its own
// Top-512; a Reindex layer re-scores only the pool with its own indexer
// query and takes a new Top-512.
//
// Selection is exact: the k-th key K* and, among items equal to K*, the
// largest id I* still taken are found by radix selection over
// order-preserving uint32 keys; an item is selected iff
//   key > K*  or  (key == K* and id <= I*),
// which is the first k items in (score descending, id ascending) order.  A
// last pass over the items in id order compacts the selected ids with a
// workgroup prefix sum, so the output list is ascending and independent of
// thread timing.
#include "csa2_launch.h"
#include "index_core.h"

namespace csa2 {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 4096;
constexpr int kCandCap = 4096;

// ---------------------------------------------------------------------------
// Item sources: item i of a query row -> (valid, key, id).  Ids increase with
// i for every source (pool blocks are ascending), so a pass in item order is a
// pass in id order.
struct Item {
  bool valid;
  uint32_t key;
  int32_t id;
};

struct SrcArgs {
  const float* keys;         // row-major [rows, stride]
  const int32_t* pool;       // [rows, k_blocks] or null
  const int32_t* vis_len;    // [rows]
  int k_blocks;
  int N_cap;
  int stride;                // elements per row of `keys`
};

template <int SRC>
struct Source {
  const float* keys;
  const int32_t* pool;
  int vis;
  int nb_cap;
  int n;

  __device__ Source(const SrcArgs& a, int r) {
    vis = min(max(a.vis_len[r], 0), a.N_cap);
    nb_cap = (a.N_cap + 7) >> 3;
    keys = a.keys + static_cast<size_t>(r) * a.stride;
    pool = a.pool ? a.pool + static_cast<size_t>(r) * a.k_blocks : nullptr;
    if (SRC == kSrcBlocks) n = (vis + 7) >> 3;
    else if (SRC == kSrcFlat) n = vis;
    else n = a.k_blocks * 8;
  }

  __device__ __forceinline__ Item get(int i) const {
    Item it;
    if (SRC == kSrcBlocks || SRC == kSrcFlat) {
      it.valid = true;
      it.id = i;
      it.key = float_to_key(keys[i]);
    } else {
      const int blk = pool[i >> 3];
      const int pos = blk * 8 + (i & 7);
      it.valid = blk >= 0 && blk < nb_cap && pos < vis;
      it.id = pos;
      const float s = SRC == kSrcPoolStored ? (it.valid ? keys[pos] : 0.0f) : keys[i];
      it.key = float_to_key(s);
    }
    return it;
  }
};

// ---------------------------------------------------------------------------
// Workgroup primitives (1024 threads).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ uint32_t wg_excl_scan(uint32_t v, uint32_t* wave_buf, uint32_t* total) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wave_buf[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kSelWaves ? wave_buf[lane] : 0;
    const uint32_t ti = wave_incl_scan(t);
    if (lane < kSelWaves) wave_buf[kSelWaves + lane] = ti - t;
    if (lane == kSelWaves - 1) wave_buf[2 * kSelWaves] = ti;
  }
  __syncthreads();
  const uint32_t r = wave_buf[kSelWaves + wave] + inc - v;
  *total = wave_buf[2 * kSelWaves];
  __syncthreads();
  return r;
}

__device__ uint32_t wg_reduce(uint32_t v, uint32_t* wave_buf, bool is_max) {
  uint32_t t;
  const uint32_t ex = wg_excl_scan(is_max ? 0u : v, wave_buf, &t);
  (void)ex;
  if (!is_max) return t;
  // max via shuffles
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(v, d, 64)));
  if (lane_id() == 0) wave_buf[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = 0;
  for (int w = 0; w < kSelWaves; ++w) m = max(m, wave_buf[w]);
  __syncthreads();
  return m;
}

// Given per-bin counts in hist[0..nbins), finds the bin holding the item of
// rank `rank` (1-based) counting from the top bin down (descending) or from
// bin 0 up (ascending).  Returns the bin; *before gets the count of items in
// bins passed before it.  nbins <= 4 * kSelThreads.
__device__ int find_rank_bin(const uint32_t* hist, int nbins, uint32_t rank, bool descending,
                             uint32_t* wave_buf, uint32_t* result, uint32_t* before) {
  const int per = (nbins + kSelThreads - 1) / kSelThreads;  // bins per thread, <= 4
  const int t = threadIdx.x;
  uint32_t c[4] = {0, 0, 0, 0};
  uint32_t s = 0;
  for (int i = 0; i < per; ++i) {
    const int idx = t * per + i;
    int bin = descending ? nbins - 1 - idx : idx;
    c[i] = (idx < nbins) ? hist[bin] : 0;
    s += c[i];
  }
  uint32_t tot;
  uint32_t p = wg_excl_scan(s, wave_buf, &tot);
  if (p < rank && rank <= p + s) {
    for (int i = 0; i < per; ++i) {
      if (rank <= p + c[i]) {
        const int idx = t * per + i;
        result[0] = static_cast<uint32_t>(descending ? nbins - 1 - idx : idx);
        result[1] = p;
        break;
      }
      p += c[i];
    }
  }
  __syncthreads();
  const int bin = static_cast<int>(result[0]);
  *before = result[1];
  __syncthreads();
  return bin;
}

// ---------------------------------------------------------------------------
template <int SRC>
__global__ __launch_bounds__(kSelThreads) void k_select(SrcArgs args, int k,
                                                        int32_t* __restrict__ out_ids,
                                                        float* __restrict__ out_keys) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t cand_key[kCandCap];
  __shared__ int32_t cand_id[kCandCap];
  __shared__ uint32_t wave_buf[2 * kSelWaves + 4];
  __shared__ uint32_t res[4];
  __shared__ uint32_t cand_count;

  const int r = blockIdx.x;
  const Source<SRC> src(args, r);
  const int n = src.n;
  const int tid = threadIdx.x;

  // Pass 0: valid count and key range.
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0;
  for (int i = tid; i < n; i += kSelThreads) {
    const Item it = src.get(i);
    if (it.valid) {
      ++cnt;
      kmin = min(kmin, it.key);
      kmax = max(kmax, it.key);
    }
  }
  const uint32_t n_valid = wg_reduce(cnt, wave_buf, false);
  kmax = wg_reduce(kmax, wave_buf, true);
  kmin = ~wg_reduce(~kmin, wave_buf, true);
  const uint32_t need = min(static_cast<uint32_t>(k), n_valid);

  // Threshold: select iff key > k_star || (key == k_star && id <= i_star).
  uint32_t k_star = 0;
  int32_t i_star = 0x7fffffff;
  if (need < n_valid && need > 0) {
    // Pass 1: histogram of (key - kmin) >> sh over at most kBins bins.
    const uint32_t range = kmax - kmin;
    int sh = 0;
    while (sh < 32 && (static_cast<uint64_t>(range) >> sh) >= kBins) ++sh;
    for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const Item it = src.get(i);
      if (it.valid) atomicAdd(&hist[(it.key - kmin) >> sh], 1u);
    }
    __syncthreads();
    const int nbins = static_cast<int>((static_cast<uint64_t>(range) >> sh) + 1);
    uint32_t above;
    const int bstar = find_rank_bin(hist, nbins, need, true, wave_buf, res, &above);
    uint32_t rem = need - above;                     // items to take at or below the bin
    const uint32_t in_bin = hist[bstar];
    // Candidates: items whose offset from kmin has the prefix bstar << sh.
    uint32_t prefix = static_cast<uint32_t>(bstar) << sh;   // offset prefix
    uint32_t pmask = sh >= 32 ? 0u : (0xffffffffu << sh);
    const bool in_lds = in_bin <= static_cast<uint32_t>(kCandCap);
    if (in_lds) {
      if (tid == 0) cand_count = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) {
        const Item it = src.get(i);
        if (it.valid && ((it.key - kmin) & pmask) == prefix) {
          const uint32_t slot = atomicAdd(&cand_count, 1u);
          cand_key[slot] = it.key - kmin;
          cand_id[slot] = it.id;
        }
      }
      __syncthreads();
    }
    // Radix passes over the low sh bits of the offset, 8 bits at a time.
    uint32_t eq_count = in_bin;
    int lo = sh;
    while (lo > 0) {
      const int bits = lo >= 8 ? 8 : lo;
      lo -= bits;
      const uint32_t dmask = (1u << bits) - 1u;
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (uint32_t c = tid; c < in_bin; c += kSelThreads) {
          const uint32_t off = cand_key[c];
          if ((off & pmask) == prefix) atomicAdd(&hist[(off >> lo) & dmask], 1u);
        }
      } else {
        for (int i = tid; i < n; i += kSelThreads) {
          const Item it = src.get(i);
          const uint32_t off = it.key - kmin;
          if (it.valid && (off & pmask) == prefix) atomicAdd(&hist[(off >> lo) & dmask], 1u);
        }
      }
      __syncthreads();
      uint32_t before;
      const int d = find_rank_bin(hist, 1 << bits, rem, true, wave_buf, res, &before);
      eq_count = hist[d];
      rem -= before;
      prefix |= static_cast<uint32_t>(d) << lo;
      pmask |= dmask << lo;
      __syncthreads();
    }
    k_star = prefix + kmin;
    // Among items equal to k_star take the `rem` lowest ids.
    if (rem < eq_count) {
      uint32_t iprefix = 0, imask = 0;
      for (int lo2 = 24; lo2 > 0;) {
        lo2 -= 8;
        for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        if (in_lds) {
          for (uint32_t c = tid; c < in_bin; c += kSelThreads) {
            const uint32_t id = static_cast<uint32_t>(cand_id[c]);
            if (cand_key[c] + kmin == k_star && (id & imask) == iprefix)
              atomicAdd(&hist[(id >> lo2) & 255u], 1u);
          }
        } else {
          for (int i = tid; i < n; i += kSelThreads) {
            const Item it = src.get(i);
            const uint32_t id = static_cast<uint32_t>(it.id);
            if (it.valid && it.key == k_star && (id & imask) == iprefix)
              atomicAdd(&hist[(id >> lo2) & 255u], 1u);
          }
        }
        __syncthreads();
        uint32_t below;
        const int d = find_rank_bin(hist, 256, rem, false, wave_buf, res, &below);
        rem -= below;
        iprefix |= static_cast<uint32_t>(d) << lo2;
        imask |= 255u << lo2;
        __syncthreads();
      }
      i_star = static_cast<int32_t>(iprefix);
    }
  }

  // Final pass: ordered compaction of the selected items.
  int32_t* orow = out_ids + static_cast<size_t>(r) * k;
  float* krow = out_keys ? out_keys + static_cast<size_t>(r) * k : nullptr;
  constexpr int kPer = 4;
  uint32_t written = 0;
  for (int base = 0; base < n; base += kSelThreads * kPer) {
    Item it[kPer];
    bool sel[kPer];
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = base + tid * kPer + e;
      it[e] = (i < n) ? src.get(i) : Item{false, 0u, 0};
      sel[e] = it[e].valid && need > 0 &&
               (it[e].key > k_star || (it[e].key == k_star && it[e].id <= i_star));
      c += sel[e] ? 1u : 0u;
    }
    uint32_t round_total;
    uint32_t off = written + wg_excl_scan(c, wave_buf, &round_total);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (sel[e] && off < static_cast<uint32_t>(k)) {
        orow[off] = it[e].id;
        if (krow) krow[off] = key_to_float(it[e].key);
        ++off;
      }
    }
    written += round_total;
  }
  for (int i = static_cast<int>(min(written, static_cast<uint32_t>(k))) + tid; i < k; i += kSelThreads) {
    orow[i] = -1;
    if (krow) krow[i] = -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// Pool re-scoring: each workgroup scores 32 pool blocks (8 tiles of 32
// positions, 4 blocks per tile); lane col takes position 8*block + col%8 of
// block 4*tile + col/8.  Rows of one block are 8 consecutive key rows.
constexpr int kRescoreBlocksPerWg = 32;

template <bool FP8>
__global__ __launch_bounds__(256) void k_pool_rescore(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ pool_blocks, int k_blocks,
    const int32_t* __restrict__ vis_len, int n_q, int N_cap, float* __restrict__ pool_scores) {
  const int r = blockIdx.y;
  const int b = r / n_q;
  const int vis = min(max(vis_len[r], 0), N_cap);
  const int nb_cap = (N_cap + 7) >> 3;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  bf16x8 qa[8];
  float wr[16];
  load_query(qa, q_idx + static_cast<size_t>(r) * kIdxHeads * kIdxDim, col, half);
  load_weights(wr, w_idx + static_cast<size_t>(r) * kIdxHeads, half);
  const int32_t* prow = pool_blocks + static_cast<size_t>(r) * k_blocks;
  const uint8_t* kb = k_idx + static_cast<size_t>(b) * N_cap * (FP8 ? 128 : 256);
  float* orow = pool_scores + static_cast<size_t>(r) * k_blocks * 8;
  const int tiles = (k_blocks + 3) / 4;
  const int t0 = blockIdx.x * (kRescoreBlocksPerWg / 4);
  const int t1 = min(t0 + kRescoreBlocksPerWg / 4, tiles);
  for (int t = t0 + wave; t < t1; t += 4) {
    const int slot = 4 * t + (col >> 3);
    const int blk = slot < k_blocks ? prow[slot] : -1;
    const int pos = blk * 8 + (col & 7);
    const bool valid = blk >= 0 && blk < nb_cap && pos < vis;
    KeyTile<FP8> kt;
    load_key_half<FP8>(kt, kb + static_cast<size_t>(valid ? pos : 0) * (FP8 ? 128 : 256), half);
    const float s = head_sum(key_tile_dot<FP8>(qa, kt), wr);
    if (half == 0 && slot < k_blocks) orow[slot * 8 + (col & 7)] = valid ? s : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_pool_rescore(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                               bool fp8, const int32_t* pool_blocks, int k_blocks,
                               const int32_t* vis_len, int B, int n_q, int N_cap,
                               float* pool_scores, hipStream_t stream) {
  dim3 grid((k_blocks + kRescoreBlocksPerWg - 1) / kRescoreBlocksPerWg, B * n_q);
  const uint8_t* kb = static_cast<const uint8_t*>(k_idx);
  if (fp8)
    hipLaunchKernelGGL(k_pool_rescore<true>, grid, dim3(256), 0, stream, q_idx, w_idx, kb,
                       pool_blocks, k_blocks, vis_len, n_q, N_cap, pool_scores);
  else
    hipLaunchKernelGGL(k_pool_rescore<false>, grid, dim3(256), 0, stream, q_idx, w_idx, kb,
                       pool_blocks, k_blocks, vis_len, n_q, N_cap, pool_scores);
  return hipGetLastError();
}

hipError_t launch_select(SelectSource src, const float* keys, const int32_t* pool_blocks,
                         int k_blocks, const int32_t* vis_len, int rows, int N_cap, int k,
                         int32_t* out_ids, float* out_keys, hipStream_t stream) {
  SrcArgs a;
  a.keys = keys;
  a.pool = pool_blocks;
  a.vis_len = vis_len;
  a.k_blocks = k_blocks;
  a.N_cap = N_cap;
  switch (src) {
    case kSrcBlocks: a.stride = (N_cap + 7) / 8; break;
    case kSrcPoolScored: a.stride = k_blocks * 8; break;
    default: a.stride = N_cap; break;
  }
  dim3 grid(rows), block(kSelThreads);
  switch (src) {
    case kSrcBlocks:
      hipLaunchKernelGGL(k_select<kSrcBlocks>, grid, block, 0, stream, a, k, out_ids, out_keys);
      break;
    case kSrcPoolStored:
      hipLaunchKernelGGL(k_select<kSrcPoolStored>, grid, block, 0, stream, a, k, out_ids, out_keys);
      break;
    case kSrcPoolScored:
      hipLaunchKernelGGL(k_select<kSrcPoolScored>, grid, block, 0, stream, a, k, out_ids, out_keys);
      break;
    default:
      hipLaunchKernelGGL(k_select<kSrcFlat>, grid, block, 0, stream, a, k, out_ids, out_keys);
      break;
  }
  return hipGetLastError();
}

}  // namespace csa2
