// Indexer scan with the block maximum fused in (decode), and the prefill-chunk
// variant that reuses each key tile for several query rows.
//
// "DeepSeek-V4.1-Flash 架构详解", §3.2: the first Full layer scans every
// visible entry; scores are aggregated per block of 8 positions (maximum).
// The scan streams the indexer keys once from HBM (128 B per FP8 entry), so
// it is bound by HBM bandwidth; the 32 heads x 128 dims contraction per entry
// runs on bf16 matrix cores after an exact FP8 -> bf16 conversion.
#include "csa2_launch.h"
#include "index_core.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <bool FP8>
__device__ __forceinline__ const uint8_t* key_row(const uint8_t* kb, int pos, int N_cap) {
  // Rows past the end of the buffer are never addressed: the last tile's
  // extra lanes re-read the final row and are masked afterwards.
  const int p = pos < N_cap ? pos : N_cap - 1;
  return kb + static_cast<size_t>(p) * (FP8 ? 128 : 256);
}

__device__ __forceinline__ void emit(float s, int pos, int vis, int half, int col, float* scores,
                                     float* block_max) {
  const bool valid = pos < vis;
  if (scores != nullptr && half == 0 && valid) scores[pos] = s;
  if (block_max != nullptr) {
    float m = valid ? s : -__builtin_inff();
    m = fmaxf(m, wave_xor(m, 1));
    m = fmaxf(m, wave_xor(m, 2));
    m = fmaxf(m, wave_xor(m, 4));
    if (half == 0 && (col & 7) == 0 && valid) block_max[pos >> 3] = m;
  }
}

// Decode: one query row per workgroup row (blockIdx.y).  The workgroup's
// four waves take interleaved 32-position tiles of its chunk.  Each tile
// (32 rows of 128 B FP8 or 256 B bf16 keys) is copied straight from HBM into
// a per-wave LDS slot with coalesced, non-temporal direct-to-LDS loads (every
// load instruction moves 1 KB of whole 128-byte lines; the keys are read
// once, so they are not kept in the caches).  The global address of each lane
// is permuted so that the slot holds a swizzled layout: 16-byte chunk c of row
// r sits at chunk position c ^ f(r), which makes the MFMA-layout reads below
// (16 B per lane, one row per lane) free of LDS bank conflicts.  DEPTH tiles
// are in flight per wave; loads complete in issue order, so waiting until at
// most DEPTH tiles' loads are outstanding guarantees the oldest has landed.
template <bool FP8>
struct ScanTile {
  static constexpr int kRowBytes = FP8 ? 128 : 256;
  static constexpr int kChunks = kRowBytes / 16;            // 16-B chunks per row
  static constexpr int kBytes = 32 * kRowBytes;              // one tile
  static constexpr int kLoads = kBytes / 1024;               // direct-to-LDS loads per tile
  __device__ static int pos(int row, int chunk) {            // swizzled byte offset
    const int f = FP8 ? ((row >> 1) & 7) : (row & 15);
    return row * kRowBytes + ((chunk ^ f) << 4);
  }
};

template <int N>
__device__ __forceinline__ void wait_tiles(int pending, int per_tile) {
  // pending in [0, N]; per_tile loads per tile.  The immediate must be a
  // constant, so branch on the (wave-uniform) count.
  if (per_tile == 4) {
    if (pending >= 2 && N >= 2) wait_vmem<8>();
    else if (pending == 1) wait_vmem<4>();
    else wait_vmem<0>();
  } else {
    if (pending >= 2 && N >= 2) wait_vmem<16>();
    else if (pending == 1) wait_vmem<8>();
    else wait_vmem<0>();
  }
}

template <bool FP8, int DEPTH>
__global__ __launch_bounds__(kThreads) void k_index_scan(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ vis_len, int n_q, int N_cap,
    int tiles_per_wg, float* __restrict__ scores, float* __restrict__ block_max) {
  using TT = ScanTile<FP8>;
  static_assert(DEPTH <= 2, "wait_tiles handles up to two tiles in flight");
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][DEPTH + 1][TT::kBytes];
  const int r = blockIdx.y;
  const int b = r / n_q;
  const int vis = min(max(vis_len[r], 0), N_cap);
  const int ntiles = (vis + 31) >> 5;
  const int t_begin = blockIdx.x * tiles_per_wg;
  const int t_end = min(t_begin + tiles_per_wg, ntiles);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  int t = t_begin + wave;
  if (t >= t_end) return;

  bf16x8 qa[8];
  float wr[16];
  load_query(qa, q_idx + static_cast<size_t>(r) * kIdxHeads * kIdxDim, col, half);
  load_weights(wr, w_idx + static_cast<size_t>(r) * kIdxHeads, half);
  const uint8_t* kb = k_idx + static_cast<size_t>(b) * N_cap * TT::kRowBytes;
  float* srow = scores ? scores + static_cast<size_t>(r) * N_cap : nullptr;
  float* brow = block_max ? block_max + static_cast<size_t>(r) * ((N_cap + 7) >> 3) : nullptr;

  // Source offset (within a tile) of this lane for each of the tile's loads.
  int goff[TT::kLoads];
  int grow[TT::kLoads];
#pragma unroll
  for (int i = 0; i < TT::kLoads; ++i) {
    const int g = 64 * i + lane;                  // destination chunk index in the slot
    const int row = g / TT::kChunks, p = g % TT::kChunks;
    const int f = FP8 ? ((row >> 1) & 7) : (row & 15);
    grow[i] = row;
    goff[i] = row * TT::kRowBytes + ((p ^ f) << 4);
  }
  auto issue = [&](int slot, int tile) {
    const int rows = N_cap - 32 * tile;           // rows of this tile inside the buffer
    const uint8_t* base = kb + static_cast<size_t>(32) * tile * TT::kRowBytes;
#pragma unroll
    for (int i = 0; i < TT::kLoads; ++i) {
      const uint8_t* src = base + (grow[i] < rows ? goff[i] : 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)src,
          (__attribute__((address_space(3))) void*)(&stage[wave][slot][i * 1024]), 16, 0,
          2 /* non-temporal */);
    }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (t + d * kWaves < t_end) issue(d, t + d * kWaves);
  int slot = 0;
  for (; t < t_end; t += kWaves) {
    const int tp = t + DEPTH * kWaves;
    if (tp < t_end) issue((slot + DEPTH) % (DEPTH + 1), tp);
    const int ahead = (t_end - 1 - t) / kWaves;   // tiles after t for this wave
    wait_tiles<DEPTH>(ahead < DEPTH ? ahead : DEPTH, TT::kLoads);
    const uint8_t* st = stage[wave][slot];
    KeyTile<FP8> kt;
#pragma unroll
    for (int j = 0; j < KeyTile<FP8>::kWords; ++j)
      kt.v[j] = *reinterpret_cast<const u32x4*>(st + TT::pos(col, (TT::kChunks / 2) * half + j));
    const float s = head_sum(key_tile_dot<FP8>(qa, kt), wr);
    emit(s, 32 * t + col, vis, half, col, srow, brow);
    slot = slot == DEPTH ? 0 : slot + 1;
  }
}

int pick_tiles_per_wg(long long total_tiles, int min_tiles, int target_wgs, int max_tiles) {
  long long t = (total_tiles + target_wgs - 1) / target_wgs;
  if (t < min_tiles) t = min_tiles;
  if (t > max_tiles) t = max_tiles;
  t = (t + kWaves - 1) / kWaves * kWaves;
  return static_cast<int>(t);
}

}  // namespace

hipError_t launch_index_score(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                              bool fp8, const int32_t* vis_len, int B, int n_q, int N_cap,
                              float* scores, float* block_max, hipStream_t stream) {
  const int tiles = (N_cap + 31) / 32;
  const uint8_t* kb = static_cast<const uint8_t*>(k_idx);
  if (n_q < 16) {
    const int rows = B * n_q;
    const int tpw = pick_tiles_per_wg(static_cast<long long>(tiles) * rows, 8, 4096, 64);
    dim3 grid((tiles + tpw - 1) / tpw, rows);
    if (fp8)
      hipLaunchKernelGGL((k_index_scan<true, 2>), grid, dim3(kThreads), 0, stream, q_idx, w_idx,
                         kb, vis_len, n_q, N_cap, tpw, scores, block_max);
    else
      hipLaunchKernelGGL((k_index_scan<false, 1>), grid, dim3(kThreads), 0, stream, q_idx, w_idx,
                         kb, vis_len, n_q, N_cap, tpw, scores, block_max);
  } else {
    return launch_index_gemm(q_idx, w_idx, kb, fp8, vis_len, B, n_q, N_cap, scores, block_max,
                             stream);
  }
  return hipGetLastError();
}

}  // namespace csa2
