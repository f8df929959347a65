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

// Decode: one query row per workgroup row (blockIdx.y); the workgroup's four
// waves take interleaved 32-position tiles of its chunk, one tile ahead in
// flight.
template <bool FP8>
__global__ __launch_bounds__(kThreads) void k_index_scan(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ vis_len, int n_q, int N_cap,
    int tiles_per_wg, float* __restrict__ scores, float* __restrict__ block_max) {
  const int r = blockIdx.y;
  const int b = r / n_q;
  const int vis = min(max(vis_len[r], 0), N_cap);
  const int ntiles = (vis + 31) >> 5;
  const int t_begin = blockIdx.x * tiles_per_wg;
  if (t_begin >= ntiles) return;
  const int t_end = min(t_begin + tiles_per_wg, ntiles);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;

  bf16x8 qa[8];
  float wr[16];
  load_query(qa, q_idx + static_cast<size_t>(r) * kIdxHeads * kIdxDim, col, half);
  load_weights(wr, w_idx + static_cast<size_t>(r) * kIdxHeads, half);
  const uint8_t* kb = k_idx + static_cast<size_t>(b) * N_cap * (FP8 ? 128 : 256);
  float* srow = scores ? scores + static_cast<size_t>(r) * N_cap : nullptr;
  float* brow = block_max ? block_max + static_cast<size_t>(r) * ((N_cap + 7) >> 3) : nullptr;

  int t = t_begin + wave;
  if (t >= t_end) return;
  KeyTile<FP8> cur, nxt;
  load_key_half<FP8>(cur, key_row<FP8>(kb, 32 * t + col, N_cap), half);
  for (; t < t_end; t += kWaves) {
    const int tn = t + kWaves;
    if (tn < t_end) load_key_half<FP8>(nxt, key_row<FP8>(kb, 32 * tn + col, N_cap), half);
    const float s = head_sum(key_tile_dot<FP8>(qa, cur), wr);
    emit(s, 32 * t + col, vis, half, col, srow, brow);
    cur = nxt;
  }
}

// Prefill chunk: a workgroup takes 16 query rows of one sequence (4 per wave)
// and a range of key tiles; each wave reuses every key tile it loads for its
// 4 rows.  Query rows only see their own visible prefix.
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerWg = kRowsPerWave * kWaves;

template <bool FP8>
__global__ __launch_bounds__(kThreads) void k_index_gemm(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ vis_len, int n_q, int N_cap,
    int tiles_per_wg, float* __restrict__ scores, float* __restrict__ block_max) {
  __shared__ float w_lds[kRowsPerWg][kIdxHeads];
  const int b = blockIdx.z;
  const int j_wg = blockIdx.y * kRowsPerWg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  const size_t row0 = static_cast<size_t>(b) * n_q;

  for (int i = threadIdx.x; i < kRowsPerWg * kIdxHeads; i += kThreads) {
    const int j = j_wg + i / kIdxHeads;
    w_lds[i / kIdxHeads][i % kIdxHeads] = j < n_q ? w_idx[(row0 + j) * kIdxHeads + i % kIdxHeads] : 0.0f;
  }
  __syncthreads();

  const int j0 = j_wg + wave * kRowsPerWave;
  int vis[kRowsPerWave];
  int vis_max = 0;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    vis[i] = (j0 + i < n_q) ? min(max(vis_len[row0 + j0 + i], 0), N_cap) : 0;
    vis_max = max(vis_max, vis[i]);
  }
  const int t_begin = blockIdx.x * tiles_per_wg;
  const int t_end = min(t_begin + tiles_per_wg, (vis_max + 31) >> 5);
  if (t_begin >= t_end) return;

  bf16x8 qa[kRowsPerWave][8];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int j = min(j0 + i, n_q - 1);
    load_query(qa[i], q_idx + (row0 + j) * kIdxHeads * kIdxDim, col, half);
  }
  const uint8_t* kb = k_idx + static_cast<size_t>(b) * N_cap * (FP8 ? 128 : 256);
  const size_t nb_cap = (N_cap + 7) >> 3;

  KeyTile<FP8> cur, nxt;
  load_key_half<FP8>(cur, key_row<FP8>(kb, 32 * t_begin + col, N_cap), half);
  for (int t = t_begin; t < t_end; ++t) {
    if (t + 1 < t_end) load_key_half<FP8>(nxt, key_row<FP8>(kb, 32 * (t + 1) + col, N_cap), half);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (32 * t >= vis[i]) continue;  // wave-uniform
      float wr[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) wr[rr] = w_lds[wave * kRowsPerWave + i][8 * (rr / 4) + 4 * half + (rr % 4)];
      const float s = head_sum(key_tile_dot<FP8>(qa[i], cur), wr);
      const size_t row = row0 + j0 + i;
      emit(s, 32 * t + col, vis[i], half, col, scores ? scores + row * N_cap : nullptr,
           block_max ? block_max + row * nb_cap : nullptr);
    }
    cur = nxt;
  }
}

int pick_tiles_per_wg(long long total_tiles, int min_tiles, int target_wgs) {
  long long t = (total_tiles + target_wgs - 1) / target_wgs;
  if (t < min_tiles) t = min_tiles;
  t = (t + kWaves - 1) / kWaves * kWaves;
  return static_cast<int>(t);
}

}  // namespace

hipError_t launch_index_score(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                              bool fp8, const int32_t* vis_len, int B, int n_q, int N_cap,
                              float* scores, float* block_max, hipStream_t stream) {
  const int tiles = (N_cap + 31) / 32;
  const uint8_t* kb = static_cast<const uint8_t*>(k_idx);
  if (n_q < kRowsPerWg) {
    const int rows = B * n_q;
    const int tpw = pick_tiles_per_wg(static_cast<long long>(tiles) * rows, 8, 2048);
    dim3 grid((tiles + tpw - 1) / tpw, rows);
    if (fp8)
      hipLaunchKernelGGL(k_index_scan<true>, grid, dim3(kThreads), 0, stream, q_idx, w_idx, kb,
                         vis_len, n_q, N_cap, tpw, scores, block_max);
    else
      hipLaunchKernelGGL(k_index_scan<false>, grid, dim3(kThreads), 0, stream, q_idx, w_idx, kb,
                         vis_len, n_q, N_cap, tpw, scores, block_max);
  } else {
    const int groups = (n_q + kRowsPerWg - 1) / kRowsPerWg;
    const int tpw = 64;
    dim3 grid((tiles + tpw - 1) / tpw, groups, B);
    if (fp8)
      hipLaunchKernelGGL(k_index_gemm<true>, grid, dim3(kThreads), 0, stream, q_idx, w_idx, kb,
                         vis_len, n_q, N_cap, tpw, scores, block_max);
    else
      hipLaunchKernelGGL(k_index_gemm<false>, grid, dim3(kThreads), 0, stream, q_idx, w_idx, kb,
                         vis_len, n_q, N_cap, tpw, scores, block_max);
  }
  return hipGetLastError();
}

}  // namespace csa2
