// Indexer scores of a prefill chunk: many query rows against the same keys,
// a dense contraction run on matrix cores.
//
// "DeepSeek-V4.1-Flash 架构详解", §3.2 and the §1 configuration table: the
// score of entry t for query row j is  s = sum_{h<32} w_jh max(0, q_jh . k_t)
// over 32 heads of 128 dims; a prefill query sees only its own visible prefix
// (vis_len[j] entries).
//
// Work decomposition.  A workgroup (4 waves) takes 28 query rows of one
// sequence (7 per wave) and a range of 32-key tiles.  Every key tile is
// copied once from memory into a 4-slot LDS ring with direct-to-LDS loads
// (each wave issues its share; waits counted by hand; one LDS barrier per
// tile) and read by all four waves, so each key is fetched once per 28 query
// rows.  A wave keeps the A operands of its 7 query rows (32 heads x 128
// dims each) in accumulation registers for the whole range and, per tile and
// row, runs 8 steps of v_mfma_f32_32x32x16_bf16 (32 heads x 32 keys) followed
// by the ReLU-weighted head sum in registers (head weights of its rows held
// in VGPRs), then one 128-byte store of the 32 scores.  Workgroup ids are
// ordered so that the key chunk varies fastest: with a multiple of 8 chunks
// each XCD always works on the same key chunk, which stays in its L2.
#include "csa2_launch.h"
#include "index_core.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 7;   // 8 would not fit the register file
constexpr int kRowsPerWg = kRowsPerWave * kWaves;
constexpr int kStages = 4;
constexpr int kChunksPerRow = 8;    // key chunks per query group (one per XCD)

// A key tile: 32 rows, 16-byte chunk c of row r stored at chunk position
// c ^ f(r), which keeps the B-operand reads (one row per lane) free of LDS
// bank conflicts.
template <bool FP8>
struct KTile {
  static constexpr int kRowBytes = FP8 ? 128 : 256;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = 32 * kRowBytes;
  static constexpr int kLoads = kBytes / 1024;            // 1 KB loads per tile
  static constexpr int kLoadsPerWave = kLoads / kWaves;   // 1 (FP8) or 2 (bf16)
  __device__ static int swz(int row) { return FP8 ? ((row >> 1) & 7) : (row & 15); }
  __device__ static int pos(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
};

// Waits until at most n (0 .. 63) vector-memory instructions of this wave
// are outstanding; n is wave-uniform, the immediate is chosen by a switch.
template <int N>
__device__ __forceinline__ void wait_le(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmem<N>();
      return;
    }
    wait_le<N - 1>(n);
  } else {
    wait_vmem<0>();
  }
}

template <bool FP8>
__global__ __launch_bounds__(kThreads, 1) void k_index_gemm(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ vis_len, int n_q, int N_cap,
    int tiles_per_wg, float* __restrict__ scores, float* __restrict__ block_max) {
  using KT = KTile<FP8>;
  static_assert(kStages == 4, "the wait accounting below assumes 3 tiles issued ahead");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStages][KT::kBytes];

  const int b = blockIdx.z;
  const int j_wg = blockIdx.y * kRowsPerWg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  const size_t row0 = static_cast<size_t>(b) * n_q;

  // Visible lengths: the workgroup's key range is set by its longest row.
  int vis_wg = (col < kRowsPerWg && j_wg + col < n_q)
                   ? min(max(vis_len[row0 + j_wg + col], 0), N_cap) : 0;
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) vis_wg = max(vis_wg, __shfl_xor(vis_wg, d, 64));
  vis_wg = __builtin_amdgcn_readfirstlane(vis_wg);
  const int t_begin = blockIdx.x * tiles_per_wg;
  const int t_end = min(t_begin + tiles_per_wg, (vis_wg + 31) >> 5);
  if (t_begin >= t_end) return;   // the same for the whole workgroup

  const int jw = j_wg + kRowsPerWave * wave;
  int vis[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
    vis[i] = __builtin_amdgcn_readfirstlane(
        (jw + i < n_q) ? min(max(vis_len[row0 + jw + i], 0), N_cap) : 0);

  // Key tiles: wave w issues loads [w LPW, (w + 1) LPW) of every tile.  Lane
  // l of load i fills chunk position g = 64 i + l (row g / kChunks, position
  // g % kChunks), i.e. it reads chunk (g % kChunks) ^ swz(row) of that row.
  const uint8_t* kb = k_idx + static_cast<size_t>(b) * N_cap * KT::kRowBytes;
  int goff[KT::kLoadsPerWave], grow[KT::kLoadsPerWave];
#pragma unroll
  for (int u = 0; u < KT::kLoadsPerWave; ++u) {
    const int g = 64 * (KT::kLoadsPerWave * wave + u) + lane;
    const int row = g / KT::kChunks, p = g % KT::kChunks;
    grow[u] = row;
    goff[u] = row * KT::kRowBytes + ((p ^ KT::swz(row)) << 4);
  }
  auto issue = [&](int t) {
    const int rows_left = N_cap - 32 * t;   // rows of this tile inside the buffer
    const uint8_t* base = kb + static_cast<size_t>(32) * t * KT::kRowBytes;
    const uint32_t dst = lds_offset(&ring[(t - t_begin) % kStages][0]);
#pragma unroll
    for (int u = 0; u < KT::kLoadsPerWave; ++u)
      dma16(base + (grow[u] < rows_left ? goff[u] : 0),
            dst + 1024 * (KT::kLoadsPerWave * wave + u));
  };
#pragma unroll
  for (int d = 0; d < kStages - 1; ++d)
    if (t_begin + d < t_end) issue(t_begin + d);

  // Query operands (lane: head col, dims 64 half + 8 s) of the wave's rows,
  // and the head weights of the 16 accumulator rows each lane holds.
  bf16x8 qa[kRowsPerWave][8];
  float wr[kRowsPerWave][16];
  {
    u32x4 qv[kRowsPerWave][8];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int j = min(jw + i, n_q - 1);
      const u32x4* p = reinterpret_cast<const u32x4*>(
          q_idx + ((row0 + j) * kIdxHeads + col) * kIdxDim + 64 * half);
#pragma unroll
      for (int s = 0; s < 8; ++s) qv[i][s] = p[s];
      load_weights(wr[i], w_idx + (row0 + j) * kIdxHeads, half);
    }
    // These plain loads finish before the loop: only direct-to-LDS loads are
    // in flight inside it.
    wait_vmem<0>();
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
      for (int s = 0; s < 8; ++s) qa[i][s] = __builtin_bit_cast(bf16x8, to_agpr(qv[i][s]));
  }
  const size_t nb_cap = (N_cap + 7) >> 3;
  const int per_row = (scores != nullptr) + (block_max != nullptr);

  // Vector-memory instructions complete in issue order, and the score stores
  // count as well.  Iteration t issues the loads of tile t + 3, then one
  // store per output for each row that sees tile t (lane 0 always has a
  // store to make, so none is skipped).  Before tile t is read, the
  // instructions issued after its loads are therefore the stores of
  // iterations t - 3 .. t - 1 and the loads of tiles t + 1 and t + 2.
  auto stores_of = [&](int tt) {
    if (tt < t_begin) return 0;
    int n = 0;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) n += (32 * tt < vis[i]) ? per_row : 0;
    return n;
  };
  for (int t = t_begin; t < t_end; ++t) {
    const int after = stores_of(t - 3) + stores_of(t - 2) + stores_of(t - 1) +
                      KT::kLoadsPerWave * (min(t_end - 1 - t, kStages - 2));
    wait_le<63>(min(after, 63));
    lds_barrier();   // every wave's share of tile t has landed; tile t - 1 is done
    if (t + kStages - 1 < t_end) issue(t + kStages - 1);

    // B operands: lane (col, half) reads dims 64 half .. + 63 of key row col.
    const uint8_t* tile = ring[(t - t_begin) % kStages];
    bf16x8 kop[8];
    if constexpr (FP8) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(tile + KT::pos(col, 4 * half + s2));
        kop[2 * s2] = fp8x8_to_bf16x8(w.x, w.y);
        kop[2 * s2 + 1] = fp8x8_to_bf16x8(w.z, w.w);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        kop[s] = *reinterpret_cast<const bf16x8*>(tile + KT::pos(col, 8 * half + s));
    }

#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (32 * t >= vis[i]) continue;   // wave-uniform
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) acc = mfma32(qa[i][s], kop[s], acc);
      const float sc = head_sum(acc, wr[i]);
      const int pos = 32 * t + col;
      const bool valid = pos < vis[i];
      const size_t row = row0 + jw + i;
      if (scores != nullptr && half == 0 && valid) scores[row * N_cap + pos] = sc;
      if (block_max != nullptr) {
        float m = valid ? sc : -__builtin_inff();
        m = fmaxf(m, wave_xor(m, 1));
        m = fmaxf(m, wave_xor(m, 2));
        m = fmaxf(m, wave_xor(m, 4));
        if (half == 0 && (col & 7) == 0 && valid) block_max[row * nb_cap + (pos >> 3)] = m;
      }
    }
  }
}

}  // namespace

hipError_t launch_index_gemm(const uint16_t* q_idx, const float* w_idx, const uint8_t* k_idx,
                             bool fp8, const int32_t* vis_len, int B, int n_q, int N_cap,
                             float* scores, float* block_max, hipStream_t stream) {
  const int tiles = (N_cap + 31) / 32;
  const int tpw = (tiles + kChunksPerRow - 1) / kChunksPerRow;
  const int groups = (n_q + kRowsPerWg - 1) / kRowsPerWg;
  dim3 grid((tiles + tpw - 1) / tpw, groups, B);
  if (fp8)
    hipLaunchKernelGGL(k_index_gemm<true>, grid, dim3(kThreads), 0, stream, q_idx, w_idx, k_idx,
                       vis_len, n_q, N_cap, tpw, scores, block_max);
  else
    hipLaunchKernelGGL(k_index_gemm<false>, grid, dim3(kThreads), 0, stream, q_idx, w_idx, k_idx,
                       vis_len, n_q, N_cap, tpw, scores, block_max);
  return hipGetLastError();
}

}  // namespace csa2
