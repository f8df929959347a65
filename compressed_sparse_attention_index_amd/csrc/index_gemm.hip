// Indexer scores of a prefill chunk: many query rows against the same keys,
// a dense contraction run on matrix cores.
//
// "DeepSeek-V4.1-Flash 架构详解", §3.2 and the §1 configuration table: the
// score of entry t for query row j is  s = sum_{h<32} w_jh max(0, q_jh . k_t)
// over 32 heads of 128 dims; a prefill query sees only its own visible prefix
// (vis_len[j] entries).
//
// Work decomposition.  A workgroup (4 waves) takes 32 query rows of one
// sequence (8 per wave) and a range of 64-key tiles.  Every key tile is
// copied once from memory into a 4-slot LDS ring with direct-to-LDS loads
// (each wave issues its share; waits counted by hand; one LDS barrier per
// tile) and read by all four waves, so each key is fetched once per 32 query
// rows.  A tile is worked on in two 32-key halves.  A wave keeps the A operands of its 8 query rows (32 heads x 128
// dims each) in accumulation registers for the whole range.  Per tile and
// row and half it runs 16 steps of v_mfma_f32_16x16x32_bf16 (two 16-head blocks x two
// 16-key blocks x four 32-dim steps).  In that shape a lane holds 8 heads of
// 2 keys, so a row needs only 8 head weights in registers, which leaves room
// for a second accumulator set and for the next tile's B operands: the
// ReLU-weighted head sum of one row runs on the vector ALU while the matrix
// core works on the next row, and the LDS reads of the next half are in
// flight while the current half is worked on.  Lane partial sums are combined across the four
// 16-lane groups with two lane-swap steps that also pack two rows into one
// 64-lane store.  Workgroup ids are ordered so that the key chunk varies
// fastest: with a multiple of 8 chunks each XCD always works on the same key
// chunk, which stays in its L2.
#include "csa2_launch.h"
#include "index_core.h"

#include <utility>

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 8;
constexpr int kRowsPerWg = kRowsPerWave * kWaves;
constexpr int kPairs = (kRowsPerWave + 1) / 2;   // store instructions per tile and output
constexpr int kStages = 4;
constexpr int kChunksPerRow = 8;    // key chunks per query group (one per XCD)

constexpr int kOutScores = 1;
constexpr int kOutBlockMax = 2;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A key tile: 64 rows, 16-byte chunk c of row r stored at chunk position
// c ^ (r & 7), so that eight lanes reading the same chunk of eight
// consecutive rows hit eight different bank groups.
template <bool FP8>
struct KTile {
  static constexpr int kRowBytes = FP8 ? 128 : 256;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = 64 * kRowBytes;
  static constexpr int kLoads = kBytes / 1024;            // 1 KB loads per tile
  static constexpr int kLoadsPerWave = kLoads / kWaves;   // 2 (FP8) or 4 (bf16)
  __device__ static int pos(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
  }
};

// The contraction over the 128 dims is split into four MFMA steps ks of 32;
// lane group g (lane / 16) supplies 8 consecutive dims of each step.  Which
// dims those are is free as long as A and B agree; they are chosen so that a
// lane's B operands are whole 16-byte chunks of the key row:
//   bf16 keys: step ks, group g -> dims 32 ks + 8 g .. + 7     (chunk 4 ks + g)
//   FP8 keys:  step ks, group g -> dims 64 (ks / 2) + 16 g + 8 (ks % 2) .. + 7
//              (steps 2u and 2u + 1 share chunk 4 u + g)
template <bool FP8>
__device__ __forceinline__ int dim_base(int ks, int g) {
  return FP8 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : 32 * ks + 8 * g;
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N - 1 in order, so
// that I can be used where a constant expression is required.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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

// Sum of the values of lanes l and l ^ 32: of a in lanes 0..31, of b in
// lanes 32..63.
__device__ __forceinline__ float swap32_sum(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum of the values of lanes l and l ^ 16: of a in 16-lane rows 0 and 2, of
// b in rows 1 and 3.
__device__ __forceinline__ float swap16_sum(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct Acc {
  f32x4 d[2][2];   // [head block][key block]
};

template <bool FP8, int OUT>
__global__ __launch_bounds__(kThreads, 1) void k_index_gemm(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ vis_len, int n_q, int N_cap,
    int tiles_per_wg, float* __restrict__ scores, float* __restrict__ block_max) {
  using KT = KTile<FP8>;
  static_assert(kStages == 4, "the wait accounting below assumes this ring depth");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStages][KT::kBytes];

  const int b = blockIdx.z;
  const int j_wg = blockIdx.y * kRowsPerWg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const size_t row0 = static_cast<size_t>(b) * n_q;

  // Visible lengths: the workgroup's key range is set by its longest row.
  const int r32 = lane & 31;
  int vis_wg = (r32 < kRowsPerWg && j_wg + r32 < n_q)
                   ? min(max(vis_len[row0 + j_wg + r32], 0), N_cap) : 0;
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) vis_wg = max(vis_wg, __shfl_xor(vis_wg, d, 64));
  vis_wg = __builtin_amdgcn_readfirstlane(vis_wg);
  const int t_begin = blockIdx.x * tiles_per_wg;
  const int t_end = min(t_begin + tiles_per_wg, (vis_wg + 63) >> 6);
  if (t_begin >= t_end) return;   // the same for the whole workgroup

  const int jw = j_wg + kRowsPerWave * wave;
  int vis[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
    vis[i] = __builtin_amdgcn_readfirstlane(
        (jw + i < n_q) ? min(max(vis_len[row0 + jw + i], 0), N_cap) : 0);
  int vis_min = vis[0];
#pragma unroll
  for (int i = 1; i < kRowsPerWave; ++i) vis_min = min(vis_min, vis[i]);

  // Key tiles: wave w issues loads [w LPW, (w + 1) LPW) of every tile.  Lane
  // l of load u fills chunk position p = 64 (w LPW + u) + l (row p /
  // kChunks), which holds chunk (p % kChunks) ^ (row & 7) of that row.
  const uint8_t* kbase = k_idx + static_cast<size_t>(b) * N_cap * KT::kRowBytes;
  int goff[KT::kLoadsPerWave], grow[KT::kLoadsPerWave];
#pragma unroll
  for (int u = 0; u < KT::kLoadsPerWave; ++u) {
    const int p = 64 * (KT::kLoadsPerWave * wave + u) + lane;
    const int row = p / KT::kChunks;
    grow[u] = row;
    goff[u] = row * KT::kRowBytes + (((p % KT::kChunks) ^ (row & 7)) << 4);
  }
  auto issue = [&](int t) {
    const int rows_left = N_cap - 64 * t;   // rows of this tile inside the buffer
    const uint8_t* base = kbase + static_cast<size_t>(64) * t * KT::kRowBytes;
    const uint32_t dst = lds_offset(&ring[static_cast<unsigned>(t - t_begin) % kStages][0]);
#pragma unroll
    for (int u = 0; u < KT::kLoadsPerWave; ++u)
      dma16(base + (grow[u] < rows_left ? goff[u] : 0),
            dst + 1024 * (KT::kLoadsPerWave * wave + u));
  };
#pragma unroll
  for (int d = 0; d < kStages; ++d)
    if (t_begin + d < t_end) issue(t_begin + d);

  // A operands: lane (c, g) of head block hb and step ks holds head
  // 16 hb + c, dims dim_base(ks, g) .. + 7.  Head weights: accumulator value
  // r of head block hb belongs to head 16 hb + 4 g + r.
  bf16x8 qa[kRowsPerWave][2][4];
  float w8[kRowsPerWave][8];
  {
    u32x4 qv[kRowsPerWave][2][4];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const size_t j = row0 + min(jw + i, n_q - 1);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qv[i][hb][ks] = *reinterpret_cast<const u32x4*>(
              q_idx + (j * kIdxHeads + 16 * hb + c) * kIdxDim + dim_base<FP8>(ks, g));
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const f32x4 w =
            *reinterpret_cast<const f32x4*>(w_idx + j * kIdxHeads + 16 * hb + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) w8[i][4 * hb + r] = w[r];
      }
    }
    // These plain loads finish before the loop: only direct-to-LDS loads are
    // in flight inside it.
    wait_vmem<0>();
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qa[i][hb][ks] = __builtin_bit_cast(bf16x8, to_agpr(qv[i][hb][ks]));
  }
  const size_t nb_cap = (N_cap + 7) >> 3;
  constexpr int per_row = ((OUT & kOutScores) ? 1 : 0) + ((OUT & kOutBlockMax) ? 1 : 0);

  // B operands of half h of tile t: lane (c, g) of key block kb and step ks
  // holds key 64 t + 32 h + 16 kb + c, dims dim_base(ks, g) .. + 7.
  auto read_kop = [&](int t, int h, bf16x8 (&kop)[2][4]) {
    const uint8_t* tile = ring[static_cast<unsigned>(t - t_begin) % kStages] + 32 * h * KT::kRowBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (FP8) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 w =
              *reinterpret_cast<const u32x4*>(tile + KT::pos(16 * kb + c, 4 * u + g));
          kop[kb][2 * u] = fp8x8_to_bf16x8(w.x, w.y);
          kop[kb][2 * u + 1] = fp8x8_to_bf16x8(w.z, w.w);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kop[kb][ks] = *reinterpret_cast<const bf16x8*>(tile + KT::pos(16 * kb + c, 4 * ks + g));
      }
    }
  };

  // One row's 16 MFMAs: four independent accumulator chains.
  auto mma_row = [&](int i, const bf16x8 (&kop)[2][4]) {
    Acc a;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) a.d[hb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          a.d[hb][kb] = mfma16(qa[i][hb][ks], kop[kb][ks], a.d[hb][kb]);
    return a;
  };

  // Lane partial sums over the lane's 8 heads, for keys c (key block 0) and
  // 16 + c (key block 1), summed over lane groups g and g ^ 2: lanes 0..31
  // then hold key c, lanes 32..63 key 16 + c.
  auto row_part = [&](int i, const Acc& a) {
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p0 = __builtin_fmaf(w8[i][4 * hb + r], relu(a.d[hb][0][r]), p0);
        p1 = __builtin_fmaf(w8[i][4 * hb + r], relu(a.d[hb][1][r]), p1);
      }
    return swap32_sum(p0, p1);
  };

  // Scores of half-tile th (keys 32 th .. + 31).  After the second swap,
  // lane l holds the score of row i - 1 + ((l / 16) & 1) for a pair (rows
  // i - 1, i), or of row i alone, at key 32 th + (l & 15) + 16 (l / 32).
  // FULL: every row sees the whole half, so no lane is masked.
  auto compute = [&](int th, const bf16x8 (&kop)[2][4], auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int key = 32 * th + c + 16 * (lane >> 5);
    Acc acc = mma_row(0, kop);
    float first = 0.0f;
    static_for<kRowsPerWave>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      Acc next;
      if constexpr (i + 1 < kRowsPerWave) next = mma_row(i + 1, kop);
      const float a = row_part(i, acc);
      if constexpr (i + 1 < kRowsPerWave) acc = next;
      constexpr bool single = (i == kRowsPerWave - 1) && (i % 2 == 0);
      if constexpr (i % 2 == 0 && !single) {
        first = a;
      } else {
        const float sc = single ? swap16_sum(a, a) : swap16_sum(first, a);
        const int ir = single ? i : i - 1 + (g & 1);
        // Arithmetic select: a conditional pick of two array elements would
        // become a per-lane array index (private memory).
        const int v_lo = single ? vis[i] : vis[i - 1];
        const int vis_r = v_lo + ((vis[i] - v_lo) & -(g & 1));
        const bool valid = FULL || key < vis_r;
        const size_t row = row0 + jw + ir;
        if constexpr (OUT & kOutScores)
          if (valid) scores[row * N_cap + key] = sc;
        if constexpr (OUT & kOutBlockMax) {
          float m = valid ? sc : -__builtin_inff();
          m = fmaxf(m, wave_xor(m, 1));
          m = fmaxf(m, wave_xor(m, 2));
          m = fmaxf(m, wave_xor(m, 4));
          if (FULL || ((c & 7) == 0 && valid)) block_max[row * nb_cap + (key >> 3)] = m;
        }
      }
    });
  };

  // Vector-memory instructions complete in issue order, and the score stores
  // count as well.  Iteration t works on half 0 of tile t, waits for tile
  // t + 1, issues the loads of tile t + 4 and works on half 1; per half and
  // output it makes one store per pair of rows with a visible key there
  // (lane 0 or 16 then stores, so none is skipped).  When tile t + 1 is
  // waited for, the instructions issued after its loads are the stores of
  // halves 2t - 5 .. 2t and the loads of tiles t + 2 and t + 3 issued in
  // iterations t - 2 and t - 1 (the loads issued before the loop have all
  // completed there).  Counting fewer than were issued would only wait
  // longer.
  auto stores_of = [&](int th) {   // th: half-tile index
    if (th < 2 * t_begin) return 0;
    if (32 * th + 32 <= vis_min) return kPairs * per_row;
    int n = 0;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; i += 2) {
      const int v = (i + 1 < kRowsPerWave) ? max(vis[i], vis[i + 1]) : vis[i];
      n += (32 * th < v) ? per_row : 0;
    }
    return n;
  };
  auto loads_in = [&](int it, int tile) {
    return (it >= t_begin && tile < t_end) ? KT::kLoadsPerWave : 0;
  };
  constexpr int kSteady = 6 * kPairs * per_row + 2 * KT::kLoadsPerWave;
  static_assert(kSteady <= 63, "vmcnt range");

  auto half = [&](int th, const bf16x8 (&kop)[2][4]) {
    if (32 * th + 32 <= vis_min)
      compute(th, kop, std::true_type{});
    else
      compute(th, kop, std::false_type{});
  };

  lds_barrier();   // the first tiles (waited for above) are visible to all waves
  bf16x8 kop_a[2][4], kop_b[2][4];
  read_kop(t_begin, 0, kop_a);
  for (int t = t_begin; t < t_end; ++t) {
    half(2 * t, kop_a);
    read_kop(t, 1, kop_b);
    if (t + 1 < t_end) {
      int after = loads_in(t - 2, t + 2) + loads_in(t - 1, t + 3);
#pragma unroll
      for (int d = 0; d < 6; ++d) after += stores_of(2 * t - 5 + d);
      if (after == kSteady)
        wait_vmem<kSteady>();
      else
        wait_le<63>(min(after, 63));
      lds_barrier();   // tile t + 1 has landed; every wave has read tile t
      if (t + kStages < t_end) issue(t + kStages);
      read_kop(t + 1, 0, kop_a);
    }
    half(2 * t + 1, kop_b);
  }
}

}  // namespace

hipError_t launch_index_gemm(const uint16_t* q_idx, const float* w_idx, const uint8_t* k_idx,
                             bool fp8, const int32_t* vis_len, int B, int n_q, int N_cap,
                             float* scores, float* block_max, hipStream_t stream) {
  const int tiles = (N_cap + 63) / 64;
  const int tpw = (tiles + kChunksPerRow - 1) / kChunksPerRow;
  const int groups = (n_q + kRowsPerWg - 1) / kRowsPerWg;
  dim3 grid((tiles + tpw - 1) / tpw, groups, B);
  const int out = (scores != nullptr ? kOutScores : 0) | (block_max != nullptr ? kOutBlockMax : 0);
#define CSA2_GEMM_LAUNCH(F, O)                                                                 \
  hipLaunchKernelGGL((k_index_gemm<F, O>), grid, dim3(kThreads), 0, stream, q_idx, w_idx, k_idx, \
                     vis_len, n_q, N_cap, tpw, scores, block_max)
  switch ((fp8 ? 4 : 0) | out) {
    case 1: CSA2_GEMM_LAUNCH(false, 1); break;
    case 2: CSA2_GEMM_LAUNCH(false, 2); break;
    case 3: CSA2_GEMM_LAUNCH(false, 3); break;
    case 5: CSA2_GEMM_LAUNCH(true, 1); break;
    case 6: CSA2_GEMM_LAUNCH(true, 2); break;
    case 7: CSA2_GEMM_LAUNCH(true, 3); break;
    default: return hipErrorInvalidValue;   // no output requested
  }
#undef CSA2_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace csa2
