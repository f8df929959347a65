// Indexer scores of a prefill chunk: many query rows against the same keys,
// a dense contraction run on matrix cores.
//
// "DeepSeek-V4.1-Flash 架构详解", §3.2 and the §1 configuration table: the
// score of entry t for query row j is  s = sum_{h<32} w_jh max(0, q_jh . k_t)
// over 32 heads of 128 dims; a prefill query sees only its own visible prefix
// (vis_len[j] entries).
//
// Work decomposition.  A workgroup (4 waves) takes 16 query rows of one
// sequence (4 per wave) and a range of 64-key tiles; two workgroups share a
// compute unit (two waves per SIMD).  Every key tile is copied once from
// memory into a 4-slot LDS ring with direct-to-LDS loads (each wave issues
// its share; waits counted by hand; one LDS barrier per tile) and read by all
// four waves, so each key is fetched once per 16 query rows.  A wave keeps
// the A operands of its 4 query rows (32 heads x 128 dims each) in
// accumulation registers for the whole range.  Keys are worked on in
// quarters of 16: per row and quarter, 8 steps of v_mfma_f32_16x16x32_bf16
// (two 16-head blocks x four 32-dim steps).  In that shape a lane holds 8
// heads of one key, so a row needs only 8 head weights in registers, which
// is what lets two waves share a SIMD: the ReLU-weighted head sums of one
// wave run on the vector ALU while the matrix core works for the other.
// The B operands of the next quarter are read from LDS while the current
// one is worked on.  Per 32-key half tile, lane partial sums are combined
// across the four 16-lane groups with two lane-swap steps that also pack two
// rows into one 64-lane store.  Workgroup ids are ordered so that the key
// chunk varies fastest: with a multiple of 8 chunks each XCD always works on
// the same key chunk, which stays in its L2.
#include "csa2_launch.h"
#include "index_core.h"

#include <utility>

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kWgPerCu = 2;   // two workgroups (two waves per SIMD) share a compute unit
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerWg = kRowsPerWave * kWaves;
constexpr int kPairs = (kRowsPerWave + 1) / 2;   // store instructions per tile and output
constexpr int kStages = 4;
constexpr int kChunksPerRow = 8;    // key chunks per query group (one per XCD)

constexpr int kOutScores = 1;
constexpr int kOutBlockMax = 2;
constexpr int kOutScoresBf16 = 4;   // scores stored as bf16 (rounded to nearest even)

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
__global__ __launch_bounds__(kThreads, kWgPerCu) void k_index_gemm(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, Pages pg, const int32_t* __restrict__ vis_len, int n_q,
    int N_cap, int tiles_per_wg, float* __restrict__ scores, float* __restrict__ block_max) {
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
  // With paging, lane l holds the pool page of the workgroup's l-th logical
  // page (the launcher keeps a paged workgroup within 32 tiles of 64 entries
  // and pages hold at least 64: at most 33 pages); a tile never straddles
  // two pages.
  const bool paged = pg.bt != nullptr;
  const int page0 = paged ? (64 * t_begin) >> pg.log2p : 0;
  int my_page = 0;
  if (paged && page0 + lane < pg.max_pages) {
    bool mapped;
    my_page = page_id(pg, b, page0 + lane, mapped);
  }
  // Rows of load u: grow0 + u * (64 / kChunks).
  int goff[KT::kLoadsPerWave];
  const int grow0 = (64 * KT::kLoadsPerWave * wave + lane) / KT::kChunks;
#pragma unroll
  for (int u = 0; u < KT::kLoadsPerWave; ++u) {
    const int p = 64 * (KT::kLoadsPerWave * wave + u) + lane;
    const int row = p / KT::kChunks;
    goff[u] = row * KT::kRowBytes + (((p % KT::kChunks) ^ (row & 7)) << 4);
  }
  auto issue = [&](int t) {
    const int rows_left = N_cap - 64 * t;   // rows of this tile inside the buffer
    const uint8_t* base = kbase + static_cast<size_t>(64) * t * KT::kRowBytes;
    if (paged) {
      const int e = 64 * t;
      const int pid = __shfl(my_page, (e >> pg.log2p) - page0, 64);
      base = k_idx + ((static_cast<size_t>(pid) << pg.log2p) + (e & ((1 << pg.log2p) - 1))) *
                         KT::kRowBytes;
    }
    const uint32_t dst = lds_offset(&ring[static_cast<unsigned>(t - t_begin) % kStages][0]);
#pragma unroll
    for (int u = 0; u < KT::kLoadsPerWave; ++u)
      dma16(base + (grow0 + u * (64 / KT::kChunks) < rows_left ? goff[u] : 0),
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
  constexpr int per_row =
      ((OUT & (kOutScores | kOutScoresBf16)) ? 1 : 0) + ((OUT & kOutBlockMax) ? 1 : 0);

  // Keys are worked on in quarters of 16 (quarter qq: keys 16 qq .. + 15,
  // rows 16 (qq % 4) .. + 15 of tile qq / 4).  B operands of a quarter: lane
  // (c, g) of step ks holds key 16 qq + c, dims dim_base(ks, g) .. + 7.  They
  // are read from LDS as raw bytes one quarter ahead and converted at use.
  constexpr int kRaw = FP8 ? 2 : 4;
  struct Raw {
    u32x4 v[kRaw];
  };
  auto read_raw = [&](int qq) {
    const uint8_t* tile = ring[static_cast<unsigned>((qq >> 2) - t_begin) % kStages];
    const int row = 16 * (qq & 3) + c;
    Raw r;
#pragma unroll
    for (int u = 0; u < kRaw; ++u)
      r.v[u] = *reinterpret_cast<const u32x4*>(tile + KT::pos(row, 4 * u + g));
    return r;
  };
  auto operands = [&](const Raw& r, bf16x8 (&kq)[4]) {
#pragma unroll
    for (int u = 0; u < kRaw; ++u) {
      if constexpr (FP8) {
        kq[2 * u] = fp8x8_to_bf16x8(r.v[u].x, r.v[u].y);
        kq[2 * u + 1] = fp8x8_to_bf16x8(r.v[u].z, r.v[u].w);
      } else {
        kq[u] = __builtin_bit_cast(bf16x8, r.v[u]);
      }
    }
  };

  // Per row, the lane partial sum over its 8 heads (16 hb + 4 g + r) for its
  // key of the quarter: 8 MFMAs (two head blocks x four steps).
  auto quarter = [&](const Raw& raw, float (&part)[kRowsPerWave]) {
    bf16x8 kq[4];
    operands(raw, kq);
    static_for<kRowsPerWave>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      f32x4 d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        d0 = mfma16(qa[i][0][ks], kq[ks], d0);
        d1 = mfma16(qa[i][1][ks], kq[ks], d1);
      }
      float p = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) p = __builtin_fmaf(w8[i][r], relu(d0[r]), p);
#pragma unroll
      for (int r = 0; r < 4; ++r) p = __builtin_fmaf(w8[i][4 + r], relu(d1[r]), p);
      part[i] = p;
    });
  };

  // Scores of half-tile th (keys 32 th .. + 31) from the partial sums of its
  // two quarters.  The first swap adds lane groups g and g ^ 2 and puts key
  // 32 th + c in lanes 0..31, key 32 th + 16 + c in lanes 32..63; the second
  // adds groups g and g ^ 1 and leaves in lane l the score of row
  // i - 1 + ((l / 16) & 1) of a pair (rows i - 1, i), or of row i alone, at
  // key 32 th + (l & 15) + 16 (l / 32).  FULL: every row sees the whole
  // half, so no lane is masked.
  auto finish = [&](int th, const float (&p0)[kRowsPerWave], const float (&p1)[kRowsPerWave],
                    auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int key = 32 * th + c + 16 * (lane >> 5);
    float first = 0.0f;
    static_for<kRowsPerWave>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const float a = swap32_sum(p0[i], p1[i]);
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
        if constexpr (OUT & kOutScoresBf16)
          if (valid) reinterpret_cast<uint16_t*>(scores)[row * N_cap + key] = bf16_rne_bits(sc);
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
  auto finish_half = [&](int th, const float (&p0)[kRowsPerWave],
                         const float (&p1)[kRowsPerWave]) {
    if (32 * th + 32 <= vis_min)
      finish(th, p0, p1, std::true_type{});
    else
      finish(th, p0, p1, std::false_type{});
  };

  // Vector-memory instructions complete in issue order, and the score stores
  // count as well.  Iteration t works on quarters 4t .. 4t + 2, waits for
  // tile t + 1, issues the loads of tile t + 4 and works on quarter 4t + 3;
  // after each odd quarter it makes per output one store per pair of rows
  // with a visible key in that half (lane 0 or 16 then stores, so none is
  // skipped).  When tile t + 1 is waited for, the instructions issued after
  // its loads are the stores of halves 2t - 5 .. 2t and the loads of tiles
  // t + 2 and t + 3 issued in iterations t - 2 and t - 1 (the loads issued
  // before the loop have all completed there).  Counting fewer than were
  // issued would only wait longer.
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

  lds_barrier();   // the first tiles (waited for above) are visible to all waves
  float p0[kRowsPerWave], p1[kRowsPerWave];
  Raw ra = read_raw(4 * t_begin), rb;
  for (int t = t_begin; t < t_end; ++t) {
    const int q = 4 * t;
    rb = read_raw(q + 1);
    quarter(ra, p0);
    ra = read_raw(q + 2);
    quarter(rb, p1);
    finish_half(2 * t, p0, p1);
    rb = read_raw(q + 3);
    quarter(ra, p0);
    if (t + 1 < t_end) {
      int after = loads_in(t - 2, t + 2) + loads_in(t - 1, t + 3);
#pragma unroll
      for (int d = 0; d < 6; ++d) after += stores_of(2 * t - 5 + d);
      if (after == kSteady)
        wait_vmem<kSteady>();
      else
        wait_vmem_le<63>(min(after, 63));
      lds_barrier();   // tile t + 1 has landed; every wave has read tile t
      if (t + kStages < t_end) issue(t + kStages);
      ra = read_raw(q + 4);
    }
    quarter(rb, p1);
    finish_half(2 * t + 1, p0, p1);
  }
}

}  // namespace

hipError_t launch_index_gemm(const uint16_t* q_idx, const float* w_idx, const uint8_t* k_idx,
                             bool fp8, const Pages& pg, const int32_t* vis_len, int B, int n_q,
                             int N_cap, float* scores, float* block_max, hipStream_t stream,
                             bool scores_bf16) {
  const int tiles = (N_cap + 63) / 64;
  int tpw = (tiles + kChunksPerRow - 1) / kChunksPerRow;
  if (pg.bt != nullptr) tpw = tpw < 32 ? tpw : 32;   // at most 33 pages per workgroup
  const int groups = (n_q + kRowsPerWg - 1) / kRowsPerWg;
  dim3 grid((tiles + tpw - 1) / tpw, groups, B);
  const int out = (scores != nullptr ? (scores_bf16 ? kOutScoresBf16 : kOutScores) : 0) |
                  (block_max != nullptr ? kOutBlockMax : 0);
#define CSA2_GEMM_LAUNCH(F, O)                                                                 \
  hipLaunchKernelGGL((k_index_gemm<F, O>), grid, dim3(kThreads), 0, stream, q_idx, w_idx, k_idx, \
                     pg, vis_len, n_q, N_cap, tpw, scores, block_max)
  switch ((fp8 ? 8 : 0) | out) {
    case 1: CSA2_GEMM_LAUNCH(false, 1); break;
    case 2: CSA2_GEMM_LAUNCH(false, 2); break;
    case 3: CSA2_GEMM_LAUNCH(false, 3); break;
    case 4: CSA2_GEMM_LAUNCH(false, 4); break;
    case 9: CSA2_GEMM_LAUNCH(true, 1); break;
    case 10: CSA2_GEMM_LAUNCH(true, 2); break;
    case 11: CSA2_GEMM_LAUNCH(true, 3); break;
    case 12: CSA2_GEMM_LAUNCH(true, 4); break;
    default: return hipErrorInvalidValue;   // no output, or bf16 scores with block maxima
  }
#undef CSA2_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace csa2
