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

constexpr int kOutScores = 1;
constexpr int kOutBlockMax = 2;
constexpr int kOutScoresBf16 = 4;   // scores stored as bf16 (rounded to nearest even)

// Stores of one position's score and of its block's maximum.  Lane 0 always
// holds a visible position of a tile that is worked on, so each requested
// output is written by exactly one store instruction per tile.
template <int OUT>
__device__ __forceinline__ void emit(float s, int pos, int vis, int half, int col, float* scores,
                                     float* block_max) {
  const bool valid = pos < vis;
  if constexpr (OUT & kOutScores)
    if (half == 0 && valid) scores[pos] = s;
  if constexpr (OUT & kOutScoresBf16)
    if (half == 0 && valid) reinterpret_cast<uint16_t*>(scores)[pos] = bf16_rne_bits(s);
  if constexpr (OUT & kOutBlockMax) {
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
// are in flight per wave while it works on one.  One tile ahead with small
// LDS slots (more resident workgroups) streams faster than two or more ahead
// with fewer workgroups.  Vector-memory instructions complete in issue order
// and the output stores count as well, so a tile has landed once no more are
// outstanding than the loads of the tiles issued after it and the stores
// made since.
// MXFP4 keys: the tile's 32 rows of 64 B of E2M1, then (at byte 2048) one
// 4-byte load per lane of the rows' scales (lanes 32..63 repeat lanes
// 0..31, landing in the next 128 bytes).
template <int KD>
struct ScanTile {
  static constexpr int kRowBytes = KeyFmt<KD>::kRowBytes;
  static constexpr int kChunks = kRowBytes / 16;            // 16-B chunks per row
  static constexpr int kDataBytes = 32 * kRowBytes;
  static constexpr int kBytes = kDataBytes + (fp4_keys(KD) ? 256 : 0);   // one tile slot
  static constexpr int kLoads = kDataBytes / 1024 + (fp4_keys(KD) ? 1 : 0);  // loads per tile
  __device__ static int swz(int row) {
    return KD == kKdFp8 ? ((row >> 1) & 7) : KD == kKdBf16 ? (row & 15) : ((row >> 2) & 3);
  }
  __device__ static int pos(int row, int chunk) {            // swizzled byte offset
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
};

template <int KD, int DEPTH, int OUT>
__global__ __launch_bounds__(kThreads) void k_index_scan(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_idx, Pages pg, const int32_t* __restrict__ vis_len, int n_q,
    int N_cap, int tiles_per_wg, float* __restrict__ scores, float* __restrict__ block_max) {
  using TT = ScanTile<KD>;
  constexpr int kStores = ((OUT & (kOutScores | kOutScoresBf16)) ? 1 : 0) +
                          ((OUT & kOutBlockMax) ? 1 : 0);
  constexpr int kSteady = DEPTH * (TT::kLoads + kStores);
  static_assert(kSteady <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][DEPTH + 1][TT::kBytes];
  const int r = blockIdx.y;
  const int b = r / n_q;
  const int vis = min(max(vis_len[r], 0), N_cap);
  const int ntiles = (vis + 31) >> 5;
  const int t_begin = blockIdx.x * tiles_per_wg;
  const int t_end = min(t_begin + tiles_per_wg, ntiles);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  int t = t_begin + wave;
  if (t >= t_end) return;

  QueryOp<KD> qa;
  float wr[16];
  load_query<KD>(qa, q_idx + static_cast<size_t>(r) * kIdxHeads * kIdxDim, col, half);
  load_weights(wr, w_idx + static_cast<size_t>(r) * kIdxHeads, half);
  // With paging, lane l holds the pool page of the workgroup's l-th logical
  // page (a workgroup spans at most 64 tiles of 32 entries, pages hold at
  // least 64 entries: at most 33 pages); a tile never straddles two pages.
  const bool paged = pg.bt != nullptr;
  const int page0 = paged ? (32 * t_begin) >> pg.log2p : 0;
  int my_page = 0;
  if (paged && page0 + lane < pg.max_pages) {
    bool mapped;
    my_page = page_id(pg, b, page0 + lane, mapped);
  }
  // Row r of the scores (bf16 scores: 2 bytes per entry).
  float* srow = scores == nullptr ? nullptr
                : (OUT & kOutScoresBf16)
                    ? reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(scores) +
                                               static_cast<size_t>(r) * N_cap)
                    : scores + static_cast<size_t>(r) * N_cap;
  float* brow = block_max ? block_max + static_cast<size_t>(r) * ((N_cap + 7) >> 3) : nullptr;

  // Source offset (within a tile) of this lane for each of the tile's
  // 16-byte loads.
  constexpr int kData = TT::kDataBytes / 1024;
  int goff[kData];
  int grow[kData];
#pragma unroll
  for (int i = 0; i < kData; ++i) {
    const int g = 64 * i + lane;                  // destination chunk index in the slot
    const int row = g / TT::kChunks, p = g % TT::kChunks;
    grow[i] = row;
    goff[i] = row * TT::kRowBytes + ((p ^ TT::swz(row)) << 4);
  }
  // MXFP4: the scales of all rows follow the rows of E2M1 in the buffer.
  const size_t total_rows = paged ? (static_cast<size_t>(pg.num_pages) << pg.log2p)
                                  : static_cast<size_t>(gridDim.y / n_q) * N_cap;
  const uint8_t* scales = k_idx + total_rows * TT::kRowBytes;
  auto issue = [&](int slot, int tile) {
    const int rows = N_cap - 32 * tile;           // rows of this tile inside the buffer
    size_t row0 = static_cast<size_t>(b) * N_cap + static_cast<size_t>(32) * tile;
    if (paged) {
      const int e = 32 * tile;
      const int pid = __shfl(my_page, (e >> pg.log2p) - page0, 64);
      row0 = (static_cast<size_t>(pid) << pg.log2p) + (e & ((1 << pg.log2p) - 1));
    }
    const uint8_t* base = k_idx + row0 * TT::kRowBytes;
#pragma unroll
    for (int i = 0; i < kData; ++i) {
      const uint8_t* src = base + (grow[i] < rows ? goff[i] : 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)src,
          (__attribute__((address_space(3))) void*)(&stage[wave][slot][i * 1024]), 16, 0,
          2 /* non-temporal */);
    }
    if constexpr (fp4_keys(KD)) {
      const int r = lane & 31;
      const uint8_t* src = scales + (row0 + (r < rows ? r : 0)) * 4;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)src,
          (__attribute__((address_space(3))) void*)(&stage[wave][slot][TT::kDataBytes]), 4, 0,
          2 /* non-temporal */);
    }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (t + d * kWaves < t_end) issue(d, t + d * kWaves);
  int slot = 0;
  for (int k = 0; t < t_end; t += kWaves, ++k) {
    const int tp = t + DEPTH * kWaves;
    if (tp < t_end) issue((slot + DEPTH) % (DEPTH + 1), tp);
    // Issued after tile t's loads: the loads of this wave's next (up to
    // DEPTH) tiles and the stores of its previous min(k, DEPTH) tiles.
    const int ahead = min((t_end - 1 - t) / kWaves, DEPTH);
    const int after = TT::kLoads * ahead + kStores * min(k, DEPTH);
    if (after == kSteady)
      wait_vmem<kSteady>();
    else
      wait_vmem_le<kSteady>(after);
    const uint8_t* st = stage[wave][slot];
    KeyTile<KD> kt;
#pragma unroll
    for (int j = 0; j < KeyTile<KD>::kWords; ++j)
      kt.v[j] = *reinterpret_cast<const u32x4*>(st + TT::pos(col, (TT::kChunks / 2) * half + j));
    if constexpr (fp4_keys(KD))
      kt.sc = *reinterpret_cast<const uint16_t*>(st + TT::kDataBytes + 4 * col + 2 * half);
    const float s = head_sum(key_tile_dot<KD>(qa, kt), wr);
    emit<OUT>(s, 32 * t + col, vis, half, col, srow, brow);
    slot = slot == DEPTH ? 0 : slot + 1;
  }
}

// Tiles per workgroup for about `target_wgs` workgroups over all rows (at
// least min_tiles, at most max_tiles, a multiple of the waves per workgroup).
// Many short workgroups balance better than one resident wave of long ones:
// units that finish early take more work.
int pick_tiles_per_wg(long long total_tiles, int min_tiles, int target_wgs, int max_tiles) {
  long long t = (total_tiles + target_wgs - 1) / target_wgs;
  if (t < min_tiles) t = min_tiles;
  if (t > max_tiles) t = max_tiles;
  t = (t + kWaves - 1) / kWaves * kWaves;
  return static_cast<int>(t);
}

}  // namespace

hipError_t launch_index_score(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                              int kd, const Pages& pg, const int32_t* vis_len, int B, int n_q,
                              int N_cap, float* scores, float* block_max, hipStream_t stream,
                              bool scores_bf16) {
  const int tiles = (N_cap + 31) / 32;
  const uint8_t* kb = static_cast<const uint8_t*>(k_idx);
  if (n_q < 16) {
    const int rows = B * n_q;
    const int out = (scores != nullptr ? (scores_bf16 ? kOutScoresBf16 : kOutScores) : 0) |
                    (block_max != nullptr ? kOutBlockMax : 0);
    const int tpw = pick_tiles_per_wg(static_cast<long long>(tiles) * rows, 8, 4096, 64);
#define CSA2_SCAN_LAUNCH(F, D, O)                                                              \
  do {                                                                                         \
    dim3 grid((tiles + tpw - 1) / tpw, rows);                                                  \
    hipLaunchKernelGGL((k_index_scan<F, D, O>), grid, dim3(kThreads), 0, stream, q_idx, w_idx, \
                       kb, pg, vis_len, n_q, N_cap, tpw, scores, block_max);                   \
  } while (0)
    switch (8 * kd + out) {
      case 1: CSA2_SCAN_LAUNCH(kKdBf16, 1, 1); break;
      case 2: CSA2_SCAN_LAUNCH(kKdBf16, 1, 2); break;
      case 3: CSA2_SCAN_LAUNCH(kKdBf16, 1, 3); break;
      case 4: CSA2_SCAN_LAUNCH(kKdBf16, 1, 4); break;
      case 9: CSA2_SCAN_LAUNCH(kKdFp8, 1, 1); break;
      case 10: CSA2_SCAN_LAUNCH(kKdFp8, 1, 2); break;
      case 11: CSA2_SCAN_LAUNCH(kKdFp8, 1, 3); break;
      case 12: CSA2_SCAN_LAUNCH(kKdFp8, 1, 4); break;
      case 17: CSA2_SCAN_LAUNCH(kKdFp4, 1, 1); break;
      case 18: CSA2_SCAN_LAUNCH(kKdFp4, 1, 2); break;
      case 19: CSA2_SCAN_LAUNCH(kKdFp4, 1, 3); break;
      case 20: CSA2_SCAN_LAUNCH(kKdFp4, 1, 4); break;
      case 25: CSA2_SCAN_LAUNCH(kKdFp4Q, 1, 1); break;
      case 26: CSA2_SCAN_LAUNCH(kKdFp4Q, 1, 2); break;
      case 27: CSA2_SCAN_LAUNCH(kKdFp4Q, 1, 3); break;
      case 28: CSA2_SCAN_LAUNCH(kKdFp4Q, 1, 4); break;
      default: return hipErrorInvalidValue;   // no output, or bf16 scores with block maxima
    }
#undef CSA2_SCAN_LAUNCH
  } else {
    if (fp4_keys(kd)) return hipErrorInvalidValue;   // rejected by the API layer first
    return launch_index_gemm(q_idx, w_idx, kb, kd == kKdFp8, pg, vis_len, B, n_q, N_cap, scores,
                             block_max, stream, scores_bf16);
  }
  return hipGetLastError();
}

}  // namespace csa2
