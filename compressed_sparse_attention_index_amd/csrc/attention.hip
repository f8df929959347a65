// Sparse multi-query attention over the selected MXFP4 main-KV entries plus
// the FP8 sliding window, with one softmax across both.
//
// "DeepSeek-V4.1-Flash 架构详解": §1 configuration table (64 query heads of
// 512 dims, window 128), §4 (main KV is MXFP4 and is dequantised before
// attention, SWA KV is FP8), §9 step 5 (decode attends to the CSA2-selected
// global KV plus this layer's SWA KV).  DeepSeek-V4 essay (mlqm.cn) §4.3: a
// compressed entry serves as both key and value; §6.4: kernels are batch
// invariant (a query gives the same bits whatever else is in the batch).
//
// Work decomposition.  A query row's 64 heads are split into four groups of
// 16; one workgroup takes one (row, head group) and walks the row's whole
// entry list
//   [ top_k selected slots, padded to a multiple of 32 | 128 window slots ]
// in tiles of 32 entries.  The four workgroups of a row get ids that differ
// by 8, so they run on the same XCD and its L2 serves the row's gathers to
// all four.  No row is ever split across workgroups over its entries: there
// are no partial results in memory, no merge kernel and no workspace, and
// the arithmetic of a row (tile order, wave assignment, merge order) depends
// only on top_k and the row's own data, never on the other rows of the call.
//
// A workgroup is 8 waves in 4 pairs; pair p takes tiles p, p + 4, ...; wave
// (p, d) of a pair covers dims half d (256 dims).  Per tile, without waiting
// on the other pairs except at two workgroup barriers:
//   1. gather: lane (m, c) = (lane % 16, lane / 16) loads, for entries m and
//      16 + m, 32 bytes of E2M1 (dims 256 d + 64 c .. + 64) and the dword
//      holding their two E8M0 scales, or 64 FP8 bytes of the same dims for
//      window entries, straight into registers, one tile ahead;
//   2. exact dequantisation to bf16 (gfx950 scaled conversions) in the
//      A-operand layout of v_mfma_f32_16x16x32_bf16 with entries on M:
//      partial S^T[entry][head] = K . q^T over the wave's dims, contraction
//      step s taking dims 256 d + 64 c + 8 s .. + 8 from lane group c (q^T,
//      the B operand, holds the same dims for the whole row); each converted
//      16-byte piece also goes to the wave's private LDS tile;
//   3. the two waves of the pair exchange their partial sums through LDS
//      (barrier), both form S = S_0 + S_1 and run the same softmax in log2
//      units against a per-head reference that moves only when a tile's
//      maximum exceeds it by more than kLazyRescale.  The accumulator layout
//      of S^T (lane (head, c) holds entries 4 c + i and 16 + 4 c + i) is
//      already the B-operand layout of P^T for the PV product;
//   4. O^T[dim][head] += V^T . P^T over the tile's 32 entries for the wave's
//      256 dims, V^T read from its own LDS tile with transposing reads
//      (ds_read_b64_tr_b16); a second barrier frees the exchange buffer.
// At the end the four pairs' (reference, sum, O^T) are merged in pair order
// through LDS and each wave writes 64 dims of the 16 heads.
#include "csa2_launch.h"
#include "csa2_device.h"

namespace csa2 {
namespace {

constexpr int kWaves = 8;
constexpr int kPairs = kWaves / 2;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsPerWg = 16;
constexpr int kGroupsPerRow = kHeads / kHeadsPerWg;
constexpr int kTile = 32;                    // entries per tile
constexpr int kHalfDims = kDim / 2;          // dims of one wave of a pair
// LDS row of one dequantised half entry (512 bytes) plus 32 bytes of padding:
// row r then starts 32 r bytes (mod 256) into the 64 banks, so the 16-byte
// stores of 8 consecutive rows, and the 32-byte pieces a transposing read
// takes from 8 consecutive rows, each fall in distinct banks with no
// address swizzle (every per-step offset is an immediate).
constexpr int kRowBytes = kHalfDims * 2 + 32;
constexpr int kTileBytes = kTile * kRowBytes;
static_assert(kMaxWindow == kTile * 4, "one window tile per pair");
constexpr int kDimTiles = kHalfDims / 16;    // 16-dim tiles of O^T per wave
// Staging in a wave's own tile region before its first dequantised store:
// the q rows of the workgroup's 16 heads over the wave's dims half (16 x
// 512 bytes, row stride kQStride) and the raw FP8 bytes of its window
// tile's 32 rows over the same half (32 x 256 bytes, stride kWStride, from
// byte kWinStage).  Each load instruction then covers whole 128-byte lines
// (instead of one 16-byte piece of 64 different lines), and the operands
// are read back from LDS in the MFMA layouts; with these strides the 16
// rows one read touches fall in distinct banks.
constexpr int kQStride = 528;
constexpr int kWStride = 272;
constexpr int kWinStage = 16 * kQStride;
static_assert(kWinStage + kTile * kWStride <= kTileBytes, "staging fits the tile");
constexpr int kSteps = kHalfDims / 32;       // contraction steps of the partial S
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;
static_assert(kGroupsPerRow == 4, "row = 4 head groups");
static_assert(kMaxWindow % kTile == 0 && kMaxTopK % kTile == 0, "whole tiles");

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* kv_fp4;
  const uint8_t* kv_scale;
  const int32_t* idx;
  const uint8_t* swa;
  const int32_t* swa_pos0;
  const int32_t* q_pos;
  uint16_t* out;
  float* lse;
  const float* sink;   // [64] per-head sink logits (natural log), or null
  Pages pg;            // main-KV page table (pg.bt == nullptr: contiguous)
  int N_cap, top_k, S_cap, n_q, window, replay_start, rows;
  float scale2;        // sm_scale * log2(e)
};

struct Smem {
  uint8_t tile[kWaves][kTileBytes];     // dequantised half entries [entry][dims]; O^T at the end
  f32x4_t xs[kWaves][2][64];            // partial S^T handed to the partner
  float ml[kPairs][kHeadsPerWg][2];     // per pair and head: reference max (log2), sum
  int32_t ids[kMaxTopK];                // the row's selected ids (-1: no entry)
  uint32_t ready[kWaves];               // last round whose partial is in xs[wave]
  uint32_t taken[kWaves];               // last round in which the wave read its partner's partial
};

struct Ctx {
  size_t row0;         // main-KV row of entry 0 of the sequence (0 with paging: ids are pool rows)
  int r, b, hg, wave, pair, d, lane, m, c;
  int sel_tiles, qpos, p0, lo;
};

// A tile's raw bytes for one lane, halves h = 0, 1 (entries m and 16 + m).
// Selected entries (MainRaw): f[h][0..1] = E2M1 bytes 128 d + 32 c .. + 32,
// sc[h] = the dword of scales covering those 64 dims: E8M0 blocks 8 d + 2 c
// and + 1 (bytes 2 (c % 2) + k), or E4M3 blocks 16 d + 4 c .. + 3 (bytes
// 0..3).  Window entries (WinRaw): v[h][0..3] = FP8 bytes 256 d + 64 c ..
// + 64.
struct MainRaw {
  u32x4 f[2][2];
  uint32_t sc[2];
  bool valid[2];
};
struct WinRaw {
  u32x4 v[2][4];
  bool valid[2];
};

struct State {
  u32x4 qb[kSteps];        // q^T B operands: head m, dims 256 d + 64 c + 8 s .. + 8
  f32x4_t o[kDimTiles];    // O^T: lane (head m, c) holds dims 256 d + 16 t + 4 c + i
  float m_ref, l;          // per head (every lane of head m holds the same)
  uint32_t exchanged;      // last round in which the pair exchanged partial sums
};

__device__ __forceinline__ f32x4_t mfma16(bf16x8 a, bf16x8 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word_of(const u32x4& w, int k) {
  return k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
}

// Two floats -> two bf16 (round to nearest even), lo in the low half.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Max and sum over the four lanes of one head (lanes m + 16 c').
__device__ __forceinline__ float head_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float head_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Issues the loads of selected-entry tile t (wave-uniform) into w.  Every
// call issues the same loads (a tile past the list reads slots that hold -1
// and so entry 0 of the sequence), so that the compiler can count the loads
// still in flight on every path and wait only for the ones it needs.
template <int FMT>
__device__ __forceinline__ void gather_rows(const AttnArgs& a, const Ctx& x, const int (&id)[2],
                                            MainRaw& w) {
  constexpr int kSc = KvFmt<FMT>::kScaleBytes;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool valid = id[h] >= 0;
    w.valid[h] = valid;
    const size_t er = x.row0 + (valid ? id[h] : 0);
    const uint8_t* src = a.kv_fp4 + er * 256 + 128 * x.d + 32 * x.c;
    w.f[h][0] = *reinterpret_cast<const u32x4*>(src);
    w.f[h][1] = *reinterpret_cast<const u32x4*>(src + 16);
    const int sc_off = FMT == kFmtE8M0 ? 8 * x.d + 4 * (x.c >> 1) : 16 * x.d + 4 * x.c;
    w.sc[h] = *reinterpret_cast<const uint32_t*>(a.kv_scale + er * kSc + sc_off);
  }
}
template <int FMT>
__device__ __forceinline__ void gather_main(const AttnArgs& a, const Ctx& x, const int32_t* ids,
                                            int t, MainRaw& w) {
  t = min(t, kMaxTopK / kTile - 1);
  const int id[2] = {ids[kTile * t + x.m], ids[kTile * t + 16 + x.m]};
  gather_rows<FMT>(a, x, id, w);
}

// Selected slot `slot` of row r (sequence b) read from global memory: the
// entry id, or with paging its pool row; -1 for no entry (an id out of
// range or on an unmapped page).
__device__ __forceinline__ int slot_id(const AttnArgs& a, int r, int b, int slot) {
  const int v = slot < a.top_k ? a.idx[static_cast<size_t>(r) * a.top_k + slot] : -1;
  if (v < 0 || v >= a.N_cap) return -1;
  if (a.pg.bt == nullptr) return v;
  bool mapped;
  const size_t row = pool_row(a.pg, b, a.N_cap, v, mapped);
  return mapped ? static_cast<int>(row) : -1;
}

// Window tile u (positions q_pos - 127 + 32 u .. + 31), dims half d: the
// validity of the lane's two slots (entries 16 h + m), and the loads of
// the 32 rows, lane l of load j taking row 4 j + l / 16, bytes 16 (l % 16)
// .. + 16 of the half.  An empty row reads the query row, which always
// exists.
struct WinLoad {
  u32x4 raw[8];
};
__device__ __forceinline__ int window_pos(const Ctx& x, int u, int j) {
  return x.qpos - (kMaxWindow - 1) + kTile * u + j;
}
__device__ __forceinline__ bool window_valid(const AttnArgs& a, const Ctx& x, int p) {
  return p >= x.lo && p <= x.qpos && p - x.p0 < a.S_cap;
}
__device__ __forceinline__ void load_window(const AttnArgs& a, const Ctx& x, int u, WinLoad& l,
                                            WinRaw& w) {
#pragma unroll
  for (int h = 0; h < 2; ++h) w.valid[h] = window_valid(a, x, window_pos(x, u, 16 * h + x.m));
  const uint8_t* qrow =
      reinterpret_cast<const uint8_t*>(a.q + static_cast<size_t>(x.r) * kHeads * kDim);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = window_pos(x, u, 4 * j + (x.lane >> 4));
    const uint8_t* row = window_valid(a, x, p)
                             ? a.swa + (static_cast<size_t>(x.b) * a.S_cap + (p - x.p0)) * 512
                             : qrow;
    l.raw[j] = *reinterpret_cast<const u32x4*>(row + 256 * x.d + 16 * (x.lane & 15));
  }
}
// Through the staging area into the operand layout: v[h][0..3] = bytes
// 64 c .. + 64 of row 16 h + m.
__device__ __forceinline__ void stage_window(const Ctx& x, const WinLoad& l, uint8_t* tile,
                                             WinRaw& w) {
  uint8_t* st = tile + kWinStage;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<u32x4*>(st + (4 * j + (x.lane >> 4)) * kWStride + 16 * (x.lane & 15)) =
        l.raw[j];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w.v[h][k] = *reinterpret_cast<const u32x4*>(st + (16 * h + x.m) * kWStride + 64 * x.c +
                                                  16 * k);
}

// Dequantisation, LDS store and the partial S^T = K . q^T of one tile.
// Step s: lane (m, c) supplies dims 256 d + 64 c + 8 s .. + 8 of entry
// 16 h + m, which is 16-byte chunk 8 c + s of its LDS row.
template <bool kMain, int FMT, class R>
__device__ __forceinline__ void qk_tile(const Ctx& x, const R& w, const State& st, uint8_t* tile,
                                        f32x4_t (&acc)[2]) {
  // Scale of step s: E8M0 per 32 dims, scale[h][s / 4]; E4M3 per 16 dims,
  // scale[h][s / 2].
  float scale[2][4];
  if constexpr (kMain && FMT == kFmtE4M3) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float f[4];
      e4m3x4_to_f32(w.sc[h], f);
#pragma unroll
      for (int k = 0; k < 4; ++k) scale[h][k] = w.valid[h] ? f[k] : 0.0f;
    }
  } else if constexpr (kMain) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // Blocks 8 d + 2 c + k: bytes 2 (c % 2) + k of the loaded dword.
      const uint32_t two = w.sc[h] >> (16 * (x.c & 1));
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // The conversion reads only the exponent field of its scale
        // operand, as an E8M0 code: the code shifted into that field is the
        // scale 2^(code - 127) for every code (0: 2^-127, 255: NaN).  An
        // empty slot gets the bits 0 (2^-127): finite values, which the
        // softmax masks by the slot's validity.
        const uint32_t code = (two >> (8 * k)) & 0xffu;
        scale[h][k] = __uint_as_float(w.valid[h] ? code << 23 : 0u);
      }
    }
  }
  // Two accumulators per half (even and odd steps), added at the end: four
  // independent MFMA chains hide the result latency of each product.
  f32x4_t part[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) part[h][0] = part[h][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 kb;
      if constexpr (kMain) {
        if constexpr (FMT == kFmtE4M3)
          kb = fp4x8_mul_to_bf16x8(word_of(w.f[h][s >> 2], s & 3), scale[h][s >> 1]);
        else
          kb = fp4x8_to_bf16x8(word_of(w.f[h][s >> 2], s & 3), scale[h][s >> 2]);
      } else {
        const u32x4& q4 = w.v[h][s >> 1];
        const uint32_t lo = (s & 1) ? q4.z : q4.x, hi = (s & 1) ? q4.w : q4.y;
        kb = fp8x8_to_bf16x8(w.valid[h] ? lo : 0u, w.valid[h] ? hi : 0u);
      }
      *reinterpret_cast<bf16x8*>(tile + (16 * h + x.m) * kRowBytes + 16 * (8 * x.c + s)) = kb;
      part[h][s & 1] = mfma16(kb, __builtin_bit_cast(bf16x8, st.qb[s]), part[h][s & 1]);
    }
    // One step at a time: unfenced, the scheduler hoists the conversions of
    // every step and runs out of registers.
    __builtin_amdgcn_sched_barrier(0);
  }
  acc[0] = part[0][0] + part[0][1];
  acc[1] = part[1][0] + part[1][1];
}

// Transposing read of V^T for one A operand: lanes of group c read rows
// (entries) 4 c + j / 4 (a) and 16 + 4 c + j / 4 (b), dims 16 t + 4 (j % 4)
// .. + 4 (j = lane % 16); lane j then holds dim 16 t + j of entries 4 c ..
// 4 c + 3 and 16 + 4 c .. + 3, the k order of P^T's B operand.
__device__ __forceinline__ bf16x8 tr_read_pair(const uint8_t* tile, int off_a, int off_b) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_a));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_b));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Softmax of the tile (S = the pair's two partial sums) and O^T += V^T . P^T.
__device__ __forceinline__ void softmax_pv(const AttnArgs& a, const Ctx& x, uint32_t vm0,
                                           uint32_t vm1, const uint8_t* tile, int off_a, int off_b,
                                           const f32x4_t (&s0)[2], const f32x4_t (&s1)[2],
                                           State& st) {
  // Validity of entry 16 h + e is bit e of vm_h; lane (m, c) holds entries
  // 16 h + 4 c + i.  The partner's partial is added in the same order in
  // both waves.  Logits are scaled into log2 units after the maximum (a
  // positive scale commutes with it) and inside the exponent's fma.
  float xv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = s0[i >> 2][i & 3] + s1[i >> 2][i & 3];
  if ((vm0 & vm1) != 0xffffu) {   // wave-uniform: some slot of the tile is empty
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool v = (((i >> 2) ? vm1 : vm0) >> (4 * x.c + (i & 3))) & 1u;
      xv[i] = v ? xv[i] : -__builtin_inff();
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3])),
                   fmaxf(fmaxf(xv[4], xv[5]), fmaxf(xv[6], xv[7])));
  // A tile is processed only when one of its slots holds an entry, so the
  // maximum (and from here on the reference) is finite.
  mx = head_max(mx) * a.scale2;
  // Reference: kept unless still -inf or exceeded by more than kLazyRescale.
  const float mr = st.m_ref;
  const float ref = (mr == -__builtin_inff() || mx > mr + kLazyRescale) ? mx : mr;
  if (ref != mr) {
    // A finite mr means O and l hold sums relative to it: rescale them.
    const float alpha = mr == -__builtin_inff() ? 1.0f : __builtin_amdgcn_exp2f(mr - ref);
    if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
      for (int t = 0; t < kDimTiles; ++t) st.o[t] *= alpha;
      st.l *= alpha;
    }
    st.m_ref = ref;
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // exp2(-inf) = 0 for an empty slot.
    xv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xv[i], a.scale2, -st.m_ref));
    sum += xv[i];
  }
  st.l += head_sum(sum);
  const u32x4 pw = {pack_bf16x2(xv[0], xv[1]), pack_bf16x2(xv[2], xv[3]),
                    pack_bf16x2(xv[4], xv[5]), pack_bf16x2(xv[6], xv[7])};
  const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
  // The wave's own LDS stores of this tile precede these reads in issue
  // order (the LDS operations of a wave complete in order).
  // V^T operands read kAhead dims tiles ahead of their product (LDS latency
  // is several products long).
  constexpr int kAhead = 4;
  bf16x8 va[kAhead];
#pragma unroll
  for (int t = 0; t < kAhead; ++t) va[t] = tr_read_pair(tile, off_a + 32 * t, off_b + 32 * t);
#pragma unroll
  for (int t = 0; t < kDimTiles; ++t) {
    const bf16x8 cur = va[t % kAhead];
    if (t + kAhead < kDimTiles)
      va[t % kAhead] = tr_read_pair(tile, off_a + 32 * (t + kAhead), off_b + 32 * (t + kAhead));
    st.o[t] = mfma16(cur, pb, st.o[t]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The pair's S = (partial of wave d = 0) + (partial of wave d = 1), the same
// sum in both waves, through one call site: the operands are selected by
// the wave's half (two calls would be two copies of the code, and the
// compiler would copy the whole O^T state between their register
// assignments every tile).
__device__ __forceinline__ void pair_softmax_pv(const AttnArgs& a, const Ctx& x, uint32_t vm0,
                                                uint32_t vm1, const uint8_t* tile, int off_a,
                                                int off_b, const f32x4_t (&mine)[2],
                                                const f32x4_t (&other)[2], State& st) {
  const bool lo = x.d == 0;
  const f32x4_t s0[2] = {lo ? mine[0] : other[0], lo ? mine[1] : other[1]};
  const f32x4_t s1[2] = {lo ? other[0] : mine[0], lo ? other[1] : mine[1]};
  softmax_pv(a, x, vm0, vm1, tile, off_a, off_b, s0, s1, st);
}

// Waits (bounded) until the LDS counter reaches `want`.  The two waves of a
// pair synchronise only with each other through these counters, so the four
// pairs of a workgroup run independently and the two waves that share a SIMD
// overlap one's products with the other's conversions.  A pair's rounds
// always complete (each wave signals every round it works on), so the wait
// ends; the bound only guards against a wave that never signals.
__device__ __forceinline__ void wait_counter(const uint32_t* ctr, uint32_t want) {
  for (int spin = 0; spin < (1 << 22); ++spin) {
    if (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= want) return;
    __builtin_amdgcn_s_sleep(1);
  }
}
__device__ __forceinline__ void signal_counter(uint32_t* ctr, uint32_t v) {
  __hip_atomic_store(ctr, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Round `round` (numbered from 1) of one pair: its tile, processed only when
// `work` (the same in both waves of the pair).  The exchange: a wave writes
// its partial S^T once its partner has taken the one of the pair's previous
// exchange, signals it, and reads the partner's once that is signalled.
template <bool kMain, int FMT, class R>
__device__ __forceinline__ void round_tile(const AttnArgs& a, const Ctx& x, Smem& sm, const R& w,
                                           bool work, uint32_t round, uint8_t* tile, int off_a,
                                           int off_b, State& st) {
  if (!work) return;
  f32x4_t acc[2];
  qk_tile<kMain, FMT, R>(x, w, st, tile, acc);
  const int partner = x.wave ^ 1;
  wait_counter(&sm.taken[partner], st.exchanged);
  st.exchanged = round;
  sm.xs[x.wave][0][x.lane] = acc[0];
  sm.xs[x.wave][1][x.lane] = acc[1];
  signal_counter(&sm.ready[x.wave], round);
  wait_counter(&sm.ready[partner], round);
  f32x4_t other[2] = {sm.xs[partner][0][x.lane], sm.xs[partner][1][x.lane]};
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): both reads have returned
  signal_counter(&sm.taken[x.wave], round);
  const uint32_t vm0 = static_cast<uint32_t>(__ballot(w.valid[0])) & 0xffffu;
  const uint32_t vm1 = static_cast<uint32_t>(__ballot(w.valid[1])) & 0xffffu;
  pair_softmax_pv(a, x, vm0, vm1, tile, off_a, off_b, acc, other, st);
}

template <int FMT>
__global__ __launch_bounds__(kThreads, 1) void k_sparse_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  Ctx x;
  // Workgroup id -> (row, head group): the four head groups of row r have
  // ids 32 (r / 8) + 8 hg + r % 8, i.e. the same id modulo 8 (one XCD).
  const int id = blockIdx.x;
  x.r = (id >> 5) * 8 + (id & 7);
  x.hg = (id >> 3) & 3;
  if (x.r >= a.rows) return;
  x.b = x.r / a.n_q;
  x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  x.pair = x.wave >> 1;
  x.d = x.wave & 1;
  x.lane = threadIdx.x & 63;
  x.m = x.lane & 15;
  x.c = x.lane >> 4;
  x.sel_tiles = (a.top_k + kTile - 1) / kTile;
  // Loads issued first, in this order: the window bounds, the slot id this
  // thread stores to LDS, the ids of the pair's first selected tile
  // (straight from global memory, so that its gather goes out as soon as
  // they arrive, without waiting for the workgroup's ids), and the q rows
  // (lane l of load j: head 2 j + l / 32, bytes 16 (l % 32) .. + 16 of the
  // wave's dims half).
  x.qpos = a.q_pos[x.r];
  x.p0 = a.swa_pos0[x.b];
  x.row0 = a.pg.bt == nullptr ? static_cast<size_t>(x.b) * a.N_cap : 0;
  const int my_id = slot_id(a, x.r, x.b, threadIdx.x);
  const int first[2] = {slot_id(a, x.r, x.b, kTile * x.pair + x.m),
                        slot_id(a, x.r, x.b, kTile * x.pair + 16 + x.m)};
  u32x4 qraw[8];
  {
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(
        a.q + (static_cast<size_t>(x.r) * kHeads + kHeadsPerWg * x.hg) * kDim) + 512 * x.d;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      qraw[j] = *reinterpret_cast<const u32x4*>(qbase + (2 * j + (x.lane >> 5)) * 1024 +
                                                16 * (x.lane & 31));
  }
  __builtin_amdgcn_sched_barrier(0);
  x.lo = max(max(x.qpos - a.window + 1, x.p0), 0);
  if (a.replay_start >= 0) x.lo = max(x.lo, a.replay_start);
  State st;
  uint8_t* tile = sm.tile[x.wave];
#pragma unroll
  for (int t = 0; t < kDimTiles; ++t) st.o[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  st.m_ref = -__builtin_inff();
  st.l = 0.0f;
  st.exchanged = 0;

  // Transposing-read offsets for dims tile 0 (tile t: + 32 t): row 4 c + j /
  // 4 (a) or 16 + 4 c + j / 4 (b), dims 4 (j % 4) .. + 4.
  const int j = x.m;
  const int off_a = (4 * x.c + (j >> 2)) * kRowBytes + 8 * (j & 3);
  const int off_b = off_a + 16 * kRowBytes;

  // Round 1: pair p takes window tile p, before the workgroup barrier that
  // publishes the ids (the window needs none); its exchange goes through
  // that barrier.  Then pair p takes selected tiles p, p + 4, ... (one
  // round each), the next tile's loads issued before the current one is
  // processed (two register buffers).
  {
    WinRaw wr;
    WinLoad wl;
    MainRaw m0, m1;
    load_window(a, x, x.pair, wl, wr);
    gather_rows<FMT>(a, x, first, m0);
    __builtin_amdgcn_sched_barrier(0);
    // q^T operands of head 16 hg + m: step s takes dims 256 d + 64 c + 8 s
    // .. + 8, i.e. 16 bytes at 128 c + 16 s of the head's staged half row.
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4*>(tile + (2 * j + (x.lane >> 5)) * kQStride + 16 * (x.lane & 31)) =
          qraw[j];
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      st.qb[s] = *reinterpret_cast<const u32x4*>(tile + x.m * kQStride + 128 * x.c + 16 * s);
    stage_window(x, wl, tile, wr);
    __builtin_amdgcn_sched_barrier(0);
    const bool work = __ballot(wr.valid[0] || wr.valid[1]) != 0;
    f32x4_t acc[2];
    if (work) {
      qk_tile<false, FMT, WinRaw>(x, wr, st, tile, acc);
      sm.xs[x.wave][0][x.lane] = acc[0];
      sm.xs[x.wave][1][x.lane] = acc[1];
    }
    sm.ids[threadIdx.x] = my_id;
    if (x.lane == 0) {
      sm.ready[x.wave] = 0;
      sm.taken[x.wave] = 0;
    }
    lds_barrier();   // ids, counters and the window partials are in LDS
    uint32_t round = 1;
    if (work) {
      const int partner = x.wave ^ 1;
      f32x4_t other[2] = {sm.xs[partner][0][x.lane], sm.xs[partner][1][x.lane]};
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): both reads have returned
      signal_counter(&sm.taken[x.wave], round);
      st.exchanged = round;
      const uint32_t vm0 = static_cast<uint32_t>(__ballot(wr.valid[0])) & 0xffffu;
      const uint32_t vm1 = static_cast<uint32_t>(__ballot(wr.valid[1])) & 0xffffu;
      pair_softmax_pv(a, x, vm0, vm1, tile, off_a, off_b, acc, other, st);
    }
    const int rounds = (x.sel_tiles + kPairs - 1) / kPairs;
    int t = x.pair;
    auto run = [&](const MainRaw& w) {
      ++round;
      const bool wk = t < x.sel_tiles && __ballot(w.valid[0] || w.valid[1]) != 0;
      round_tile<true, FMT>(a, x, sm, w, wk, round, tile, off_a, off_b, st);
      t += kPairs;
    };
    for (int i = 0; i < rounds; i += 2) {
      gather_main<FMT>(a, x, sm.ids, t + kPairs, m1);
      __builtin_amdgcn_sched_barrier(0);
      run(m0);
      if (i + 1 >= rounds) break;
      gather_main<FMT>(a, x, sm.ids, t + kPairs, m0);
      __builtin_amdgcn_sched_barrier(0);
      run(m1);
    }
  }

  // Merge of the four pairs' partial results, in pair order.  Each wave
  // leaves its O^T in its tile ([dims tile][lane], fp32) and each pair its
  // (reference, sum) per head; wave (p, d) then finishes dims tiles 4 p ..
  // 4 p + 3 of its half.
  f32x4_t* mine = reinterpret_cast<f32x4_t*>(tile);
#pragma unroll
  for (int tt = 0; tt < kDimTiles; ++tt) mine[tt * 64 + x.lane] = st.o[tt];
  if (x.d == 0 && x.c == 0) {
    sm.ml[x.pair][x.m][0] = st.m_ref;
    sm.ml[x.pair][x.m][1] = st.l;
  }
  __syncthreads();
  const int head = kHeadsPerWg * x.hg + x.m;
  float mi[kPairs], li[kPairs];
  float M = a.sink != nullptr ? a.sink[head] * kLog2e : -__builtin_inff();
  const float s2 = M;
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    mi[i] = sm.ml[i][x.m][0];
    li[i] = sm.ml[i][x.m][1];
    M = fmaxf(M, mi[i]);
  }
  float wt[kPairs];
  float L = 0.0f;
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    wt[i] = mi[i] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mi[i] - M);
    L += wt[i] * li[i];
  }
  if (s2 != -__builtin_inff()) L += __builtin_amdgcn_exp2f(s2 - M);
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint16_t* orow = a.out + (static_cast<size_t>(x.r) * kHeads + head) * kDim + kHalfDims * x.d;
#pragma unroll
  for (int tt = 0; tt < kDimTiles / kPairs; ++tt) {
    const int dt = (kDimTiles / kPairs) * x.pair + tt;
    f32x4_t v = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kPairs; ++i)
      v += wt[i] * reinterpret_cast<const f32x4_t*>(sm.tile[2 * i + x.d])[dt * 64 + x.lane];
    v *= inv;
    *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * x.c) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
  if (a.lse != nullptr && x.wave == 0 && x.c == 0)
    a.lse[static_cast<size_t>(x.r) * kHeads + head] =
        L > 0.0f ? (M + log2f(L)) * kLn2 : -__builtin_inff();
}

}  // namespace

size_t attn_workspace_bytes(int rows, int top_k) {
  (void)rows;
  (void)top_k;
  return 0;
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                              int N_cap, const int32_t* idx, int top_k, const uint8_t* swa_kv,
                              int S_cap, const int32_t* swa_pos0, const int32_t* q_pos,
                              float sm_scale, int window, int replay_start, const float* sink,
                              int kv_fmt, const Pages& pg, int B, int n_q, uint16_t* out,
                              float* lse, void* ws, hipStream_t stream) {
  (void)ws;
  // Prefill-shaped calls (many query rows per sequence) take the one-row-
  // per-workgroup kernel; the choice depends on n_q only, never on B.
  if (n_q >= kRowsKernelMinNq)
    return launch_attn_rows(q, kv_fp4, kv_scale, N_cap, idx, top_k, swa_kv, S_cap, swa_pos0,
                            q_pos, sm_scale, window, replay_start, sink, kv_fmt, pg, B, n_q, out,
                            lse, stream);
  AttnArgs a;
  a.q = q; a.kv_fp4 = kv_fp4; a.kv_scale = kv_scale; a.idx = idx; a.swa = swa_kv;
  a.swa_pos0 = swa_pos0; a.q_pos = q_pos; a.out = out; a.lse = lse; a.sink = sink;
  a.pg = pg;
  a.N_cap = N_cap; a.top_k = top_k; a.S_cap = S_cap; a.n_q = n_q;
  a.window = window; a.replay_start = replay_start;
  a.rows = B * n_q;
  a.scale2 = sm_scale * kLog2e;
  // Rows in groups of 8 (one per XCD), 4 head groups each.
  const long long wgs = static_cast<long long>((a.rows + 7) / 8) * 8 * kGroupsPerRow;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (kv_fmt == kFmtE8M0)
    hipLaunchKernelGGL(k_sparse_attn<kFmtE8M0>, dim3(static_cast<unsigned>(wgs)), dim3(kThreads),
                       0, stream, a);
  else
    hipLaunchKernelGGL(k_sparse_attn<kFmtE4M3>, dim3(static_cast<unsigned>(wgs)), dim3(kThreads),
                       0, stream, a);
  return hipGetLastError();
}

}  // namespace csa2
