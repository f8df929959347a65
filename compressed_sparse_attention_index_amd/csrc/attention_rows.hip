// Sparse multi-query attention of prefill-shaped calls (n_q >= 16 query
// rows per sequence): one workgroup per query row, all 64 heads.  Decode
// rows use the head-group kernel of attention.hip.
//
// "DeepSeek-V4.1-Flash 架构详解": §1 configuration table (64 query heads of
// 512 dims, window 128), §4 (main KV is MXFP4 and is dequantised before
// attention, SWA KV is FP8), §3.1 (an encoder prefill chunk attends for many
// query tokens at once).  DeepSeek-V4 essay (mlqm.cn) §4.3: a compressed
// entry serves as both key and value; §6.4: batch-invariant kernels.
//
// Work decomposition.  A workgroup (4 waves) takes one query row, all 64
// heads, and the row's whole entry list in 64-entry chunks
//   [ top_k selected slots, padded to a multiple of 32 | 128 window slots ].
// A row is never split over workgroups, so its arithmetic does not depend on
// how many rows the call has.  Every entry of a chunk is gathered,
// dequantised and written to LDS once, and serves all 64 heads.  Per chunk,
// wave w = (e, dh) with e = w / 2, dh = w % 2:
//   1. stages the raw bytes of entry tile e (32 entries) x dims half dh with
//      direct-to-LDS loads, two chunks ahead, into a private staging slot
//      (no registers held; waits counted by hand);
//   2. finishes the previous chunk's O^T[dims][head] += V^T . P^T for dims
//      quarter w and all 64 heads, with V^T read from the shared LDS buffer
//      through transposing reads (ds_read_b64_tr_b16), each read feeding the
//      MFMAs of both head tiles; a barrier follows (the buffer is free);
//   3. dequantises its tile exactly to bf16 with the gfx950 conversion
//      instructions, in one pass that writes the shared buffer and forms the
//      partial S^T[entry][head] over its 256 dims for all 64 heads on
//      32x32x16 bf16 MFMA (q^T for 64 heads x 256 dims sits in accumulation
//      registers for the whole row);
//   4. hands the partial of head tile 1 - dh to its partner (e, 1 - dh) and
//      receives the partner's partial of head tile dh (one LDS exchange,
//      one barrier);
//   5. runs the online softmax (fp32, log2 domain) for entry tile e x head
//      tile dh and publishes P (bf16, in the accumulator's lane order) with
//      the tile's reference max and sum (a third barrier).
// Every wave keeps the running max and sum of all 64 heads, updated
// identically in all four waves from the published per-tile values.  The
// reference max moves only when a tile's max exceeds it by more than
// kLazyRescale, so the accumulators are rarely rescaled.
// LDS rows are 1024 bytes (one entry); 16-byte chunk k of row r sits at
// k ^ kswz(r), which keeps the row-wise stores and the transposing reads free
// of bank conflicts.  Before the first chunk and after the last one the same
// buffer stages the query row and the output rows, so that both move to and
// from HBM as whole 1 KB rows.
#include "csa2_launch.h"
#include "csa2_device.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;         // entries per chunk: two 32-entry tiles
constexpr int kTile = 32;
constexpr int kRow = 1024;         // LDS bytes of one dequantised entry (512 bf16)
constexpr int kBuf = kChunk * kRow;
constexpr int kStage = 8192;       // staging bytes per wave and chunk
// Direct-to-LDS loads per wave and tile: selected tiles 4 x 16 B of E2M1
// plus one (E8M0) or two (E4M3) dwords of scales; window tiles 8 x 16 B.
template <int FMT> constexpr int kMainLoads = FMT == kFmtE8M0 ? 5 : 6;
constexpr int kWindowLoads = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxChunks = (kMaxTopK + kMaxWindow + kChunk - 1) / kChunk;
constexpr float kLazyRescale = 8.0f;

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
  const float* sink; // [64] per-head sink logits (natural log), or null
  Pages pg;          // main-KV page table (pg.bt == nullptr: contiguous)
  int N_cap, top_k, S_cap, n_q, window, replay_start;
  int rows, n_chunks;
  float scale2;      // sm_scale * log2(e)
};

struct Smem {
  uint8_t kv[kBuf];              // dequantised entries of a chunk [entry][dims], swizzled
  uint8_t stage[2][4][kStage];   // raw bytes [chunk parity][wave]
  f32x4_t sx[4][4][64];          // partial S^T handed to the partner, [wave][i / 4][lane]
  u32x4 pb[2][2][2][64];         // P^T (bf16) [entry tile][head tile][16-entry step][lane]
  float pml[2][2][32][2];        // (reference max, sum) [entry tile][head tile][head]
  int ids[kMaxChunks * kChunk];  // selected ids of the workgroup's chunks (-1: none)
};

struct Ctx {
  size_t row0;   // main-KV row of entry 0 of the sequence (0 with paging: ids are pool rows)
  int r, b, tkp, qpos, lo, p0, slot0, wave, lane, c, half, e, dh;
};

struct State {
  u32x4 qb[2][16];   // q^T: head 32 h + c, dims 256 dh + 128 half + 8 k + [0, 8)
  f32x16 o[4][2];    // O^T: dims 128 w + 32 m + 8 (i / 4) + 4 half + i % 4, head 32 h + c
  float m_run[2], l_run[2];   // heads c and 32 + c
};

// Swizzle of the 16-byte chunks of LDS row r (a bijection of r's low four
// bits): a row-wise store by 16 lanes, and each 16- or 32-lane group of a
// transposing read, touches every bank at most once.
__device__ __forceinline__ int kswz(int r) {
  return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 3);
}

__device__ __forceinline__ bool tile_is_main(const Ctx& x, int ch) {
  return kChunk * ch + kTile * x.e < x.tkp;
}

__device__ __forceinline__ uint32_t word_of(const u32x4& w4, int k) {
  return k == 0 ? w4.x : k == 1 ? w4.y : k == 2 ? w4.z : w4.w;
}

// Two floats -> two bf16 (round to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32 (converting the halves one by one takes four).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 tr_read_pair(const uint8_t* v, int off0, int off1) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v + off0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v + off1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Issues the wave's direct-to-LDS loads of its tile of chunk ch (entry tile
// e, dims half dh) into staging slot `stg` and returns whether the lane's
// slot holds an entry.  Slot layout: load i of lane l lands at 1024 i + 16 l
// (selected tiles: 4 x 16 B of E2M1 and, at 4096 + 4 l, the 4 E8M0 scales of
// its 128 dims, or at 4096 + 4 l and 4352 + 4 l its 8 E4M3 scales; window
// tiles: 8 x 16 B of FP8).  An empty slot reads a row that always
// exists (entry 0 of the sequence, or the query row), so every tile of a kind
// issues a fixed number of loads; it is zeroed when dequantised.
template <int FMT>
__device__ __forceinline__ bool issue_tile(const AttnArgs& a, const Ctx& x, Smem& sm, int ch,
                                           int stg) {
  const int slot = kChunk * ch + kTile * x.e + x.c;
  const uint32_t dst = lds_offset(sm.stage[stg][x.wave]);
  if (tile_is_main(x, ch)) {
    const int id = sm.ids[slot - x.slot0];
    const bool valid = id >= 0;
    const size_t er = x.row0 + (valid ? id : 0);
    const uint8_t* src = a.kv_fp4 + er * 256 + 128 * x.dh + 64 * x.half;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(src + 16 * i, dst + 1024 * i);
    if (FMT == kFmtE8M0) {
      dma4(a.kv_scale + er * 16 + 8 * x.dh + 4 * x.half, dst + 4096);
    } else {
      const uint8_t* sc = a.kv_scale + er * 32 + 16 * x.dh + 8 * x.half;
      dma4(sc, dst + 4096);
      dma4(sc + 4, dst + 4352);
    }
    return valid;
  }
  const int j = slot - x.tkp;
  const int p = x.qpos - (kMaxWindow - 1) + j;
  const bool valid = j < kMaxWindow && p >= x.lo && p <= x.qpos && p - x.p0 < a.S_cap;
  const uint8_t* row =
      valid ? a.swa + (static_cast<size_t>(x.b) * a.S_cap + (p - x.p0)) * 512
            : reinterpret_cast<const uint8_t*>(a.q + static_cast<size_t>(x.r) * kHeads * kDim);
  const uint8_t* src = row + 256 * x.dh + 128 * x.half;
#pragma unroll
  for (int i = 0; i < 8; ++i) dma16(src + 16 * i, dst + 1024 * i);
  return valid;
}

// Dequantisation of the lane's entry from its staging slot, 16 bytes of raw
// data (a unit) at a time: a unit holds 8-dim groups k = 4 u .. 4 u + 3 of
// E2M1 (selected entries) or k = 2 u, 2 u + 1 of FP8 (window); group k is
// dims 256 dh + 128 half + 8 k, whose scale is E8M0 block k / 4 or E4M3
// block k / 2 of the lane's 128 dims.  Empty slots get the scale bits 0
// (read as 2^-127 by the E8M0 conversion, 0 by the E4M3 multiply) or zeroed
// FP8 bytes: finite values, which the softmax masks by the slot's validity.
template <bool kMain, int FMT>
struct Dequant {
  static constexpr int kPerUnit = kMain ? 4 : 2;
  static constexpr int kUnits = 16 / kPerUnit;
  float scale[8];
  const uint8_t* sp;
  bool valid;
  __device__ __forceinline__ Dequant(const uint8_t* slot, int lane, bool lane_valid)
      : sp(slot + 16 * lane), valid(lane_valid) {
    if (kMain && FMT == kFmtE8M0) {
      const uint32_t sc = *reinterpret_cast<const uint32_t*>(slot + 4096 + 4 * lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t code = (sc >> (8 * i)) & 0xffu;
        uint32_t bits = code == 0 ? 0x00400000u : (code == 255 ? 0x7fc00000u : code << 23);
        scale[i] = __uint_as_float(lane_valid ? bits : 0u);
      }
    } else if (kMain) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float f[4];
        e4m3x4_to_f32(*reinterpret_cast<const uint32_t*>(slot + 4096 + 256 * q + 4 * lane), f);
#pragma unroll
        for (int i = 0; i < 4; ++i) scale[4 * q + i] = lane_valid ? f[i] : 0.0f;
      }
    }
  }
  __device__ __forceinline__ u32x4 unit(int u) const {
    return *reinterpret_cast<const u32x4*>(sp + 1024 * u);
  }
  __device__ __forceinline__ bf16x8 convert(const u32x4& w, int k) const {
    if (kMain && FMT == kFmtE4M3) return fp4x8_mul_to_bf16x8(word_of(w, k & 3), scale[k >> 1]);
    if (kMain) return fp4x8_to_bf16x8(word_of(w, k & 3), scale[k >> 2]);
    const uint32_t lo = (k & 1) ? w.z : w.x, hi = (k & 1) ? w.w : w.y;
    return fp8x8_to_bf16x8(valid ? lo : 0u, valid ? hi : 0u);
  }
};

// Moves the running max and sum past the chunk just finished (from the
// per-tile reference maxima and sums its waves published) and rescales the
// accumulators when the max moves.  Where a tile's reference differs from the
// new max, the wave that published that tile's P rescales it in LDS before
// anyone reads it.  All waves run this on the same values, so they take the
// same branches (and barrier) and keep identical (m, l).
__device__ __forceinline__ void pv_prep(const Ctx& x, Smem& sm, State& st) {
  float b[2][2];   // [head tile][entry tile]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float c0 = sm.pml[0][h][x.c][0], s0 = sm.pml[0][h][x.c][1];
    const float c1 = sm.pml[1][h][x.c][0], s1 = sm.pml[1][h][x.c][1];
    const float mn = fmaxf(c0, c1);   // never below m_run
    const float mr = st.m_run[h];
    const float alpha =
        mn == mr ? 1.0f : (mr == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mr - mn));
    b[h][0] = c0 == mn ? 1.0f : (c0 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(c0 - mn));
    b[h][1] = c1 == mn ? 1.0f : (c1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(c1 - mn));
    st.l_run[h] = st.l_run[h] * alpha + (s0 * b[h][0] + s1 * b[h][1]);
    st.m_run[h] = mn;
    // (While the max is still -inf nothing has been accumulated: O is zero.)
    if (__ballot(alpha != 1.0f && mr != -__builtin_inff()) != 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m) st.o[m][h] *= alpha;
    }
  }
  const bool fix = b[0][0] != 1.0f || b[0][1] != 1.0f || b[1][0] != 1.0f || b[1][1] != 1.0f;
  if (__ballot(fix) != 0) {
    const float be = x.dh ? (x.e ? b[1][1] : b[1][0]) : (x.e ? b[0][1] : b[0][0]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 w = sm.pb[x.e][x.dh][t][x.lane];
      u32x4 r;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t u = word_of(w, k);
        const uint32_t v = pack_bf16x2(__uint_as_float(u << 16) * be,
                                       __uint_as_float(u & 0xffff0000u) * be);
        if (k == 0) r.x = v;
        else if (k == 1) r.y = v;
        else if (k == 2) r.z = v;
        else r.w = v;
      }
      sm.pb[x.e][x.dh][t][x.lane] = r;
    }
    lds_barrier();
  }
}

// Transposing-read offsets of the wave's V^T operands for 32-dim block m of
// dims quarter w, 16-entry step j: lane (i16 = lane % 16) reads 8 bytes at
// entry 16 j + 4 half + i16 / 4 (a) and 16 j + 8 + 4 half + i16 / 4 (b), dims
// 128 w + 32 m + 16 ((lane / 16) % 2) + 4 (i16 % 4).  The 8 values a lane
// receives are entries 16 j + 8 (i / 4) + 4 half + i % 4, the order of the
// accumulator elements 8 t + i of P (j = 2 e + t).  Bits 6-7 of an offset
// are the block m XORed with the row's swizzle, so block m is base ^ (64 m),
// and step j adds 16 rows.
struct TrOffs {
  int a, b;
  __device__ __forceinline__ int off_a(int m, int j) const { return (a ^ (64 * m)) + 16 * kRow * j; }
  __device__ __forceinline__ int off_b(int m, int j) const { return (b ^ (64 * m)) + 16 * kRow * j; }
};

__device__ __forceinline__ TrOffs tr_offsets(const Ctx& x) {
  const int i16 = x.lane & 15;
  const int cl = 2 * ((x.lane >> 4) & 1) + ((i16 & 3) >> 1);
  const int byte = 8 * (i16 & 1);
  const int ra = 4 * x.half + (i16 >> 2), rb = ra + 8;
  TrOffs t;
  t.a = ra * kRow + 16 * (16 * x.wave + (cl ^ kswz(ra))) + byte;
  t.b = rb * kRow + 16 * (16 * x.wave + (cl ^ kswz(rb))) + byte;
  return t;
}

// The loops below are software-pipelined by hand (the next raw unit and the
// next V^T operand are read one step ahead) and fenced per step, so that the
// scheduler does not hoist every LDS read of the chunk and run out of
// registers.

// Chunk ch's tile: dequantised once, written to the LDS buffer (16-byte chunk
// k of the lane's row at st_off ^ (k << 4)) and multiplied into the partial
// S^T of both head tiles.
template <bool kMain, int FMT>
__device__ __forceinline__ void qk_store(const Ctx& x, Smem& sm, const State& st,
                                         const uint8_t* slot, bool valid, int st_off,
                                         f32x16 (&acc)[2]) {
  using D = Dequant<kMain, FMT>;
  const D dq(slot, x.lane, valid);
  u32x4 raw[2];
  raw[0] = dq.unit(0);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int u = k / D::kPerUnit;
    if (k % D::kPerUnit == 0 && u + 1 < D::kUnits) raw[(u + 1) & 1] = dq.unit(u + 1);
    const bf16x8 kb = dq.convert(raw[u & 1], k);
    *reinterpret_cast<bf16x8*>(sm.kv + (st_off ^ (k << 4))) = kb;
    acc[0] = mfma32(kb, __builtin_bit_cast(bf16x8, st.qb[0][k]), acc[0]);
    acc[1] = mfma32(kb, __builtin_bit_cast(bf16x8, st.qb[1][k]), acc[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T . P^T for the chunk in the LDS buffer (P^T of 16-entry step
// j = 2 e + t is pb[e][h][t]).
__device__ __forceinline__ void pv(const Ctx& x, const Smem& sm, State& st, const TrOffs& tr) {
  bf16x8 va[2];
  u32x4 pbv[2][2];
  va[0] = tr_read_pair(sm.kv, tr.off_a(0, 0), tr.off_b(0, 0));
  pbv[0][0] = sm.pb[0][0][0][x.lane];
  pbv[0][1] = sm.pb[0][1][0][x.lane];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int j = k >> 2, m = k & 3;
    if (k + 1 < 16) {
      const int j1 = (k + 1) >> 2, m1 = (k + 1) & 3;
      va[(k + 1) & 1] = tr_read_pair(sm.kv, tr.off_a(m1, j1), tr.off_b(m1, j1));
      if (m == 0 && j + 1 < 4) {
        pbv[(j + 1) & 1][0] = sm.pb[(j + 1) >> 1][0][(j + 1) & 1][x.lane];
        pbv[(j + 1) & 1][1] = sm.pb[(j + 1) >> 1][1][(j + 1) & 1][x.lane];
      }
    }
    st.o[m][0] = mfma32(va[k & 1], __builtin_bit_cast(bf16x8, pbv[j & 1][0]), st.o[m][0]);
    st.o[m][1] = mfma32(va[k & 1], __builtin_bit_cast(bf16x8, pbv[j & 1][1]), st.o[m][1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Chunk ch, staged in slot S; kPV: the previous chunk's PV comes first.
// `valid` (the lane's slot validity) is replaced by that of chunk ch + 2,
// whose loads go to the same slot once it has been read.
template <bool kMain, bool kPV, int FMT>
__device__ __forceinline__ void attend_chunk(const AttnArgs& a, const Ctx& x, Smem& sm, State& st,
                                             bool& valid, int ch, int c1, int S, int st_off,
                                             const TrOffs& tr) {
  if (kPV) {
    pv_prep(x, sm, st);
    pv(x, sm, st, tr);
    // Every wave is done reading the buffer: it takes this chunk.
    lds_barrier();
  }
  // This chunk's loads have landed once only chunk ch + 1's are outstanding.
  if (ch + 1 < c1) {
    if (tile_is_main(x, ch + 1)) wait_vmem<kMainLoads<FMT>>();
    else wait_vmem<kWindowLoads>();
  } else {
    wait_vmem<0>();
  }
  asm volatile("" ::: "memory");
  const uint8_t* slot = sm.stage[S][x.wave];
  const uint32_t vmask = static_cast<uint32_t>(__ballot(valid));
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  qk_store<kMain, FMT>(x, sm, st, slot, valid, st_off, acc);
  // The staging slot has been read; chunk ch + 2 goes there.
  if (ch + 2 < c1) valid = issue_tile<FMT>(a, x, sm, ch + 2, S);

  // Exchange with the partner wave (e, 1 - dh): it gets this wave's partial
  // of head tile 1 - dh, this wave gets its partial of head tile dh
  // (a + b == b + a exactly, so the order of the two halves is immaterial).
  auto give = [&](const f32x16& g) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sm.sx[x.wave][i][x.lane] = f32x4_t{g[4 * i], g[4 * i + 1], g[4 * i + 2], g[4 * i + 3]};
  };
  if (x.dh) give(acc[0]);
  else give(acc[1]);
  lds_barrier();

  // Sums S of head 32 dh + c for entries rho = 8 (i / 4) + 4 half + i % 4 of
  // the tile; empty slots get S = -inf.
  float xv[16];
  auto sum_halves = [&](const f32x16& keep) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4_t other = sm.sx[x.wave ^ 1][i][x.lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[4 * i + j] = keep[4 * i + j] + other[j];
    }
  };
  if (x.dh) sum_halves(acc[1]);
  else sum_halves(acc[0]);
  if (vmask != 0xffffffffu) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rho = 8 * (i >> 2) + 4 * x.half + (i & 3);
      if (!((vmask >> rho) & 1u)) xv[i] = -__builtin_inff();
    }
  }
  float smax = xv[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) smax = fmaxf(smax, xv[i]);
  smax = fmaxf(smax, other_half(smax));
  // Logits are S * scale2 (log2 units, scale2 > 0, so the tile's max logit
  // is smax * scale2).  The tile's reference: the running max, unless that
  // is still -inf or the tile exceeds it by more than kLazyRescale.
  const float tmax = smax * a.scale2;
  const float mr = x.dh ? st.m_run[1] : st.m_run[0];
  const float cand = (mr == -__builtin_inff() || tmax > mr + kLazyRescale) ? tmax : mr;
  const float mref = cand == -__builtin_inff() ? 0.0f : cand;
  float tsum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    xv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xv[i], a.scale2, -mref));
    tsum += xv[i];
  }
  tsum += other_half(tsum);
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
    sm.pb[x.e][x.dh][t2][x.lane] =
        u32x4{pack_bf16x2(xv[8 * t2], xv[8 * t2 + 1]), pack_bf16x2(xv[8 * t2 + 2], xv[8 * t2 + 3]),
              pack_bf16x2(xv[8 * t2 + 4], xv[8 * t2 + 5]),
              pack_bf16x2(xv[8 * t2 + 6], xv[8 * t2 + 7])};
  if (x.half == 0) {
    sm.pml[x.e][x.dh][x.c][0] = cand;
    sm.pml[x.e][x.dh][x.c][1] = tsum;
  }
  lds_barrier();
}

template <int FMT>
__global__ __launch_bounds__(kThreads, 1) void k_attn_rows(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) Smem sm;

  Ctx x;
  x.r = blockIdx.x;
  x.b = x.r / a.n_q;
  x.row0 = a.pg.bt == nullptr ? static_cast<size_t>(x.b) * a.N_cap : 0;
  x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  x.lane = threadIdx.x & 63;
  x.c = x.lane & 31;
  x.half = x.lane >> 5;
  x.e = x.wave >> 1;
  x.dh = x.wave & 1;
  x.tkp = (a.top_k + kTile - 1) / kTile * kTile;
  x.qpos = a.q_pos[x.r];
  x.p0 = a.swa_pos0[x.b];
  x.lo = max(max(x.qpos - a.window + 1, x.p0), 0);
  if (a.replay_start >= 0) x.lo = max(x.lo, a.replay_start);
  const int c0 = 0;
  const int c1 = a.n_chunks;
  x.slot0 = kChunk * c0;

  // The selected ids of chunks [c0, c1) go to LDS first, so that no gather
  // waits on a global id load; out-of-range ids (and, with paging, ids on
  // unmapped pages) become -1 (no entry), and with paging the others become
  // pool rows.  The id loads and the q loads are all issued before any is
  // used.
  constexpr int kPer = (kMaxChunks * kChunk + kThreads - 1) / kThreads;
  int sid[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int slot = x.slot0 + threadIdx.x + kThreads * u;
    sid[u] = -1;
    if (slot < kChunk * c1 && slot < a.top_k)
      sid[u] = a.idx[static_cast<size_t>(x.r) * a.top_k + slot];
  }
  // The query row (64 heads x 1 KB) goes to the K/V buffer, which is free
  // until the first chunk is stored: wave w fetches head rows 16 w .. 16 w +
  // 15 with one coalesced 1 KB load per row, lane l taking 16-byte chunk
  // l ^ kswz(row) so that chunk C of a row lands at slot C ^ kswz(row).
  {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q + static_cast<size_t>(x.r) * kHeads * kDim);
    const uint32_t kv0 = lds_offset(sm.kv);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 16 * x.wave + i;
      dma16(qrow + row * kRow + 16 * (x.lane ^ kswz(row)), kv0 + row * kRow);
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + kThreads * u;
    if (i >= kChunk * (c1 - c0)) continue;
    int v = (sid[u] >= 0 && sid[u] < a.N_cap) ? sid[u] : -1;
    if (v >= 0 && a.pg.bt != nullptr) {
      bool mapped;
      const size_t row = pool_row(a.pg, x.b, a.N_cap, v, mapped);
      v = mapped ? static_cast<int>(row) : -1;
    }
    sm.ids[i] = v;
  }
  // The ids and the query row have landed (every wave's) before the first
  // gather is issued: no other vector-memory load is in flight inside the
  // loop.
  wait_vmem<0>();
  __syncthreads();

  bool valid0 = issue_tile<FMT>(a, x, sm, c0, 0);
  bool valid1 = false;
  if (c0 + 1 < c1) valid1 = issue_tile<FMT>(a, x, sm, c0 + 1, 1);
  // q^T operands (head 32 h + c, dims 256 dh + 128 half + 8 k).  q is only
  // ever an MFMA operand, which may come from accumulation registers:
  // keeping it there leaves the VGPRs to the accumulators and the operands
  // in flight.
  State st;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 32 * h + x.c;
    u32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[k] = *reinterpret_cast<const u32x4*>(
          sm.kv + row * kRow + 16 * ((32 * x.dh + 16 * x.half + k) ^ kswz(row)));
#pragma unroll
    for (int k = 0; k < 16; ++k) st.qb[h][k] = to_agpr(v[k]);
  }
  // Every wave has its q before the first chunk goes to the buffer.
  lds_barrier();
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    st.o[m][0] = f32x16{};
    st.o[m][1] = f32x16{};
  }
  st.m_run[0] = st.m_run[1] = -__builtin_inff();
  st.l_run[0] = st.l_run[1] = 0.0f;

  const TrOffs tr = tr_offsets(x);
  // Row-wise store offset of the lane's entry 32 e + c, dims 256 dh + 128 half.
  const int srow = kTile * x.e + x.c;
  const int st_off = srow * kRow + 512 * x.dh + 256 * x.half + 16 * kswz(srow);

  // Chunks [c0, cm) hold selected entries in this wave's tile, [cm, c1) window
  // entries.
  const int cm = min(max((x.tkp - kTile * x.e + kChunk - 1) / kChunk, c0), c1);
  if (c0 < cm) attend_chunk<true, false, FMT>(a, x, sm, st, valid0, c0, c1, 0, st_off, tr);
  else attend_chunk<false, false, FMT>(a, x, sm, st, valid0, c0, c1, 0, st_off, tr);
  int ch = c0 + 1;
  for (; ch < cm; ++ch) {
    const int S = (ch - c0) & 1;
    bool v = S ? valid1 : valid0;
    attend_chunk<true, true, FMT>(a, x, sm, st, v, ch, c1, S, st_off, tr);
    if (S) valid1 = v;
    else valid0 = v;
  }
  for (; ch < c1; ++ch) {
    const int S = (ch - c0) & 1;
    bool v = S ? valid1 : valid0;
    attend_chunk<false, true, FMT>(a, x, sm, st, v, ch, c1, S, st_off, tr);
    if (S) valid1 = v;
    else valid0 = v;
  }
  pv_prep(x, sm, st);
  pv(x, sm, st, tr);

  // Output, through the K/V buffer once every wave is done with it: lane
  // (c, half) holds head 32 h + c, dims 128 w + 32 m + 8 i4 + 4 half + [0,
  // 4), i.e. half of 16-byte chunk 16 w + 4 m + i4 of the head's row; rows
  // are then stored whole, one coalesced 1 KB store per head row.
  lds_barrier();
  // The row is normalised by its softmax sum, which a sink logit s (log2
  // units s2) extends: with m' = max(m, s2) the sum is l 2^(m - m') +
  // 2^(s2 - m') and O (relative to m) is scaled by 2^(m - m') / sum.
  float fo[2], lse2[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float mr = st.m_run[h], l = st.l_run[h];
    const float s2 = a.sink != nullptr ? a.sink[32 * h + x.c] * kLog2e : -__builtin_inff();
    const float mn = fmaxf(mr, s2);
    const float al = mr == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mr - mn);
    const float sum = l * al + (s2 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(s2 - mn));
    fo[h] = sum > 0.0f ? al / sum : 0.0f;
    lse2[h] = sum > 0.0f ? mn + log2f(sum) : -__builtin_inff();
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 32 * h + x.c;
    const float f = fo[h];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x16& o = st.o[m][h];
        *reinterpret_cast<u32x2*>(sm.kv + row * kRow +
                                  16 * ((16 * x.wave + 4 * m + i4) ^ kswz(row)) + 8 * x.half) =
            u32x2{pack_bf16x2(o[4 * i4] * f, o[4 * i4 + 1] * f),
                  pack_bf16x2(o[4 * i4 + 2] * f, o[4 * i4 + 3] * f)};
      }
    if (x.wave == 0 && x.half == 0 && a.lse != nullptr)
      a.lse[static_cast<size_t>(x.r) * kHeads + row] = lse2[h] * kLn2;
  }
  lds_barrier();
  uint16_t* dst = a.out + static_cast<size_t>(x.r) * kHeads * kDim;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 16 * x.wave + i;
    *reinterpret_cast<u32x4*>(dst + row * kDim + 8 * x.lane) =
        *reinterpret_cast<const u32x4*>(sm.kv + row * kRow + 16 * (x.lane ^ kswz(row)));
  }
}

}  // namespace

hipError_t launch_attn_rows(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                            int N_cap, const int32_t* idx, int top_k, const uint8_t* swa_kv,
                            int S_cap, const int32_t* swa_pos0, const int32_t* q_pos,
                            float sm_scale, int window, int replay_start, const float* sink,
                            int kv_fmt, const Pages& pg, int B, int n_q, uint16_t* out, float* lse,
                            hipStream_t stream) {
  const int rows = B * n_q;
  AttnArgs a;
  a.q = q; a.kv_fp4 = kv_fp4; a.kv_scale = kv_scale; a.idx = idx; a.swa = swa_kv;
  a.swa_pos0 = swa_pos0; a.q_pos = q_pos; a.out = out; a.lse = lse;
  a.N_cap = N_cap; a.top_k = top_k; a.S_cap = S_cap; a.n_q = n_q;
  a.window = window; a.replay_start = replay_start;
  a.sink = sink;
  a.pg = pg;
  a.scale2 = sm_scale * kLog2e;
  a.rows = rows;
  const int tkp = (top_k + kTile - 1) / kTile * kTile;
  a.n_chunks = (tkp + kMaxWindow + kChunk - 1) / kChunk;
  if (kv_fmt == kFmtE8M0)
    hipLaunchKernelGGL(k_attn_rows<kFmtE8M0>, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(k_attn_rows<kFmtE4M3>, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace csa2
