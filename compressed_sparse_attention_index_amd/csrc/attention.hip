// Sparse multi-query attention over the selected MXFP4 main-KV entries plus
// the FP8 sliding window, with one softmax across both.
//
// "DeepSeek-V4.1-Flash 架构详解": §1 configuration table (64 query heads of
// 512 dims, window 128), §4 (main KV is MXFP4 and is dequantised before
// attention, SWA KV is FP8), §9 step 5 (decode attends to the CSA2-selected
// global KV plus this layer's SWA KV).  DeepSeek-V4 essay (mlqm.cn) §4.3: a
// compressed entry serves as both key and value.
//
// Work decomposition.  A workgroup (4 waves) takes one query row, one tile of
// 32 heads and a range of 64-entry chunks of the row's entry list
//   [ top_k selected slots, padded to a multiple of 32 | 128 window slots ].
// The two head-tile workgroups of a (row, split) get ids 8 apart, so they run
// on the same XCD and the second one finds the gathered entries in its L2.
// Wave w = (e, dh) owns entry tile e (32 entries) and dims half dh of every
// chunk, and keeps its own online-softmax state for the entries of tile e:
//   1. it gathers the raw bytes of its 32 entries x 256 dims with
//      direct-to-LDS loads, two tiles ahead, into a private staging slot
//      (no registers held; waits counted by hand);
//   2. it dequantises them exactly to bf16 with the gfx950 conversion
//      instructions (lane: entry lane % 32, 128 dims per lane half), keeps
//      them in its own region of an LDS tile and forms the partial
//      S^T[entry][head] over its 256 dims on 32x32x16 bf16 MFMA with q^T in
//      registers; the partner wave (e, 1 - dh) supplies the other 256 dims
//      through LDS (the only exchange inside the loop);
//   3. online softmax in fp32 (log2 domain) over tile e, identical in both
//      waves of the pair; P stays in registers, in the accumulator's own lane
//      order, which is the B-operand order of the next step once the entry
//      order inside an MFMA step is permuted to match;
//   4. O^T[dim][head] += V^T . P^T for its 256 dims, V^T read back from its
//      own LDS region with transposing reads (ds_read_b64_tr_b16), so K and V
//      share one copy and no other wave waits for it.
// At the end the two entry-tile states of each dims half are merged through
// LDS.  LDS tile rows are 1088 bytes apart and 16-byte chunk k of row r sits
// at k ^ ((r / 4) % 4); together these keep both the row-wise stores and the
// transposing reads free of bank conflicts, and let the transposing reads of
// a lane differ only by immediate offsets.
// Rows split over several workgroups write (m, l, O) partials that a second
// kernel merges in split order; when there are enough rows every workgroup
// covers whole rows and no partials are written.  The partial O (relative to
// its split's own max) is rounded to bf16, like the output itself: half the
// bytes of fp32 partials for a rounding error of the same size as the
// output's; m and l stay fp32.
#include "csa2_launch.h"
#include "csa2_device.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;
constexpr int kTile = 32;
constexpr int kHeadTile = 32;
constexpr int kRowBytes = 1088;    // pitch of the dequantised entries in the LDS tile
constexpr int kStage = 8192;       // staging bytes per wave and tile
constexpr int kMainLoads = 5;      // direct-to-LDS loads per wave: selected tile
constexpr int kWindowLoads = 8;    //                                 window tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kFillWgs = 256;      // rows are split until about this many workgroups exist
constexpr int kMaxSplits = 64;
constexpr int kMaxChunks = (kMaxTopK + kMaxWindow + kChunk - 1) / kChunk;
// The softmax reference max of a wave moves only when a tile's max exceeds it
// by more than this (log2 units): P then stays below 2^kLazyRescale, well
// inside bf16 and fp32 range at unchanged relative precision, and the
// accumulators are rescaled rarely instead of on every new max.
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
  uint16_t* part_o;  // [rows, nsplit, 64, 512] bf16, or null
  float* part_ml;    // [rows, nsplit, 64, 2] or null
  int N_cap, top_k, S_cap, n_q, window, replay_start;
  int rows, n_chunks, cps, nsplit;
  float scale2;      // sm_scale * log2(e)
};

// Pointers to the kernel's LDS arrays.
struct Lds {
  uint8_t* v;                       // dequantised chunk, [entry][dim], swizzled
  uint8_t (*stage)[4][kStage];      // raw bytes per stage and wave
  f32x4_t (*sx)[4][64];             // partial S^T per wave, [wave][i / 4][lane]
  int* ids;                         // selected ids of the workgroup's chunks (-1: none)
};

struct RowCtx {
  int r, b, tkp, qpos, lo, p0, dh, e, half, slot0, wave, lane;
};

struct State {
  bf16x8 qb[16];
  f32x16 o[8];
  float m_run, l_run;
};

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// Whether the wave's tile of chunk ch holds selected entries (else window).
__device__ __forceinline__ bool tile_is_main(const RowCtx& x, int ch) {
  return kChunk * ch + kTile * x.e < x.tkp;
}

// Issues the wave's direct-to-LDS loads of its tile of chunk ch into staging
// slot `stg` and returns whether the lane's slot holds an entry.  Slot
// layout: load i of lane l lands at 1024 i + 16 l (selected tiles: 4 x 16 B
// of E2M1 and, at 4096 + 4 l, the 4 E8M0 scales; window tiles: 8 x 16 B of
// FP8).  An empty slot reads a row that always exists (entry 0 of the
// sequence, or the query row), so every tile of a kind issues a fixed number
// of loads; it is zeroed when dequantised.
__device__ __forceinline__ bool issue_tile(const AttnArgs& a, const RowCtx& x, const Lds& s,
                                           int ch, int stg) {
  const int c = x.lane & 31;
  const int slot = kChunk * ch + kTile * x.e + c;
  const uint32_t dst = lds_offset(s.stage[stg][x.wave]);
  if (tile_is_main(x, ch)) {
    const int id = s.ids[slot - x.slot0];
    const bool valid = id >= 0;
    const size_t er = static_cast<size_t>(x.b) * a.N_cap + (valid ? id : 0);
    const uint8_t* src = a.kv_fp4 + er * 256 + 128 * x.dh + 64 * x.half;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(src + 16 * i, dst + 1024 * i);
    dma4(a.kv_scale + er * 16 + 8 * x.dh + 4 * x.half, dst + 4096);
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

__device__ __forceinline__ uint32_t word_of(const u32x4& w4, int k) {
  return k == 0 ? w4.x : k == 1 ? w4.y : k == 2 ? w4.z : w4.w;
}

__device__ __forceinline__ bf16x8 tr_read_pair(const uint8_t* v, int off0, int off1) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v + off0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v + off1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 l = static_cast<__bf16>(lo), h = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h)) << 16);
}

// The wave's tile of chunk ch, staged in slot `stg`; `valid` is the lane's
// slot validity and is replaced by that of chunk ch + 2, whose loads go to
// the same slot once this tile is dequantised.
__device__ __forceinline__ void attend_tile(const AttnArgs& a, const RowCtx& x, const Lds& s,
                                            State& st, bool& valid, int ch, int c1, int stg) {
  const int wave = x.wave, lane = x.lane;
  const int c = lane & 31;
  const uint32_t vmask = static_cast<uint32_t>(__ballot(valid));
  const bool lane_valid = valid;
  const int rho0 = 4 * x.half;   // entry of sacc[i]: 8 (i / 4) + 4 half + i % 4

  // This tile's loads have landed once only chunk ch + 1's are outstanding.
  if (ch + 1 < c1) {
    if (tile_is_main(x, ch + 1)) wait_vmem<kMainLoads>();
    else wait_vmem<kWindowLoads>();
  } else {
    wait_vmem<0>();
  }
  asm volatile("" ::: "memory");

  // Dequantise (empty slots give zeros: scale 0 for E2M1, which has no NaN;
  // zeroed bytes for FP8), keep in the wave's LDS region, partial S^T.  The
  // dims-half-0 wave starts the sums of empty slots at -inf, so that S is
  // -inf exactly there and no per-element mask is needed afterwards.
  f32x16 sacc = {}, sacc2 = {};
  if (x.dh == 0 && vmask != 0xffffffffu) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rho = 8 * (i >> 2) + rho0 + (i & 3);
      if (!((vmask >> rho) & 1u)) sacc[i] = -__builtin_inff();
    }
  }
  const uint8_t* sp = s.stage[stg][wave] + 16 * lane;
  const int row = kTile * x.e + c;
  uint8_t* vrow = s.v + row * kRowBytes + 16 * (32 * x.dh + 16 * x.half);
  const int g = swz(row);
  if (tile_is_main(x, ch)) {
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const u32x4*>(sp + 1024 * i);
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(s.stage[stg][wave] + 4096 + 4 * lane);
    float scale[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      scale[i] = lane_valid ? e8m0_to_float((sc >> (8 * i)) & 0xffu) : 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bf16x8 kb = fp4x8_to_bf16x8(word_of(w[k >> 2], k & 3), scale[k >> 2]);
      *reinterpret_cast<bf16x8*>(vrow + 16 * (k ^ g)) = kb;
      if (k & 1) sacc2 = mfma32(kb, st.qb[k], sacc2);
      else sacc = mfma32(kb, st.qb[k], sacc);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const u32x2 w2 = *reinterpret_cast<const u32x2*>(sp + 1024 * (k >> 1) + 8 * (k & 1));
      const bf16x8 kb = fp8x8_to_bf16x8(lane_valid ? w2.x : 0u, lane_valid ? w2.y : 0u);
      *reinterpret_cast<bf16x8*>(vrow + 16 * (k ^ g)) = kb;
      if (k & 1) sacc2 = mfma32(kb, st.qb[k], sacc2);
      else sacc = mfma32(kb, st.qb[k], sacc);
    }
  }
  // Two accumulation chains (even and odd steps) keep two MFMAs in flight;
  // they are added in a fixed order.
  sacc += sacc2;
  if (ch + 2 < c1) valid = issue_tile(a, x, s, ch + 2, stg);

  // Exchange of the partial sums with the partner wave (e, 1 - dh): the
  // first barrier makes sure it has read the previous tile's values.
  lds_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s.sx[wave][i][lane] = f32x4_t{sacc[4 * i], sacc[4 * i + 1], sacc[4 * i + 2], sacc[4 * i + 3]};
  lds_barrier();

  // Sums S of head c for entries rho = 8 (i / 4) + 4 half + i % 4 of the tile
  // (a + b == b + a exactly, so both waves of the pair get the same S).
  float xv[16];
  float smax = -__builtin_inff();
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const f32x4_t other = s.sx[wave ^ 1][gi][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xv[4 * gi + j] = sacc[4 * gi + j] + other[j];
      smax = fmaxf(smax, xv[4 * gi + j]);
    }
  }
  smax = fmaxf(smax, other_half(smax));
  // Logits are S * scale2 (log2 units, scale2 > 0, so the max of the logits
  // is smax * scale2).  Reference max: set by the first tile with an entry
  // (O and l are still zero then), moved later only past kLazyRescale, with
  // O and l rescaled.
  const float tmax = smax * a.scale2;
  if (st.m_run == -__builtin_inff()) {
    st.m_run = tmax;
  } else if (__ballot(tmax > st.m_run + kLazyRescale) != 0) {
    const float m_new = fmaxf(st.m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[m][i] *= alpha;
    st.m_run = m_new;
  }
  // p = 2^(S scale2 - m): empty slots have S = -inf and give exactly 0.  The
  // max is still -inf only if no tile so far had an entry, this one included;
  // its p are then all 0 with any finite reference.
  const float m_ref = st.m_run == -__builtin_inff() ? 0.0f : st.m_run;
  float tsum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    xv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(xv[i], a.scale2, -m_ref));
    tsum += xv[i];
  }
  tsum += other_half(tsum);
  st.l_run += tsum;

  // O^T[dims 256 dh + 32 m + .., head] += V^T . P^T over the tile's entries.
  // Lane (i16 = lane % 16) reads 8 bytes at row r = 32 e + 16 t + 4 half +
  // i16 / 4 (and r + 8), dims 256 dh + 32 m + 16 ((lane / 16) % 2) + 4 (i16 %
  // 4), i.e. 16-byte chunk 32 dh + 4 m + cl; swz(r) = half and swz(r + 8) =
  // half + 2 for every t, so m and t only move the address by constants.
  const int i16 = lane & 15;
  const int rq = i16 >> 2;
  const int cl = 2 * ((lane >> 4) & 1) + ((i16 & 3) >> 1);
  const int byte = 8 * (i16 & 1);
  const int r0 = kTile * x.e + 4 * x.half + rq;
  const int base_a = r0 * kRowBytes + 16 * (32 * x.dh + (cl ^ x.half)) + byte;
  const int base_b = (r0 + 8) * kRowBytes + 16 * (32 * x.dh + (cl ^ (x.half + 2))) + byte;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16x8 va[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int off = 16 * kRowBytes * t + 64 * m;
      va[m] = tr_read_pair(s.v, base_a + off, base_b + off);
    }
    const bf16x8 pbv = __builtin_bit_cast(
        bf16x8, u32x4{pack_bf16x2(xv[8 * t], xv[8 * t + 1]), pack_bf16x2(xv[8 * t + 2], xv[8 * t + 3]),
                      pack_bf16x2(xv[8 * t + 4], xv[8 * t + 5]),
                      pack_bf16x2(xv[8 * t + 6], xv[8 * t + 7])});
#pragma unroll
    for (int m = 0; m < 8; ++m) st.o[m] = mfma32(va[m], pbv, st.o[m]);
  }
}

// Merge of the two entry-tile states of each dims half, then the output (or
// the split partial): wave (E, dh) keeps the 32-dim blocks m with m / 4 == E
// and hands the others to wave (1 - E, dh) through the no longer needed LDS
// tile.  Both waves of a pair hold the same (m, l).
template <int E>
__device__ __forceinline__ void finish(const AttnArgs& a, const RowCtx& x, const State& st,
                                       uint8_t* lds_tile, float (*ml)[2][32], int split,
                                       int head) {
  const int c = x.lane & 31;
  f32x4_t* xo = reinterpret_cast<f32x4_t*>(lds_tile);   // [wave][4 blocks][4][64 lanes]
#pragma unroll
  for (int mm = 0; mm < 4; ++mm)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      xo[((x.wave * 4 + mm) * 4 + i4) * 64 + x.lane] =
          f32x4_t{st.o[4 * (1 - E) + mm][4 * i4], st.o[4 * (1 - E) + mm][4 * i4 + 1],
                  st.o[4 * (1 - E) + mm][4 * i4 + 2], st.o[4 * (1 - E) + mm][4 * i4 + 3]};
  if (x.half == 0) {
    ml[x.wave][0][c] = st.m_run;
    ml[x.wave][1][c] = st.l_run;
  }
  lds_barrier();
  const int pw = x.wave ^ 2;   // partner: same dims half, other entry tile
  const float m_o = ml[pw][0][c], l_o = ml[pw][1][c];
  const float m_all = fmaxf(st.m_run, m_o);
  const float w_me = st.m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(st.m_run - m_all);
  const float w_o = m_o == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_o - m_all);
  // Sums are formed in entry-tile order (tile 0 first) in both waves.
  const float l_all = E == 0 ? st.l_run * w_me + l_o * w_o : l_o * w_o + st.l_run * w_me;

  // This wave's dims: 256 dh + 128 E + 32 mm + 8 (i / 4) + 4 half + i % 4.
  const int dim0 = 256 * x.dh + 128 * E;
  const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
  const size_t ps = static_cast<size_t>(x.r) * a.nsplit + split;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4_t other = xo[((pw * 4 + mm) * 4 + i4) * 64 + x.lane];
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float mine = st.o[4 * E + mm][4 * i4 + j] * w_me, theirs = other[j] * w_o;
        v[j] = E == 0 ? mine + theirs : theirs + mine;
      }
      const int d = dim0 + 32 * mm + 8 * i4 + 4 * x.half;
      if (a.nsplit == 1) {
        *reinterpret_cast<u32x2*>(a.out + (static_cast<size_t>(x.r) * kHeads + head) * kDim + d) =
            u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
      } else {
        *reinterpret_cast<u32x2*>(a.part_o + (ps * kHeads + head) * kDim + d) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
  if (x.dh == 0 && E == 0 && x.half == 0) {
    if (a.nsplit == 1) {
      if (a.lse != nullptr)
        a.lse[static_cast<size_t>(x.r) * kHeads + head] =
            l_all > 0.0f ? (m_all + log2f(l_all)) * kLn2 : -__builtin_inff();
    } else {
      a.part_ml[(ps * kHeads + head) * 2 + 0] = m_all;
      a.part_ml[(ps * kHeads + head) * 2 + 1] = l_all;
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_sparse_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t l_v[kChunk * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t l_stage[2][4][kStage];
  __shared__ __attribute__((aligned(16))) f32x4_t l_sx[4][4][64];
  __shared__ int l_ids[kMaxChunks * kChunk];
  __shared__ float l_ml[4][2][32];
  const Lds s{l_v, l_stage, l_sx, l_ids};

  // Work id: the two head tiles of a (row, split) are 8 ids apart (same XCD).
  const int id = blockIdx.x;
  const int ht = (id >> 3) & 1;
  const int pair = (id >> 4) * 8 + (id & 7);
  if (pair >= a.rows * a.nsplit) return;
  RowCtx x;
  x.r = pair / a.nsplit;
  const int split = pair - x.r * a.nsplit;
  x.b = x.r / a.n_q;
  x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  x.lane = threadIdx.x & 63;
  x.dh = x.wave & 1;
  x.e = x.wave >> 1;
  x.half = x.lane >> 5;
  x.tkp = (a.top_k + kTile - 1) / kTile * kTile;
  x.qpos = a.q_pos[x.r];
  x.p0 = a.swa_pos0[x.b];
  x.lo = max(max(x.qpos - a.window + 1, x.p0), 0);
  if (a.replay_start >= 0) x.lo = max(x.lo, a.replay_start);
  const int c0 = split * a.cps;
  const int c1 = min(c0 + a.cps, a.n_chunks);
  const int c = x.lane & 31;
  const int head = kHeadTile * ht + c;

  // The selected ids of chunks [c0, c1) go to LDS first, so that no gather
  // waits on a global id load; out-of-range ids become -1 (no entry).  The
  // id loads and the q loads below are all issued before any is used.
  x.slot0 = kChunk * c0;
  constexpr int kPer = (kMaxChunks * kChunk + kThreads - 1) / kThreads;
  int sid[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int slot = x.slot0 + threadIdx.x + kThreads * u;
    sid[u] = -1;
    if (slot < kChunk * c1 && slot < a.top_k)
      sid[u] = a.idx[static_cast<size_t>(x.r) * a.top_k + slot];
  }
  // q^T operand (lane = head, dims 256 dh + 128 half + 8 k).
  State st;
  {
    const u32x4* p = reinterpret_cast<const u32x4*>(
        a.q + (static_cast<size_t>(x.r) * kHeads + head) * kDim + 256 * x.dh + 128 * x.half);
    // q is only ever an MFMA operand, which may come from accumulation
    // registers: defining it there leaves the VGPRs to the accumulators and
    // to the LDS reads in flight.  All 16 loads are issued first.
    u32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = p[k];
#pragma unroll
    for (int k = 0; k < 16; ++k) st.qb[k] = __builtin_bit_cast(bf16x8, to_agpr(v[k]));
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + kThreads * u;
    if (i < kChunk * (c1 - c0)) s.ids[i] = sid[u] < a.N_cap ? sid[u] : -1;
  }
  // q and the ids have landed before the first gather is issued: no other
  // vector-memory load is in flight inside the loop.
  wait_vmem<0>();
  __syncthreads();

  bool valid0 = issue_tile(a, x, s, c0, 0);
  bool valid1 = false;
  if (c0 + 1 < c1) valid1 = issue_tile(a, x, s, c0 + 1, 1);
#pragma unroll
  for (int m = 0; m < 8; ++m) st.o[m] = f32x16{};
  st.m_run = -__builtin_inff();
  st.l_run = 0.0f;

  // One loop body for both staging slots (slot = chunk parity): with the
  // body duplicated per slot the compiler no longer proves the staging slots
  // apart from the other LDS arrays and drains the loads in flight.
  for (int ch = c0; ch < c1; ++ch) {
    const int stg = (ch - c0) & 1;
    bool v = stg ? valid1 : valid0;
    attend_tile(a, x, s, st, v, ch, c1, stg);
    if (stg) valid1 = v;
    else valid0 = v;
  }

  lds_barrier();   // all transposing reads of the tile are done
  if (x.e == 0) finish<0>(a, x, st, s.v, l_ml, split, head);
  else finish<1>(a, x, st, s.v, l_ml, split, head);
}

// Merge of split partials in split order: one workgroup per (row, head),
// 64 threads x 8 dims.  Lane s < nsplit fetches split s's (m, l); the merge
// weights are formed in registers and the partial outputs are read with all
// loads of a group of splits issued together.
__global__ __launch_bounds__(64) void k_attn_combine(AttnArgs a) {
  const int r = blockIdx.x / kHeads;
  const int head = blockIdx.x % kHeads;
  const int t = threadIdx.x;
  const size_t ps0 = static_cast<size_t>(r) * a.nsplit;
  float ms = -__builtin_inff(), lsv = 0.0f;
  if (t < a.nsplit) {
    ms = a.part_ml[((ps0 + t) * kHeads + head) * 2];
    lsv = a.part_ml[((ps0 + t) * kHeads + head) * 2 + 1];
  }
  float mx = ms;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
  const float wgt_mine = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - mx);
  float L = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  constexpr int kGroup = 4;
  for (int s0 = 0; s0 < a.nsplit; s0 += kGroup) {
    u32x4 u[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int sp = min(s0 + g, a.nsplit - 1);
      u[g] = *reinterpret_cast<const u32x4*>(a.part_o + ((ps0 + sp) * kHeads + head) * kDim + 8 * t);
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const float wgt = __shfl(wgt_mine, s0 + g, 64);
      const float lsg = __shfl(lsv, s0 + g, 64);
      if (s0 + g < a.nsplit) {
        L += wgt * lsg;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = word_of(u[g], j);
          acc[2 * j] += wgt * __uint_as_float(w << 16);
          acc[2 * j + 1] += wgt * __uint_as_float(w & 0xffff0000u);
        }
      }
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<u32x4*>(a.out + (static_cast<size_t>(r) * kHeads + head) * kDim + 8 * t) =
      u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
            pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  if (t == 0 && a.lse != nullptr)
    a.lse[static_cast<size_t>(r) * kHeads + head] =
        L > 0.0f ? (mx + log2f(L)) * kLn2 : -__builtin_inff();
}

// Splits per row: none once the (row, head tile) workgroups alone reach about
// kFillWgs, otherwise enough to get there (at most one chunk per split).
void plan(int rows, int top_k, int* n_chunks, int* cps, int* nsplit) {
  const int tkp = (top_k + kTile - 1) / kTile * kTile;
  *n_chunks = (tkp + kMaxWindow + kChunk - 1) / kChunk;
  const long long per_split = 2LL * rows;
  long long want = (kFillWgs + per_split - 1) / per_split;
  if (want < 1) want = 1;
  if (want > *n_chunks) want = *n_chunks;
  if (want > kMaxSplits) want = kMaxSplits;
  *cps = (*n_chunks + static_cast<int>(want) - 1) / static_cast<int>(want);
  *nsplit = (*n_chunks + *cps - 1) / *cps;
}

}  // namespace

size_t attn_workspace_bytes(int rows, int top_k) {
  int n_chunks, cps, nsplit;
  plan(rows, top_k, &n_chunks, &cps, &nsplit);
  if (nsplit == 1) return 0;
  return static_cast<size_t>(rows) * nsplit * kHeads * (kDim * sizeof(uint16_t) + 2 * sizeof(float));
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                              int N_cap, const int32_t* idx, int top_k, const uint8_t* swa_kv,
                              int S_cap, const int32_t* swa_pos0, const int32_t* q_pos,
                              float sm_scale, int window, int replay_start, int B, int n_q,
                              uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  const int rows = B * n_q;
  AttnArgs a;
  a.q = q; a.kv_fp4 = kv_fp4; a.kv_scale = kv_scale; a.idx = idx; a.swa = swa_kv;
  a.swa_pos0 = swa_pos0; a.q_pos = q_pos; a.out = out; a.lse = lse;
  a.N_cap = N_cap; a.top_k = top_k; a.S_cap = S_cap; a.n_q = n_q;
  a.window = window; a.replay_start = replay_start;
  a.scale2 = sm_scale * kLog2e;
  a.rows = rows;
  plan(rows, top_k, &a.n_chunks, &a.cps, &a.nsplit);
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (a.nsplit > 1) {
    a.part_o = static_cast<uint16_t*>(ws);
    a.part_ml = reinterpret_cast<float*>(a.part_o + static_cast<size_t>(rows) * a.nsplit * kHeads * kDim);
  }
  const long long pairs = static_cast<long long>(rows) * a.nsplit;
  const long long wgs = (pairs + 7) / 8 * 16;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_sparse_attn, dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, stream,
                     a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nsplit == 1) return err;
  hipLaunchKernelGGL(k_attn_combine, dim3(rows * kHeads), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa2
