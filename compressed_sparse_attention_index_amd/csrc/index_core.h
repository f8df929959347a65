// Indexer scoring core shared by the scan, prefill and pool re-scoring kernels.
//
// Score of entry t for one query row ("DeepSeek-V4.1-Flash 架构详解", §3.2;
// 32 x 128 indexer from the §1 configuration table):
//   s_t = sum_{h<32} w_h * max(0, q_h . k_t)
// One 32x32x16 bf16 MFMA step multiplies the 32 heads (A rows) by 32
// positions (B columns) over 16 dims; 8 steps cover the 128 dims.  The dims
// are split between the two wave halves: lane half `half` covers dims
// [64*half, 64*half + 64) of its position, step s using dims 64*half + 8*s
// .. +7, so each lane reads one contiguous 64-dim run of its key row.  The
// A operand (query) uses the same dim assignment.  The accumulator gives each
// lane 16 of the 32 heads of its position; the ReLU-weighted sum over those
// 16 plus the other half's 16 completes the head sum in registers.
#pragma once
#include "csa2_device.h"

namespace csa2 {

// Indexer-key storage types (csa2_kdtype): bf16 (256 B per entry), FP8
// E4M3FN (128 B), MXFP4 (64 B of E2M1 plus 4 E8M0 scales, one per 32 dims;
// the scales of all R rows of a buffer follow its R rows of E2M1).
// kKdFp4Q: MXFP4 keys with the query quantised to MXFP4 as well, the
// contraction on the scaled FP4 matrix instructions (products of two E2M1
// values with power-of-two scales are exact in fp32, so the result is the
// sum of the products of the dequantised values).
constexpr int kKdBf16 = 0;
constexpr int kKdFp8 = 1;
constexpr int kKdFp4 = 2;
constexpr int kKdFp4Q = 3;
constexpr bool fp4_keys(int kd) { return kd == kKdFp4 || kd == kKdFp4Q; }
template <int KD>
struct KeyFmt {
  static constexpr int kRowBytes = KD == kKdBf16 ? 256 : KD == kKdFp8 ? 128 : 64;
};

template <int KD>
struct KeyTile {
  static constexpr int kWords = KD == kKdBf16 ? 8 : KD == kKdFp8 ? 4 : 2;  // 16-B words per lane
  u32x4 v[kWords];
  uint32_t sc;   // MXFP4: the two E8M0 codes of the lane's half (low byte: dims 64 half .. + 32)
};

// Loads the lane's 64-dim half of one indexer-key row (MXFP4: and its two
// scale bytes from `scale_row`, the row's 4 scales).
template <int KD>
__device__ __forceinline__ void load_key_half(KeyTile<KD>& t, const uint8_t* row, int half,
                                              const uint8_t* scale_row = nullptr) {
  const u32x4* p = reinterpret_cast<const u32x4*>(row + (KeyFmt<KD>::kRowBytes / 2) * half);
#pragma unroll
  for (int i = 0; i < KeyTile<KD>::kWords; ++i) t.v[i] = p[i];
  if constexpr (fp4_keys(KD))
    t.sc = *reinterpret_cast<const uint16_t*>(scale_row + 2 * half);
}

// Query operand of the lane: its head row (lane % 32), dims of its half
// (64 half .. + 63).  bf16 for the bf16 contraction; for kKdFp4Q the same
// 64 dims as two MXFP4 blocks of 32 (16 bytes of E2M1 each, element 2j in
// the low nibble of byte j) and their two E8M0 codes (low byte: the first
// block).
template <int KD>
struct QueryOp {
  bf16x8 qa[8];
};
template <>
struct QueryOp<kKdFp4Q> {
  u32x4 q4[2];
  uint32_t sc;
};

// One OCP MXFP4 block of 32 bf16 values (w: four 16-byte words, exact in
// fp32): shared exponent X = floor(log2(amax)) - 2, clamped to [-127, 127]
// (-127 for an all-zero or subnormal amax); each v / 2^X rounded to the
// nearest E2M1 value, ties to the even code, saturating at 6 (the gfx950
// scaled conversion does this step).  A value that rounds to zero may keep
// its sign; -0 and +0 multiply alike, so it is left as it is.  Returns the
// E8M0 code X + 127.
__device__ __forceinline__ uint32_t mxfp4_block(const u32x4 (&w)[4], u32x4& out) {
  auto lo = [](uint32_t u) { return __uint_as_float(u << 16); };
  auto hi = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fmaxf(fabsf(lo(w[i][k])), fabsf(hi(w[i][k]))));
  const int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  const int X = ef == 0 ? -127 : max(ef - 127 - 2, -127);
  const float scale = X > -127 ? __uint_as_float(static_cast<uint32_t>(X + 127) << 23)
                               : __uint_as_float(0x00400000u);   // 2^X (2^-127 is subnormal)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, lo(w[i].x), hi(w[i].x), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo(w[i].y), hi(w[i].y), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo(w[i].z), hi(w[i].z), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo(w[i].w), hi(w[i].w), scale, 3);
    out[i] = r;
  }
  return static_cast<uint32_t>(X + 127);
}

template <int KD>
__device__ __forceinline__ void load_query(QueryOp<KD>& q, const uint16_t* q_row_base, int col,
                                           int half) {
  const u32x4* p = reinterpret_cast<const u32x4*>(q_row_base + col * kIdxDim + 64 * half);
  if constexpr (KD == kKdFp4Q) {
    // All eight loads in flight together, then the two blocks.
    u32x4 w[2][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i / 4][i % 4] = p[i];
    q.sc = mxfp4_block(w[0], q.q4[0]) | (mxfp4_block(w[1], q.q4[1]) << 8);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) q.qa[s] = __builtin_bit_cast(bf16x8, p[s]);
  }
}

// Head weights of the 16 accumulator rows this lane holds.
__device__ __forceinline__ void load_weights(float wr[16], const float* w_row, int half) {
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w_row[8 * (r / 4) + 4 * half + (r % 4)];
}

template <int KD>
__device__ __forceinline__ f32x16 key_tile_dot(const QueryOp<KD>& q, const KeyTile<KD>& t) {
  f32x16 acc = {};
  if constexpr (KD == kKdFp4Q) {
    // Two v_mfma_scale_f32_32x32x64_f8f6f4 steps with E2M1 operands: lane
    // (c, half) gives 32 consecutive dims (one MX block) of head c (A) and of
    // position c (B) and their block scales; step j covers dims
    // 64 half + 32 j .. + 31 in both halves.
    typedef int i32x8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const i32x8 a = {static_cast<int>(q.q4[j].x), static_cast<int>(q.q4[j].y),
                       static_cast<int>(q.q4[j].z), static_cast<int>(q.q4[j].w), 0, 0, 0, 0};
      const i32x8 b = {static_cast<int>(t.v[j].x), static_cast<int>(t.v[j].y),
                       static_cast<int>(t.v[j].z), static_cast<int>(t.v[j].w), 0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a, b, acc, 4 /* A: E2M1 */, 4 /* B: E2M1 */, 0,
          static_cast<int>((q.sc >> (8 * j)) & 0xffu), 0,
          static_cast<int>((t.sc >> (8 * j)) & 0xffu));
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 kb;
      if constexpr (KD == kKdFp8) {
        const u32x4 w = t.v[s / 2];
        kb = (s & 1) ? fp8x8_to_bf16x8(w.z, w.w) : fp8x8_to_bf16x8(w.x, w.y);
      } else if constexpr (KD == kKdFp4) {
        // Dims 64 half + 8 s .. + 7: word s % 4 of chunk s / 4, scale s / 4
        // (the conversion reads the E8M0 code from the exponent field).
        const u32x4 w = t.v[s / 4];
        const uint32_t word = (s & 3) == 0 ? w.x : (s & 3) == 1 ? w.y : (s & 3) == 2 ? w.z : w.w;
        kb = fp4x8_to_bf16x8(word, __uint_as_float(((t.sc >> (8 * (s / 4))) & 0xffu) << 23));
      } else {
        kb = __builtin_bit_cast(bf16x8, t.v[s]);
      }
      acc = mfma32(q.qa[s], kb, acc);
    }
  }
  return acc;
}

// max(0, x) as one integer max on the bit pattern: IEEE floats of either
// sign order like their bits read as signed integers, so every negative
// value (and -0) maps to +0 and every other value is kept.
__device__ __forceinline__ float relu(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// ReLU-weighted head sum; every lane returns the full 32-head score of its
// position (lanes l and l^32 hold the same value).
__device__ __forceinline__ float head_sum(const f32x16& acc, const float wr[16]) {
  float p = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) p = __builtin_fmaf(wr[r], relu(acc[r]), p);
  return p + other_half(p);
}

}  // namespace csa2
