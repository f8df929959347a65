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
constexpr int kKdBf16 = 0;
constexpr int kKdFp8 = 1;
constexpr int kKdFp4 = 2;
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
  if constexpr (KD == kKdFp4)
    t.sc = *reinterpret_cast<const uint16_t*>(scale_row + 2 * half);
}

// Query operand: the lane's head row (lane % 32), dims of its half.
__device__ __forceinline__ void load_query(bf16x8 qa[8], const uint16_t* q_row_base, int col,
                                           int half) {
  const u32x4* p = reinterpret_cast<const u32x4*>(q_row_base + col * kIdxDim + 64 * half);
#pragma unroll
  for (int s = 0; s < 8; ++s) qa[s] = __builtin_bit_cast(bf16x8, p[s]);
}

// Head weights of the 16 accumulator rows this lane holds.
__device__ __forceinline__ void load_weights(float wr[16], const float* w_row, int half) {
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w_row[8 * (r / 4) + 4 * half + (r % 4)];
}

template <int KD>
__device__ __forceinline__ f32x16 key_tile_dot(const bf16x8 qa[8], const KeyTile<KD>& t) {
  f32x16 acc = {};
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
    acc = mfma32(qa[s], kb, acc);
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
