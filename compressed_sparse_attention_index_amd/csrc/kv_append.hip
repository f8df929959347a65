// KV append: the new tokens' main-KV entries are encoded as MXFP4 and their
// sliding-window entries as FP8, and written into the caches that the
// attention kernels read.
//
// "DeepSeek-V4.1-Flash 架构详解", §4: main KV is stored as MXFP4 (E2M1
// elements with block scales) and SWA KV as FP8 (E4M3FN).  Two block-scale
// formats: one E8M0 scale per 32 elements (OCP MX v1.0) or one E4M3FN scale
// per 16 elements (the page's §4 layout).  Encoding rules:
//   MXFP4: per 32 elements the shared exponent X = floor(log2(amax)) - 2
//     (2 is the largest E2M1 exponent), clamped to [-127, 127]; an all-zero
//     block takes X = -127.  The E8M0 code is X + 127.  Each element v / 2^X
//     is rounded to the nearest E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6},
//     a tie going to the even code, saturating at 6; a value that rounds to
//     zero is stored as +0.  Element 2j sits in the low nibble of byte j.
//   E2M1 with E4M3 scales: per 16 elements the scale s is amax / 6 rounded
//     to E4M3FN as below, so that the block's largest element lands at the
//     top of the E2M1 range; each element goes to the E2M1 magnitude nearest
//     to |v| / s (ties to the even code, saturating at 6), sign kept, a zero
//     stored as +0; a block whose scale is 0 stores +0 everywhere.
//   FP8 E4M3FN: saturate to +-448, then round to the nearest value, a tie
//     going to the even code; the sign is kept for values that round to 0.
// Inputs are bf16, so every step below is exact in fp32 up to the rounding
// to the target grid: the scaling by 2^-X is a power of two; amax / 6 is
// the correctly rounded fp32 quotient, which never crosses an E4M3 midpoint
// (a bf16 amax is either exactly 6 times a midpoint or at least one bf16 ulp
// from it); and |v| is compared with t s, midpoint t times the E4M3 scale,
// a product of at most 7 significant bits and so exact.
//
// A wave encodes kPer entries one after another: for each, lane l holds
// elements 8 l .. 8 l + 7 (one 16-byte load of the bf16 row), so a
// 32-element block is four lanes and every load and store of the wave is
// one contiguous row.
#include "csa2_launch.h"
#include "csa2_device.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kPer = 4;   // entries per wave

__device__ __forceinline__ uint32_t word_of4(const u32x4& w, int k) {
  return k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP8 E4M3FN code of x (saturating, round to nearest even, sign kept).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {   // below 2^-6: subnormal codes, steps of 2^-9 (8 is 2^-6)
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;   // -6 .. 8
    const float frac = __uint_as_float((__float_as_uint(a) & 0x007fffffu) | 0x3f800000u);  // [1, 2)
    uint32_t m = static_cast<uint32_t>(__builtin_rintf((frac - 1.0f) * 8.0f));
    int ee = e;
    if (m == 8u) {   // rounded up to the next binade
      m = 0u;
      ++ee;
    }
    code = (static_cast<uint32_t>(ee + 7) << 3) | m;
  }
  return sign | code;
}

// Encodes one main entry (lane l: elements 8 l .. 8 l + 7 in w) into row
// `row` of the main cache.
__device__ __forceinline__ void put_main(const u32x4& w, int lane, size_t row,
                                         uint8_t* __restrict__ kv_fp4,
                                         uint8_t* __restrict__ kv_scale) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = word_of4(w, k);
    v[2 * k] = bf16_lo(u);
    v[2 * k + 1] = bf16_hi(u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = fmaxf(amax, wave_xor(amax, 1));
  amax = fmaxf(amax, wave_xor(amax, 2));   // the block's four lanes agree
  // floor(log2 amax) - 2 from the exponent field; a zero or subnormal amax
  // (field 0) gives -127 after the clamp.
  const int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  const int X = ef == 0 ? -127 : max(ef - 127 - 2, -127);
  const float scale = X > -127 ? __uint_as_float(static_cast<uint32_t>(X + 127) << 23)
                               : __uint_as_float(0x00400000u);   // 2^X (2^-127 is subnormal)
  // The gfx950 scaled conversion rounds v / scale to the nearest E2M1 value
  // (ties to the even code, saturating at 6), two elements into byte k.  A
  // negative value that rounds to zero comes out as -0; it is stored as +0.
  uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], scale, 0);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], scale, 1);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], scale, 2);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], scale, 3);
  const uint32_t mag = packed & 0x77777777u;
  const uint32_t nonzero = (mag | (mag >> 1) | (mag >> 2)) & 0x11111111u;
  packed = mag | (packed & (nonzero << 3));
  __builtin_nontemporal_store(packed,
                              reinterpret_cast<uint32_t*>(kv_fp4 + row * (kDim / 2) + 4 * lane));
  // Scale code of block q from lane 4 q: one store instruction covering the
  // row's 16 bytes.
  if ((lane & 3) == 0) kv_scale[row * (kDim / 32) + (lane >> 2)] = static_cast<uint8_t>(X + 127);
}

// Encodes one main entry with E4M3 scales per 16 elements (lane l: elements
// 8 l .. 8 l + 7 in w, half of block l / 2) into row `row`.
__device__ __forceinline__ void put_main_e4m3(const u32x4& w, int lane, size_t row,
                                              uint8_t* __restrict__ kv_fp4,
                                              uint8_t* __restrict__ kv_scale) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = word_of4(w, k);
    v[2 * k] = bf16_lo(u);
    v[2 * k + 1] = bf16_hi(u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = fmaxf(amax, wave_xor(amax, 1));   // the block's two lanes agree
  const uint32_t code = e4m3_code(amax / 6.0f);
  float sv[4];
  e4m3x4_to_f32(code, sv);
  const float s = sv[0];
  // E2M1 midpoints 0.25 .. 5 and whether a tie there rounds up (to the even
  // code 2, 4 or 6) or down (to 0, 2 or 4).
  constexpr float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  constexpr bool kTieUp[7] = {false, true, false, true, false, true, false};
  uint32_t packed = 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float a = fabsf(v[k]);
    uint32_t mag = 0u;
#pragma unroll
    for (int m = 0; m < 7; ++m) {
      const float t = kMid[m] * s;
      mag += kTieUp[m] ? (a >= t ? 1u : 0u) : (a > t ? 1u : 0u);
    }
    if (code == 0u) mag = 0u;
    const uint32_t nib = mag | ((v[k] < 0.0f && mag != 0u) ? 8u : 0u);
    packed |= nib << (4 * k);
  }
  __builtin_nontemporal_store(packed,
                              reinterpret_cast<uint32_t*>(kv_fp4 + row * (kDim / 2) + 4 * lane));
  if ((lane & 1) == 0) kv_scale[row * (kDim / 16) + (lane >> 1)] = static_cast<uint8_t>(code);
}

// Wave w of workgroup x takes entries g0 .. g0 + kPer - 1 (g = b n_new + i)
// with g0 = kPer (kWaves x + w); the main-entry loads of all of them are
// issued together (rows clamped to the last entry, unused past it).  New
// entries are read once and the cache rows are not read back here, so both
// move with non-temporal loads and stores.
template <int FMT>
__global__ __launch_bounds__(64 * kWaves) void k_kv_append(
    const uint16_t* __restrict__ kv_new, const uint16_t* __restrict__ swa_new,
    const int32_t* __restrict__ pos, int B, int n_new, int N_cap, Pages pg,
    uint8_t* __restrict__ kv_fp4,
    uint8_t* __restrict__ kv_scale, uint8_t* __restrict__ swa, int S_cap,
    const int32_t* __restrict__ swa_pos0) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long total = static_cast<long long>(B) * n_new;
  const long long g0 = (static_cast<long long>(blockIdx.x) * kWaves + wave) * kPer;
  if (g0 >= total) return;   // the whole wave
  const uint8_t* kv_src = reinterpret_cast<const uint8_t*>(kv_new) + 16 * lane;
  u32x4 w[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const long long g = min(g0 + e, total - 1);
    w[e] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(kv_src + static_cast<size_t>(g) * kDim * 2));
  }
  // (sequence, token) of entry g0, then of the next entries by stepping.
  const int b0 = static_cast<int>(g0 / n_new);
  const int i0 = static_cast<int>(g0 - static_cast<long long>(b0) * n_new);
  int bs[kPer], is[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    int b = b0, i = i0 + e;
    while (i >= n_new) {   // n_new < kPer: an entry may lie several sequences on
      i -= n_new;
      ++b;
    }
    bs[e] = b;
    is[e] = i;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if (g0 + e >= total) break;
    const long long p = static_cast<long long>(pos[bs[e]]) + is[e];
    if (p < 0 || p >= N_cap) continue;
    bool mapped;
    const size_t row = pool_row(pg, bs[e], N_cap, static_cast<int>(p), mapped);
    if (!mapped) continue;   // an unmapped page: the entry is skipped
    if (FMT == kFmtE8M0) put_main(w[e], lane, row, kv_fp4, kv_scale);
    else put_main_e4m3(w[e], lane, row, kv_fp4, kv_scale);
  }
  if (swa_new == nullptr) return;
  // Window entries: only the rows inside the window are read.
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const long long g = g0 + e;
    if (g >= total) break;
    const int b = bs[e];
    const long long p = static_cast<long long>(pos[b]) + is[e];
    const long long j = p - swa_pos0[b];
    if (j < 0 || j >= S_cap) continue;
    const u32x4 sw = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(swa_new) +
                                                     static_cast<size_t>(g) * kDim * 2 + 16 * lane);
    u32x2 out = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t u = word_of4(sw, k);
      const uint32_t two = e4m3_code(bf16_lo(u)) | (e4m3_code(bf16_hi(u)) << 8);
      if (k < 2) out.x |= two << (16 * k);
      else out.y |= two << (16 * (k - 2));
    }
    *reinterpret_cast<u32x2*>(swa + (static_cast<size_t>(b) * S_cap + static_cast<size_t>(j)) *
                                        kDim + 8 * lane) = out;
  }
}

}  // namespace

hipError_t launch_kv_append(const uint16_t* kv_new, const uint16_t* swa_new, const int32_t* pos,
                            int B, int n_new, int N_cap, int kv_fmt, const Pages& pg,
                            uint8_t* kv_fp4,
                            uint8_t* kv_scale, uint8_t* swa, int S_cap, const int32_t* swa_pos0,
                            hipStream_t stream) {
  const long long waves = (static_cast<long long>(B) * n_new + kPer - 1) / kPer;
  const long long wgs = (waves + kWaves - 1) / kWaves;
  if (wgs < 1) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (kv_fmt == kFmtE8M0)
    hipLaunchKernelGGL(k_kv_append<kFmtE8M0>, dim3(static_cast<unsigned>(wgs)), dim3(64 * kWaves),
                       0, stream, kv_new, swa_new, pos, B, n_new, N_cap, pg, kv_fp4, kv_scale, swa,
                       S_cap, swa_pos0);
  else
    hipLaunchKernelGGL(k_kv_append<kFmtE4M3>, dim3(static_cast<unsigned>(wgs)), dim3(64 * kWaves),
                       0, stream, kv_new, swa_new, pos, B, n_new, N_cap, pg, kv_fp4, kv_scale, swa,
                       S_cap, swa_pos0);
  return hipGetLastError();
}

}  // namespace csa2
