// Device-side helpers shared by the CSA2 kernels (gfx950 / CDNA4 only).
//
// Number formats (OCP definitions; the method stores main KV as MXFP4 and SWA
// KV as FP8 -- "DeepSeek-V4.1-Flash 架构详解", §4):
//   FP8 E4M3FN -> bf16 and E2M1 (with a block scale) -> bf16 use the
//   gfx950 scaled-conversion instructions.  Every E4M3FN value is a bf16
//   value, and so is every E2M1 x 2^(c - 127) for E8M0 codes c <= 252 (the
//   largest, 6 x 2^125, is below the bf16 maximum; code 0 gives bf16
//   subnormals): those conversions are exact.  Codes 253 and 254 overflow
//   bf16 for E2M1 magnitudes >= 4 and >= 2 respectively.  Every E2M1 x E4M3
//   product (at most 2 x 4 significant bits, magnitudes 2^-10 .. 2688) is a
//   bf16 value too.
// Matrix cores: v_mfma_f32_32x32x16_bf16, wave64.  Operand layout (lane l):
//   A[m][k]: m = l % 32, k = 8 * (l / 32) + i, i = 0..7
//   B[k][n]: n = l % 32, k = 8 * (l / 32) + i
//   D[m][n]: n = l % 32, m = 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2_launch.h"

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kIdxHeads = 32;     // indexer heads
constexpr int kIdxDim = 128;      // indexer dim
constexpr int kHeads = 64;        // attention query heads
constexpr int kDim = 512;         // attention head dim = entry dim
constexpr int kBlock = 8;         // positions per pool block
constexpr int kMaxTopK = 512;
constexpr int kMaxPoolBlocks = 2048;
constexpr int kMaxWindow = 128;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Four FP8 E4M3FN bytes -> four bf16 (two packed words).
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// fp32 -> bf16 bits, rounded to the nearest bf16 value with ties to the even
// pattern (the gfx950 conversion instruction).
__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Eight FP8 bytes (two words) -> eight bf16 as an MFMA operand.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x2 a = fp8x4_to_bf16(w0), b = fp8x4_to_bf16(w1);
  u32x4 v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, v);
}

// Eight E2M1 nibbles (one word, element 2j in the low nibble of byte j) with
// one power-of-two block scale -> eight bf16.  The gfx950 scaled conversion
// reads only the exponent field of its fp32 scale operand (as an E8M0 code):
// the mantissa and the sign are ignored and +0 reads as 2^-127.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  u32x4 v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8, v);
}

// Eight E2M1 nibbles times an arbitrary fp32 scale s -> eight bf16.  The
// elements are converted at unit scale (exact) and multiplied by s in fp32;
// for an E4M3 scale the product of the two has at most 6 significant bits
// and lies within [2^-10, 2688], so the product and its bf16 rounding are
// both exact, and s = 0 gives zeros.
__device__ __forceinline__ bf16x8 fp4x8_mul_to_bf16x8(uint32_t w, float s) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  uint32_t r[4];
#define CSA2_FP4_PAIR(I)                                                                \
  {                                                                                     \
    const f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, I);             \
    r[I] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f * s, bf16x2_t));      \
  }
  CSA2_FP4_PAIR(0)
  CSA2_FP4_PAIR(1)
  CSA2_FP4_PAIR(2)
  CSA2_FP4_PAIR(3)
#undef CSA2_FP4_PAIR
  u32x4 v = {r[0], r[1], r[2], r[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Main-KV scale layouts (csa2_kvfmt): E8M0 per 32 elements (16 bytes per
// entry) or E4M3FN per 16 elements (32 bytes per entry).
constexpr int kFmtE8M0 = 0;
constexpr int kFmtE4M3 = 1;
template <int FMT> struct KvFmt;
template <> struct KvFmt<kFmtE8M0> { static constexpr int kScaleBytes = 16, kBlock = 32; };
template <> struct KvFmt<kFmtE4M3> { static constexpr int kScaleBytes = 32, kBlock = 16; };

// Four FP8 E4M3FN bytes -> four floats (exact; the gfx950 conversion).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float (&f)[4]) {
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// E8M0 code -> 2^(code-127) as a float (code 0 gives the subnormal 2^-127,
// code 255 gives NaN).
__device__ __forceinline__ float e8m0_to_float(uint32_t code) {
  const uint32_t bits = code == 0 ? 0x00400000u : (code == 255 ? 0x7fc00000u : code << 23);
  return __uint_as_float(bits);
}

// Order-preserving map of fp32 to uint32: larger score -> larger key; -0 and
// +0 map to the same key.
__device__ __forceinline__ uint32_t float_to_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float other_half(float v) {
  uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float wave_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Waits until at most N vector-memory instructions of this wave are still
// outstanding (they complete in issue order).  Direct-to-LDS loads are not
// tracked by the compiler's own waits, so their consumers call this.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Waits until at most n (0 .. N) vector-memory instructions of this wave are
// outstanding, for a wave-uniform n known only at run time: the immediate is
// chosen by a chain of compares (callers test their common count first).
template <int N>
__device__ __forceinline__ void wait_vmem_le(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmem<N>();
      return;
    }
    wait_vmem_le<N - 1>(n);
  } else {
    wait_vmem<0>();
  }
}

// Byte offset of an LDS object within the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// Direct-to-LDS loads (lane l's 16 or 4 bytes land at lds + 16 l or + 4 l;
// lds must be wave-uniform).  They are issued as assembly on purpose: the
// compiler then does not track them, so it never drains them before
// unrelated LDS accesses or barriers.  Their consumers wait with wait_vmem,
// and a kernel that uses them issues no other vector-memory loads while any
// of them is in flight (the compiler's own waits would miscount).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its direct-to-LDS loads in flight (which the caller
// waits for with wait_vmem before the barrier when other waves read them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Moves a value into accumulation registers.  Used for MFMA operands that
// are loop-invariant (an MFMA may read A and B from there), which leaves the
// VGPRs to the accumulators and to loads in flight.
__device__ __forceinline__ u32x4 to_agpr(u32x4 v) {
  u32x4 w;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w.x) : "v"(v.x));
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w.y) : "v"(v.y));
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w.z) : "v"(v.z));
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(w.w) : "v"(v.w));
  return w;
}

// Physical page of logical page j of sequence b.  `mapped` says whether the
// table holds an id in [0, num_pages); an id outside is clamped into that
// range, so that no address is ever out of bounds.
__device__ __forceinline__ int page_id(const Pages& pg, int b, int j, bool& mapped) {
  const int v = pg.bt[static_cast<size_t>(b) * pg.max_pages + j];
  mapped = v >= 0 && v < pg.num_pages;
  return min(max(v, 0), pg.num_pages - 1);
}

// Row of entry e (0 <= e < N_cap) of sequence b: in the page pool, or
// b * N_cap + e without paging.
__device__ __forceinline__ size_t pool_row(const Pages& pg, int b, int N_cap, int e,
                                           bool& mapped) {
  if (pg.bt == nullptr) {
    mapped = true;
    return static_cast<size_t>(b) * N_cap + e;
  }
  const int p = page_id(pg, b, e >> pg.log2p, mapped);
  return (static_cast<size_t>(p) << pg.log2p) + (e & ((1 << pg.log2p) - 1));
}

}  // namespace csa2
