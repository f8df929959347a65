// Sparse multi-query attention over the selected MXFP4 main-KV entries plus
// the FP8 sliding window, with one softmax across both.
//
// "DeepSeek-V4.1-Flash 架构详解": §1 configuration table (64 query heads of
// 512 dims, window 128), §4 (main KV is MXFP4 and is dequantised before
// attention, SWA KV is FP8), §9 step 5 (decode attends to the CSA2-selected
// global KV plus this layer's SWA KV).  DeepSeek-V4 essay (mlqm.cn) §4.3: a
// compressed entry serves as both key and value.
//
// Work decomposition.  A workgroup (4 waves) takes one query row and a range
// of 64-entry chunks of the row's entry list
//   [ top_k selected slots, padded to a multiple of 32 | 128 window slots ].
// Wave w owns head tile h = w & 1 (32 heads) and entry tile e = w >> 1 of each
// chunk.  Per chunk:
//   1. the wave gathers its 32 entries straight into MFMA A-operand registers
//      (lane: entry lane%32, dims [256*half, +256)), dequantises them exactly
//      to bf16 with the gfx950 conversion instructions, and writes its share
//      of them to an LDS tile [64 entries][512 dims];
//   2. S^T[entry][head] = K . q^T on 32x32x16 bf16 MFMA; q of the row is
//      staged once in LDS (rows padded so the operand reads are conflict-free)
//      and each lane ends up with 16 logits of one head;
//   3. online softmax in fp32 (log2 domain); the two waves sharing a head tile
//      exchange per-head maxima and sums through LDS;
//   4. O^T[dim][head] += V^T . P^T: P^T is the softmax output still in
//      registers (the entry order inside an MFMA step is permuted to match
//      the accumulator layout), V^T comes from the LDS tile with transposing
//      reads (ds_read_b64_tr_b16), so K and V share one copy.  The wave
//      accumulates dims [256*e, +256) of its head tile.
// Rows with several workgroups write (m, l, O) partials that a second kernel
// merges in split order.
#include "csa2_launch.h"
#include "csa2_device.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;
constexpr int kTile = 32;
constexpr int kVPitch = 544;   // bf16 per LDS row: 1088 B, rows 64 B apart mod 256
constexpr int kQPitch = 520;   // bf16 per q row in LDS: 1040 B, rows 16 B apart mod 256
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTargetWgs = 512;

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
  float* part_o;     // [rows, nsplit, 64, 512] or null
  float* part_ml;    // [rows, nsplit, 64, 2] or null
  int N_cap, top_k, S_cap, n_q, window, replay_start;
  int n_chunks, cps, nsplit;
  float scale2;      // sm_scale * log2(e)
};

struct RawTile {
  u32x4 v[16];       // main: 8 words x 16 B of E2M1; window: 16 x 16 B of FP8
  u32x2 sc;          // main: 8 E8M0 scales
};

__device__ __forceinline__ bool load_entry(const AttnArgs& a, RawTile& t, int r, int b, int slot,
                                           int tkp, int half, int qpos, int lo) {
#pragma unroll
  for (int i = 0; i < 16; ++i) t.v[i] = u32x4{0, 0, 0, 0};
  t.sc = u32x2{0, 0};
  if (slot < tkp) {
    const int id = slot < a.top_k ? a.idx[static_cast<size_t>(r) * a.top_k + slot] : -1;
    if (id < 0 || id >= a.N_cap) return false;
    const size_t row = static_cast<size_t>(b) * a.N_cap + id;
    const u32x4* p = reinterpret_cast<const u32x4*>(a.kv_fp4 + row * 256 + 128 * half);
#pragma unroll
    for (int i = 0; i < 8; ++i) t.v[i] = p[i];
    t.sc = *reinterpret_cast<const u32x2*>(a.kv_scale + row * 16 + 8 * half);
    return true;
  }
  const int p = qpos - (kMaxWindow - 1) + (slot - tkp);
  const int p0 = a.swa_pos0[b];
  if (slot - tkp >= kMaxWindow || p < lo || p > qpos || p - p0 >= a.S_cap) return false;
  const size_t row = static_cast<size_t>(b) * a.S_cap + (p - p0);
  const u32x4* src = reinterpret_cast<const u32x4*>(a.swa + row * 512 + 256 * half);
#pragma unroll
  for (int i = 0; i < 16; ++i) t.v[i] = src[i];
  return true;
}

// Dims 256*half + 8*s .. +7 of the lane's entry as an MFMA operand.
__device__ __forceinline__ bf16x8 dequant_step(const RawTile& t, bool is_main, int s) {
  if (is_main) {
    const u32x4 w4 = t.v[s >> 2];
    const uint32_t w = (s & 3) == 0 ? w4.x : (s & 3) == 1 ? w4.y : (s & 3) == 2 ? w4.z : w4.w;
    const int q = s >> 2;   // scale index within the half
    const uint32_t code = ((q < 4 ? t.sc.x : t.sc.y) >> (8 * (q & 3))) & 0xffu;
    return fp4x8_to_bf16x8(w, e8m0_to_float(code));
  }
  const u32x4 w4 = t.v[s >> 1];
  return (s & 1) ? fp8x8_to_bf16x8(w4.z, w4.w) : fp8x8_to_bf16x8(w4.x, w4.y);
}

__device__ __forceinline__ bf16x8 tr_read_pair(const uint16_t* vbuf, int row, int col) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(vbuf + row * kVPitch + col));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(vbuf + (row + 8) * kVPitch + col));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(kThreads, 1) void k_sparse_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[kChunk * kVPitch];
  __shared__ __attribute__((aligned(16))) uint16_t qbuf[kHeads * kQPitch];
  __shared__ __attribute__((aligned(16))) uint32_t pbuf[4][64][8];
  __shared__ float xbuf[4][32];
  __shared__ float lbuf[4][32];

  const int r = blockIdx.y;
  const int split = blockIdx.x;
  const int b = r / a.n_q;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = wave & 1, e = wave >> 1, partner = wave ^ 2;
  const int half = lane >> 5, c = lane & 31;
  const int tkp = (a.top_k + kTile - 1) / kTile * kTile;
  const int ent = tkp + kMaxWindow;
  const int c0 = split * a.cps;
  const int c1 = min(c0 + a.cps, a.n_chunks);
  const int qpos = a.q_pos[r];
  int lo = max(max(qpos - a.window + 1, a.swa_pos0[b]), 0);
  if (a.replay_start >= 0) lo = max(lo, a.replay_start);

  // q of all 64 heads staged in LDS (coalesced 16-B loads); the q^T operand
  // of a step is read from there: lane = head 32h + c, dims 256*half + 8*s.
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.q + static_cast<size_t>(r) * kHeads * kDim);
#pragma unroll
    for (int i = 0; i < kHeads * kDim / 8 / kThreads; ++i) {
      const int g = i * kThreads + threadIdx.x;         // 16-B chunk: head g/64, dims 8*(g%64)
      *reinterpret_cast<u32x4*>(qbuf + (g >> 6) * kQPitch + 8 * (g & 63)) = src[g];
    }
  }
  const uint16_t* qrow = qbuf + (32 * h + c) * kQPitch + 256 * half;

  f32x16 o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.0f;

  RawTile raw;
  bool valid = load_entry(a, raw, r, b, kChunk * c0 + kTile * e + c, tkp, half, qpos, lo);

  for (int ch = c0; ch < c1; ++ch) {
    const int base = kChunk * ch + kTile * e;
    const bool is_main = base < tkp;
    const uint32_t vmask = static_cast<uint32_t>(__ballot(valid));

    __syncthreads();  // the previous chunk's readers of vbuf / pbuf are done
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const bf16x8 kb = dequant_step(raw, is_main, s);
      if ((s & 1) == h)
        *reinterpret_cast<bf16x8*>(vbuf + (kTile * e + c) * kVPitch + 256 * half + 8 * s) = kb;
      sacc = mfma32(kb, *reinterpret_cast<const bf16x8*>(qrow + 8 * s), sacc);
    }
    if (ch + 1 < c1)
      valid = load_entry(a, raw, r, b, base + kChunk + c, tkp, half, qpos, lo);

    // Logits of head 32h + c for entries rho = 8*(i/4) + 4*half + (i%4) of tile e.
    float x[16];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rho = 8 * (i >> 2) + 4 * half + (i & 3);
      x[i] = ((vmask >> rho) & 1u) ? sacc[i] * a.scale2 : -__builtin_inff();
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, other_half(tmax));
    if (half == 0) xbuf[wave][c] = tmax;
    __syncthreads();
    const float cmax = fmaxf(tmax, xbuf[partner][c]);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = (m_run == -__builtin_inff()) ? 0.0f : exp2f(m_run - m_new);
    float p[16];
    float tsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = (x[i] == -__builtin_inff()) ? 0.0f : exp2f(x[i] - m_new);
      tsum += p[i];
    }
    tsum += other_half(tsum);
    uint32_t pw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const __bf16 lo16 = static_cast<__bf16>(p[2 * k]);
      const __bf16 hi16 = static_cast<__bf16>(p[2 * k + 1]);
      pw[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo16)) |
              (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi16)) << 16);
    }
    *reinterpret_cast<u32x4*>(&pbuf[wave][lane][0]) = u32x4{pw[0], pw[1], pw[2], pw[3]};
    *reinterpret_cast<u32x4*>(&pbuf[wave][lane][4]) = u32x4{pw[4], pw[5], pw[6], pw[7]};
    if (half == 0) lbuf[wave][c] = tsum;
    __syncthreads();
    const float l0 = e == 0 ? tsum : lbuf[partner][c];
    const float l1 = e == 0 ? lbuf[partner][c] : tsum;
    l_run = l_run * alpha + (l0 + l1);
    m_run = m_new;

#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[m][i] *= alpha;

    // O^T[dims 256e + 32m + .., head] += V^T . P^T over the 64 entries.
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      const int src_wave = (et == e) ? wave : partner;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(&pbuf[src_wave][lane][0]);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(&pbuf[src_wave][lane][4]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, t == 0 ? w0 : w1);
        const int i16 = lane & 15;
        const int row = kTile * et + 16 * t + 4 * half + (i16 >> 2);
        const int colbase = 256 * e + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const bf16x8 va = tr_read_pair(vbuf, row, colbase + 32 * m);
          o[m] = mfma32(va, pb, o[m]);
        }
      }
    }
  }

  const int head = 32 * h + c;
  if (a.nsplit == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    uint16_t* orow = a.out + (static_cast<size_t>(r) * kHeads + head) * kDim + 256 * e;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        uint32_t w[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const __bf16 x0 = static_cast<__bf16>(o[m][4 * i4 + 2 * j] * inv);
          const __bf16 x1 = static_cast<__bf16>(o[m][4 * i4 + 2 * j + 1] * inv);
          w[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x0)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x1)) << 16);
        }
        *reinterpret_cast<u32x2*>(orow + 32 * m + 8 * i4 + 4 * half) = u32x2{w[0], w[1]};
      }
    if (a.lse != nullptr && e == 0 && half == 0)
      a.lse[static_cast<size_t>(r) * kHeads + head] =
          l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -__builtin_inff();
  } else {
    const size_t ps = static_cast<size_t>(r) * a.nsplit + split;
    float* prow = a.part_o + (ps * kHeads + head) * kDim + 256 * e;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4_t*>(prow + 32 * m + 8 * i4 + 4 * half) =
            f32x4_t{o[m][4 * i4], o[m][4 * i4 + 1], o[m][4 * i4 + 2], o[m][4 * i4 + 3]};
    if (e == 0 && half == 0) {
      a.part_ml[(ps * kHeads + head) * 2 + 0] = m_run;
      a.part_ml[(ps * kHeads + head) * 2 + 1] = l_run;
    }
  }
}

// Merge of split partials in split order: one workgroup per (row, head),
// 64 threads x 8 dims.  Lane s < nsplit fetches split s's (m, l); the merge
// weights are formed in registers and the partial outputs are read with all
// loads of a group of splits issued together.
constexpr int kMaxSplits = 64;

__global__ __launch_bounds__(64) void k_attn_combine(AttnArgs a) {
  const int r = blockIdx.x / kHeads;
  const int head = blockIdx.x % kHeads;
  const int t = threadIdx.x;
  const size_t ps0 = static_cast<size_t>(r) * a.nsplit;
  float ms = -__builtin_inff(), ls = 0.0f;
  if (t < a.nsplit) {
    ms = a.part_ml[((ps0 + t) * kHeads + head) * 2];
    ls = a.part_ml[((ps0 + t) * kHeads + head) * 2 + 1];
  }
  float mx = ms;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
  const float wgt_mine = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - mx);
  float L = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  constexpr int kGroup = 4;
  for (int s0 = 0; s0 < a.nsplit; s0 += kGroup) {
    f32x4_t u[kGroup], v[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int s = min(s0 + g, a.nsplit - 1);
      const f32x4_t* po = reinterpret_cast<const f32x4_t*>(
          a.part_o + ((ps0 + s) * kHeads + head) * kDim + 8 * t);
      u[g] = po[0];
      v[g] = po[1];
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const float wgt = __shfl(wgt_mine, s0 + g, 64);
      const float lsg = __shfl(ls, s0 + g, 64);
      if (s0 + g < a.nsplit) {
        L += wgt * lsg;
        acc[0] += wgt * u[g][0]; acc[1] += wgt * u[g][1]; acc[2] += wgt * u[g][2]; acc[3] += wgt * u[g][3];
        acc[4] += wgt * v[g][0]; acc[5] += wgt * v[g][1]; acc[6] += wgt * v[g][2]; acc[7] += wgt * v[g][3];
      }
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const __bf16 x0 = static_cast<__bf16>(acc[2 * j] * inv);
    const __bf16 x1 = static_cast<__bf16>(acc[2 * j + 1] * inv);
    w[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x0)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x1)) << 16);
  }
  *reinterpret_cast<u32x4*>(a.out + (static_cast<size_t>(r) * kHeads + head) * kDim + 8 * t) =
      u32x4{w[0], w[1], w[2], w[3]};
  if (t == 0 && a.lse != nullptr)
    a.lse[static_cast<size_t>(r) * kHeads + head] =
        L > 0.0f ? (mx + log2f(L)) * kLn2 : -__builtin_inff();
}

void plan(int rows, int top_k, int* n_chunks, int* cps, int* nsplit) {
  const int tkp = (top_k + kTile - 1) / kTile * kTile;
  *n_chunks = (tkp + kMaxWindow + kChunk - 1) / kChunk;
  const long long total = static_cast<long long>(rows) * (*n_chunks);
  long long c = (total + kTargetWgs - 1) / kTargetWgs;
  if (c < 1) c = 1;
  if (c > *n_chunks) c = *n_chunks;
  if ((*n_chunks + c - 1) / c > kMaxSplits) c = (*n_chunks + kMaxSplits - 1) / kMaxSplits;
  *cps = static_cast<int>(c);
  *nsplit = (*n_chunks + *cps - 1) / *cps;
}

}  // namespace

size_t attn_workspace_bytes(int rows, int top_k) {
  int n_chunks, cps, nsplit;
  plan(rows, top_k, &n_chunks, &cps, &nsplit);
  if (nsplit == 1) return 0;
  return static_cast<size_t>(rows) * nsplit * kHeads * (kDim + 2) * sizeof(float);
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
  plan(rows, top_k, &a.n_chunks, &a.cps, &a.nsplit);
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (a.nsplit > 1) {
    a.part_o = static_cast<float*>(ws);
    a.part_ml = a.part_o + static_cast<size_t>(rows) * a.nsplit * kHeads * kDim;
  }
  hipLaunchKernelGGL(k_sparse_attn, dim3(a.nsplit, rows), dim3(kThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nsplit == 1) return err;
  hipLaunchKernelGGL(k_attn_combine, dim3(rows * kHeads), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa2
