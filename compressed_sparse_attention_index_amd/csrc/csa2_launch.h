// Internal launchers behind the C ABI (host side).  Arguments are validated by
// the API layer before any of these is called.  A kv_fmt argument is a
// csa2_kvfmt value (0: E8M0 per 32, 1: E4M3 per 16).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Page table of a paged cache (csa2_paging in include/csa2.h): entry e of
// sequence b sits in pool row bt[b * max_pages + (e >> log2p)] * 2^log2p +
// (e & (2^log2p - 1)).  bt == nullptr: contiguous arrays, row b * N_cap + e.
struct Pages {
  const int32_t* bt;
  int log2p, max_pages, num_pages;
};

// kd: csa2_kdtype (0 bf16, 1 FP8, 2 MXFP4; MXFP4 only for n_q < 16).
// scores_bf16: `scores` receives bf16 bit patterns (2 bytes per entry, the
// fp32 score rounded to nearest even) and block_max must be null.
hipError_t launch_index_score(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                              int kd, const Pages& pg, const int32_t* vis_len, int B, int n_q,
                              int N_cap, float* scores, float* block_max, hipStream_t stream,
                              bool scores_bf16 = false);

// Prefill-chunk scoring on matrix cores (n_q >= 16 rows per sequence); see
// index_gemm.hip.
hipError_t launch_index_gemm(const uint16_t* q_idx, const float* w_idx, const uint8_t* k_idx,
                             bool fp8, const Pages& pg, const int32_t* vis_len, int B, int n_q,
                             int N_cap, float* scores, float* block_max, hipStream_t stream,
                             bool scores_bf16 = false);

// Block Top-K (pool of blocks); see topk.hip.
size_t block_topk_workspace_bytes(int rows, int N_cap);
int block_topk_max_blocks();
hipError_t launch_block_topk(const float* block_max, const int32_t* vis_len, int rows, int N_cap,
                             int k, int32_t* out, void* ws, hipStream_t stream);
// The same selection with the library's own fixed-size device scratch array
// instead of a caller's workspace (no allocation); see topk.hip.
bool block_topk_noalloc_fits(int rows, int N_cap);
hipError_t launch_block_topk_noalloc(const float* block_max, const int32_t* vis_len, int rows,
                                     int N_cap, int k, int32_t* out, hipStream_t stream);

// Pool Top-K.  mode 0: keys are stored scores; 1 / 2 / 3 / 4: the pool
// positions are re-scored with q_idx / w_idx on FP8 / bf16 / MXFP4 keys /
// MXFP4 keys with the query quantised to MXFP4.
size_t pool_topk_workspace_bytes(int rows, int k_blocks);
hipError_t launch_pool_topk(int mode, const float* scores, const uint16_t* q_idx,
                            const float* w_idx, const void* k_idx, const Pages& pg,
                            const int32_t* pool_blocks,
                            int k_blocks, const int32_t* vis_len, int rows, int n_q, int N_cap,
                            int top_k, int32_t* out, float* out_key, void* ws,
                            hipStream_t stream);

// Flat Top-K over [0, vis) of every row (prefill rows).
// bf16: `scores` holds bf16 bit patterns (uint16) instead of fp32.
hipError_t launch_flat_topk(const void* scores, const int32_t* vis_len, int rows, int N_cap,
                            int k, int32_t* out, float* out_key, hipStream_t stream,
                            bool bf16 = false);

size_t attn_workspace_bytes(int rows, int top_k);

// Attention of prefill-shaped calls (n_q >= kRowsKernelMinNq): one
// workgroup per query row, all 64 heads; see attention_rows.hip.  Decode
// rows use the head-group kernel of attention.hip.
constexpr int kRowsKernelMinNq = 16;
hipError_t launch_attn_rows(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                            int N_cap, const int32_t* idx, int top_k, const uint8_t* swa_kv,
                            int S_cap, const int32_t* swa_pos0, const int32_t* q_pos,
                            float sm_scale, int window, int replay_start, const float* sink,
                            int kv_fmt, const Pages& pg, int B, int n_q, uint16_t* out, float* lse,
                            hipStream_t stream);

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                              int N_cap, const int32_t* idx, int top_k, const uint8_t* swa_kv,
                              int S_cap, const int32_t* swa_pos0, const int32_t* q_pos,
                              float sm_scale, int window, int replay_start, const float* sink,
                              int kv_fmt, const Pages& pg, int B, int n_q, uint16_t* out,
                              float* lse, void* ws, hipStream_t stream);

// KV append: MXFP4 main entries and FP8 window entries of new tokens; see
// kv_append.hip.
hipError_t launch_kv_append(const uint16_t* kv_new, const uint16_t* swa_new, const int32_t* pos,
                            int B, int n_new, int N_cap, int kv_fmt, const Pages& pg,
                            uint8_t* kv_fp4,
                            uint8_t* kv_scale, uint8_t* swa, int S_cap, const int32_t* swa_pos0,
                            hipStream_t stream);

}  // namespace csa2
