// Internal launchers behind the C ABI (host side).  Arguments are validated by
// the API layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

hipError_t launch_index_score(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                              bool fp8, const int32_t* vis_len, int B, int n_q, int N_cap,
                              float* scores, float* block_max, hipStream_t stream);

// Re-scores the pool positions of every query row into pool_scores
// [B * n_q, k_blocks * 8] (-inf for empty or invisible slots).
hipError_t launch_pool_rescore(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                               bool fp8, const int32_t* pool_blocks, int k_blocks,
                               const int32_t* vis_len, int B, int n_q, int N_cap,
                               float* pool_scores, hipStream_t stream);

enum SelectSource { kSrcBlocks = 0, kSrcPoolStored = 1, kSrcPoolScored = 2, kSrcFlat = 3 };

// Exact Top-k selection, one workgroup per query row.  See topk.hip.
hipError_t launch_select(SelectSource src, const float* keys, const int32_t* pool_blocks,
                         int k_blocks, const int32_t* vis_len, int rows, int N_cap, int k,
                         int32_t* out_ids, float* out_keys, hipStream_t stream);

size_t attn_workspace_bytes(int rows, int top_k);

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                              int N_cap, const int32_t* idx, int top_k, const uint8_t* swa_kv,
                              int S_cap, const int32_t* swa_pos0, const int32_t* q_pos,
                              float sm_scale, int window, int replay_start, int B, int n_q,
                              uint16_t* out, float* lse, void* ws, hipStream_t stream);

}  // namespace csa2
