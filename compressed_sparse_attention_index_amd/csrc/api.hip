// C ABI of the CSA2 decode hot path: host-side validation and dispatch.
// Every check runs before anything is enqueued; see include/csa2.h for the
// contract of each entry point.
#include "../../include/csa2.h"
#include "csa2_launch.h"
#include "csa2_device.h"

#include <stdint.h>

static_assert(csa2::kFmtE8M0 == CSA2_KV_MXFP4_E8M0_32 && csa2::kFmtE4M3 == CSA2_KV_FP4_E4M3_16,
              "kernel format ids follow csa2_kvfmt");

namespace {

constexpr int32_t kMaxNcap = 1 << 22;       // block ids fit the selection bitmap in LDS
constexpr int32_t kMaxGridY = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

csa2_status from_hip(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// A page table: NULL (contiguous) or a valid csa2_paging whose logical
// capacity is N_cap.  Fills `pg` (bt = nullptr for NULL).
csa2_status check_paging(const csa2_paging* paging, int32_t N_cap, csa2::Pages* pg) {
  *pg = csa2::Pages{nullptr, 0, 0, 0};
  if (!paging) return CSA2_OK;
  if (!paging->block_table) return CSA2_ERR_NULL;
  if (!aligned16(paging->block_table)) return CSA2_ERR_ALIGN;
  const int32_t P = paging->page_entries;
  if (P < 64 || P > 65536 || (P & (P - 1)) != 0) return CSA2_ERR_SHAPE;
  if (paging->max_pages < 1 || paging->num_pages < 1) return CSA2_ERR_SHAPE;
  if (static_cast<int64_t>(paging->max_pages) * P != N_cap) return CSA2_ERR_SHAPE;
  if (static_cast<int64_t>(paging->num_pages) * P > 0x7fffffffLL) return CSA2_ERR_SHAPE;
  int log2p = 0;
  while ((1 << log2p) < P) ++log2p;
  *pg = csa2::Pages{paging->block_table, log2p, paging->max_pages, paging->num_pages};
  return CSA2_OK;
}

csa2_status check_rows(int32_t B, int32_t n_q) {
  if (B < 1 || n_q < 1) return CSA2_ERR_SHAPE;
  if (static_cast<int64_t>(B) * n_q > (1LL << 30)) return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

csa2_status attn_common(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                        int32_t N_cap, const int32_t* idx, int32_t top_k, const uint8_t* swa_kv,
                        int32_t S_cap, const int32_t* swa_pos0, const int32_t* q_pos,
                        float sm_scale, const csa2_attn_opts* opts, int32_t B, int32_t n_q,
                        uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (!q || !kv_fp4 || !kv_scale || !swa_pos0 || !q_pos || !out) return CSA2_ERR_NULL;
  if (top_k > 0 && !idx) return CSA2_ERR_NULL;
  if (S_cap > 0 && !swa_kv) return CSA2_ERR_NULL;
  csa2_status st = check_rows(B, n_q);
  if (st != CSA2_OK) return st;
  if (N_cap < 1 || N_cap > kMaxNcap || top_k < 0 || top_k > 512 || S_cap < 0) return CSA2_ERR_SHAPE;
  if (static_cast<int64_t>(B) * n_q > kMaxGridY) return CSA2_ERR_SHAPE;
  // A softmax scale is positive and finite (1 / sqrt(512) on these layers);
  // the kernel relies on it to keep empty slots at -inf.
  if (!(sm_scale > 0.0f) || !(sm_scale < __builtin_inff())) return CSA2_ERR_SHAPE;
  int32_t window = 128, replay_start = -1, kv_fmt = CSA2_KV_MXFP4_E8M0_32;
  const float* sink = nullptr;
  csa2::Pages pg{nullptr, 0, 0, 0};
  if (opts) {
    if ((opts->kv_fmt != CSA2_KV_MXFP4_E8M0_32 && opts->kv_fmt != CSA2_KV_FP4_E4M3_16) ||
        (opts->flags & ~(CSA2_ATTN_SINK | CSA2_ATTN_PAGED)) != 0)
      return CSA2_ERR_UNSUPPORTED;
    if (opts->flags & CSA2_ATTN_PAGED) {
      if (!opts->paging) return CSA2_ERR_NULL;
      const csa2_status ps = check_paging(opts->paging, N_cap, &pg);
      if (ps != CSA2_OK) return ps;
    }
    kv_fmt = opts->kv_fmt;
    if (opts->window < 0 || opts->window > 128 || opts->replay_start < -1) return CSA2_ERR_SHAPE;
    window = opts->window;
    replay_start = opts->replay_start;
    if (opts->flags & CSA2_ATTN_SINK) {
      sink = opts->sink;
      if (!sink) return CSA2_ERR_NULL;
    }
  }
  const void* ptrs[] = {q, kv_fp4, kv_scale, idx, swa_kv, swa_pos0, q_pos, out, lse, sink};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return CSA2_ERR_ALIGN;
  const size_t need = csa2::attn_workspace_bytes(B * n_q, top_k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return CSA2_ERR_ALIGN;
  return from_hip(csa2::launch_sparse_attn(q, kv_fp4, kv_scale, N_cap, idx, top_k, swa_kv, S_cap,
                                           swa_pos0, q_pos, sm_scale, window, replay_start, sink,
                                           kv_fmt, pg, B, n_q, out, lse, ws, stream));
}

// Validation and launch of the scan; bf16: scores are bf16 bit patterns
// (no block maxima).
csa2_status index_score_impl(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                             csa2_kdtype k_dtype, const csa2_paging* paging,
                             const int32_t* vis_len, int32_t B, int32_t n_q, int32_t N_cap,
                             float* scores, float* block_max, bool bf16, hipStream_t stream) {
  if (!q_idx || !w_idx || !k_idx || !vis_len) return CSA2_ERR_NULL;
  if (!scores && !block_max) return CSA2_ERR_NULL;
  if (k_dtype != CSA2_KDTYPE_BF16 && k_dtype != CSA2_KDTYPE_FP8_E4M3 &&
      k_dtype != CSA2_KDTYPE_MXFP4 && k_dtype != CSA2_KDTYPE_MXFP4_QK)
    return CSA2_ERR_UNSUPPORTED;
  // MXFP4 keys: decode rows only (the prefill-shaped kernel reads bf16 / FP8).
  if ((k_dtype == CSA2_KDTYPE_MXFP4 || k_dtype == CSA2_KDTYPE_MXFP4_QK) && n_q >= 16)
    return CSA2_ERR_UNSUPPORTED;
  csa2_status st = check_rows(B, n_q);
  if (st != CSA2_OK) return st;
  if (N_cap < 1 || N_cap > kMaxNcap) return CSA2_ERR_SHAPE;
  if (n_q < 16 && static_cast<int64_t>(B) * n_q > kMaxGridY) return CSA2_ERR_SHAPE;
  if (n_q >= 16 && (B > kMaxGridY || ceil_div(n_q, 16) > kMaxGridY)) return CSA2_ERR_SHAPE;
  const void* ptrs[] = {q_idx, w_idx, k_idx, vis_len, scores, block_max};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return CSA2_ERR_ALIGN;
  csa2::Pages pg;
  st = check_paging(paging, N_cap, &pg);
  if (st != CSA2_OK) return st;
  return from_hip(csa2::launch_index_score(q_idx, w_idx, k_idx, static_cast<int>(k_dtype), pg,
                                           vis_len, B, n_q, N_cap, scores, block_max, stream,
                                           bf16));
}

}  // namespace

extern "C" {

csa2_status csa2_index_score(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                             csa2_kdtype k_dtype, const csa2_paging* paging,
                             const int32_t* vis_len, int32_t B, int32_t n_q, int32_t N_cap,
                             float* scores, float* block_max, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return index_score_impl(q_idx, w_idx, k_idx, k_dtype, paging, vis_len, B, n_q, N_cap, scores,
                          block_max, false, stream);
}

csa2_status csa2_index_score_bf16(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                                  csa2_kdtype k_dtype, const csa2_paging* paging,
                                  const int32_t* vis_len, int32_t B, int32_t n_q, int32_t N_cap,
                                  uint16_t* scores, hipStream_t stream) {
  if (!scores) return CSA2_ERR_NULL;
  return index_score_impl(q_idx, w_idx, k_idx, k_dtype, paging, vis_len, B, n_q, N_cap,
                          reinterpret_cast<float*>(scores), nullptr, true, stream);
}

csa2_status csa2_flat_topk_bf16(const uint16_t* scores, const int32_t* vis_len, int32_t B,
                                int32_t n_q, int32_t N_cap, int32_t top_k, int32_t* idx_out,
                                float* idx_score, hipStream_t stream) {
  if (!scores || !vis_len || !idx_out) return CSA2_ERR_NULL;
  csa2_status st = check_rows(B, n_q);
  if (st != CSA2_OK) return st;
  if (N_cap < 1 || N_cap > kMaxNcap || top_k < 1 || top_k > 512) return CSA2_ERR_SHAPE;
  const int32_t rows = B * n_q;
  if (rows > kMaxGridY) return CSA2_ERR_SHAPE;
  const void* ptrs[] = {scores, vis_len, idx_out, idx_score};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return CSA2_ERR_ALIGN;
  return from_hip(csa2::launch_flat_topk(scores, vis_len, rows, N_cap, top_k, idx_out, idx_score,
                                         stream, true));
}

csa2_status csa2_block_topk(const float* block_max, const int32_t* vis_len, int32_t B,
                            int32_t n_q, int32_t N_cap, int32_t k_blocks, int32_t* pool_blocks,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!block_max || !vis_len || !pool_blocks) return CSA2_ERR_NULL;
  csa2_status st = check_rows(B, n_q);
  if (st != CSA2_OK) return st;
  if (N_cap < 1 || N_cap > kMaxNcap || k_blocks < 1 || k_blocks > 2048) return CSA2_ERR_SHAPE;
  if (static_cast<int64_t>(B) * n_q > kMaxGridY) return CSA2_ERR_SHAPE;
  const void* ptrs[] = {block_max, vis_len, pool_blocks, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return CSA2_ERR_ALIGN;
  const size_t need = csa2::block_topk_workspace_bytes(B * n_q, N_cap);
  if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  return from_hip(csa2::launch_block_topk(block_max, vis_len, B * n_q, N_cap, k_blocks,
                                          pool_blocks, ws, stream));
}

csa2_status csa2_block_topk_noalloc(const float* block_max, const int32_t* vis_len, int32_t B,
                                    int32_t n_q, int32_t N_cap, int32_t k_blocks,
                                    int32_t* pool_blocks, hipStream_t stream) {
  if (!block_max || !vis_len || !pool_blocks) return CSA2_ERR_NULL;
  csa2_status st = check_rows(B, n_q);
  if (st != CSA2_OK) return st;
  if (N_cap < 1 || N_cap > kMaxNcap || k_blocks < 1 || k_blocks > 2048) return CSA2_ERR_SHAPE;
  if (static_cast<int64_t>(B) * n_q > kMaxGridY) return CSA2_ERR_SHAPE;
  const void* ptrs[] = {block_max, vis_len, pool_blocks};
  for (const void* p : ptrs)
    if (!aligned16(p)) return CSA2_ERR_ALIGN;
  if (!csa2::block_topk_noalloc_fits(B * n_q, N_cap)) return CSA2_ERR_WORKSPACE;
  return from_hip(csa2::launch_block_topk_noalloc(block_max, vis_len, B * n_q, N_cap, k_blocks,
                                                  pool_blocks, stream));
}

csa2_status csa2_reindex_topk(csa2_mode mode, const float* scores, const uint16_t* q_idx,
                              const float* w_idx, const void* k_idx, csa2_kdtype k_dtype,
                              const csa2_paging* paging, const int32_t* pool_blocks,
                              int32_t k_blocks, const int32_t* vis_len, int32_t B, int32_t n_q,
                              int32_t N_cap, int32_t top_k, int32_t* idx_out, float* idx_score,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  if (mode != CSA2_MODE_FULL && mode != CSA2_MODE_REINDEX) return CSA2_ERR_UNSUPPORTED;
  if (!vis_len || !idx_out) return CSA2_ERR_NULL;
  csa2_status st = check_rows(B, n_q);
  if (st != CSA2_OK) return st;
  if (N_cap < 1 || N_cap > kMaxNcap || top_k < 1 || top_k > 512) return CSA2_ERR_SHAPE;
  const int32_t rows = B * n_q;
  const void* ptrs[] = {scores, q_idx, w_idx, k_idx, pool_blocks, vis_len, idx_out, idx_score, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return CSA2_ERR_ALIGN;
  csa2::Pages pg;
  st = check_paging(paging, N_cap, &pg);
  if (st != CSA2_OK) return st;
  if (!pool_blocks) {
    if (!scores) return CSA2_ERR_NULL;
    return from_hip(csa2::launch_flat_topk(scores, vis_len, rows, N_cap, top_k, idx_out,
                                           idx_score, stream));
  }
  if (k_blocks < 1 || k_blocks > 2048) return CSA2_ERR_SHAPE;
  if (rows > kMaxGridY) return CSA2_ERR_SHAPE;
  const bool stored = mode == CSA2_MODE_FULL && scores;
  if (!stored) {
    if (!q_idx || !w_idx || !k_idx) return CSA2_ERR_NULL;
    if (k_dtype != CSA2_KDTYPE_BF16 && k_dtype != CSA2_KDTYPE_FP8_E4M3 &&
        k_dtype != CSA2_KDTYPE_MXFP4 && k_dtype != CSA2_KDTYPE_MXFP4_QK)
      return CSA2_ERR_UNSUPPORTED;
  }
  const size_t need = csa2::pool_topk_workspace_bytes(rows, k_blocks);
  if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  const int kmode = stored ? 0
                          : k_dtype == CSA2_KDTYPE_FP8_E4M3 ? 1
                          : k_dtype == CSA2_KDTYPE_BF16 ? 2
                          : k_dtype == CSA2_KDTYPE_MXFP4 ? 3 : 4;
  return from_hip(csa2::launch_pool_topk(kmode, scores, q_idx, w_idx, k_idx, pg, pool_blocks,
                                         k_blocks,
                                         vis_len, rows, n_q, N_cap, top_k, idx_out, idx_score, ws,
                                         stream));
}

csa2_status csa2_sparse_attn_decode(const uint16_t* q, const uint8_t* kv_fp4,
                                    const uint8_t* kv_scale, int32_t N_cap, const int32_t* idx,
                                    int32_t top_k, const uint8_t* swa_kv, int32_t S_cap,
                                    const int32_t* swa_pos0, const int32_t* q_pos, float sm_scale,
                                    const csa2_attn_opts* opts, int32_t B, int32_t n_q,
                                    uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  return attn_common(q, kv_fp4, kv_scale, N_cap, idx, top_k, swa_kv, S_cap, swa_pos0, q_pos,
                     sm_scale, opts, B, n_q, out, lse, ws, ws_bytes, stream);
}

csa2_status csa2_reuse_attn(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                            int32_t N_cap, const int32_t* idx, int32_t top_k,
                            const uint8_t* swa_kv, int32_t S_cap, const int32_t* swa_pos0,
                            const int32_t* q_pos, float sm_scale, const csa2_attn_opts* opts,
                            int32_t B, int32_t n_q, uint16_t* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  return attn_common(q, kv_fp4, kv_scale, N_cap, idx, top_k, swa_kv, S_cap, swa_pos0, q_pos,
                     sm_scale, opts, B, n_q, out, lse, ws, ws_bytes, stream);
}

csa2_status csa2_kv_append(const uint16_t* kv_new, const uint16_t* swa_new, const int32_t* pos,
                           int32_t B, int32_t n_new, int32_t N_cap, int32_t kv_fmt,
                           const csa2_paging* paging, uint8_t* kv_fp4, uint8_t* kv_scale,
                           uint8_t* swa_kv, int32_t S_cap, const int32_t* swa_pos0,
                           hipStream_t stream) {
  if (!kv_new || !pos || !kv_fp4 || !kv_scale) return CSA2_ERR_NULL;
  if (swa_new && (!swa_kv || !swa_pos0)) return CSA2_ERR_NULL;
  csa2_status st = check_rows(B, n_new);
  if (st != CSA2_OK) return st;
  if (N_cap < 1 || N_cap > kMaxNcap || S_cap < 0) return CSA2_ERR_SHAPE;
  if (kv_fmt != CSA2_KV_MXFP4_E8M0_32 && kv_fmt != CSA2_KV_FP4_E4M3_16) return CSA2_ERR_UNSUPPORTED;
  const void* ptrs[] = {kv_new, swa_new, pos, kv_fp4, kv_scale, swa_kv, swa_pos0};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return CSA2_ERR_ALIGN;
  csa2::Pages pg;
  st = check_paging(paging, N_cap, &pg);
  if (st != CSA2_OK) return st;
  return from_hip(csa2::launch_kv_append(kv_new, swa_new, pos, B, n_new, N_cap, kv_fmt, pg,
                                         kv_fp4, kv_scale,
                                         swa_new ? swa_kv : nullptr, S_cap, swa_pos0, stream));
}

size_t csa2_workspace_size(csa2_op op, int32_t B, int32_t n_q, int32_t N_cap, int32_t top_k,
                           int32_t k_blocks) {
  if (B < 1 || n_q < 1 || N_cap < 1) return static_cast<size_t>(-1);
  const size_t rows = static_cast<size_t>(B) * n_q;
  switch (op) {
    case CSA2_OP_INDEX_SCORE:
      return 0;
    case CSA2_OP_BLOCK_TOPK:
      return csa2::block_topk_workspace_bytes(static_cast<int>(rows), N_cap);
    case CSA2_OP_REINDEX_TOPK:
      if (k_blocks < 0 || k_blocks > 2048) return static_cast<size_t>(-1);
      return csa2::pool_topk_workspace_bytes(static_cast<int>(rows), k_blocks);
    case CSA2_OP_SPARSE_ATTN:
      if (top_k < 0 || top_k > 512) return static_cast<size_t>(-1);
      return csa2::attn_workspace_bytes(static_cast<int>(rows), top_k);
  }
  return static_cast<size_t>(-1);
}

const char* csa2_status_string(csa2_status status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "a required pointer is NULL";
    case CSA2_ERR_SHAPE: return "invalid size or shape";
    case CSA2_ERR_UNSUPPORTED: return "unsupported dtype, format, mode or option";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_ALIGN: return "pointer not 16-byte aligned";
    case CSA2_ERR_HIP: return "HIP runtime or kernel launch error";
    case CSA2_ERR_STATE: return "layer state lacks the pool or indices the mode reuses";
  }
  return "unknown status";
}

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

}  // extern "C"
