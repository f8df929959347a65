// Layer driver: the static layer schedule of the model and one layer's CSA2
// work by mode, with the pool and the Top-K indices carried from layer to
// layer in a caller-owned state.  Host code only; it enqueues the library's
// own entry points, so their validation and kernels are the ones used.
//
// "DeepSeek-V4.1-Flash 架构详解", §1: 40 layers, a 20-layer causal encoder
// and a 20-layer decoder; only the encoder's first two layers are pure
// sliding-window attention; the encoder's 18 other layers form three groups
// of six (Full, then five Reuse), the decoder's 20 five groups of four (the
// first Full + three Reuse, the others Reindex + three Reuse).  §3 mode
// table: a Reuse layer reuses the most recent Top-K, a Reindex layer
// re-scores the most recent pool, and every layer has its own query and SWA
// KV.
#include "../../include/csa2.h"
#include "csa2_launch.h"

#include <stdint.h>

namespace {

constexpr int32_t kLayers = 40;
constexpr int32_t kEncoderLayers = 20;
constexpr int32_t kSwaLayers = 2;
constexpr int32_t kEncoderGroup = 6;
constexpr int32_t kDecoderGroup = 4;

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// The workspace holds the block Top-K's and the pool Top-K's, one after the
// other (both used by a Full layer).
struct WsSplit {
  size_t bt, pool;
};

bool ws_split(int32_t B, int32_t n_q, int32_t N_cap, int32_t k_blocks, int32_t top_k,
              WsSplit* w) {
  const size_t bt = csa2_workspace_size(CSA2_OP_BLOCK_TOPK, B, n_q, N_cap, top_k, k_blocks);
  const size_t pool = csa2_workspace_size(CSA2_OP_REINDEX_TOPK, B, n_q, N_cap, top_k, k_blocks);
  if (bt == static_cast<size_t>(-1) || pool == static_cast<size_t>(-1)) return false;
  w->bt = align256(bt);
  w->pool = pool;
  return true;
}

csa2_status attend(const csa2_layer_args* a, const int32_t* idx, int32_t top_k, uint16_t* out,
                   float* lse, hipStream_t stream) {
  csa2_attn_opts o{};
  o.window = a->window;
  o.replay_start = a->replay_start;
  o.kv_fmt = a->kv_fmt;
  o.flags = (a->sink ? CSA2_ATTN_SINK : 0u) | (a->kv_paging ? CSA2_ATTN_PAGED : 0u);
  o.sink = a->sink;
  o.paging = a->kv_paging;
  return csa2_sparse_attn_decode(a->q, a->kv_fp4, a->kv_scale, a->N_cap, idx, top_k, a->swa_kv,
                                 a->S_cap, a->swa_pos0, a->q_pos, a->sm_scale, &o, a->B, a->n_q,
                                 out, lse, nullptr, 0, stream);
}

}  // namespace

extern "C" {

int32_t csa2_layer_mode(int32_t layer) {
  if (layer < 0 || layer >= kLayers) return -1;
  if (layer < kSwaLayers) return CSA2_MODE_SWA;
  if (layer < kEncoderLayers)
    return (layer - kSwaLayers) % kEncoderGroup == 0 ? CSA2_MODE_FULL : CSA2_MODE_REUSE;
  const int32_t d = layer - kEncoderLayers;
  if (d % kDecoderGroup != 0) return CSA2_MODE_REUSE;
  return d == 0 ? CSA2_MODE_FULL : CSA2_MODE_REINDEX;
}

size_t csa2_layer_workspace_size(int32_t B, int32_t n_q, int32_t N_cap, int32_t k_blocks,
                                 int32_t top_k) {
  WsSplit w;
  if (!ws_split(B, n_q, N_cap, k_blocks, top_k, &w)) return static_cast<size_t>(-1);
  return w.bt + w.pool;
}

csa2_status csa2_run_layer(csa2_mode mode, const csa2_layer_args* a, csa2_layer_state* st,
                           uint16_t* out, float* lse, hipStream_t stream) {
  if (!a || !st) return CSA2_ERR_NULL;
  if (mode == CSA2_MODE_SWA) return attend(a, nullptr, 0, out, lse, stream);
  if (mode != CSA2_MODE_FULL && mode != CSA2_MODE_REINDEX && mode != CSA2_MODE_REUSE)
    return CSA2_ERR_UNSUPPORTED;
  if (!st->idx) return CSA2_ERR_NULL;
  if (st->top_k < 1 || st->top_k > 512) return CSA2_ERR_SHAPE;
  if (mode == CSA2_MODE_REUSE) {
    if (!st->has_idx) return CSA2_ERR_STATE;
    return attend(a, st->idx, st->top_k, out, lse, stream);
  }
  const bool prefill = a->n_q >= 16;
  if (mode == CSA2_MODE_REINDEX && (!st->has_pool || prefill)) return CSA2_ERR_STATE;
  WsSplit w{0, 0};
  if (!prefill && !ws_split(a->B, a->n_q, a->N_cap, st->k_blocks, st->top_k, &w))
    return CSA2_ERR_SHAPE;
  if (!prefill && (!st->ws || st->ws_bytes < w.bt + w.pool)) return CSA2_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(st->ws);
  csa2_status s;
  if (mode == CSA2_MODE_FULL) {
    if (prefill) {
      // Prefill-shaped rows: scores of every visible entry, flat Top-k.
      if (!st->scores) return CSA2_ERR_NULL;
      s = csa2_index_score(a->q_idx, a->w_idx, a->k_idx, a->k_dtype, a->k_paging, a->vis_len, a->B,
                           a->n_q, a->N_cap, st->scores, nullptr, nullptr, 0, stream);
      if (s != CSA2_OK) return s;
      s = csa2_reindex_topk(CSA2_MODE_FULL, st->scores, nullptr, nullptr, nullptr, a->k_dtype,
                            nullptr, nullptr, 0, a->vis_len, a->B, a->n_q, a->N_cap, st->top_k,
                            st->idx, nullptr, nullptr, 0, stream);
      if (s != CSA2_OK) return s;
      st->has_pool = 0;
    } else {
      if (!st->block_max || !st->pool_blocks) return CSA2_ERR_NULL;
      s = csa2_index_score(a->q_idx, a->w_idx, a->k_idx, a->k_dtype, a->k_paging, a->vis_len, a->B,
                           a->n_q, a->N_cap, nullptr, st->block_max, nullptr, 0, stream);
      if (s != CSA2_OK) return s;
      s = csa2_block_topk(st->block_max, a->vis_len, a->B, a->n_q, a->N_cap, st->k_blocks,
                          st->pool_blocks, ws, w.bt, stream);
      if (s != CSA2_OK) return s;
      st->has_pool = 1;
      s = csa2_reindex_topk(CSA2_MODE_FULL, nullptr, a->q_idx, a->w_idx, a->k_idx, a->k_dtype,
                            a->k_paging, st->pool_blocks, st->k_blocks, a->vis_len, a->B, a->n_q,
                            a->N_cap, st->top_k, st->idx, nullptr, ws + w.bt, w.pool, stream);
      if (s != CSA2_OK) return s;
    }
  } else {   // CSA2_MODE_REINDEX (the state holds a pool: checked above)
    s = csa2_reindex_topk(CSA2_MODE_REINDEX, nullptr, a->q_idx, a->w_idx, a->k_idx, a->k_dtype,
                          a->k_paging, st->pool_blocks, st->k_blocks, a->vis_len, a->B, a->n_q,
                          a->N_cap, st->top_k, st->idx, nullptr, ws + w.bt, w.pool, stream);
    if (s != CSA2_OK) return s;
  }
  st->has_idx = 1;
  return attend(a, st->idx, st->top_k, out, lse, stream);
}

}  // extern "C"
