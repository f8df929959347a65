/*
 * csa2.h -- C ABI of the CSA2 decode hot path on MI355X (gfx950).
 *
 * CSA2 (Compressed Sparse Attention 2) as described for DeepSeek-V4.1-Flash:
 *   1. the hierarchical sparse indexer scores every visible main-KV entry with
 *      a 32-head x 128-dim indexer query against one shared 128-dim indexer
 *      key per entry, and takes the maximum score of each block of 8
 *      positions;
 *   2. a two-level Top-K keeps at most 2,048 blocks (a pool of at most 16,384
 *      candidate positions) and then the Top-512 positions inside the pool;
 *   3. sparse multi-query attention of 64 query heads of 512 dims over the
 *      512 selected MXFP4 main-KV entries plus the 128-token FP8 sliding
 *      window, with one softmax across both.
 * Sources: "DeepSeek-V4.1-Flash 架构详解：CED、CSA2 与 890 字节 KV Cache"
 * (gentlecold.top) -- §1 configuration table (64 x 512 query heads, 32 x 128
 * indexer, top-k 512, pool <= 2048 blocks x 8, window 128), §3 mode table
 * (Full / Reindex / Reuse), §3.2 Hierarchical Sparse Indexer, §4 MXFP4 main
 * KV dequantised before attention and FP8 SWA KV; the DeepSeek-V4 essay at
 * mlqm.cn (news 871487) §3.2 (indexer), §3.3 (window of the most recent 128
 * uncompressed tokens), §4.3 (a compressed entry is both key and value).
 * The indexer score formula is not printed on those pages; this library
 * computes s_t = sum_h w_h * max(0, qI_h . KI_t).
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers to contiguous, row-major,
 *     batch-major arrays with the shapes given below; the caller owns them.
 *     bf16 values are passed as their uint16 bit patterns.
 *   - Pointers must be 16-byte aligned (256 bytes recommended).
 *   - Every call is asynchronous: it validates its host-side arguments,
 *     enqueues kernels on `stream` and returns.  It never synchronises,
 *     never allocates and never frees device memory.  Calls are ordered only
 *     by their stream.
 *   - On an argument error the call returns a status other than CSA2_OK and
 *     enqueues nothing.  A failed kernel launch returns CSA2_ERR_HIP.  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Device-side index and length arguments are sanitised in the kernels,
 *     never trusted for addressing: vis_len is clamped to [0, N_cap]; an index
 *     outside [0, N_cap) is an empty slot; window positions outside the stored
 *     window slots are skipped.
 *   - Scratch memory comes only from the caller's workspace `ws` of
 *     `ws_bytes` bytes, sized with csa2_workspace_size().  Calls that may run
 *     at the same time must not share a workspace.  Apart from
 *     csa2_block_topk, results never depend on the workspace contents on
 *     entry.  csa2_block_topk needs a workspace that was zero-filled once
 *     when allocated or last used by a csa2_block_topk call (see there).
 *   - Sizes: N_cap <= 4,194,304 entries (4x the pages' maximum context of
 *     1,048,576 tokens), B * n_q <= 65,535 for the decode-shaped calls.
 *   - The library keeps no state; it is thread-safe.
 *   - Query rows: B sequences x n_q query tokens per sequence.  Decode uses
 *     n_q = 1; an encoder prefill chunk uses n_q > 1 with per-query visible
 *     lengths.
 *   - Index lists are reported in ascending order and padded with -1.  Ties
 *     in a selection are broken by the lower index, so results are
 *     deterministic.
 */
#ifndef CSA2_H_
#define CSA2_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 7

/* Symbols of the C ABI; everything else in the library is hidden. */
#define CSA2_API __attribute__((visibility("default")))

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,         /* a required pointer is NULL */
  CSA2_ERR_SHAPE = 2,        /* a size is negative, zero where it must not be, or too large */
  CSA2_ERR_UNSUPPORTED = 3,  /* dtype, format, mode or option this build does not implement */
  CSA2_ERR_WORKSPACE = 4,    /* workspace missing or smaller than csa2_workspace_size() */
  CSA2_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned */
  CSA2_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed */
  CSA2_ERR_STATE = 7         /* csa2_run_layer: the layer state lacks what the mode reuses */
} csa2_status;

/* Storage type of the indexer keys. */
typedef enum {
  CSA2_KDTYPE_BF16 = 0,      /* 128 x bf16 = 256 bytes per entry */
  CSA2_KDTYPE_FP8_E4M3 = 1,  /* 128 x FP8 E4M3FN (OCP) = 128 bytes per entry */
  /* FP4 indexer QK path (DeepSeek-V4 essay, mlqm.cn, §10.2: the Lightning
     Indexer's QK path in FP4): OCP MXFP4, 64 bytes of E2M1 (element 2j in
     the low nibble of byte j) plus 4 E8M0 scales (one per 32 dims) per
     entry.  A buffer of R entries (R = B * N_cap, or num_pages *
     page_entries with paging) holds the R rows of E2M1 first and then the R
     rows of 4 scale bytes: 68 * R bytes.  Decode rows only (n_q < 16);
     prefill-shaped calls return CSA2_ERR_UNSUPPORTED. */
  CSA2_KDTYPE_MXFP4 = 2,
  /* The same essay passage with the query on the FP4 path as well: keys
     stored exactly as for CSA2_KDTYPE_MXFP4, and each query row quantised
     to MXFP4 inside the kernel (OCP MX rules per 32 dims of each head:
     shared exponent floor(log2(amax)) - 2 clamped to [-127, 127], elements
     rounded to the nearest E2M1 value, ties to even, saturating at 6).  The
     QK products run on the gfx950 scaled FP4 matrix instructions; each
     product of two dequantised values is exact, the sums are fp32.  Decode
     rows only, as above. */
  CSA2_KDTYPE_MXFP4_QK = 3
} csa2_kdtype;

/* Storage format of main-KV entries (512 dims each).  Both store E2M1
   elements two per byte (element 2j in the low nibble of byte j), 256 bytes
   per entry, and the block scales in a separate array. */
typedef enum {
  /* OCP MXFP4: one E8M0 scale per 32 elements, 16 bytes per entry; element
     i = E2M1 * 2^(scale[i/32] - 127). */
  CSA2_KV_MXFP4_E8M0_32 = 0,
  /* One FP8 E4M3FN scale per 16 elements and no global scale
     ("DeepSeek-V4.1-Flash 架构详解", §4): 32 bytes of scales per entry,
     288 bytes per entry in all; element i = E2M1 * E4M3FN(scale[i/16]). */
  CSA2_KV_FP4_E4M3_16 = 1
} csa2_kvfmt;

/* CSA2 layer modes ("DeepSeek-V4.1-Flash 架构详解", §3 mode table). */
typedef enum {
  CSA2_MODE_FULL = 0,     /* own indexer Q/K and Top-K; builds the pool */
  CSA2_MODE_REINDEX = 1,  /* own indexer Q; re-scores only the pool against the Full layer's indexer K */
  CSA2_MODE_REUSE = 2,    /* no indexer; reuses the most recent Top-K indices */
  CSA2_MODE_SWA = 3       /* sliding-window attention only (no global KV) */
} csa2_mode;

/* Operation ids for csa2_workspace_size(). */
typedef enum {
  CSA2_OP_INDEX_SCORE = 0,
  CSA2_OP_BLOCK_TOPK = 1,
  CSA2_OP_REINDEX_TOPK = 2,
  CSA2_OP_SPARSE_ATTN = 3
} csa2_op;

/*
 * Paged caches.  The DeepSeek-V4 essay (mlqm.cn, §7.1) keeps the compressed
 * KV and the indexer K of every request in a paged cache (the sliding-window
 * KV stays in a per-request state cache).  A main-KV or indexer-K argument
 * with paging points to a pool of num_pages pages of page_entries
 * consecutive entries each (pool arrays [num_pages * page_entries, ...]).
 * Entry e of sequence b lives in pool row
 *   block_table[b * max_pages + e / page_entries] * page_entries + e % page_entries
 * and the sequence's logical capacity is N_cap = max_pages * page_entries
 * (a call's N_cap must equal it).  Rows never straddle pages, so every
 * kernel reads whole tiles from one page.
 *   block_table  [B, max_pages] int32 device memory: physical page of each
 *                logical page, or -1 (unmapped)
 *   page_entries a power of two, 64 .. 65536
 *   max_pages    >= 1
 *   num_pages    >= 1, num_pages * page_entries <= 2^31 - 1
 * Every page holding an entry that a call reads (a visible position of the
 * scan or pool re-scoring) must be mapped: an id outside [0, num_pages) is
 * clamped into it for addressing (nothing is read out of bounds) and the
 * results that depend on it are unspecified.  Attention treats a selected
 * id on an unmapped page as an empty slot; the KV append skips entries whose
 * page is unmapped.  NULL paging = contiguous [B, N_cap, ...] arrays.
 */
typedef struct {
  const int32_t* block_table;
  int32_t page_entries;
  int32_t max_pages;
  int32_t num_pages;
} csa2_paging;

/* Bits of csa2_attn_opts.flags. */
#define CSA2_ATTN_SINK 1u   /* opts->sink is read (per-head sink logits) */
#define CSA2_ATTN_PAGED 2u  /* opts->paging is read: kv_fp4 / kv_scale are page pools */

/* Options of the attention entry points; NULL means the defaults.  The
   first four fields have the layout of ABI 1, whose last field (then
   `reserved`, always 0) is now `flags`: an ABI-1 caller's struct, which
   ends there, is read correctly because `sink` is read only when
   flags & CSA2_ATTN_SINK. */
typedef struct {
  int32_t window;        /* SWA window in tokens, 0..128; default 128 */
  int32_t replay_start;  /* first token a replayed window may see (window
                            [max(s, i-W+1), i]); -1 = no truncation (default) */
  int32_t kv_fmt;        /* csa2_kvfmt of kv_fp4 / kv_scale; default CSA2_KV_MXFP4_E8M0_32;
                            another value gives CSA2_ERR_UNSUPPORTED */
  uint32_t flags;        /* CSA2_ATTN_* bits; other bits must be 0 */
  const float* sink;     /* with CSA2_ATTN_SINK: [64] fp32 per-head sink logits (device
                            memory), see csa2_sparse_attn_decode; otherwise not read */
  const csa2_paging* paging;  /* with CSA2_ATTN_PAGED: the main-KV page table (host
                                 memory, read during the call); otherwise not read */
} csa2_attn_opts;

/*
 * csa2_index_score -- indexer scan (score every visible entry) with the block
 * maximum over 8 positions fused in.
 *   Computes, for query row r = b * n_q + j and every visible entry
 *   t < vis_len[r]:
 *     s[r][t] = sum_{h<32} w_idx[r][h] * max(0, sum_{d<128} q_idx[r][h][d] * k_idx[b][t][d])
 *     block_max[r][i] = max_{t in [8i, min(8i+8, vis_len[r]))} s[r][t]
 *   ("DeepSeek-V4.1-Flash 架构详解", §3.2: the Full layer scans every visible
 *   entry and aggregates scores per block of 8 positions.)  Products are exact
 *   in fp32 and accumulated in fp32.
 * Arguments
 *   q_idx     [B, n_q, 32, 128] bf16 indexer queries
 *   w_idx     [B, n_q, 32] fp32 per-head weights
 *   k_idx     [B, N_cap, 128] indexer keys of dtype k_dtype, or a page pool
 *   paging    NULL, or the page table of k_idx (see csa2_paging)
 *   vis_len   [B, n_q] int32 visible entries per query row
 *   scores    [B, n_q, N_cap] fp32 output or NULL; entries t >= vis_len are not written
 *   block_max [B, n_q, ceil(N_cap/8)] fp32 output or NULL; blocks past the
 *             visible ones are not written.  At least one output must be given.
 *   ws        unused (may be NULL; csa2_workspace_size returns 0)
 */
CSA2_API csa2_status csa2_index_score(const uint16_t* q_idx, const float* w_idx, const void* k_idx,
                             csa2_kdtype k_dtype, const csa2_paging* paging,
                             const int32_t* vis_len, int32_t B, int32_t n_q,
                             int32_t N_cap, float* scores, float* block_max, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * csa2_index_score_bf16 -- the scan of csa2_index_score with the scores kept
 *   in BF16: each score s[r][t] (computed exactly as above, fp32) is stored
 *   rounded to the nearest bf16 value (ties to the even pattern).  The
 *   BF16-score variant of the indexer (DeepSeek-V4 essay, mlqm.cn, §10.2:
 *   FP32 index scores replaced by BF16 make the Top-k selector about twice as
 *   fast at a KV-entry recall of 99.7%): half the score bytes written and
 *   read.  Opt-in: a Top-k over bf16 scores is measured by its recall against
 *   the fp32 selection, not by parity (bf16 rounding merges close scores
 *   into ties, which the selection then breaks by position).
 * Arguments as csa2_index_score, except
 *   scores    [B, n_q, N_cap] uint16 (bf16 bit patterns) output, required;
 *             entries t >= vis_len are not written.  No block maxima.
 * Errors as csa2_index_score (CSA2_ERR_NULL for a missing scores).
 */
CSA2_API csa2_status csa2_index_score_bf16(const uint16_t* q_idx, const float* w_idx,
                                           const void* k_idx, csa2_kdtype k_dtype,
                                           const csa2_paging* paging, const int32_t* vis_len,
                                           int32_t B, int32_t n_q, int32_t N_cap,
                                           uint16_t* scores, hipStream_t stream);

/*
 * csa2_flat_topk_bf16 -- the flat Top-k of csa2_reindex_topk (no pool: every
 *   visible entry of a query row is a candidate; the encoder prefill path,
 *   "DeepSeek-V4.1-Flash 架构详解", §3.1/§3.2) over bf16 scores: the first
 *   min(top_k, vis_len[r]) entries in (score descending, position
 *   ascending) order, compared as the bf16 values, reported in ascending
 *   position order and padded with -1.  (DeepSeek-V4 essay §10.2; see
 *   csa2_index_score_bf16.)
 * Arguments
 *   scores    [B, n_q, N_cap] uint16 bf16 bit patterns (device memory), as
 *             written by csa2_index_score_bf16; entries >= vis_len not read
 *   vis_len   [B, n_q] int32
 *   top_k     1 .. 512
 *   idx_out   [B, n_q, top_k] int32 output
 *   idx_score [B, n_q, top_k] fp32 output of the selected scores (the bf16
 *             values; -inf for padding) or NULL
 * Errors: CSA2_ERR_NULL (scores, vis_len or idx_out missing), CSA2_ERR_SHAPE
 *   (sizes out of range), CSA2_ERR_ALIGN (a pointer not 16-byte aligned),
 *   CSA2_ERR_HIP (launch failure).
 */
CSA2_API csa2_status csa2_flat_topk_bf16(const uint16_t* scores, const int32_t* vis_len,
                                         int32_t B, int32_t n_q, int32_t N_cap, int32_t top_k,
                                         int32_t* idx_out, float* idx_score, hipStream_t stream);

/*
 * csa2_block_topk -- first level of the Top-K: the pool of blocks.
 *   Orders the nb = ceil(vis_len/8) visible blocks of each query row by
 *   (block_max descending, block id ascending) and keeps the first
 *   min(k_blocks, nb) ("DeepSeek-V4.1-Flash 架构详解", §3.2: at most 2,048
 *   blocks of 8 positions, at most 16,384 candidates).
 * Arguments
 *   block_max   [B, n_q, ceil(N_cap/8)] fp32 (as written by csa2_index_score)
 *   vis_len     [B, n_q] int32
 *   k_blocks    1..2048
 *   pool_blocks [B, n_q, k_blocks] int32 output: ascending block ids, -1 padded
 *   ws          csa2_workspace_size(CSA2_OP_BLOCK_TOPK, ...) bytes (required).
 *               Its first 2 * B * n_q * 4096 words are histograms that must
 *               start at zero; every call leaves them zeroed, so a workspace
 *               zero-filled once (hipMemset) when allocated, or last used by
 *               csa2_block_topk, is always ready.  Other contents are caught
 *               by the histograms' totals (they must equal the visible block
 *               count and the candidate count of the row): such a row is
 *               still selected exactly, by a slower pass over every visible
 *               block.  Stale bins whose totals happen to match are not
 *               caught and give an unspecified pool.
 */
CSA2_API csa2_status csa2_block_topk(const float* block_max, const int32_t* vis_len, int32_t B,
                            int32_t n_q, int32_t N_cap, int32_t k_blocks, int32_t* pool_blocks,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_block_topk_noalloc -- csa2_block_topk with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *   Same arguments (minus ws / ws_bytes), result and errors as
 *   csa2_block_topk.  Scratch memory is a fixed 16 MiB device array inside
 *   the library (one per GPU, held until the process ends; its address is
 *   resolved on the first call on each device).  The call allocates
 *   nothing.  Limits: B * n_q <= 64 and B * n_q * ceil(N_cap / 8) * 12 <=
 *   16 MiB - 2,162,688 bytes (e.g. 8 rows at N_cap = 1,048,576 or 64 rows at
 *   131,072); larger calls return CSA2_ERR_WORKSPACE and enqueue nothing.
 *   Every call on a GPU shares that GPU's array: calls that may overlap on
 *   one GPU (other streams, other threads) race and must be serialised by
 *   the caller.  The array's histograms are zero when the library is loaded
 *   and every call leaves them zeroed.
 */
CSA2_API csa2_status csa2_block_topk_noalloc(const float* block_max, const int32_t* vis_len,
                                             int32_t B, int32_t n_q, int32_t N_cap,
                                             int32_t k_blocks, int32_t* pool_blocks,
                                             hipStream_t stream);

/*
 * csa2_reindex_topk -- second level of the Top-K.
 *   With a pool (pool_blocks != NULL) the candidates are the visible
 *   positions of the pool's blocks:
 *     CSA2_MODE_FULL    keys are scores[r][t] when scores != NULL; with
 *                       scores == NULL the pool positions are re-scored with
 *                       q_idx / w_idx (the Full layer's own query) on k_idx.
 *                       By construction this equals the Top-k over all
 *                       visible positions when k_blocks * 8 >= top_k.
 *     CSA2_MODE_REINDEX keys are the pool positions re-scored with this
 *                       layer's q_idx / w_idx against the Full layer's k_idx
 *                       ("DeepSeek-V4.1-Flash 架构详解", §3.2: a Reindex
 *                       layer re-scores only the pool).
 *   Without a pool (pool_blocks == NULL, FULL or REINDEX) the candidates are
 *   all positions [0, vis_len) keyed by scores (flat Top-k of an encoder
 *   prefill chunk; scores required).
 *   The first min(top_k, #candidates) candidates in (key descending,
 *   position ascending) order are kept.  CSA2_MODE_REUSE runs no indexer and
 *   returns CSA2_ERR_UNSUPPORTED.
 * Arguments
 *   scores      [B, n_q, N_cap] fp32 or NULL (see above)
 *   q_idx, w_idx, k_idx, k_dtype, paging  as for csa2_index_score (may be
 *               NULL when the keys come from scores)
 *   pool_blocks [B, n_q, k_blocks] int32 ascending block ids, -1 padded, or NULL
 *   vis_len     [B, n_q] int32
 *   top_k       1..512
 *   idx_out     [B, n_q, top_k] int32 output: ascending positions, -1 padded
 *   idx_score   [B, n_q, top_k] fp32 output of the selected keys (-inf for
 *               padding) or NULL
 *   ws          csa2_workspace_size(CSA2_OP_REINDEX_TOPK, ...) bytes, required
 *               with a pool (unused without one)
 */
CSA2_API csa2_status csa2_reindex_topk(csa2_mode mode, const float* scores, const uint16_t* q_idx,
                              const float* w_idx, const void* k_idx, csa2_kdtype k_dtype,
                              const csa2_paging* paging, const int32_t* pool_blocks,
                              int32_t k_blocks,
                              const int32_t* vis_len, int32_t B, int32_t n_q, int32_t N_cap,
                              int32_t top_k, int32_t* idx_out, float* idx_score, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn_decode -- sparse multi-query attention of a Full or
 * Reindex layer.
 *   For query row r = b * n_q + j and head h < 64, the entry set is
 *     E = { main entry idx[r][i] : 0 <= idx[r][i] < N_cap }
 *         + { window token p : max(q_pos[r]-W+1, swa_pos0[b], replay_start, 0) <= p <= q_pos[r],
 *                               p - swa_pos0[b] < S_cap }
 *   (no de-duplication between the two parts).  Each entry v is used as key
 *   and value.  Main entries are E2M1 with block scales, v[i] = E2M1(nibble i)
 *   * 2^(kv_scale[i/32] - 127) (CSA2_KV_MXFP4_E8M0_32, the default) or
 *   E2M1(nibble i) * E4M3FN(kv_scale[i/16]) (CSA2_KV_FP4_E4M3_16, opts->kv_fmt);
 *   window entries are FP8 E4M3FN, slot p - swa_pos0[b] of swa_kv.  Then
 *     l_e = sm_scale * q[r][h] . v_e,  out[r][h] = sum_e softmax(l)_e v_e,
 *     lse[r][h] = log sum_e exp(l_e)   (natural log; -inf for an empty set,
 *                                       whose output is 0)
 *   With CSA2_ATTN_SINK, head h also has a sink logit s_h: the normaliser gains
 *   exp(s_h) and no value, i.e. out = sum_e exp(l_e) v_e / (sum_e exp(l_e) +
 *   exp(s_h)) and lse = log(sum_e exp(l_e) + exp(s_h)); s_h = -inf is no
 *   sink (DeepSeek-V4 essay (mlqm.cn) §4.3: a learnable attention sink on
 *   which each head may put part of its probability mass).
 *   ("DeepSeek-V4.1-Flash 架构详解", §1 (64 x 512 heads, window 128), §4
 *   (dequantised before attention), §9 step 5 (selected global KV plus this
 *   layer's SWA KV); V4 essay §4.3 (an entry is both key and value).)
 *   Dequantisation is exact in bf16; q.k and p.v run on bf16 matrix cores
 *   with fp32 accumulation and an fp32 online softmax; out is rounded to bf16.
 * Arguments
 *   q         [B, n_q, 64, 512] bf16
 *   kv_fp4    [B, N_cap, 256] uint8 packed E2M1 (or a page pool, opts->paging)
 *   kv_scale  [B, N_cap, 16] uint8 E8M0, or [B, N_cap, 32] uint8 E4M3FN (same
 *             paging as kv_fp4)
 *   idx       [B, n_q, top_k] int32 entry indices, -1 = empty slot; top_k 0..512
 *   swa_kv    [B, S_cap, 512] uint8 FP8 E4M3FN; slot i holds token swa_pos0[b] + i
 *   swa_pos0  [B] int32
 *   q_pos     [B, n_q] int32 token position of each query
 *   sm_scale  softmax scale, finite and > 0 (else CSA2_ERR_SHAPE)
 *   opts      NULL or options (window, replay_start, kv_fmt, sink, paging)
 *   out       [B, n_q, 64, 512] bf16 output
 *   lse       [B, n_q, 64] fp32 output or NULL
 *   ws        csa2_workspace_size(CSA2_OP_SPARSE_ATTN, ...) bytes
 */
CSA2_API csa2_status csa2_sparse_attn_decode(const uint16_t* q, const uint8_t* kv_fp4,
                                    const uint8_t* kv_scale, int32_t N_cap, const int32_t* idx,
                                    int32_t top_k, const uint8_t* swa_kv, int32_t S_cap,
                                    const int32_t* swa_pos0, const int32_t* q_pos, float sm_scale,
                                    const csa2_attn_opts* opts, int32_t B, int32_t n_q,
                                    uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/*
 * csa2_reuse_attn -- attention of a Reuse layer: the same computation and
 * arguments as csa2_sparse_attn_decode, with idx taken from the most recent
 * Full or Reindex layer and this layer's own q and swa_kv; no indexer runs
 * ("DeepSeek-V4.1-Flash 架构详解", §3 mode table and §3.2).
 */
CSA2_API csa2_status csa2_reuse_attn(const uint16_t* q, const uint8_t* kv_fp4, const uint8_t* kv_scale,
                            int32_t N_cap, const int32_t* idx, int32_t top_k,
                            const uint8_t* swa_kv, int32_t S_cap, const int32_t* swa_pos0,
                            const int32_t* q_pos, float sm_scale, const csa2_attn_opts* opts,
                            int32_t B, int32_t n_q, uint16_t* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * csa2_kv_append -- encode and store the KV entries of new tokens.
 *   For sequence b and new token i < n_new at position p = pos[b] + i:
 *     main KV    if 0 <= p < N_cap:  kv_fp4[b][p], kv_scale[b][p] <- kv_new[b][i]
 *                encoded in format kv_fmt
 *     window KV  if swa_new != NULL and 0 <= p - swa_pos0[b] < S_cap:
 *                swa_kv[b][p - swa_pos0[b]] <- FP8 E4M3FN of swa_new[b][i]
 *   Positions outside a cache are skipped.  ("DeepSeek-V4.1-Flash 架构详解",
 *   §4: main KV is stored as MXFP4, SWA KV as FP8.)  Encoding (OCP MX v1.0,
 *   OCP FP8):
 *     MXFP4 (CSA2_KV_MXFP4_E8M0_32): per 32 elements X = floor(log2(max |v|))
 *       - 2 clamped to [-127, 127] (-127 for an all-zero block), E8M0 code
 *       X + 127; each v / 2^X rounds to the nearest E2M1 value, ties to the
 *       even code, saturating at 6; a value that rounds to zero is stored
 *       as +0.
 *     CSA2_KV_FP4_E4M3_16: per 16 elements the scale s is max |v| / 6
 *       rounded to FP8 E4M3FN (rule below); each |v| / s rounds to the
 *       nearest E2M1 value, ties to the even code, saturating at 6, sign
 *       kept, zero stored as +0; a block with s = 0 stores +0 everywhere.
 *     FP8: saturate to +-448, round to nearest, ties to even; the sign is
 *       kept for values that round to zero.
 *   Inputs must be finite (a non-finite value leaves its block's or
 *   element's codes unspecified).  The caches' layouts are those the
 *   attention entry points read.
 * Arguments
 *   kv_new    [B, n_new, 512] bf16 main-KV entries
 *   swa_new   [B, n_new, 512] bf16 window entries, or NULL (no window writes)
 *   pos       [B] int32 position of each sequence's first new token
 *   kv_fmt    csa2_kvfmt of the main cache (else CSA2_ERR_UNSUPPORTED)
 *   paging    NULL, or the page table of kv_fp4 / kv_scale (see csa2_paging);
 *             the window cache is never paged
 *   kv_fp4    [B, N_cap, 256] uint8, kv_scale [B, N_cap, 16] (E8M0) or
 *             [B, N_cap, 32] (E4M3FN) uint8 (written)
 *   swa_kv    [B, S_cap, 512] uint8 (written; may be NULL when swa_new is)
 *   swa_pos0  [B] int32 (may be NULL when swa_new is)
 */
CSA2_API csa2_status csa2_kv_append(const uint16_t* kv_new, const uint16_t* swa_new,
                           const int32_t* pos, int32_t B, int32_t n_new, int32_t N_cap,
                           int32_t kv_fmt, const csa2_paging* paging, uint8_t* kv_fp4,
                           uint8_t* kv_scale,
                           uint8_t* swa_kv, int32_t S_cap, const int32_t* swa_pos0,
                           hipStream_t stream);

/*
 * Layer driver.  The model's 40 layers follow one static schedule
 * ("DeepSeek-V4.1-Flash 架构详解", §3.1 and §1): layers 0 and 1 are pure
 * sliding-window attention; the 18 other encoder layers (2..19, m = 2) form
 * three groups of six, a Full layer then five Reuse layers; the 20 decoder
 * layers (20..39, m = 1) form five groups of four, the first a Full layer
 * and the others a Reindex layer, each followed by three Reuse layers.  A
 * Reuse layer reuses the most recent Top-K indices, a Reindex layer the most
 * recent pool, and every layer computes its own query and SWA KV (§3 mode
 * table).  csa2_layer_mode gives a layer's mode; csa2_run_layer enqueues one
 * layer's CSA2 work and carries the pool and the indices from layer to layer
 * in a caller-owned state.
 */

/* Mode of layer `layer` (0..39) of the schedule; -1 for another index. */
CSA2_API int32_t csa2_layer_mode(int32_t layer);

/* Inputs of one layer: the shared caches (the indexer K and main KV, which
   the Full layer's projections wrote) and this layer's own query and window. */
typedef struct {
  const void* k_idx;             /* indexer K, as for csa2_index_score */
  csa2_kdtype k_dtype;
  const csa2_paging* k_paging;   /* NULL: contiguous */
  const uint8_t* kv_fp4;         /* main KV, as for csa2_sparse_attn_decode */
  const uint8_t* kv_scale;
  int32_t kv_fmt;                /* csa2_kvfmt */
  const csa2_paging* kv_paging;  /* NULL: contiguous */
  int32_t N_cap;
  const int32_t* vis_len;        /* [B, n_q] visible entries per query row */
  const uint16_t* q_idx;         /* [B, n_q, 32, 128] bf16: Full and Reindex layers */
  const float* w_idx;            /* [B, n_q, 32] fp32: Full and Reindex layers */
  const uint16_t* q;             /* [B, n_q, 64, 512] bf16 */
  const uint8_t* swa_kv;         /* [B, S_cap, 512] FP8, this layer's window */
  int32_t S_cap;
  const int32_t* swa_pos0;       /* [B] */
  const int32_t* q_pos;          /* [B, n_q] */
  float sm_scale;
  int32_t window;                /* 0..128 */
  int32_t replay_start;          /* -1: none */
  const float* sink;             /* [64] per-head sink logits, or NULL */
  int32_t B, n_q;
} csa2_layer_args;

/* State carried across layers: device buffers owned by the caller, sized
   for the largest layer.  The driver sets has_pool / has_idx (host fields)
   when it enqueues the work that fills them; a caller starts with both 0. */
typedef struct {
  float* block_max;      /* [B, n_q, ceil(N_cap/8)] (decode rows: n_q < 16) */
  float* scores;         /* [B, n_q, N_cap] (prefill-shaped rows: n_q >= 16) or NULL */
  int32_t* pool_blocks;  /* [B, n_q, k_blocks] */
  int32_t k_blocks;      /* 1..2048 (2048 in the model) */
  int32_t* idx;          /* [B, n_q, top_k] */
  int32_t top_k;         /* 1..512 (512 in the model) */
  void* ws;              /* csa2_layer_workspace_size(...) bytes, zero-filled once */
  size_t ws_bytes;
  int32_t has_pool;
  int32_t has_idx;
} csa2_layer_state;

/*
 * csa2_run_layer -- one layer's CSA2 work, by mode:
 *   CSA2_MODE_FULL     decode rows (n_q < 16): scan with block maxima,
 *                      block Top-K (pool), Top-k re-scored in the pool;
 *                      prefill-shaped rows (n_q >= 16): scan with scores,
 *                      flat Top-k (no pool; state->scores required); then
 *                      attention.  Sets has_idx (and has_pool for decode rows).
 *   CSA2_MODE_REINDEX  re-scores the state's pool with this layer's q_idx /
 *                      w_idx, Top-k, attention (needs has_pool).
 *   CSA2_MODE_REUSE    attention over the state's indices (needs has_idx).
 *   CSA2_MODE_SWA      attention over the window only.
 * Returns CSA2_ERR_STATE when the state lacks what the mode reuses; other
 * errors as for the calls it makes (nothing of a failed call is enqueued,
 * but earlier calls of the same layer may have been).
 *   out, lse   as for csa2_sparse_attn_decode
 */
CSA2_API csa2_status csa2_run_layer(csa2_mode mode, const csa2_layer_args* args,
                                    csa2_layer_state* state, uint16_t* out, float* lse,
                                    hipStream_t stream);

/* Workspace bytes of csa2_run_layer for the given sizes (the largest of the
   calls it makes); (size_t)-1 for invalid sizes. */
CSA2_API size_t csa2_layer_workspace_size(int32_t B, int32_t n_q, int32_t N_cap, int32_t k_blocks,
                                          int32_t top_k);

/* Workspace bytes an operation needs for the given sizes (0 if none);
   returns (size_t)-1 for an unknown op or invalid sizes. */
CSA2_API size_t csa2_workspace_size(csa2_op op, int32_t B, int32_t n_q, int32_t N_cap, int32_t top_k,
                           int32_t k_blocks);

/* Static description of a status code. */
CSA2_API const char* csa2_status_string(csa2_status status);

/* CSA2_ABI_VERSION of the built library. */
CSA2_API int32_t csa2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H_ */
