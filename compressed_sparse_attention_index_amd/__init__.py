"""Python binding of libcsa2.so, the CSA2 decode hot path for MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/csa2.h.  Tensors are torch tensors on
the GPU (torch supplies device memory and the current stream); bf16 arrays
are passed as int16/uint16/bfloat16 tensors of their bit patterns.  If the
library is not built this module raises instead of computing anything.
"""
import ctypes
import os

import torch

__all__ = [
    "KDTYPE_BF16", "KDTYPE_FP8", "KDTYPE_MXFP4", "KDTYPE_MXFP4_QK", "Mxfp4Keys", "KV_MXFP4_E8M0_32", "KV_FP4_E4M3_16", "MODE_FULL", "MODE_REINDEX", "MODE_REUSE",
    "OP_INDEX_SCORE", "OP_BLOCK_TOPK", "OP_REINDEX_TOPK", "OP_SPARSE_ATTN",
    "Csa2Error", "Paging", "lib", "abi_version", "workspace_size", "index_score", "block_topk",
    "block_topk_noalloc",
    "reindex_topk", "sparse_attn_decode", "reuse_attn", "kv_append",
    "MODE_SWA", "layer_mode", "LayerState", "run_layer",
]

KDTYPE_BF16, KDTYPE_FP8, KDTYPE_MXFP4, KDTYPE_MXFP4_QK = 0, 1, 2, 3
KV_MXFP4_E8M0_32, KV_FP4_E4M3_16 = 0, 1   # main-KV scale formats (csa2_kvfmt)
MODE_FULL, MODE_REINDEX, MODE_REUSE, MODE_SWA = 0, 1, 2, 3
OP_INDEX_SCORE, OP_BLOCK_TOPK, OP_REINDEX_TOPK, OP_SPARSE_ATTN = 0, 1, 2, 3

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_F = ctypes.c_float

_SIGNATURES = {
    "csa2_index_score": [_P, _P, _P, _I, _P, _P, _I, _I, _I, _P, _P, _P, _S, _P],
    "csa2_index_score_bf16": [_P, _P, _P, _I, _P, _P, _I, _I, _I, _P, _P],
    "csa2_flat_topk_bf16": [_P, _P, _I, _I, _I, _I, _P, _P, _P],
    "csa2_block_topk": [_P, _P, _I, _I, _I, _I, _P, _P, _S, _P],
    "csa2_block_topk_noalloc": [_P, _P, _I, _I, _I, _I, _P, _P],
    "csa2_reindex_topk": [_I, _P, _P, _P, _P, _I, _P, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _S,
                          _P],
    "csa2_sparse_attn_decode": [_P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _F, _P, _I, _I, _P, _P,
                                _P, _S, _P],
    "csa2_reuse_attn": [_P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _F, _P, _I, _I, _P, _P, _P, _S, _P],
    "csa2_kv_append": [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P],
    "csa2_workspace_size": [_I, _I, _I, _I, _I, _I],
    "csa2_layer_mode": [_I],
    "csa2_layer_workspace_size": [_I, _I, _I, _I, _I],
    "csa2_run_layer": [_I, _P, _P, _P, _P, _P],
    "csa2_status_string": [_I],
    "csa2_abi_version": [],
}
_RESTYPES = {"csa2_workspace_size": _S, "csa2_status_string": ctypes.c_char_p,
             "csa2_abi_version": _I, "csa2_layer_workspace_size": _S}


ATTN_SINK = 1    # csa2_attn_opts.flags bit: the sink pointer is read
ATTN_PAGED = 2   # csa2_attn_opts.flags bit: the paging pointer is read


class PagingStruct(ctypes.Structure):
    """csa2_paging."""
    _fields_ = [("block_table", ctypes.c_void_p), ("page_entries", _I), ("max_pages", _I),
                ("num_pages", _I)]


class AttnOpts(ctypes.Structure):
    _fields_ = [("window", _I), ("replay_start", _I), ("kv_fmt", _I), ("flags", ctypes.c_uint32),
                ("sink", ctypes.c_void_p), ("paging", ctypes.POINTER(PagingStruct))]


class Paging:
    """A page table (include/csa2.h, csa2_paging): block_table [B, max_pages]
    int32 on the GPU, page_entries entries per page, num_pages pages in the
    pool.  The logical capacity per sequence is max_pages * page_entries."""

    def __init__(self, block_table, page_entries, num_pages):
        self.block_table = block_table
        self.page_entries = int(page_entries)
        self.num_pages = int(num_pages)
        self.max_pages = int(block_table.shape[1])
        self.n_cap = self.max_pages * self.page_entries
        self.struct = PagingStruct(_ptr(block_table, (torch.int32,), "block_table"),
                                   self.page_entries, self.max_pages, self.num_pages)

    def ref(self):
        return ctypes.byref(self.struct)


def _paging(paging):
    return paging.ref() if paging is not None else None


class Mxfp4Keys:
    """Indexer keys in MXFP4 (CSA2_KDTYPE_MXFP4): `buf` is a uint8 GPU tensor
    of 68 * rows bytes (rows = B * N_cap, or the page pool's rows), the rows'
    64 bytes of E2M1 first, then their 4 E8M0 scale bytes.  fp4_query: the
    query is quantised to MXFP4 too and QK runs on FP4 matrix instructions
    (CSA2_KDTYPE_MXFP4_QK)."""

    def __init__(self, buf, rows, n_cap, fp4_query=False):
        assert buf.dtype == torch.uint8 and buf.numel() == 68 * rows
        self.buf, self.rows, self.n_cap = buf, int(rows), int(n_cap)
        self.fp4_query = bool(fp4_query)

    def with_fp4_query(self, on=True):
        """The same key buffer, with or without the FP4 query."""
        return Mxfp4Keys(self.buf, self.rows, self.n_cap, fp4_query=on)


def _keys(k_idx):
    """(pointer, csa2_kdtype, N_cap or None) of an indexer-key argument."""
    if k_idx is None:
        return None, KDTYPE_BF16, None
    if isinstance(k_idx, Mxfp4Keys):
        kd = KDTYPE_MXFP4_QK if k_idx.fp4_query else KDTYPE_MXFP4
        return _ptr(k_idx.buf, (torch.uint8,), "k_idx"), kd, k_idx.n_cap
    kd = KDTYPE_BF16 if k_idx.dtype in _BITS16 else KDTYPE_FP8
    return _ptr(k_idx, _BITS16 + _U8, "k_idx"), kd, k_idx.shape[1]


class AttnOptsV1(ctypes.Structure):
    """The 16-byte options struct of ABI 1 (no sink pointer)."""
    _fields_ = [("window", _I), ("replay_start", _I), ("kv_fmt", _I), ("reserved", _I)]


class Csa2Error(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def lib():
    """The loaded libcsa2.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_sparse_attention_index_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, _I)
        _lib = l
    return _lib


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise Csa2Error(name, st, lib().csa2_status_string(st).decode())


def abi_version():
    return lib().csa2_abi_version()


def workspace_size(op, B, n_q, N_cap, top_k=512, k_blocks=2048):
    return lib().csa2_workspace_size(op, B, n_q, N_cap, top_k, k_blocks)


def _ptr(t, dtypes, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


_BITS16 = (torch.int16, torch.uint16, torch.bfloat16)
_U8 = (torch.uint8, torch.float8_e4m3fn)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _workspace(ws, nbytes, device):
    # Zero-filled: the block Top-K histograms must start at zero to take the
    # fast path (every call leaves them zeroed again).
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def index_score(q_idx, w_idx, k_idx, vis_len, scores=None, block_max=None, paging=None,
                stream=None):
    """Indexer scan: scores [B, n_q, N_cap] and/or block_max [B, n_q, ceil(N_cap/8)].
    With paging, k_idx is a page pool [num_pages * page_entries, 128]."""
    B, n_q = q_idx.shape[0], q_idx.shape[1]
    kp, kd, kn = _keys(k_idx)
    N_cap = paging.n_cap if paging is not None else kn
    _call("csa2_index_score", _ptr(q_idx, _BITS16, "q_idx"), _ptr(w_idx, _F32, "w_idx"),
          kp, kd, _paging(paging),
          _ptr(vis_len, _I32, "vis_len"), B, n_q, N_cap,
          _ptr(scores, _F32, "scores"), _ptr(block_max, _F32, "block_max"), None, 0,
          _stream(stream))


class PreparedCall:
    """A C call with its arguments checked and packed once; run() makes only
    the call, on the current stream (or `stream`)."""

    def __init__(self, name, args, keep):
        self._fn, self._name, self._args, self.keep = getattr(lib(), name), name, args, keep

    def run(self, stream=None):
        st = self._fn(*self._args, _stream(stream))
        if st != 0:
            raise Csa2Error(self._name, st, lib().csa2_status_string(st).decode())


def index_score_call(q_idx, w_idx, k_idx, vis_len, scores=None, block_max=None, paging=None):
    """index_score prepared once (see PreparedCall)."""
    B, n_q = q_idx.shape[0], q_idx.shape[1]
    kp, kd, kn = _keys(k_idx)
    N_cap = paging.n_cap if paging is not None else kn
    args = (_ptr(q_idx, _BITS16, "q_idx"), _ptr(w_idx, _F32, "w_idx"), kp, kd, _paging(paging),
            _ptr(vis_len, _I32, "vis_len"), B, n_q, N_cap, _ptr(scores, _F32, "scores"),
            _ptr(block_max, _F32, "block_max"), None, 0)
    return PreparedCall("csa2_index_score", args,
                        (q_idx, w_idx, k_idx, vis_len, scores, block_max, paging))


def index_score_bf16(q_idx, w_idx, k_idx, vis_len, scores, paging=None, stream=None):
    """The scan with scores stored as bf16 bit patterns: scores [B, n_q, N_cap]
    (int16 / uint16 / bfloat16 GPU tensor), each the fp32 score rounded to
    nearest even."""
    B, n_q = q_idx.shape[0], q_idx.shape[1]
    kp, kd, kn = _keys(k_idx)
    N_cap = paging.n_cap if paging is not None else kn
    _call("csa2_index_score_bf16", _ptr(q_idx, _BITS16, "q_idx"), _ptr(w_idx, _F32, "w_idx"),
          kp, kd, _paging(paging), _ptr(vis_len, _I32, "vis_len"), B, n_q, N_cap,
          _ptr(scores, _BITS16, "scores"), _stream(stream))


def flat_topk_bf16(scores, vis_len, top_k, idx_out, idx_score=None, stream=None):
    """Flat Top-top_k over bf16 scores [B, n_q, N_cap] (ties by position),
    ascending, -1 padded; idx_score (fp32) optional."""
    B, n_q, N_cap = scores.shape[0], scores.shape[1], scores.shape[2]
    _call("csa2_flat_topk_bf16", _ptr(scores, _BITS16, "scores"), _ptr(vis_len, _I32, "vis_len"),
          B, n_q, N_cap, top_k, _ptr(idx_out, _I32, "idx_out"),
          _ptr(idx_score, _F32, "idx_score"), _stream(stream))


def block_topk(block_max, vis_len, N_cap, k_blocks, pool_blocks, ws=None, stream=None):
    """Pool of the top min(k_blocks, nb) blocks per query row, ascending, -1 padded."""
    B, n_q = block_max.shape[0], block_max.shape[1]
    ws, nbytes = _workspace(ws, workspace_size(OP_BLOCK_TOPK, B, n_q, N_cap, 0, k_blocks),
                            block_max.device)
    _call("csa2_block_topk", _ptr(block_max, _F32, "block_max"), _ptr(vis_len, _I32, "vis_len"),
          B, n_q, N_cap, k_blocks, _ptr(pool_blocks, _I32, "pool_blocks"),
          _ptr(ws, (torch.uint8,), "ws"), nbytes, _stream(stream))


def block_topk_noalloc(block_max, vis_len, N_cap, k_blocks, pool_blocks, stream=None):
    """block_topk on the library's own fixed device scratch array (no workspace,
    no allocation); limits and sharing rules in include/csa2.h."""
    B, n_q = block_max.shape[0], block_max.shape[1]
    _call("csa2_block_topk_noalloc", _ptr(block_max, _F32, "block_max"),
          _ptr(vis_len, _I32, "vis_len"), B, n_q, N_cap, k_blocks,
          _ptr(pool_blocks, _I32, "pool_blocks"), _stream(stream))


def reindex_topk(mode, vis_len, N_cap, top_k, idx_out, scores=None, q_idx=None, w_idx=None,
                 k_idx=None, pool_blocks=None, idx_score=None, paging=None, ws=None, stream=None):
    """Top-k inside the pool (Full / Reindex) or over [0, vis) without a pool."""
    B, n_q = vis_len.shape[0], vis_len.shape[1]
    k_blocks = pool_blocks.shape[-1] if pool_blocks is not None else 0
    kp, kd, _ = _keys(k_idx)
    need = workspace_size(OP_REINDEX_TOPK, B, n_q, N_cap, top_k, k_blocks)
    ws, nbytes = _workspace(ws, need if pool_blocks is not None else 0, vis_len.device)
    _call("csa2_reindex_topk", mode, _ptr(scores, _F32, "scores"), _ptr(q_idx, _BITS16, "q_idx"),
          _ptr(w_idx, _F32, "w_idx"), kp, kd, _paging(paging),
          _ptr(pool_blocks, _I32, "pool_blocks"), k_blocks, _ptr(vis_len, _I32, "vis_len"),
          B, n_q, N_cap, top_k, _ptr(idx_out, _I32, "idx_out"),
          _ptr(idx_score, _F32, "idx_score"), _ptr(ws, (torch.uint8,), "ws"), nbytes,
          _stream(stream))


def _attn_args(q, kv_fp4, kv_scale, idx, swa_kv, swa_pos0, q_pos, sm_scale, out, lse=None,
               window=128, replay_start=-1, sink=None, kv_fmt=KV_MXFP4_E8M0_32, paging=None,
               ws=None):
    """Checked and packed arguments of an attention call (all but the stream),
    and the objects they point into."""
    B, n_q = q.shape[0], q.shape[1]
    N_cap = paging.n_cap if paging is not None else kv_fp4.shape[1]
    top_k = idx.shape[-1] if idx is not None else 0
    S_cap = swa_kv.shape[1] if swa_kv is not None else 0
    need = workspace_size(OP_SPARSE_ATTN, B, n_q, N_cap, top_k, 0)
    ws, nbytes = _workspace(ws, need, q.device)
    sp = _ptr(sink, _F32, "sink")
    flags = (ATTN_SINK if sp else 0) | (ATTN_PAGED if paging is not None else 0)
    opts = AttnOpts(window, replay_start, kv_fmt, flags, sp,
                    ctypes.pointer(paging.struct) if paging is not None else None)
    args = (_ptr(q, _BITS16, "q"), _ptr(kv_fp4, _U8, "kv_fp4"),
            _ptr(kv_scale, _U8, "kv_scale"), N_cap, _ptr(idx, _I32, "idx"), top_k,
            _ptr(swa_kv, _U8, "swa_kv"), S_cap, _ptr(swa_pos0, _I32, "swa_pos0"),
            _ptr(q_pos, _I32, "q_pos"), float(sm_scale), ctypes.byref(opts), B, n_q,
            _ptr(out, _BITS16, "out"), _ptr(lse, _F32, "lse"), _ptr(ws, (torch.uint8,), "ws"),
            nbytes)
    keep = (q, kv_fp4, kv_scale, idx, swa_kv, swa_pos0, q_pos, out, lse, sink, paging, ws, opts)
    return args, keep


def _attn(name, *args, stream=None, **kw):
    a, _ = _attn_args(*args, **kw)
    _call(name, *a, _stream(stream))


def sparse_attn_decode(*args, **kw):
    """Attention of a Full / Reindex layer over idx plus the SWA window."""
    _attn("csa2_sparse_attn_decode", *args, **kw)


def reuse_attn(*args, **kw):
    """Attention of a Reuse layer (indices from an earlier layer, no indexer)."""
    _attn("csa2_reuse_attn", *args, **kw)


def sparse_attn_call(*args, **kw):
    """sparse_attn_decode prepared once (see PreparedCall)."""
    return PreparedCall("csa2_sparse_attn_decode", *_attn_args(*args, **kw))


def reuse_attn_call(*args, **kw):
    """reuse_attn prepared once (see PreparedCall)."""
    return PreparedCall("csa2_reuse_attn", *_attn_args(*args, **kw))


def kv_append(kv_new, pos, kv_fp4, kv_scale, swa_new=None, swa_kv=None, swa_pos0=None,
              kv_fmt=KV_MXFP4_E8M0_32, paging=None, stream=None):
    """Encodes new tokens' entries (kv_new [B, n_new, 512] bf16 -> E2M1 rows
    pos[b] + i of kv_fp4 with scales in kv_scale, format kv_fmt; swa_new ->
    FP8 rows of swa_kv)."""
    B, n_new = kv_new.shape[0], kv_new.shape[1]
    N_cap = paging.n_cap if paging is not None else kv_fp4.shape[1]
    S_cap = swa_kv.shape[1] if swa_kv is not None else 0
    _call("csa2_kv_append", _ptr(kv_new, _BITS16, "kv_new"), _ptr(swa_new, _BITS16, "swa_new"),
          _ptr(pos, _I32, "pos"), B, n_new, N_cap, kv_fmt, _paging(paging),
          _ptr(kv_fp4, _U8, "kv_fp4"),
          _ptr(kv_scale, _U8, "kv_scale"), _ptr(swa_kv, _U8, "swa_kv"), S_cap,
          _ptr(swa_pos0, _I32, "swa_pos0"), _stream(stream))


class LayerArgs(ctypes.Structure):
    """csa2_layer_args."""
    _fields_ = [("k_idx", _P), ("k_dtype", _I), ("k_paging", ctypes.POINTER(PagingStruct)),
                ("kv_fp4", _P), ("kv_scale", _P), ("kv_fmt", _I),
                ("kv_paging", ctypes.POINTER(PagingStruct)), ("N_cap", _I), ("vis_len", _P),
                ("q_idx", _P), ("w_idx", _P), ("q", _P), ("swa_kv", _P), ("S_cap", _I),
                ("swa_pos0", _P), ("q_pos", _P), ("sm_scale", _F), ("window", _I),
                ("replay_start", _I), ("sink", _P), ("B", _I), ("n_q", _I)]


class LayerStateStruct(ctypes.Structure):
    """csa2_layer_state."""
    _fields_ = [("block_max", _P), ("scores", _P), ("pool_blocks", _P), ("k_blocks", _I),
                ("idx", _P), ("top_k", _I), ("ws", _P), ("ws_bytes", _S), ("has_pool", _I),
                ("has_idx", _I)]


def layer_mode(layer):
    """Mode of layer 0..39 in the model's schedule (-1 otherwise)."""
    return lib().csa2_layer_mode(layer)


class LayerState:
    """Device buffers carried across layers (the pool and the Top-K indices)
    for B x n_q query rows over N_cap entries."""

    def __init__(self, B, n_q, N_cap, k_blocks=2048, top_k=512, device="cuda"):
        z = lambda *shape, dt=torch.int32: torch.empty(*shape, dtype=dt, device=device)
        self.prefill = n_q >= 16
        self.block_max = None if self.prefill else z(B, n_q, (N_cap + 7) // 8, dt=torch.float32)
        self.scores = z(B, n_q, N_cap, dt=torch.float32) if self.prefill else None
        self.pool_blocks = z(B, n_q, k_blocks)
        self.idx = z(B, n_q, top_k)
        n = lib().csa2_layer_workspace_size(B, n_q, N_cap, k_blocks, top_k)
        self.ws = torch.zeros(max(int(n), 16), dtype=torch.uint8, device=device)
        self.struct = LayerStateStruct(
            _ptr(self.block_max, _F32, "block_max"), _ptr(self.scores, _F32, "scores"),
            _ptr(self.pool_blocks, _I32, "pool_blocks"), k_blocks, _ptr(self.idx, _I32, "idx"),
            top_k, self.ws.data_ptr(), self.ws.numel(), 0, 0)


def layer_call(state, k_idx, kv_fp4, kv_scale, vis_len, q, swa_kv, swa_pos0, q_pos, sm_scale,
               out, lse=None, q_idx=None, w_idx=None, kv_fmt=KV_MXFP4_E8M0_32, window=128,
               replay_start=-1, sink=None, k_paging=None, kv_paging=None):
    """A prepared csa2_run_layer call: the arguments are checked and packed
    once; LayerCall.run(mode, stream) then makes only the C call (for loops
    that issue the same layer's call on the same buffers many times)."""
    B, n_q = q.shape[0], q.shape[1]
    N_cap = kv_paging.n_cap if kv_paging is not None else kv_fp4.shape[1]
    kp, kd, _ = _keys(k_idx)
    a = LayerArgs(kp, kd,
                  ctypes.pointer(k_paging.struct) if k_paging is not None else None,
                  _ptr(kv_fp4, _U8, "kv_fp4"), _ptr(kv_scale, _U8, "kv_scale"), kv_fmt,
                  ctypes.pointer(kv_paging.struct) if kv_paging is not None else None, N_cap,
                  _ptr(vis_len, _I32, "vis_len"), _ptr(q_idx, _BITS16, "q_idx"),
                  _ptr(w_idx, _F32, "w_idx"), _ptr(q, _BITS16, "q"), _ptr(swa_kv, _U8, "swa_kv"),
                  swa_kv.shape[1], _ptr(swa_pos0, _I32, "swa_pos0"), _ptr(q_pos, _I32, "q_pos"),
                  float(sm_scale), window, replay_start, _ptr(sink, _F32, "sink"), B, n_q)
    return LayerCall(a, state, _ptr(out, _BITS16, "out"), _ptr(lse, _F32, "lse"),
                     (k_idx, kv_fp4, kv_scale, vis_len, q, swa_kv, swa_pos0, q_pos, out, lse,
                      q_idx, w_idx, sink, k_paging, kv_paging))


class LayerCall:
    """See layer_call; holds references to the tensors it points to."""

    def __init__(self, args, state, out_ptr, lse_ptr, keep):
        self.args, self.state, self.keep = args, state, keep
        self._a, self._s = ctypes.byref(args), ctypes.byref(state.struct)
        self._out, self._lse = out_ptr, lse_ptr
        self._fn = lib().csa2_run_layer

    def run(self, mode, stream=None):
        st = self._fn(mode, self._a, self._s, self._out, self._lse, _stream(stream))
        if st != 0:
            raise Csa2Error("csa2_run_layer", st, lib().csa2_status_string(st).decode())


def run_layer(mode, state, k_idx, kv_fp4, kv_scale, vis_len, q, swa_kv, swa_pos0, q_pos,
              sm_scale, out, lse=None, q_idx=None, w_idx=None, kv_fmt=KV_MXFP4_E8M0_32,
              window=128, replay_start=-1, sink=None, k_paging=None, kv_paging=None,
              stream=None):
    """One layer's CSA2 work by mode (include/csa2.h, csa2_run_layer)."""
    layer_call(state, k_idx, kv_fp4, kv_scale, vis_len, q, swa_kv, swa_pos0, q_pos, sm_scale,
               out, lse=lse, q_idx=q_idx, w_idx=w_idx, kv_fmt=kv_fmt, window=window,
               replay_start=replay_start, sink=sink, k_paging=k_paging,
               kv_paging=kv_paging).run(mode, stream)
