"""libcsa Python binding: CSA / HCA attention kernels for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libcsa.so`` (built by ``build.py``).  PyTorch supplies device memory and the
current stream.  There is no CPU fallback: importing this package fails
loudly when the library is missing.

Calls (same names as the C ABI in include/csa.h):
  csa_compress, csa_index_scores, csa_topk, csa_sparse_mqa, hca_dense_mqa
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libcsa.so not found at {LIB_PATH}: build it with "
                      "`python -m compressed_sparse_long_compress_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

CSA_OK, CSA_EINVAL, CSA_EUNSUPPORTED, CSA_EHIP, CSA_EWORKSPACE = 0, -1, -2, -3, -4


class _Kv(ctypes.Structure):
    _fields_ = [("nope", ctypes.c_void_p), ("rope", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("cap", ctypes.c_int64), ("pages", ctypes.c_void_p), ("page", ctypes.c_int32)]


class _IdxKeys(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("cap", ctypes.c_int64),
                ("pages", ctypes.c_void_p), ("page", ctypes.c_int32)]


_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_lib.csa_compress.argtypes = [_vp, _vp, _i64, _i64, _i32, _i32, _f32, _i32, _Kv, _vp]
_lib.csa_compress_channel.argtypes = [_vp, _vp, _i64, _i64, _i32, _i32, _f32, _i32, _Kv, _vp]
_lib.csa_compress_index_keys.argtypes = [_vp, _vp, _i64, _i64, _i32, _i32, _i32, _IdxKeys, _vp]
_lib.csa_index_scores.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _IdxKeys, _i32, _i64, _vp, _vp, _sz, _vp]
_lib.csa_index_scores_grouped.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _IdxKeys, _i32, _i64, _i32, _vp,
                                          _vp, _sz, _vp]
_lib.csa_index_topk_workspace.restype = _sz
_lib.csa_index_topk_workspace.argtypes = [_i64, _i64, _i32, _i32]
_lib.csa_index_topk.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _IdxKeys, _i32, _i64, _i32, _vp, _vp, _sz,
                                _vp]
_lib.csa_index_bwd_workspace.restype = _sz
_lib.csa_index_bwd_workspace.argtypes = [_i64, _i32]
_lib.csa_index_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _IdxKeys, _i32, _vp, _vp, _i32, _vp, _vp, _vp,
                               _i64, _vp, _sz, _vp]
_lib.csa_topk_workspace.restype = _sz
_lib.csa_topk_workspace.argtypes = [_i64, _i64, _i32]
_lib.csa_topk.argtypes = [_vp, _i64, _i64, _vp, _i32, _i32, _vp, _vp, _sz, ctypes.c_uint32, _vp]
CSA_TOPK_PREPARED = 1
_lib.csa_topk_noalloc.argtypes = [_vp, _i64, _i64, _vp, _i32, _i32, _vp, _vp]
_lib.csa_mqa_workspace.restype = _sz
_lib.csa_mqa_workspace.argtypes = [_i64, _i32, _i32, _i64]
_lib.csa_sparse_mqa.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _i32, _i32, _Kv, _Kv, _i32, _f32, _f32, _vp,
                                _vp, _vp, _sz, _vp]
_lib.hca_dense_mqa.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _Kv, _Kv, _i32, _f32, _f32, _vp, _vp,
                               _vp, _sz, _vp]
_lib.csa_mqa_bwd_workspace.restype = _sz
_lib.csa_mqa_bwd_workspace.argtypes = [_i64, _i64, _i32]
_lib.csa_mqa_bwd.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _i32, _i32, _Kv, _Kv, _i32, _f32, _f32, _vp, _vp,
                             _vp, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp]
_lib.csa_pages_bytes.restype = _sz
_lib.csa_pages_bytes.argtypes = [_i32, _i32, _i32]
_lib.csa_pages_store.argtypes = [_Kv, _IdxKeys, _i32, _i32, _vp, _i32, _vp, _sz, _vp]
_lib.csa_pages_load.argtypes = [_Kv, _IdxKeys, _i32, _i32, _vp, _i32, _vp, _sz, _vp]
_lib.csa_mfma_probe_flops.restype = _i64
_lib.csa_mfma_probe_flops.argtypes = [_i32, _i32, _i64]
_lib.csa_mfma_probe.argtypes = [_i32, _i32, _i64, _vp, _i64, _vp]
_lib.csa_last_error.restype = ctypes.c_char_p
_lib.csa_version.restype = ctypes.c_int

EXPORTS = ["csa_compress", "csa_compress_channel", "csa_compress_index_keys", "csa_index_scores", "csa_index_scores_grouped", "csa_index_topk_workspace", "csa_index_topk", "csa_index_bwd_workspace",
           "csa_index_bwd", "csa_topk_workspace", "csa_topk", "csa_topk_noalloc", "csa_mqa_workspace",
           "csa_sparse_mqa", "hca_dense_mqa", "csa_mqa_bwd_workspace", "csa_mqa_bwd", "csa_pages_bytes", "csa_pages_store", "csa_pages_load",
           "csa_mfma_probe_flops", "csa_mfma_probe", "csa_last_error", "csa_version"]


class CsaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libcsa error {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != CSA_OK:
        raise CsaError(rc, _lib.csa_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def version():
    return _lib.csa_version()


def mfma_probe(kind, blocks, iters, sink):
    """One launch of the matrix-core throughput probe (kind 0: fp16 16x16x32, 1: MXFP4 32x32x64)
    on the current stream; sink: float32 tensor of >= blocks x 256 elements.  Returns the
    launch's flop count."""
    _need(sink, "sink", torch.float32, 1)
    _check(_lib.csa_mfma_probe(int(kind), int(blocks), int(iters), _ptr(sink), sink.numel(), _stream()))
    return int(_lib.csa_mfma_probe_flops(int(kind), int(blocks), int(iters)))


class KvCache:
    """Mixed-precision entries: nope uint8 [rows, d-64], rope bf16 [rows, 64], scale fp32 [rows].

    Contiguous: rows = n_seq*cap, slot i of sequence s at row s*cap + i.  Paged
    (pages int32 [n_seq, cap // page], page a power of two): slot i of sequence s
    at row pages[s, i // page] * page + i % page; sequences may share pages."""

    def __init__(self, nope, rope, scale, cap, pages=None, page=0):
        _need(nope, "nope", torch.uint8, 2)
        _need(rope, "rope", torch.bfloat16, 2)
        _need(scale, "scale", torch.float32, 1)
        if rope.shape[1] != 64 or nope.shape[0] != rope.shape[0] or scale.shape[0] != rope.shape[0]:
            raise ValueError("inconsistent KvCache arrays")
        if pages is None:
            if cap <= 0 or rope.shape[0] % cap != 0:
                raise ValueError("rows must be a multiple of cap")
        else:
            _need(pages, "pages", torch.int32, 2)
            if page <= 0 or page & (page - 1) or cap % page or pages.shape[1] != cap // page:
                raise ValueError("page must be a power of two dividing cap; pages [n_seq, cap // page]")
            if rope.shape[0] % page:
                raise ValueError("rows must be whole pages")
        self.nope, self.rope, self.scale, self.cap = nope, rope, scale, int(cap)
        self.pages, self.page = pages, int(page) if pages is not None else 0

    @property
    def d(self):
        return self.nope.shape[1] + 64

    @classmethod
    def empty(cls, n_seq, cap, d, device="cuda"):
        rows = n_seq * cap
        return cls(torch.zeros(rows, d - 64, dtype=torch.uint8, device=device),
                   torch.zeros(rows, 64, dtype=torch.bfloat16, device=device),
                   torch.zeros(rows, dtype=torch.float32, device=device), cap)

    def c(self):
        return _Kv(self.nope.data_ptr(), self.rope.data_ptr(), self.scale.data_ptr(), self.cap,
                   self.pages.data_ptr() if self.pages is not None else None, self.page)


class IndexKeys:
    """MXFP4 indexer keys: data uint8 [rows, d_i/2], scale uint8 [rows, d_i/32].

    Contiguous: rows = n_seq*cap, key of entry j of sequence s at row s*cap + j.  Paged (pages int32
    [n_seq, cap // page], page a power of two): at row pages[s, j // page] * page + j % page."""

    def __init__(self, data, scale, cap, pages=None, page=0):
        _need(data, "keys.data", torch.uint8, 2)
        _need(scale, "keys.scale", torch.uint8, 2)
        if data.shape[0] != scale.shape[0] or data.shape[1] != scale.shape[1] * 16:
            raise ValueError("inconsistent IndexKeys arrays")
        if pages is not None:
            _need(pages, "keys.pages", torch.int32, 2)
            if page <= 0 or page & (page - 1) or cap % page or pages.shape[1] != cap // page:
                raise ValueError("page must be a power of two dividing cap; pages [n_seq, cap // page]")
            if data.shape[0] % page:
                raise ValueError("rows must be whole pages")
        self.data, self.scale, self.cap = data, scale, int(cap)
        self.pages, self.page = pages, int(page) if pages is not None else 0

    @property
    def d_i(self):
        return self.data.shape[1] * 2

    def c(self):
        return _IdxKeys(self.data.data_ptr(), self.scale.data_ptr(), self.cap,
                        self.pages.data_ptr() if self.pages is not None else None, self.page)


def csa_compress(kv, logits, tok0, m, seq, out, rope_base=10000.0):
    """Compress tokens [tok0, tok0+n_tok) (kv bf16 [n_tok, d], logits fp32 [n_tok]) into `out` (KvCache)."""
    _need(kv, "kv", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 1)
    n_tok, d = kv.shape
    if logits.shape[0] != n_tok or d != out.d:
        raise ValueError("kv / logits / out shapes disagree")
    _check(_lib.csa_compress(_ptr(kv), _ptr(logits), int(tok0), int(n_tok), int(m), int(d), float(rope_base),
                             int(seq), out.c(), _stream()))
    return out


def csa_compress_channel(kv, logits, tok0, m, seq, out, rope_base=10000.0):
    """csa_compress with per-channel weights: logits fp32 [n_tok, d]."""
    _need(kv, "kv", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 2)
    n_tok, d = kv.shape
    if tuple(logits.shape) != (n_tok, d) or d != out.d:
        raise ValueError("kv / logits / out shapes disagree")
    _check(_lib.csa_compress_channel(_ptr(kv), _ptr(logits), int(tok0), int(n_tok), int(m), int(d), float(rope_base),
                                     int(seq), out.c(), _stream()))
    return out


def csa_compress_index_keys(k, logits, tok0, m, seq, out):
    """Raw index-key tokens (bf16 [n_tok, d_i], logits fp32 [n_tok]) -> MXFP4 rows of `out` (IndexKeys)."""
    _need(k, "k", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 1)
    n_tok, d_i = k.shape
    if logits.shape[0] != n_tok or d_i != out.d_i:
        raise ValueError("k / logits / out shapes disagree")
    _check(_lib.csa_compress_index_keys(_ptr(k), _ptr(logits), int(tok0), int(n_tok), int(m), int(d_i), int(seq),
                                        out.c(), _stream()))
    return out


def csa_index_scores(q, q_scale, w, seq, pos, keys, m, n_cols, out=None, topk_ws=None):
    """MXFP4 indexer scores: q uint8 [T, h_i, d_i/2], q_scale uint8 [T, h_i, d_i/32], w fp32 [T, h_i] -> fp32 [T, n_cols].

    topk_ws: the workspace of the csa_topk call that follows; the indexer then
    also writes the selection's row summary into it, and that call passes
    prepared=True."""
    _need(q, "q", torch.uint8, 3)
    _need(q_scale, "q_scale", torch.uint8, 3)
    _need(w, "w", torch.float32, 2)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int64, 1)
    T, h_i, half = q.shape
    d_i = half * 2
    if d_i != keys.d_i or tuple(q_scale.shape) != (T, h_i, d_i // 32) or tuple(w.shape) != (T, h_i):
        raise ValueError("indexer query shapes disagree")
    if seq.shape[0] != T or pos.shape[0] != T:
        raise ValueError("seq / pos must have T entries")
    if out is None:
        out = torch.empty(T, n_cols, dtype=torch.float32, device=q.device)
    _need(out, "scores", torch.float32, 2)
    if tuple(out.shape) != (T, n_cols):
        raise ValueError("scores must be [T, n_cols]")
    _check(_lib.csa_index_scores(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(seq), _ptr(pos), T, h_i, d_i, keys.c(), int(m),
                                 int(n_cols), _ptr(out), _ptr(topk_ws), topk_ws.numel() if topk_ws is not None else 0,
                                 _stream()))
    return out


def csa_index_scores_grouped(q, q_scale, w, seq, pos, keys, m, n_cols, group, out=None, topk_ws=None):
    """csa_index_scores for rows in groups of `group` (1, 2 or 4) that share a sequence
    (multi-token decode): each group streams its keys once.  Same result as
    csa_index_scores for any seq / pos."""
    _need(q, "q", torch.uint8, 3)
    _need(q_scale, "q_scale", torch.uint8, 3)
    _need(w, "w", torch.float32, 2)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int64, 1)
    T, h_i, half = q.shape
    d_i = half * 2
    if d_i != keys.d_i or tuple(q_scale.shape) != (T, h_i, d_i // 32) or tuple(w.shape) != (T, h_i):
        raise ValueError("indexer query shapes disagree")
    if seq.shape[0] != T or pos.shape[0] != T:
        raise ValueError("seq / pos must have T entries")
    if out is None:
        out = torch.empty(T, n_cols, dtype=torch.float32, device=q.device)
    _need(out, "scores", torch.float32, 2)
    if tuple(out.shape) != (T, n_cols):
        raise ValueError("scores must be [T, n_cols]")
    _check(_lib.csa_index_scores_grouped(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(seq), _ptr(pos), T, h_i, d_i, keys.c(),
                                         int(m), int(n_cols), int(group), _ptr(out), _ptr(topk_ws),
                                         topk_ws.numel() if topk_ws is not None else 0, _stream()))
    return out


def csa_index_topk_workspace(T, n_cols, k, h_i):
    return int(_lib.csa_index_topk_workspace(int(T), int(n_cols), int(k), int(h_i)))


def csa_index_topk(q, q_scale, w, seq, pos, keys, m, n_cols, k, out=None, ws=None):
    """Indexer + top-k without score rows -> int32 [T, k] (what csa_index_scores + csa_topk give).

    ws: a uint8 workspace of csa_index_topk_workspace(T, n_cols, k, h_i) bytes (allocated when None)."""
    _need(q, "q", torch.uint8, 3)
    _need(q_scale, "q_scale", torch.uint8, 3)
    _need(w, "w", torch.float32, 2)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int64, 1)
    T, h_i, half = q.shape
    d_i = half * 2
    if d_i != keys.d_i or tuple(q_scale.shape) != (T, h_i, d_i // 32) or tuple(w.shape) != (T, h_i):
        raise ValueError("indexer query shapes disagree")
    if seq.shape[0] != T or pos.shape[0] != T:
        raise ValueError("seq / pos must have T entries")
    if out is None:
        out = torch.empty(T, k, dtype=torch.int32, device=q.device)
    _need(out, "idx", torch.int32, 2)
    if tuple(out.shape) != (T, k):
        raise ValueError("idx must be [T, k]")
    if ws is None:
        ws = torch.empty(max(csa_index_topk_workspace(T, n_cols, k, h_i), 1), dtype=torch.uint8, device=q.device)
    _check(_lib.csa_index_topk(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(seq), _ptr(pos), T, h_i, d_i, keys.c(),
                               int(m), int(n_cols), int(k), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def csa_index_bwd(q, q_scale, w, seq, pos, keys, m, idx, g, key_rows=None, dkeys=None, ws=None):
    """Gradient of the indexer scores at the selected columns idx [T, n_sel] given g = dL/dscore there
    -> (dq fp32 [T, h_i, d_i], dw fp32 [T, h_i], dkeys fp32 [key_rows, d_i]); dkeys is accumulated into
    when given (zeros otherwise)."""
    _need(q, "q", torch.uint8, 3)
    _need(q_scale, "q_scale", torch.uint8, 3)
    _need(w, "w", torch.float32, 2)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int64, 1)
    _need(idx, "idx", torch.int32, 2)
    _need(g, "g", torch.float32, 2)
    T, h_i, half = q.shape
    d_i = half * 2
    if d_i != keys.d_i or tuple(q_scale.shape) != (T, h_i, d_i // 32) or tuple(w.shape) != (T, h_i):
        raise ValueError("indexer query shapes disagree")
    if idx.shape[0] != T or tuple(g.shape) != tuple(idx.shape):
        raise ValueError("idx and g must be [T, n_sel]")
    if key_rows is None:
        key_rows = keys.data.shape[0]
    dq = torch.empty(T, h_i, d_i, dtype=torch.float32, device=q.device)
    dw = torch.empty(T, h_i, dtype=torch.float32, device=q.device)
    if dkeys is None:
        dkeys = torch.zeros(key_rows, d_i, dtype=torch.float32, device=q.device)
    _need(dkeys, "dkeys", torch.float32, 2)
    if tuple(dkeys.shape) != (key_rows, d_i):
        raise ValueError("dkeys must be [key_rows, d_i]")
    if ws is None:
        ws = torch.empty(csa_index_bwd_workspace(key_rows, d_i), dtype=torch.uint8, device=q.device)
    _check(_lib.csa_index_bwd(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(seq), _ptr(pos), T, h_i, d_i, keys.c(), int(m),
                              _ptr(idx), _ptr(g), int(idx.shape[1]), _ptr(dq), _ptr(dw), _ptr(dkeys), int(key_rows),
                              _ptr(ws), ws.numel(), _stream()))
    return dq, dw, dkeys


def csa_index_bwd_workspace(key_rows, d_i):
    return int(_lib.csa_index_bwd_workspace(int(key_rows), int(d_i)))


def csa_topk_workspace(T, n_cols, k):
    return int(_lib.csa_topk_workspace(int(T), int(n_cols), int(k)))


def topk_workspace(T, n_cols, k, device="cuda"):
    """A top-k workspace (its contents need no initialisation)."""
    need = csa_topk_workspace(T, n_cols, k)
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def csa_topk(scores, pos, m, k, out=None, ws=None, prepared=False):
    """Top-k per row (score desc, index asc) in ascending index order, -1 padded -> int32 [T, k].

    ws: a uint8 workspace of csa_topk_workspace(T, n_cols, k) bytes (allocated when None)."""
    _need(scores, "scores", torch.float32, 2)
    _need(pos, "pos", torch.int64, 1)
    T, n_cols = scores.shape
    if out is None:
        out = torch.empty(T, k, dtype=torch.int32, device=scores.device)
    _need(out, "idx", torch.int32, 2)
    if ws is None:
        ws = topk_workspace(T, n_cols, k, scores.device)
    _check(_lib.csa_topk(_ptr(scores), T, n_cols, _ptr(pos), int(m), int(k), _ptr(out), _ptr(ws), ws.numel(),
                         CSA_TOPK_PREPARED if prepared else 0, _stream()))
    return out


def csa_topk_noalloc(scores, pos, m, k, out=None):
    """csa_topk through the entry point that allocates nothing (the library's own scratch array)."""
    _need(scores, "scores", torch.float32, 2)
    _need(pos, "pos", torch.int64, 1)
    T, n_cols = scores.shape
    if out is None:
        out = torch.empty(T, k, dtype=torch.int32, device=scores.device)
    _need(out, "idx", torch.int32, 2)
    _check(_lib.csa_topk_noalloc(_ptr(scores), T, n_cols, _ptr(pos), int(m), int(k), _ptr(out), _stream()))
    return out


def csa_mqa_workspace(T, H, d, max_keys):
    return int(_lib.csa_mqa_workspace(int(T), int(H), int(d), int(max_keys)))


def _mqa_outputs(q, out, lse):
    T, H, d = q.shape
    if out is None:
        out = torch.empty(T, H, d, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(T, H, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    return out, lse


def _win(win, comp):
    return win.c() if win is not None else _Kv(None, None, None, 1)


def csa_sparse_mqa(q, seq, pos, idx, m, comp, win, window, sm_scale, rope_base=10000.0, out=None, lse=None, ws=None):
    """CSA attention over selected entries (idx int32 [T, k]) plus the window -> (out fp32 [T,H,d], lse fp32 [T,H])."""
    _need(q, "q", torch.bfloat16, 3)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int64, 1)
    _need(idx, "idx", torch.int32, 2)
    T, H, d = q.shape
    k = idx.shape[1]
    out, lse = _mqa_outputs(q, out, lse)
    need = csa_mqa_workspace(T, H, d, k + window)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = ws.numel() if ws is not None else 0
    _check(_lib.csa_sparse_mqa(_ptr(q), _ptr(seq), _ptr(pos), T, H, d, _ptr(idx), k, int(m), comp.c(), _win(win, comp),
                               int(window), float(sm_scale), float(rope_base), _ptr(out), _ptr(lse), _ptr(ws),
                               ws_bytes, _stream()))
    return out, lse


def hca_dense_mqa(q, seq, pos, m, max_vis, comp, win, window, sm_scale, rope_base=10000.0, out=None, lse=None,
                  ws=None):
    """HCA attention over every visible compressed entry plus the window -> (out, lse)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int64, 1)
    T, H, d = q.shape
    out, lse = _mqa_outputs(q, out, lse)
    need = csa_mqa_workspace(T, H, d, max_vis + window)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = ws.numel() if ws is not None else 0
    _check(_lib.hca_dense_mqa(_ptr(q), _ptr(seq), _ptr(pos), T, H, d, int(m), int(max_vis), comp.c(),
                              _win(win, comp), int(window), float(sm_scale), float(rope_base), _ptr(out), _ptr(lse),
                              _ptr(ws), ws_bytes, _stream()))
    return out, lse


def csa_mqa_bwd_workspace(comp_rows, win_rows, d):
    return int(_lib.csa_mqa_bwd_workspace(int(comp_rows), int(win_rows), int(d)))


def csa_mqa_bwd(q, seq, pos, idx, m, comp, win, window, sm_scale, out, lse, dout, rope_base=10000.0, dq=None,
                dcomp=None, dwin=None, ws=None):
    """Gradient of the attention step -> (dq fp32 [T,H,d], dcomp fp32 [comp rows, d], dwin fp32 [win rows, d]).

    idx int32 [T, k] (the selected entries) or None (every visible entry); out / lse are the forward's.
    dcomp / dwin are accumulated into (fresh zeros when not given; dwin None when window is 0); their
    row counts bound the cache rows.  ws: csa_mqa_bwd_workspace bytes (allocated when None)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(seq, "seq", torch.int32, 1)
    _need(pos, "pos", torch.int64, 1)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    _need(dout, "dout", torch.float32, 3)
    k = 0
    if idx is not None:
        _need(idx, "idx", torch.int32, 2)
        k = idx.shape[1]
    T, H, d = q.shape
    if dq is None:
        dq = torch.empty(T, H, d, dtype=torch.float32, device=q.device)
    if dcomp is None:
        dcomp = torch.zeros(comp.nope.shape[0], d, dtype=torch.float32, device=q.device)
    if dwin is None and window > 0:
        dwin = torch.zeros(win.nope.shape[0], d, dtype=torch.float32, device=q.device)
    comp_rows = dcomp.shape[0]
    win_rows = dwin.shape[0] if (dwin is not None and window > 0) else 0
    if ws is None:
        ws = torch.empty(csa_mqa_bwd_workspace(comp_rows, win_rows, d), dtype=torch.uint8, device=q.device)
    _check(_lib.csa_mqa_bwd(_ptr(q), _ptr(seq), _ptr(pos), T, H, d, _ptr(idx), k, int(m), comp.c(), _win(win, comp),
                            int(window), float(sm_scale), float(rope_base), _ptr(out), _ptr(lse), _ptr(dout),
                            _ptr(dq), _ptr(dcomp), comp_rows, _ptr(dwin), win_rows, _ptr(ws), ws.numel(), _stream()))
    return dq, dcomp, dwin


# ---- shared-prefix pages on the host and on disk ----
_PAGES_MAGIC = b"CSAPAGE1"


def _page_args(kv, keys):
    d = kv.d
    d_i = keys.d_i if keys is not None else 0
    kc = keys.c() if keys is not None else _IdxKeys(None, None, 0, None, 0)
    return d, d_i, kc


def csa_pages_bytes(page, d, d_i):
    return int(_lib.csa_pages_bytes(int(page), int(d), int(d_i)))


def csa_pages_store(kv, keys, page_ids, host):
    """Copy physical pages page_ids of kv (KvCache, paged) and keys (IndexKeys or None) into host
    (a uint8 CPU tensor, pinned for asynchronous copies); synchronise before reading it."""
    d, d_i, kc = _page_args(kv, keys)
    ids = (ctypes.c_int32 * len(page_ids))(*[int(p) for p in page_ids])
    _check(_lib.csa_pages_store(kv.c(), kc, d, d_i, ids, len(page_ids), ctypes.c_void_p(host.data_ptr()),
                                host.numel(), _stream()))


def csa_pages_load(kv, keys, page_ids, host):
    """Copy host (the layout csa_pages_store writes) into physical pages page_ids of kv and keys."""
    d, d_i, kc = _page_args(kv, keys)
    ids = (ctypes.c_int32 * len(page_ids))(*[int(p) for p in page_ids])
    _check(_lib.csa_pages_load(kv.c(), kc, d, d_i, ids, len(page_ids), ctypes.c_void_p(host.data_ptr()),
                               host.numel(), _stream()))


def save_pages(path, kv, keys, page_ids):
    """Write pages page_ids of kv and keys to a file: an 8-byte tag, (d, d_i, page, n) as int32, then
    the pages in the layout of csa_pages_store."""
    import numpy as np

    d, d_i, _ = _page_args(kv, keys)
    n = len(page_ids)
    host = torch.empty(csa_pages_bytes(kv.page, d, d_i) * n, dtype=torch.uint8, pin_memory=True)
    csa_pages_store(kv, keys, page_ids, host)
    torch.cuda.current_stream().synchronize()
    with open(path, "wb") as f:
        f.write(_PAGES_MAGIC)
        f.write(np.array([d, d_i, kv.page, n], np.int32).tobytes())
        f.write(host.numpy().tobytes())


def load_pages(path, kv, keys, page_ids):
    """Read a file written by save_pages into pages page_ids of kv and keys (same d, d_i, page and count)."""
    import numpy as np

    with open(path, "rb") as f:
        if f.read(8) != _PAGES_MAGIC:
            raise ValueError(f"{path}: not a page file")
        d, d_i, page, n = (int(x) for x in np.frombuffer(f.read(16), np.int32))
        exp = _page_args(kv, keys)
        if (d, d_i, page, n) != (exp[0], exp[1], kv.page, len(page_ids)):
            raise ValueError(f"{path}: holds d={d} d_i={d_i} page={page} x{n}, the destination differs")
        data = f.read()
    host = torch.empty(len(data), dtype=torch.uint8, pin_memory=True)
    host.numpy()[:] = np.frombuffer(data, np.uint8)
    csa_pages_load(kv, keys, page_ids, host)
    torch.cuda.current_stream().synchronize()
