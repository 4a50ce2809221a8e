"""ctypes binding of libkvc.so: argument marshalling only.

Every function here checks the tensors it is handed (device, dtype, shape,
innermost stride), turns them into raw pointers and strides, and calls the C
entry point of the same name on torch's current HIP stream. All of the
compressor's work runs in the library's HIP kernels; there is no fallback,
and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

KVC_OK = 0
KVC_ERR_INVALID_ARG = -1
KVC_ERR_UNSUPPORTED = -2
KVC_ERR_WORKSPACE = -3
KVC_ERR_ALIGN = -4
KVC_ERR_HIP = -5
KVC_MAX_KV_HEADS = 64
KVC_MAX_ROWS = 256
KVC_MAX_POOL = 31
KVC_NOALLOC_SCRATCH_BYTES = 16 << 20
KVC_SCORE_SOFTMAX = 0
KVC_SCORE_LOGIT = 1
KVC_SCORE_LOGIT_INT8 = 2
KVC_FLAG_FUSED_SELECT = 1  # select and gather inside the fused scan launch, scores on chip
KVC_SCAN_STREAM = 1
KVC_SCAN_PER_HEAD = 2
KVC_SCAN_LOGIT = 3


class KvcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class LayerDesc(ctypes.Structure):
    """Mirror of ``kvc_layer_desc``."""
    _fields_ = [
        ("s", ctypes.c_int64),
        ("w", ctypes.c_int32),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("n_sink", ctypes.c_int32),
        ("n_recent", ctypes.c_int32),
        ("pool", ctypes.c_int32),
        ("score_mode", ctypes.c_int32),
        ("pos_offset", ctypes.c_int64),
        ("q_tok_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("k_tok_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64),
        ("v_tok_stride", ctypes.c_int64),
        ("v_head_stride", ctypes.c_int64),
        ("flags", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class LayerPlan(ctypes.Structure):
    """Mirror of ``kvc_layer_plan``."""
    _fields_ = [
        ("scan", ctypes.c_int32),
        ("heads_per_wg", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("hist_in_scan", ctypes.c_int32),
        ("fused_scans", ctypes.c_int32),
        ("fused_select", ctypes.c_int32),
        ("keys_per_wg", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class PrefillDesc(ctypes.Structure):
    """kvc_prefill_desc: one layer's attention shape and rotary base."""
    _fields_ = [
        ("s", ctypes.c_int64),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("scale", ctypes.c_float),
    ]


def make_desc(s, w, hq, hkv, d, block=256, scale=0.0, n_sink=0, n_recent=0, pool=1,
              pos_offset=0, q_strides=(0, 0), k_strides=(0, 0), v_strides=(0, 0),
              score_mode=0, flags=0) -> LayerDesc:
    return LayerDesc(s=s, w=w, hq=hq, hkv=hkv, d=d, block=block, scale=scale, n_sink=n_sink,
                     n_recent=n_recent, pool=pool, score_mode=score_mode, pos_offset=pos_offset,
                     q_tok_stride=q_strides[0], q_head_stride=q_strides[1],
                     k_tok_stride=k_strides[0], k_head_stride=k_strides[1],
                     v_tok_stride=v_strides[0], v_head_stride=v_strides[1], flags=flags, reserved=0)


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; build it with `python -m compression_kvc_score_amd.build` "
            "(there is no fallback implementation)")
    # torch brings its own HIP runtime; load it first so libkvc binds to the
    # same libamdhip64 (one runtime per process, shared streams).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(LayerDesc)
    PD = ctypes.POINTER(PrefillDesc)
    sig = {
        "kvc_version": (ctypes.c_int, []),
        "kvc_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "kvc_last_error": (ctypes.c_char_p, []),
        "kvc_workspace_size": (SZ, [D]),
        "kvc_plan_layer": (ctypes.c_int, [D, ctypes.POINTER(LayerPlan)]),
        "kvc_retained_offsets": (ctypes.c_int, [D, P, P]),
        "kvc_budgets_inverse_stability": (ctypes.c_int, [P, I32, I64, P]),
        "kvc_score_pass1": (ctypes.c_int, [D, P, P, P, P, P, SZ, P]),
        "kvc_score_pass2": (ctypes.c_int, [D, P, P, P, P, P, P]),
        "kvc_score_layer": (ctypes.c_int, [D, P, P, P, P, P, P, SZ, P]),
        "kvc_select_topk": (ctypes.c_int, [D, P, P, P, P, SZ, P]),
        "kvc_gather_retained": (ctypes.c_int, [D, P, P, P, P, P, P, P, P]),
        "kvc_compress_layer": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "kvc_compress_layers": (ctypes.c_int, [D, I32, P, P, P, P, P, P, P, P, P, SZ, P, P]),
        "kvc_compress_layer_noalloc": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, P, P, P]),
        "kvc_overlap_coefficient": (ctypes.c_int, [D, P, P, P, P, P]),
        "kvc_chunk_workspace_size": (SZ, [D, I64]),
        "kvc_evict_chunk": (ctypes.c_int, [D, P, P, P, I32, I64, I64, P, P, P, P, P, P, P, SZ, P]),
        "kvc_chunked_workspace_size": (SZ, [D, I64, I32]),
        "kvc_compress_chunked": (ctypes.c_int, [D, I64, P, P, P, I32, P, P, P, P, SZ, P]),
        "kvc_rmsnorm": (ctypes.c_int, [P, P, P, I64, I32, ctypes.c_float, P]),
        "kvc_rope_append": (ctypes.c_int, [PD, P, I64, I64, P, P, P, P]),
        "kvc_chunk_attention": (ctypes.c_int, [PD, P, P, P, I64, I64, P, P]),
        "kvc_swiglu": (ctypes.c_int, [P, P, I64, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def lib():
    return _load()


def _check(status: int):
    if status != KVC_OK:
        L = _load()
        msg = L.kvc_last_error().decode() or L.kvc_strerror(status).decode()
        raise KvcError(status, msg)


# ------------------------------------------------------------------ tensors

def _dev_ptr(t, name, dtype_size=None, inner_contig=True):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if dtype_size is not None and t.element_size() != dtype_size:
        raise ValueError(f"{name}: expected {dtype_size}-byte elements, got {t.dtype}")
    if inner_contig and t.dim() > 0 and t.stride(-1) != 1 and t.size(-1) > 1:
        raise ValueError(f"{name}: the innermost dimension must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _bf16_ptr(t, name):
    import torch
    if t is not None and t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError(f"{name} must hold bf16 values (torch.bfloat16 or 16-bit bit patterns)")
    return _dev_ptr(t, name, 2)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _host_i32(arr, n, name):
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int64))
    if a.shape != (n,):
        raise ValueError(f"{name} must have {n} entries")
    if np.any(a < np.iinfo(np.int32).min) or np.any(a > np.iinfo(np.int32).max):
        raise ValueError(f"{name} does not fit in int32")
    return np.ascontiguousarray(a.astype(np.int32))


def desc_for(q_win, k, v=None, *, block=256, scale=0.0, n_sink=0, n_recent=0, pool=1,
             pos_offset=0, score_mode=0, flags=0) -> LayerDesc:
    """Descriptor for tensors Q_win [W, hq, D] and K (V) [S, hkv, D] with their
    strides (the head dimension must be contiguous)."""
    w, hq, d = q_win.shape
    s, hkv, dk = k.shape
    if dk != d:
        raise ValueError("Q_win and K head dimensions differ")
    vs = (v.stride(0), v.stride(1)) if v is not None else (0, 0)
    return make_desc(s, w, hq, hkv, d, block=block, scale=scale, n_sink=n_sink,
                     n_recent=n_recent, pool=pool, pos_offset=pos_offset, score_mode=score_mode, flags=flags,
                     q_strides=(q_win.stride(0), q_win.stride(1)),
                     k_strides=(k.stride(0), k.stride(1)), v_strides=vs)


# ------------------------------------------------------------------ host-only calls

def kvc_version() -> int:
    return _load().kvc_version()


def kvc_strerror(status: int) -> str:
    return _load().kvc_strerror(status).decode()


def kvc_workspace_size(desc: LayerDesc) -> int:
    n = _load().kvc_workspace_size(ctypes.byref(desc))
    if n == 0:
        _check(KVC_ERR_INVALID_ARG)
    return n


def kvc_plan_layer(desc: LayerDesc) -> LayerPlan:
    plan = LayerPlan()
    _check(_load().kvc_plan_layer(ctypes.byref(desc), ctypes.byref(plan)))
    return plan


def kvc_retained_offsets(desc: LayerDesc, budgets) -> np.ndarray:
    b = _host_i32(budgets, desc.hkv, "budgets")
    off = np.zeros(desc.hkv + 1, dtype=np.int64)
    _check(_load().kvc_retained_offsets(ctypes.byref(desc), b.ctypes.data_as(ctypes.c_void_p),
                                        off.ctypes.data_as(ctypes.c_void_p)))
    return off


def kvc_budgets_inverse_stability(s_stable, total: int) -> np.ndarray:
    st = np.ascontiguousarray(np.asarray(s_stable, dtype=np.float64))
    out = np.zeros(st.shape[0], dtype=np.int32)
    _check(_load().kvc_budgets_inverse_stability(st.ctypes.data_as(ctypes.c_void_p), st.shape[0],
                                                 int(total), out.ctypes.data_as(ctypes.c_void_p)))
    return out


# ------------------------------------------------------------------ device calls

def kvc_score_pass1(desc, q_win, k, m_out, z_out, ws):
    L = _load()
    _check(L.kvc_score_pass1(ctypes.byref(desc), _bf16_ptr(q_win, "q_win"), _bf16_ptr(k, "k"),
                             _dev_ptr(m_out, "m_out", 4), _dev_ptr(z_out, "z_out", 4),
                             _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def kvc_score_pass2(desc, q_win, k, m, z, scores):
    L = _load()
    _check(L.kvc_score_pass2(ctypes.byref(desc), _bf16_ptr(q_win, "q_win"), _bf16_ptr(k, "k"),
                             _dev_ptr(m, "m", 4), _dev_ptr(z, "z", 4),
                             _dev_ptr(scores, "scores", 4), _stream()))


def kvc_score_layer(desc, q_win, k, m_out, z_out, scores_out, ws):
    """Both scans as kvc_compress_layer runs them; m_out, z_out, scores_out may be None."""
    L = _load()
    _check(L.kvc_score_layer(ctypes.byref(desc), _bf16_ptr(q_win, "q_win"), _bf16_ptr(k, "k"),
                             _dev_ptr(m_out, "m_out", 4), _dev_ptr(z_out, "z_out", 4),
                             _dev_ptr(scores_out, "scores_out", 4),
                             _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def kvc_select_topk(desc, scores, budgets, idx_out, ws):
    L = _load()
    b = _host_i32(budgets, desc.hkv, "budgets")
    _check(L.kvc_select_topk(ctypes.byref(desc), _dev_ptr(scores, "scores", 4),
                             b.ctypes.data_as(ctypes.c_void_p), _dev_ptr(idx_out, "idx_out", 4),
                             _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def kvc_gather_retained(desc, k, v, idx, budgets, k_out, v_out, pos_out):
    L = _load()
    b = _host_i32(budgets, desc.hkv, "budgets")
    _check(L.kvc_gather_retained(ctypes.byref(desc), _bf16_ptr(k, "k"), _bf16_ptr(v, "v"),
                                 _dev_ptr(idx, "idx", 4), b.ctypes.data_as(ctypes.c_void_p),
                                 _bf16_ptr(k_out, "k_out"), _bf16_ptr(v_out, "v_out"),
                                 _dev_ptr(pos_out, "pos_out", 4), _stream()))


def kvc_compress_layer(desc, q_win, k, v, budgets, idx_out, k_out, v_out, pos_out, ws,
                       m_out=None, z_out=None, scores_out=None):
    L = _load()
    b = _host_i32(budgets, desc.hkv, "budgets")
    _check(L.kvc_compress_layer(ctypes.byref(desc), _bf16_ptr(q_win, "q_win"), _bf16_ptr(k, "k"),
                                _bf16_ptr(v, "v"), b.ctypes.data_as(ctypes.c_void_p),
                                _dev_ptr(m_out, "m_out", 4), _dev_ptr(z_out, "z_out", 4),
                                _dev_ptr(scores_out, "scores_out", 4),
                                _dev_ptr(idx_out, "idx_out", 4), _bf16_ptr(k_out, "k_out"),
                                _bf16_ptr(v_out, "v_out"), _dev_ptr(pos_out, "pos_out", 4),
                                _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def kvc_compress_layer_noalloc(desc, q_win, k, v, budgets, idx_out, k_out, v_out, pos_out,
                               m_out=None, z_out=None, scores_out=None):
    """kvc_compress_layer with the library's fixed per-device scratch as the
    workspace (no allocation anywhere)."""
    L = _load()
    b = _host_i32(budgets, desc.hkv, "budgets")
    _check(L.kvc_compress_layer_noalloc(ctypes.byref(desc), _bf16_ptr(q_win, "q_win"), _bf16_ptr(k, "k"),
                                        _bf16_ptr(v, "v"), b.ctypes.data_as(ctypes.c_void_p),
                                        _dev_ptr(m_out, "m_out", 4), _dev_ptr(z_out, "z_out", 4),
                                        _dev_ptr(scores_out, "scores_out", 4),
                                        _dev_ptr(idx_out, "idx_out", 4), _bf16_ptr(k_out, "k_out"),
                                        _bf16_ptr(v_out, "v_out"), _dev_ptr(pos_out, "pos_out", 4), _stream()))


def kvc_overlap_coefficient(desc, idx_a, idx_b, budgets, out):
    """Per-KV-head overlap coefficient of two packed retained index sets."""
    L = _load()
    b = _host_i32(budgets, desc.hkv, "budgets")
    _check(L.kvc_overlap_coefficient(ctypes.byref(desc), _dev_ptr(idx_a, "idx_a", 4), _dev_ptr(idx_b, "idx_b", 4),
                                     b.ctypes.data_as(ctypes.c_void_p), _dev_ptr(out, "out", 4), _stream()))


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = p.value
    return arr


def _sweep_args(desc, layers, budgets, outs, ws):
    """Marshalled arguments of kvc_compress_layers (without the stream)."""
    n = len(layers)
    if len(outs) != n:
        raise ValueError("one LayerOutputs per layer")
    b = np.ascontiguousarray(np.asarray(budgets, dtype=np.int64))
    if b.shape != (n, desc.hkv):
        raise ValueError(f"budgets must have shape ({n}, {desc.hkv})")
    if np.any(b < np.iinfo(np.int32).min) or np.any(b > np.iinfo(np.int32).max):
        raise ValueError("budgets do not fit in int32")
    b = np.ascontiguousarray(b.astype(np.int32))
    cols = [_ptr_array([_bf16_ptr(l[j], name) for l in layers]) for j, name in enumerate(("q_win", "k", "v"))]
    idx = _ptr_array([_dev_ptr(o.idx, "idx", 4) for o in outs])
    kh = _ptr_array([_bf16_ptr(o.k_hat, "k_hat") for o in outs])
    vh = _ptr_array([_bf16_ptr(o.v_hat, "v_hat") for o in outs])
    pos = _ptr_array([_dev_ptr(o.pos, "pos", 4) for o in outs])
    keep = (layers, outs, ws, b, cols, idx, kh, vh, pos)
    args = (ctypes.byref(desc), n, cols[0], cols[1], cols[2], b.ctypes.data_as(ctypes.c_void_p),
            idx, kh, vh, pos, _dev_ptr(ws, "ws"), ws.numel() * ws.element_size())
    return args, keep


def _stream_handle(s):
    """A torch stream, a raw handle or None as a ctypes pointer (None: NULL)."""
    if s is None:
        return None
    return ctypes.c_void_p(s.cuda_stream if hasattr(s, "cuda_stream") else int(s))


def kvc_compress_layers(desc, layers, budgets, outs, ws, aux_stream=None):
    """layers: sequence of (q_win, k, v) tensors of one shape; budgets:
    [n_layers][hkv]; outs: one LayerOutputs per layer; ws: sweep workspace
    (alloc_sweep_workspace); aux_stream: the caller's second stream (a
    torch.cuda.Stream) or None (every layer on the current stream)."""
    args, _keep = _sweep_args(desc, layers, budgets, outs, ws)
    _check(_load().kvc_compress_layers(*args, _stream(), _stream_handle(aux_stream)))


# ------------------------------------------------------------------ immediate eviction

def kvc_chunk_workspace_size(desc: LayerDesc, cap: int) -> int:
    n = _load().kvc_chunk_workspace_size(ctypes.byref(desc), int(cap))
    if n == 0:
        _check(KVC_ERR_INVALID_ARG)
    return n


def kvc_evict_chunk(desc, q_win, k_chunk, v_chunk, budget, n_kept, cap, cur, nxt, ws):
    """One chunk boundary. cur, nxt: (k, v, pos) arenas of `cap` rows per
    head (nxt and ws may be None when the boundary only appends)."""
    L = _load()
    nk, nv, npos = nxt if nxt is not None else (None, None, None)
    _check(L.kvc_evict_chunk(ctypes.byref(desc), _bf16_ptr(q_win, "q_win"), _bf16_ptr(k_chunk, "k_chunk"),
                             _bf16_ptr(v_chunk, "v_chunk"), int(budget), int(n_kept), int(cap),
                             _bf16_ptr(cur[0], "k_cur"), _bf16_ptr(cur[1], "v_cur"), _dev_ptr(cur[2], "pos_cur", 4),
                             _bf16_ptr(nk, "k_next"), _bf16_ptr(nv, "v_next"), _dev_ptr(npos, "pos_next", 4),
                             _dev_ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream()))


def kvc_chunked_workspace_size(desc: LayerDesc, chunk: int, budget: int) -> int:
    n = _load().kvc_chunked_workspace_size(ctypes.byref(desc), int(chunk), int(budget))
    if n == 0:
        _check(KVC_ERR_INVALID_ARG)
    return n


def kvc_compress_chunked(desc, chunk, q_windows, k, v, budget, k_out, v_out, pos_out, ws):
    """Immediate eviction over a resident prompt; q_windows [n_chunks * w, hq, D]."""
    L = _load()
    _check(L.kvc_compress_chunked(ctypes.byref(desc), int(chunk), _bf16_ptr(q_windows, "q_windows"),
                                  _bf16_ptr(k, "k"), _bf16_ptr(v, "v"), int(budget), _bf16_ptr(k_out, "k_out"),
                                  _bf16_ptr(v_out, "v_out"), _dev_ptr(pos_out, "pos_out", 4),
                                  _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def alloc_arena(hkv: int, cap: int, d: int, device="cuda"):
    """(K, V, positions) of an arena: bf16 [hkv, cap, d] twice, int32 [hkv, cap]."""
    import torch
    return (torch.empty((hkv, cap, d), dtype=torch.bfloat16, device=device),
            torch.empty((hkv, cap, d), dtype=torch.bfloat16, device=device),
            torch.empty((hkv, cap), dtype=torch.int32, device=device))


class PreparedChunked:
    """Pre-marshalled kvc_compress_chunked call over fixed buffers (the
    tensors must stay alive while this object is used)."""

    def __init__(self, desc, chunk, q_windows, k, v, budget, k_out, v_out, pos_out, ws):
        self._L = _load()
        self.desc = desc
        self._keep = (q_windows, k, v, k_out, v_out, pos_out, ws)
        self._args = (ctypes.byref(desc), int(chunk), _bf16_ptr(q_windows, "q_windows"), _bf16_ptr(k, "k"),
                      _bf16_ptr(v, "v"), int(budget), _bf16_ptr(k_out, "k_out"), _bf16_ptr(v_out, "v_out"),
                      _dev_ptr(pos_out, "pos_out", 4), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size())

    def kvc_compress_chunked(self, stream=None):
        st = ctypes.c_void_p(stream) if stream is not None else _stream()
        _check(self._L.kvc_compress_chunked(*self._args, st))


# ------------------------------------------------------------------ prefill layer pieces

def kvc_rmsnorm(x, w, y, eps=1e-5):
    """x, y [rows, dim] bf16 (y may be x); w [dim]."""
    rows, dim = x.shape
    _check(_load().kvc_rmsnorm(_bf16_ptr(x, "x"), _bf16_ptr(w, "w"), _bf16_ptr(y, "y"), rows, dim, eps, _stream()))


def kvc_rope_append(pdesc, qkv, c0, q_out, k_cache, v_cache):
    """qkv [n, (hq + 2 hkv) d]; q_out [n, hq, d]; caches [s, hkv, d]."""
    _check(_load().kvc_rope_append(ctypes.byref(pdesc), _bf16_ptr(qkv, "qkv"), int(c0), qkv.shape[0],
                                   _bf16_ptr(q_out, "q_out"), _bf16_ptr(k_cache, "k_cache"),
                                   _bf16_ptr(v_cache, "v_cache"), _stream()))


def kvc_chunk_attention(pdesc, q, k_cache, v_cache, c0, o_out):
    """q, o_out [n, hq, d] at positions c0 + t; caches [s, hkv, d]."""
    _check(_load().kvc_chunk_attention(ctypes.byref(pdesc), _bf16_ptr(q, "q"), _bf16_ptr(k_cache, "k_cache"),
                                       _bf16_ptr(v_cache, "v_cache"), int(c0), q.shape[0],
                                       _bf16_ptr(o_out, "o_out"), _stream()))


def kvc_swiglu(gu, a):
    """gu [rows, 2 ffn] -> a [rows, ffn]."""
    rows, two_f = gu.shape
    _check(_load().kvc_swiglu(_bf16_ptr(gu, "gu"), _bf16_ptr(a, "a"), rows, two_f // 2, _stream()))


# ------------------------------------------------------------------ convenience

@dataclass
class LayerOutputs:
    m: object
    z: object
    scores: object
    idx: object
    k_hat: object
    v_hat: object
    pos: object
    offsets: np.ndarray


def alloc_workspace(desc: LayerDesc, device="cuda"):
    import torch
    return torch.empty(kvc_workspace_size(desc), dtype=torch.uint8, device=device)


SWEEP_STREAMS = 2  # layers in flight in kvc_compress_layers


def alloc_sweep_workspace(desc: LayerDesc, device="cuda"):
    import torch
    return torch.empty(SWEEP_STREAMS * kvc_workspace_size(desc), dtype=torch.uint8, device=device)


def alloc_outputs(desc: LayerDesc, budgets, device="cuda", with_intermediates=True) -> LayerOutputs:
    import torch
    off = kvc_retained_offsets(desc, budgets)
    rows = int(off[-1])
    f32 = dict(dtype=torch.float32, device=device)
    return LayerOutputs(
        m=torch.empty((desc.hq, desc.w), **f32) if with_intermediates else None,
        z=torch.empty((desc.hq, desc.w), **f32) if with_intermediates else None,
        scores=torch.empty((desc.hkv, desc.s), **f32) if with_intermediates else None,
        idx=torch.empty(rows, dtype=torch.int32, device=device),
        k_hat=torch.empty((rows, desc.d), dtype=torch.bfloat16, device=device),
        v_hat=torch.empty((rows, desc.d), dtype=torch.bfloat16, device=device),
        pos=torch.empty(rows, dtype=torch.int32, device=device),
        offsets=off,
    )


def compress_layer(desc, q_win, k, v, budgets, out: LayerOutputs, ws):
    kvc_compress_layer(desc, q_win, k, v, budgets, out.idx, out.k_hat, out.v_hat, out.pos, ws,
                       m_out=out.m, z_out=out.z, scores_out=out.scores)
    return out


class PreparedLayer:
    """Pre-marshalled calls for one layer's buffers: the tensors are checked
    once, and each method is then a single C call on the given (or current)
    stream. The tensors must stay alive while this object is used."""

    def __init__(self, desc, q_win, k, v, budgets, out: LayerOutputs, ws):
        L = _load()
        self._L = L
        self.desc = desc
        self._d = ctypes.byref(desc)
        self._b = _host_i32(budgets, desc.hkv, "budgets")
        bp = self._b.ctypes.data_as(ctypes.c_void_p)
        self._keep = (q_win, k, v, out, ws)
        q, kk, vv = _bf16_ptr(q_win, "q_win"), _bf16_ptr(k, "k"), _bf16_ptr(v, "v")
        m, z, sc = (_dev_ptr(out.m, "m", 4), _dev_ptr(out.z, "z", 4),
                    _dev_ptr(out.scores, "scores", 4))
        idx, kh, vh, pos = (_dev_ptr(out.idx, "idx", 4), _bf16_ptr(out.k_hat, "k_hat"),
                            _bf16_ptr(out.v_hat, "v_hat"), _dev_ptr(out.pos, "pos", 4))
        w, wn = _dev_ptr(ws, "ws"), ws.numel() * ws.element_size()
        self._a1 = (self._d, q, kk, m, z, w, wn)
        self._a2 = (self._d, q, kk, m, z, sc)
        self._as = (self._d, q, kk, m, z, sc, w, wn)
        self._a3 = (self._d, sc, bp, idx, w, wn)
        self._a4 = (self._d, kk, vv, idx, bp, kh, vh, pos)
        self._af = (self._d, q, kk, vv, bp, m, z, sc, idx, kh, vh, pos, w, wn)

    @staticmethod
    def _s(stream):
        return ctypes.c_void_p(stream) if stream is not None else _stream()

    def kvc_score_pass1(self, stream=None):
        _check(self._L.kvc_score_pass1(*self._a1, self._s(stream)))

    def kvc_score_pass2(self, stream=None):
        _check(self._L.kvc_score_pass2(*self._a2, self._s(stream)))

    def kvc_score_layer(self, stream=None):
        _check(self._L.kvc_score_layer(*self._as, self._s(stream)))

    def kvc_select_topk(self, stream=None):
        _check(self._L.kvc_select_topk(*self._a3, self._s(stream)))

    def kvc_gather_retained(self, stream=None):
        _check(self._L.kvc_gather_retained(*self._a4, self._s(stream)))

    def kvc_compress_layer(self, stream=None):
        _check(self._L.kvc_compress_layer(*self._af, self._s(stream)))


class PreparedSweep:
    """Pre-marshalled kvc_compress_layers call over fixed buffers (the tensors
    must stay alive while this object is used)."""

    def __init__(self, desc, layers, budgets, outs, ws):
        self._L = _load()
        self.desc = desc
        self.n_layers = len(layers)
        self._args, self._keep = _sweep_args(desc, layers, budgets, outs, ws)

    def kvc_compress_layers(self, stream=None, aux_stream=None):
        st = ctypes.c_void_p(stream) if stream is not None else _stream()
        _check(self._L.kvc_compress_layers(*self._args, st, _stream_handle(aux_stream)))
