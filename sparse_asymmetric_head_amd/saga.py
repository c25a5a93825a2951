"""Thin Python binding of the SAGA C ABI (include/saga.h).

Argument marshalling only: shapes are read off torch tensors, device pointers
and the current HIP stream are passed through ctypes, status codes become
exceptions.  Every step of the computation runs in the HIP library
(``lib/libsaga.so``); if that library is missing this module raises -- there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libsaga.so")

SAGA_OK = 0
SAGA_ERR_INVALID_ARG = -1
SAGA_ERR_UNSUPPORTED = -2
SAGA_ERR_WORKSPACE = -3
SAGA_ERR_HIP = -4

EXPORTS = (
    "saga_status_string", "saga_version", "saga_workspace_bytes", "saga_dense_workspace_bytes",
    "saga_workspace_init", "saga_refresh_threshold", "saga_decode_step",
    "saga_dense_gqa_baseline", "saga_workspace_layout", "saga_selection_mask", "saga_select",
    "saga_attend", "saga_read_probe", "saga_decode_step_pivot", "saga_full_attention",
    "saga_full_attention_workspace_bytes", "saga_cache_workspace_bytes", "saga_append_kv",
    "saga_decode_step_cache", "saga_merge_workspace_bytes", "saga_merge_key_heads",
    "saga_decode_step_noalloc", "saga_read_probe_shape",
)
STATIC_WORKSPACE_BYTES = 128 << 20  # SAGA_STATIC_WORKSPACE_BYTES
PROBE_SINK_WORDS = 256  # SAGA_PROBE_SINK_WORDS


class SagaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class WsLayout(ctypes.Structure):
    _fields_ = [
        ("bytes", ctypes.c_size_t),
        ("scores_off", ctypes.c_size_t),
        ("scores_ld", ctypes.c_int64),
        ("seg_off", ctypes.c_size_t),
        ("seg_words", ctypes.c_int64),
        ("chunk_len", ctypes.c_int64),
        ("n_chunk", ctypes.c_int64),
        ("n_seg", ctypes.c_int64),
        ("seg_cap", ctypes.c_int64),
        ("seg_group", ctypes.c_int64),
    ]


_lib = None


def lib(path: str | None = None):
    """Load libsaga.so (raises FileNotFoundError when it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} not found: build it with `python -m sparse_asymmetric_head_amd.build`")
    L = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.saga_status_string.argtypes = [i32]
    L.saga_status_string.restype = ctypes.c_char_p
    L.saga_version.restype = i32
    L.saga_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i64, i64]
    L.saga_workspace_bytes.restype = sz
    L.saga_dense_workspace_bytes.argtypes = [i32, i32, i32, i32, i64]
    L.saga_dense_workspace_bytes.restype = sz
    L.saga_workspace_init.argtypes = [vp, sz, vp]
    L.saga_workspace_init.restype = i32
    L.saga_refresh_threshold.argtypes = [vp, vp, i32, i32, i32, i32, i64, i64, vp, vp, sz, vp]
    L.saga_refresh_threshold.restype = i32
    L.saga_decode_step.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, i64, vp, i32, vp,
                                   vp, vp, sz, vp]
    L.saga_decode_step.restype = i32
    L.saga_decode_step_pivot.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, i64, vp, vp,
                                         i32, vp, vp, vp, sz, vp]
    L.saga_decode_step_pivot.restype = i32
    L.saga_select.argtypes = [vp, vp, i32, i32, i32, i32, i32, i64, i64, vp, i32, vp, sz, vp]
    L.saga_select.restype = i32
    L.saga_attend.argtypes = [vp, i32, i32, i32, i32, i32, i64, i64, vp, vp, vp, sz, vp]
    L.saga_attend.restype = i32
    L.saga_dense_gqa_baseline.argtypes = [vp, vp, vp, i32, i32, i32, i32, i64, vp, vp, sz, vp]
    L.saga_dense_gqa_baseline.restype = i32
    L.saga_workspace_layout.argtypes = [i32, i32, i32, i32, i32, i64, i64,
                                        ctypes.POINTER(WsLayout)]
    L.saga_workspace_layout.restype = i32
    L.saga_selection_mask.argtypes = [vp, sz, i32, i32, i32, i32, i32, i64, i64, vp, vp]
    L.saga_selection_mask.restype = i32
    L.saga_full_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i64]
    L.saga_full_attention_workspace_bytes.restype = sz
    L.saga_full_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, vp, vp, sz, vp]
    L.saga_full_attention.restype = i32
    L.saga_cache_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i64, i64]
    L.saga_cache_workspace_bytes.restype = sz
    L.saga_append_kv.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, vp]
    L.saga_append_kv.restype = i32
    L.saga_decode_step_cache.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, i64, i64, vp,
                                         vp, i32, vp, vp, vp, sz, vp]
    L.saga_decode_step_cache.restype = i32
    L.saga_decode_step_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i64, i64, vp,
                                           vp, i32, vp, vp, vp]
    L.saga_decode_step_noalloc.restype = i32
    L.saga_read_probe_shape.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp]
    L.saga_read_probe_shape.restype = i32
    L.saga_read_probe.argtypes = [vp, i64, vp, vp]
    L.saga_read_probe.restype = i32
    L.saga_merge_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    L.saga_merge_workspace_bytes.restype = sz
    L.saga_merge_key_heads.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32,
                                       ctypes.POINTER(ctypes.c_int32), vp, vp, vp, vp, vp, sz, vp]
    L.saga_merge_key_heads.restype = i32
    if path is None:
        _lib = L
    return L


def status_string(status: int) -> str:
    return lib().saga_status_string(int(status)).decode()


def _check(st: int, where: str) -> None:
    if st != SAGA_OK:
        raise SagaError(st, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ----------------------------------------------------------------- workspace

def saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N) -> int:
    return int(lib().saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N))


def saga_dense_workspace_bytes(B, h_q, h_kv, d, l_kv) -> int:
    return int(lib().saga_dense_workspace_bytes(B, h_q, h_kv, d, l_kv))


def saga_workspace_layout(B, h_q, h_k, h_v, d, l_kv, N) -> WsLayout:
    out = WsLayout()
    _check(lib().saga_workspace_layout(B, h_q, h_k, h_v, d, l_kv, N, ctypes.byref(out)),
           "saga_workspace_layout")
    return out


def saga_workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check(lib().saga_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "saga_workspace_init")


def alloc_workspace(nbytes: int, device="cuda", stream=None) -> torch.Tensor:
    """A device byte buffer of nbytes (rounded up to 256), initialised for use."""
    n = (int(nbytes) + 255) // 256 * 256
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    saga_workspace_init(ws, stream)
    return ws


def _dims(Q, K, V=None):
    if Q.dtype != torch.bfloat16 or K.dtype != torch.bfloat16:
        raise TypeError("Q and K must be bfloat16")
    if Q.dim() != 3 or K.dim() != 4:
        raise ValueError("Q must be [B][h_q][d] and K [B][h_k][l_kv][d]")
    B, h_q, d = Q.shape
    if K.shape[0] != B or K.shape[3] != d:
        raise ValueError("Q and K disagree on B or d")
    if V is not None:
        if V.dtype != torch.bfloat16 or V.dim() != 4:
            raise TypeError("V must be bfloat16 [B][h_v][l_kv][d]")
        if V.shape[0] != B or V.shape[2] != K.shape[2] or V.shape[3] != d:
            raise ValueError("V disagrees with K")
    for t in (Q, K, V):
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return B, h_q, d


def _arr(t, dtype, shape, name, optional=False):
    """Check a per-row tensor the library reads or writes (tau, O, counts, pivot):
    the C ABI trusts its size, so a short or mistyped buffer is refused here."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{name} must be a contiguous device tensor")


def _ws(ws):
    if ws is None:
        raise ValueError("a workspace is required (alloc_workspace)")
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise TypeError("the workspace must be a contiguous 1-D uint8 device tensor")


# ----------------------------------------------------------------- entry points

def saga_refresh_threshold(Q, K, N: int, tau, ws, stream=None) -> None:
    B, h_q, d = _dims(Q, K)
    h_k, l_kv = K.shape[1], K.shape[2]
    _arr(tau, torch.float32, (B, h_q), "tau")
    _ws(ws)
    _check(lib().saga_refresh_threshold(_ptr(Q), _ptr(K), B, h_q, h_k, d, l_kv, int(N),
                                        _ptr(tau), _ptr(ws), ws.numel(), _stream(stream)),
           "saga_refresh_threshold")


def saga_decode_step(Q, K, V, N: int, tau, refresh: bool, O, counts=None, ws=None,
                     stream=None) -> None:
    B, h_q, d = _dims(Q, K, V)
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    _arr(tau, torch.float32, (B, h_q), "tau")
    _arr(O, torch.float32, (B, h_q, d), "O")
    _arr(counts, torch.int32, (B, h_q), "counts", optional=True)
    _ws(ws)
    _check(lib().saga_decode_step(_ptr(Q), _ptr(K), _ptr(V), B, h_q, h_k, h_v, d, l_kv, int(N),
                                  _ptr(tau), 1 if refresh else 0, _ptr(O), _ptr(counts),
                                  _ptr(ws), ws.numel(), _stream(stream)),
           "saga_decode_step")


def saga_decode_step_pivot(Q, K, V, N: int, tau, pivot, refresh: int, O, counts=None, ws=None,
                           stream=None) -> None:
    """refresh: 0 compare with tau, 1 exact refresh (records the pivot), 2 exact
    refresh from the pivot; pivot is an int32 [B][h_q][N] tensor."""
    B, h_q, d = _dims(Q, K, V)
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    _arr(tau, torch.float32, (B, h_q), "tau")
    _arr(pivot, torch.int32, (B, h_q, int(N)), "pivot", optional=int(refresh) == 0)
    _arr(O, torch.float32, (B, h_q, d), "O")
    _arr(counts, torch.int32, (B, h_q), "counts", optional=True)
    _ws(ws)
    _check(lib().saga_decode_step_pivot(_ptr(Q), _ptr(K), _ptr(V), B, h_q, h_k, h_v, d, l_kv,
                                        int(N), _ptr(tau), _ptr(pivot), int(refresh), _ptr(O),
                                        _ptr(counts), _ptr(ws), ws.numel(), _stream(stream)),
           "saga_decode_step_pivot")


def saga_decode_step_noalloc(Q, K, V, N: int, tau, pivot, refresh: int, O, counts=None,
                             stream=None) -> None:
    """saga_decode_step_pivot on the library's static per-GPU workspace (no workspace
    argument; the call allocates nothing).  Calls on one GPU must not overlap."""
    B, h_q, d = _dims(Q, K, V)
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    _arr(tau, torch.float32, (B, h_q), "tau")
    _arr(pivot, torch.int32, (B, h_q, int(N)), "pivot", optional=int(refresh) == 0)
    _arr(O, torch.float32, (B, h_q, d), "O")
    _arr(counts, torch.int32, (B, h_q), "counts", optional=True)
    _check(lib().saga_decode_step_noalloc(_ptr(Q), _ptr(K), _ptr(V), B, h_q, h_k, h_v, d, l_kv,
                                          int(N), _ptr(tau), _ptr(pivot), int(refresh), _ptr(O),
                                          _ptr(counts), _stream(stream)),
           "saga_decode_step_noalloc")


def saga_select(Q, K, h_v: int, N: int, tau, refresh: bool, ws, stream=None) -> None:
    B, h_q, d = _dims(Q, K)
    h_k, l_kv = K.shape[1], K.shape[2]
    _arr(tau, torch.float32, (B, h_q), "tau")
    _ws(ws)
    _check(lib().saga_select(_ptr(Q), _ptr(K), B, h_q, h_k, int(h_v), d, l_kv, int(N), _ptr(tau),
                             1 if refresh else 0, _ptr(ws), ws.numel(), _stream(stream)),
           "saga_select")


def saga_attend(V, B: int, h_q: int, h_k: int, N: int, O, counts, ws, stream=None) -> None:
    if V.dtype != torch.bfloat16 or V.dim() != 4 or not V.is_contiguous():
        raise TypeError("V must be contiguous bfloat16 [B][h_v][l_kv][d]")
    h_v, l_kv, d = V.shape[1], V.shape[2], V.shape[3]
    _arr(O, torch.float32, (B, h_q, d), "O")
    _arr(counts, torch.int32, (B, h_q), "counts", optional=True)
    _ws(ws)
    _check(lib().saga_attend(_ptr(V), int(B), int(h_q), int(h_k), h_v, d, l_kv, int(N), _ptr(O),
                             _ptr(counts), _ptr(ws), ws.numel(), _stream(stream)),
           "saga_attend")


def saga_dense_gqa_baseline(Q, K, V, O, ws, stream=None) -> None:
    B, h_q, d = _dims(Q, K, V)
    h_kv, l_kv = K.shape[1], K.shape[2]
    _arr(O, torch.float32, (B, h_q, d), "O")
    _ws(ws)
    _check(lib().saga_dense_gqa_baseline(_ptr(Q), _ptr(K), _ptr(V), B, h_q, h_kv, d, l_kv,
                                         _ptr(O), _ptr(ws), ws.numel(), _stream(stream)),
           "saga_dense_gqa_baseline")


def saga_selection_mask(ws, B, h_q, h_k, h_v, d, l_kv, N, mask, stream=None) -> None:
    _ws(ws)
    if mask.dtype != torch.uint8 or mask.numel() < B * h_q * l_kv or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous uint8 tensor of B*h_q*l_kv bytes")
    _check(lib().saga_selection_mask(_ptr(ws), ws.numel(), B, h_q, h_k, h_v, d, l_kv, int(N),
                                     _ptr(mask), _stream(stream)),
           "saga_selection_mask")


def saga_full_attention_workspace_bytes(B, h_q, h_k, h_v, d, l_kv) -> int:
    return int(lib().saga_full_attention_workspace_bytes(B, h_q, h_k, h_v, d, l_kv))


def saga_full_attention(Q, K, V, O, ws, stream=None) -> None:
    """Dense attention with decoupled heads: key head floor(j*h_k/h_q), value
    head floor(j*h_v/h_q); Q [B][h_q][d], K [B][h_k][l_kv][d], V [B][h_v][l_kv][d]."""
    B, h_q, d = _dims(Q, K, V)
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    _arr(O, torch.float32, (B, h_q, d), "O")
    _ws(ws)
    _check(lib().saga_full_attention(_ptr(Q), _ptr(K), _ptr(V), B, h_q, h_k, h_v, d, l_kv,
                                     _ptr(O), _ptr(ws), ws.numel(), _stream(stream)),
           "saga_full_attention")


def saga_cache_workspace_bytes(B, h_q, h_k, h_v, d, cap, N) -> int:
    return int(lib().saga_cache_workspace_bytes(B, h_q, h_k, h_v, d, cap, int(N)))


def saga_append_kv(K, V, k_new, v_new, pos: int, stream=None) -> None:
    """K [B][h_k][cap][d], V [B][h_v][cap][d]; k_new [B][h_k][d], v_new [B][h_v][d] (bf16)."""
    B, h_k, cap, d = K.shape
    h_v = V.shape[1]
    for t in (K, V, k_new, v_new):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError("caches and new rows must be contiguous bfloat16")
    if tuple(V.shape) != (B, h_v, cap, d) or tuple(k_new.shape) != (B, h_k, d) or \
            tuple(v_new.shape) != (B, h_v, d):
        raise ValueError("k_new must be [B][h_k][d] and v_new [B][h_v][d] for caches "
                         "[B][h][cap][d]")
    _check(lib().saga_append_kv(_ptr(K), _ptr(V), _ptr(k_new), _ptr(v_new), B, h_k, h_v, d, cap,
                                int(pos), _stream(stream)), "saga_append_kv")


def saga_decode_step_cache(Q, K, V, length: int, N: int, tau, pivot, refresh: int, O,
                           counts=None, ws=None, stream=None) -> None:
    """saga_decode_step_pivot over the first `length` rows of caches with room for
    K.shape[2] rows per head."""
    B, h_q, d = _dims(Q, K, V)
    h_k, cap, h_v = K.shape[1], K.shape[2], V.shape[1]
    _arr(tau, torch.float32, (B, h_q), "tau")
    _arr(pivot, torch.int32, (B, h_q, int(N)), "pivot", optional=int(refresh) == 0)
    _arr(O, torch.float32, (B, h_q, d), "O")
    _arr(counts, torch.int32, (B, h_q), "counts", optional=True)
    _ws(ws)
    _check(lib().saga_decode_step_cache(_ptr(Q), _ptr(K), _ptr(V), B, h_q, h_k, h_v, d, cap,
                                        int(length), int(N), _ptr(tau), _ptr(pivot), int(refresh),
                                        _ptr(O), _ptr(counts), _ptr(ws), ws.numel(),
                                        _stream(stream)), "saga_decode_step_cache")


def saga_read_probe(buf, sink, stream=None) -> None:
    """Measurement utility: stream-read buf once (the achievable-read reference);
    sink (uint32/int32, PROBE_SINK_WORDS entries) receives per-workgroup XOR folds."""
    assert sink.numel() >= PROBE_SINK_WORDS and sink.element_size() == 4
    _check(lib().saga_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 _stream(stream)), "saga_read_probe")


def saga_read_probe_shape(buf, sink, blocks: int, waves: int, loads: int, chunked: bool,
                          stream=None) -> None:
    """Measurement utility: the plain read with a chosen launch shape; sink (32-bit,
    PROBE_SINK_WORDS entries, cleared first) receives XOR folds (XOR of all = XOR of buf)."""
    assert sink.numel() >= PROBE_SINK_WORDS and sink.element_size() == 4
    _check(lib().saga_read_probe_shape(_ptr(buf), buf.numel() * buf.element_size(), int(blocks),
                                       int(waves), int(loads), 1 if chunked else 0, _ptr(sink),
                                       _stream(stream)), "saga_read_probe_shape")


# ----------------------------------------------------------------- conveniences

class Decoder:
    """Holds a workspace and the per-row threshold for one (shape, N) and runs
    Atop-N decode steps with a refresh every R calls (the first call refreshes)."""

    def __init__(self, B, h_q, h_k, h_v, d, l_kv, N, R, device="cuda"):
        self.shape = (B, h_q, h_k, h_v, d, l_kv)
        self.N, self.R, self.t = int(N), int(R), 0
        self.ws = alloc_workspace(saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N), device)
        self.tau = torch.zeros(B, h_q, dtype=torch.float32, device=device)
        self.O = torch.empty(B, h_q, d, dtype=torch.float32, device=device)
        self.counts = torch.empty(B, h_q, dtype=torch.int32, device=device)

    def step(self, Q, K, V, stream=None):
        refresh = (self.t % self.R) == 0
        saga_decode_step(Q, K, V, self.N, self.tau, refresh, self.O, self.counts, self.ws, stream)
        self.t += 1
        return self.O
