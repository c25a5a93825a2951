"""fp64 CPU oracle for SAGA + Atop-N decode attention -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never does, and this package imports nothing from it.

The arithmetic lives in ``saga_oracle.c`` (plain C, double precision, libm),
compiled by ``oracle/build.py`` into ``oracle/libsaga_oracle.so``.  This module
only marshals numpy arrays into that library.  Inputs are raw bf16 bit
patterns (``uint16``) so the oracle consumes exactly the tensors the GPU sees.

Source of every definition: "More Value per Key: Asymmetric Sparse Attention
for Faster LLM Decoding" (picx.dev summary): eqs. 2-4 (scores, softmax, PV),
eq. 6 (top-N indices), Methodology > Atop-N Attention items 1-2 and eq. 7
(threshold compare, periodic exact refresh, sparse softmax-PV), SAGA
Architecture (separate key and value head counts); the growing cache of the
decode loop from Introduction > Background (cached keys and values reused).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsaga_oracle.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")


def load(path: str | None = None):
    """Load (building first if absent) the compiled oracle library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(p)
    i64, i32, dbl, flt = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float
    lib.sao_num_threads.restype = i32
    lib.sao_set_num_threads.argtypes = [i32]
    lib.sao_scores_row.argtypes = [_u16p, _u16p, i32, i64, _f64p]
    lib.sao_scores.argtypes = [_u16p, _u16p, i32, i32, i32, i32, i64, _f64p]
    lib.sao_nth_largest.argtypes = [_f64p, i64, i64]
    lib.sao_nth_largest.restype = dbl
    lib.sao_nth_largest_f32.argtypes = [_f32p, i64, i64]
    lib.sao_nth_largest_f32.restype = flt
    lib.sao_attend_row.argtypes = [_f64p, _u8p, _u16p, i32, i64, _f64p]
    lib.sao_attend_row.restype = i64
    lib.sao_select_row.argtypes = [_f64p, i64, dbl, _u8p]
    lib.sao_select_row.restype = i64
    lib.sao_trajectory.argtypes = [_u16p, _u16p, _u16p, i32, i32, i32, i32, i32, i32, i64, i64,
                                   i32, _f64p, _f64p, _i64p, ctypes.c_void_p]
    lib.sao_trajectory.restype = i32
    lib.sao_trajectory_growing.argtypes = [_u16p, _u16p, _u16p, i32, i32, i32, i32, i32, i32,
                                           i64, i64, i64, i32, _f64p, _f64p, _i64p,
                                           ctypes.c_void_p]
    lib.sao_trajectory_growing.restype = i32
    lib.sao_given_mask.argtypes = [_u16p, _u16p, _u16p, i32, i32, i32, i32, i32, i64, _u8p,
                                   _f64p, _i64p]
    lib.sao_given_mask.restype = i32
    lib.sao_dense.argtypes = [_u16p, _u16p, _u16p, i32, i32, i32, i32, i64, _f64p]
    lib.sao_dense.restype = i32
    if path is None:
        _lib = lib
    return lib


def _u16(x) -> np.ndarray:
    """Accept a numpy uint16/int16 array or a torch bf16 tensor; return uint16 bits."""
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch

        x = x.detach().to("cpu").contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(x)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns (uint16), got {a.dtype}")
    return a


def bf16_bits_to_f64(x) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    a = _u16(x)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def num_threads(lib=None) -> int:
    return (lib or load()).sao_num_threads()


def set_num_threads(n: int, lib=None) -> None:
    (lib or load()).sao_set_num_threads(int(n))


def scores(Q, K, h_k: int, lib=None) -> np.ndarray:
    """A[b][j][t] = <q_{b,j}, k_{b,kh(j),t}> / sqrt(d) in fp64 (eq. 2).
    Q: [B][h_q][d] bf16 bits; K: [B][h_k][l_kv][d] bf16 bits."""
    lib = lib or load()
    Q, K = _u16(Q), _u16(K)
    B, h_q, d = Q.shape
    l_kv = K.shape[2]
    assert K.shape == (B, h_k, l_kv, d)
    A = np.empty((B, h_q, l_kv), np.float64)
    lib.sao_scores(Q, K, B, h_q, h_k, d, l_kv, A)
    return A


def nth_largest(row, N: int, lib=None) -> float:
    """The N-th largest entry of a 1-D row by full descending sort (eq. 6)."""
    lib = lib or load()
    r = np.ascontiguousarray(row)
    if r.dtype == np.float32:
        return float(lib.sao_nth_largest_f32(r, r.size, int(N)))
    r = r.astype(np.float64)
    return float(lib.sao_nth_largest(r, r.size, int(N)))


def nth_largest_f32(row, N: int, lib=None) -> np.float32:
    lib = lib or load()
    r = np.ascontiguousarray(row, dtype=np.float32)
    return np.float32(lib.sao_nth_largest_f32(r, r.size, int(N)))


def attend_row(a, mask, Vhead, lib=None):
    """softmax(a[S]) V[S] for one row (eq. 7). Returns (o[d], |S|)."""
    lib = lib or load()
    a = np.ascontiguousarray(a, dtype=np.float64)
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    V = _u16(Vhead)
    l_kv, d = V.shape
    o = np.empty(d, np.float64)
    cnt = lib.sao_attend_row(a, m, V, d, l_kv, o)
    return o, int(cnt)


def trajectory(Q, K, V, h_k: int, h_v: int, N: int, R: int, want_mask: bool = False, lib=None):
    """Run T Atop-N decode steps with a static cache.

    Q: [T][B][h_q][d], K: [B][h_k][l_kv][d], V: [B][h_v][l_kv][d] (bf16 bits).
    Returns dict(O [T][B][h_q][d] f64, tau [T][B][h_q] f64, count [T][B][h_q] i64,
    mask [T][B][h_q][l_kv] u8 or None)."""
    lib = lib or load()
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    T, B, h_q, d = Q.shape
    l_kv = K.shape[2]
    assert K.shape == (B, h_k, l_kv, d) and V.shape == (B, h_v, l_kv, d)
    O = np.empty((T, B, h_q, d), np.float64)
    tau = np.empty((T, B, h_q), np.float64)
    cnt = np.empty((T, B, h_q), np.int64)
    mask = np.empty((T, B, h_q, l_kv), np.uint8) if want_mask else None
    rc = lib.sao_trajectory(Q, K, V, T, B, h_q, h_k, h_v, d, l_kv, int(N), int(R), O, tau, cnt,
                            mask.ctypes.data if mask is not None else None)
    if rc != 0:
        raise ValueError("oracle trajectory rejected its arguments")
    return {"O": O, "tau": tau, "count": cnt, "mask": mask}


def trajectory_growing(Q, K, V, h_k: int, h_v: int, l0: int, N: int, R: int,
                       want_mask: bool = False, lib=None):
    """Run T Atop-N decode steps over a growing cache: step t appends the row
    at position l0 + t and attends over the first l0 + t + 1 rows.

    Q: [T][B][h_q][d]; K: [B][h_k][cap][d], V: [B][h_v][cap][d] (bf16 bits),
    rows 0 .. l0 + T - 1 used.  Returns dict(O, tau, count, mask [T][B][h_q][cap]
    or None) as trajectory()."""
    lib = lib or load()
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    T, B, h_q, d = Q.shape
    cap = K.shape[2]
    assert K.shape == (B, h_k, cap, d) and V.shape == (B, h_v, cap, d)
    O = np.empty((T, B, h_q, d), np.float64)
    tau = np.empty((T, B, h_q), np.float64)
    cnt = np.empty((T, B, h_q), np.int64)
    mask = np.empty((T, B, h_q, cap), np.uint8) if want_mask else None
    rc = lib.sao_trajectory_growing(Q, K, V, T, B, h_q, h_k, h_v, d, cap, int(l0), int(N), int(R),
                                    O, tau, cnt, mask.ctypes.data if mask is not None else None)
    if rc != 0:
        raise ValueError("oracle growing trajectory rejected its arguments")
    return {"O": O, "tau": tau, "count": cnt, "mask": mask}


def given_mask(Q, K, V, h_k: int, h_v: int, mask, lib=None):
    """One decode step with an externally chosen selection S = mask (eq. 7).
    Q: [B][h_q][d]; mask: [B][h_q][l_kv] (nonzero = selected)."""
    lib = lib or load()
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    B, h_q, d = Q.shape
    l_kv = K.shape[2]
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    assert m.shape == (B, h_q, l_kv)
    O = np.empty((B, h_q, d), np.float64)
    cnt = np.empty((B, h_q), np.int64)
    if lib.sao_given_mask(Q, K, V, B, h_q, h_k, h_v, d, l_kv, m, O, cnt) != 0:
        raise ValueError("oracle given-mask rejected its arguments")
    return O, cnt


def dense(Q, K, V, lib=None) -> np.ndarray:
    """Dense GQA decode (eqs. 2-4) with h_kv shared key/value heads."""
    lib = lib or load()
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    B, h_q, d = Q.shape
    h_kv, l_kv = K.shape[1], K.shape[2]
    O = np.empty((B, h_q, d), np.float64)
    if lib.sao_dense(Q, K, V, B, h_q, h_kv, d, l_kv, O) != 0:
        raise ValueError("oracle dense rejected its arguments")
    return O
