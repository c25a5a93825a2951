"""Thin Python binding of the GQA -> SAGA key-head merge (include/saga_merge.h).

Argument marshalling only; every step runs in the HIP library (libsaga.so),
and this module raises if that library is missing.
"""
from __future__ import annotations

import ctypes

import torch

from .saga import _check, _ptr, _stream, lib


def saga_merge_workspace_bytes(n: int, h_q: int, h_kt: int, d: int, d_model: int) -> int:
    return int(lib().saga_merge_workspace_bytes(n, h_q, h_kt, d, d_model))


def saga_merge_key_heads(X, Q, W_K, h_kt: int, W_merged, pairs, pair_loss, total_loss, ws,
                         pairs_in=None, stream=None) -> None:
    """X bf16 [n][d_model], Q bf16 [n][h_q][d], W_K bf16 [h_kt*d][d_model] (device);
    outputs W_merged fp32 [h_kt/2*d][d_model], pairs int32 [h_kt/2][2],
    pair_loss fp64 [h_kt][h_kt], total_loss fp64 [1]; pairs_in: optional host
    sequence of h_kt/2 pairs that replaces the optimal matching."""
    n, d_model = X.shape
    _, h_q, d = Q.shape
    if Q.shape[0] != n or tuple(W_K.shape) != (h_kt * d, d_model):
        raise ValueError("inconsistent shapes for X, Q and W_K")
    for t in (X, Q, W_K):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("X, Q and W_K must be contiguous bf16 tensors")
    pin = None
    if pairs_in is not None:
        flat = [int(x) for p in pairs_in for x in p]
        pin = (ctypes.c_int32 * len(flat))(*flat)
        if len(flat) != h_kt:
            raise ValueError("pairs_in must list h_kt/2 pairs")
    _check(lib().saga_merge_key_heads(_ptr(X), _ptr(Q), _ptr(W_K), n, h_q, h_kt, d, d_model, pin,
                                      _ptr(W_merged), _ptr(pairs), _ptr(pair_loss),
                                      _ptr(total_loss), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "saga_merge_key_heads")


class KeyMerge:
    """Owns the outputs and the workspace of one merge shape."""

    def __init__(self, n: int, h_q: int, h_kt: int, d: int, d_model: int, device="cuda"):
        self.shape = (n, h_q, h_kt, d, d_model)
        nbytes = saga_merge_workspace_bytes(n, h_q, h_kt, d, d_model)
        if nbytes == 0:
            raise ValueError(f"unsupported merge shape {self.shape}")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.W_merged = torch.empty(h_kt // 2 * d, d_model, dtype=torch.float32, device=device)
        self.pairs = torch.empty(h_kt // 2, 2, dtype=torch.int32, device=device)
        self.pair_loss = torch.empty(h_kt, h_kt, dtype=torch.float64, device=device)
        self.total_loss = torch.empty(1, dtype=torch.float64, device=device)

    def __call__(self, X, Q, W_K, pairs_in=None, stream=None):
        saga_merge_key_heads(X, Q, W_K, self.shape[2], self.W_merged, self.pairs, self.pair_loss,
                             self.total_loss, self.ws, pairs_in=pairs_in, stream=stream)
        return self
