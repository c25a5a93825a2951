"""Shared machinery of the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle under the acceptance rules:

  * tau (refresh steps): bit-identical to element N-1 of a CPU descending sort
    of the GPU's own fp32 score row;
  * selection: the GPU set S may differ from the oracle's only at entries with
    |A - tau| <= 1e-4 (A, tau the oracle's fp64 values);
  * output: max over rows of ||O_gpu - O_ref||_inf / ||O_ref||_inf <= 2e-3, with
    O_ref the oracle run on the GPU's own S (given-mask mode), and also against
    the oracle's own trajectory output wherever the two sets agree;
  * counts: exactly |S_gpu|.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_asymmetric_head_amd import saga

SEL_BAND = 1e-4
OUT_RTOL = 2e-3


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    saga.lib()  # raises if the HIP library is missing


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def read_scores(ws: torch.Tensor, shape, N) -> np.ndarray:
    B, h_q, h_k, h_v, d, l_kv = shape
    lay = saga.saga_workspace_layout(B, h_q, h_k, h_v, d, l_kv, N)
    rows = B * h_q
    n = rows * lay.scores_ld * 4
    raw = ws[lay.scores_off:lay.scores_off + n].view(torch.float32)
    return raw.reshape(rows, lay.scores_ld)[:, :l_kv].cpu().numpy()


def read_mask(ws: torch.Tensor, shape, N) -> np.ndarray:
    B, h_q, h_k, h_v, d, l_kv = shape
    m = torch.empty(B * h_q * l_kv, dtype=torch.uint8, device=ws.device)
    saga.saga_selection_mask(ws, B, h_q, h_k, h_v, d, l_kv, N, m)
    return m.reshape(B, h_q, l_kv).cpu().numpy()


def run_gpu_trajectory(Q, K, V, N, R, mask_steps=None, score_steps=None):
    """Q [T][B][h_q][d], K, V on the GPU.  Returns per-step O, counts, tau and,
    for the requested steps, the selection mask and (refresh steps) the
    GPU's fp32 scores."""
    T, B, h_q, d = Q.shape
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    shape = (B, h_q, h_k, h_v, d, l_kv)
    dev = Q.device
    ws = saga.alloc_workspace(saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N), dev)
    tau = torch.zeros(B, h_q, dtype=torch.float32, device=dev)
    O = torch.empty(B, h_q, d, dtype=torch.float32, device=dev)
    cnt = torch.empty(B, h_q, dtype=torch.int32, device=dev)
    out = {"O": [], "count": [], "tau": [], "mask": {}, "scores": {}}
    for t in range(T):
        refresh = (t % R) == 0
        saga.saga_decode_step(Q[t], K, V, N, tau, refresh, O, cnt, ws)
        out["O"].append(O.cpu().numpy().astype(np.float64))
        out["count"].append(cnt.cpu().numpy().astype(np.int64))
        out["tau"].append(tau.cpu().numpy().copy())
        if mask_steps is None or t in mask_steps:
            out["mask"][t] = read_mask(ws, shape, N)
        if refresh and (score_steps is None or t in score_steps):
            out["scores"][t] = read_scores(ws, shape, N)
    torch.cuda.synchronize()
    return out


def rel_err(o, ref) -> float:
    """max over rows of ||o - ref||_inf / ||ref||_inf (rows with ref == 0 use abs)."""
    o = o.reshape(-1, o.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    num = np.abs(o - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(r.max()) if r.size else 0.0


def check_tau_bits(scores_row: np.ndarray, tau_gpu: np.float32, N: int, where=""):
    want = oracle.nth_largest_f32(scores_row, N)
    got = np.float32(tau_gpu)
    assert got.view(np.uint32) == want.view(np.uint32), \
        f"tau mismatch {where}: gpu {got!r} cpu-sort {want!r}"
    assert (scores_row >= got).sum() >= N and (scores_row > got).sum() < N, where


def check_selection(mask_gpu, a_ref, tau_ref, where=""):
    """mask_gpu, a_ref [l_kv]; tau_ref scalar (oracle fp64 values)."""
    want = a_ref >= tau_ref
    got = mask_gpu.astype(bool)
    diff = got != want
    if diff.any():
        gap = np.abs(a_ref[diff] - tau_ref)
        assert gap.max() <= SEL_BAND, \
            f"selection differs beyond the band {where}: {int(diff.sum())} entries, max |A-tau| {gap.max()}"
    return int(diff.sum())
