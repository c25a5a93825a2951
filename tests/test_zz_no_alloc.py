"""The allocation-free decode step (the library's static per-GPU workspace)
against saga_decode_step_pivot on a caller-owned workspace, through the C ABI:
two trajectories in a row, the second on a smaller input (the static array keeps
the first call's contents), each step's tau, counts, O and pivot bit for bit;
and a shape whose workspace exceeds the static array is refused before anything
is enqueued."""
import pytest
import torch

from gpu_helpers import require_gpu
from sparse_asymmetric_head_amd import saga
from sparse_asymmetric_head_amd import workload as wl

pytestmark = pytest.mark.gpu


def _trajectory(x, N, modes):
    Q, K, V = x["Q"], x["K"], x["V"]
    T, B, h_q, d = Q.shape
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    print(f"[no-alloc] B={B} h_q={h_q} h_k={h_k} h_v={h_v} d={d} l_kv={l_kv} N={N} "
          f"modes={modes}", flush=True)
    ws = saga.alloc_workspace(saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N))
    st = {}
    for which in ("ws", "static"):
        st[which] = dict(tau=torch.zeros(B, h_q, device="cuda"),
                         piv=torch.full((B, h_q, N), -1, dtype=torch.int32, device="cuda"),
                         O=torch.empty(B, h_q, d, device="cuda"),
                         cnt=torch.empty(B, h_q, dtype=torch.int32, device="cuda"))
    for t, mode in enumerate(modes):
        a, b = st["ws"], st["static"]
        saga.saga_decode_step_pivot(Q[t], K, V, N, a["tau"], a["piv"], mode, a["O"], a["cnt"], ws)
        b["O"].fill_(float("nan"))
        b["cnt"].fill_(-1)
        saga.saga_decode_step_noalloc(Q[t], K, V, N, b["tau"], b["piv"], mode, b["O"], b["cnt"])
        torch.cuda.synchronize()
        for k in ("tau", "piv", "O", "cnt"):
            assert torch.equal(a[k], b[k]), f"{k} differs at step {t} (mode {mode})"


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    require_gpu()
    cfg = wl.config("llama32-1b-128k-16L")
    x = wl.make_layer(cfg, 3, device="cuda", steps=4)
    _trajectory(x, cfg.N, modes=(1, 0, 2, 0))
    del x
    y = wl.make_random(2, 6, 4, 5, 64, 3001, seed=5, device="cuda", steps=4, planted=8)
    _trajectory(y, 37, modes=(1, 0, 2, 0))


def test_noalloc_refuses_shapes_beyond_the_static_workspace():
    require_gpu()
    # the batch-16 stress shape needs ~517 MiB of workspace
    need = saga.saga_workspace_bytes(16, 32, 2, 32, 128, 65536, 1024)
    assert need > saga.STATIC_WORKSPACE_BYTES
    st = saga.lib().saga_decode_step_noalloc(16, 16, 16, 16, 32, 2, 32, 128, 65536, 1024, 16, 16,
                                             0, 16, None, None)
    assert st == saga.SAGA_ERR_WORKSPACE
    # the largest bench shape that fits
    assert saga.saga_workspace_bytes(4, 12, 1, 4, 128, 131072, 512) <= saga.STATIC_WORKSPACE_BYTES
