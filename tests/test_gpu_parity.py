"""HIP path vs the fp64 oracle, through the C ABI.  Needs an MI355X.

Small cases run whole trajectories against the oracle element by element;
the full-size workloads (32K/128K context, batch 16) compare sampled rows the
oracle computes one by one, in the launch configuration the benchmark uses
(the library picks it from the shape)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (OUT_RTOL, bits, check_selection, check_tau_bits, read_mask, read_scores,
                         rel_err, require_gpu, run_gpu_trajectory)
from sparse_asymmetric_head_amd import saga
from sparse_asymmetric_head_amd import workload as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def full_check(Q, K, V, N, R, tag=""):
    T, B, h_q, d = Q.shape
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    print(f"[parity] {tag} B={B} h_q={h_q} h_k={h_k} h_v={h_v} d={d} l_kv={l_kv} N={N} R={R} T={T}",
          flush=True)
    g = run_gpu_trajectory(Q, K, V, N, R)
    Qh, Kh, Vh = bits(Q), bits(K), bits(V)
    ref = oracle.trajectory(Qh, Kh, Vh, h_k, h_v, N, R, want_mask=True)
    flips = 0
    for t in range(T):
        A = oracle.scores(Qh[t], Kh, h_k)
        if t % R == 0:
            S = g["scores"][t].reshape(B, h_q, l_kv)
            scale = np.maximum(1.0, np.abs(A).max(axis=-1, keepdims=True))
            assert (np.abs(S - A) <= 1e-5 * scale).all(), f"scores t={t}"
            for b in range(B):
                for j in range(h_q):
                    check_tau_bits(S[b, j], g["tau"][t][b, j], N, f"t={t} b={b} j={j}")
        m = g["mask"][t]
        for b in range(B):
            for j in range(h_q):
                flips += check_selection(m[b, j], A[b, j], ref["tau"][t, b, j], f"t={t} b={b} j={j}")
        assert np.array_equal(g["count"][t], m.sum(-1)), f"counts t={t}"
        Og, cg = oracle.given_mask(Qh[t], Kh, Vh, h_k, h_v, m)
        assert np.array_equal(cg, g["count"][t])
        assert rel_err(g["O"][t], Og) <= OUT_RTOL, f"output t={t}: {rel_err(g['O'][t], Og)}"
        agree = (m == ref["mask"][t]).all(-1)
        if agree.any():
            assert rel_err(g["O"][t][agree], ref["O"][t][agree]) <= OUT_RTOL
    return flips


def test_tiny_config_full_trajectory():
    cfg = wl.config("tiny")
    x = wl.make_layer(cfg, 0, device="cuda")
    full_check(x["Q"], x["K"], x["V"], cfg.N, cfg.R, "tiny")


SMALL = [
    # B, h_q, h_k, h_v, d, l_kv, N, R, T, planted
    (2, 6, 4, 5, 64, 3001, 37, 3, 7, 8),       # non-integer head ratio, ragged tail
    (1, 12, 1, 4, 128, 5000, 100, 4, 6, 32),   # Qwen-like group of 12
    (2, 32, 2, 32, 128, 4100, 64, 5, 6, 32),   # group of 16, one value head per query
    (1, 40, 1, 8, 64, 2500, 50, 2, 3, 16),     # group of 40 (four N-tiles)
    (1, 24, 1, 24, 128, 1800, 30, 2, 3, 16),   # group of 24 (two N-tiles)
    (1, 8, 8, 8, 64, 777, 20, 2, 3, 4),        # MHA: h_k = h_v = h_q
    (1, 8, 2, 2, 64, 1500, 1500, 1, 2, 0),     # N = l_kv: dense GQA
    (1, 4, 1, 2, 64, 300, 1, 1, 2, 0),         # N = 1
    (3, 4, 2, 3, 128, 17, 5, 2, 3, 2),         # l_kv shorter than one tile
    (1, 4, 2, 2, 64, 1, 1, 1, 2, 0),           # a single cache position
    (1, 32768, 512, 1024, 64, 40, 6, 2, 2, 0),  # the largest head count, groups of 64
    (4, 32, 4, 16, 64, 2000, 600, 2, 3, 16),   # 128 rows, few long segments: a block per row in attend
    (1, 8, 2, 4, 128, 1200, 900, 2, 3, 8),     # d = 128, few rows, long segments
    (16, 32, 2, 32, 128, 2000, 200, 2, 3, 16), # 512 rows: a block per row in the attend kernel
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_small_trajectories(case):
    B, h_q, h_k, h_v, d, l_kv, N, R, T, P = case
    x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=hash(case) % 10007, device="cuda",
                       steps=T, planted=P, drift=0.05)
    full_check(x["Q"], x["K"], x["V"], N, R, "small")


def test_longest_cache():
    """The longest cache the plan accepts at d = 128 (l_kv d 2 bytes just below 2^31 per
    head): 64-bit offsets, 1024 segments per row, a ragged last chunk; every position
    checked against the oracle."""
    l_kv = (1 << 23) - 5
    x = wl.make_random(1, 2, 1, 1, 128, l_kv, seed=11, device="cuda", steps=2, planted=64,
                       drift=0.05)
    full_check(x["Q"], x["K"], x["V"], 1000, 2, "longest cache")


def test_llama_32k_full_trajectory():
    cfg = wl.config("llama32-1b-32k")
    x = wl.make_layer(cfg, 0, device="cuda")
    flips = full_check(x["Q"], x["K"], x["V"], cfg.N, cfg.R, cfg.name)
    print(f"[parity] {cfg.name}: boundary flips within the band: {flips}", flush=True)


def sampled_check(cfg, layer, steps, rows):
    x = wl.make_layer(cfg, layer, device="cuda")
    Q, K, V = x["Q"], x["K"], x["V"]
    T, B, h_q, d = Q.shape
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    N, R = cfg.N, cfg.R
    print(f"[parity] {cfg.name} layer={layer} steps={steps} rows={rows}", flush=True)
    need = set(steps)
    g = run_gpu_trajectory(Q, K, V, N, R, mask_steps=need,
                           score_steps={R * (t // R) for t in steps})
    Qh = bits(Q)
    for row in rows:
        b, j = divmod(row, h_q)
        kh, vh = (j * h_k) // h_q, (j * h_v) // h_q
        Kr = bits(K[b, kh])[None, None]
        Vr = bits(V[b, vh])
        for t in steps:
            tr = R * (t // R)
            a_tr = oracle.scores(Qh[tr, b, j][None, None], Kr, 1)[0, 0]
            tau_ref = oracle.nth_largest(a_tr, N)
            a_t = oracle.scores(Qh[t, b, j][None, None], Kr, 1)[0, 0] if t != tr else a_tr
            if t == tr:
                s = g["scores"][t][row]
                assert np.abs(s - a_t).max() <= 1e-5 * max(1.0, np.abs(a_t).max())
                check_tau_bits(s, g["tau"][t][b, j], N, f"{cfg.name} t={t} row={row}")
            m = g["mask"][t][b, j]
            check_selection(m, a_t, tau_ref, f"{cfg.name} t={t} row={row}")
            assert g["count"][t][b, j] == m.sum()
            o_ref, c_ref = oracle.attend_row(a_t, m, Vr)
            assert c_ref == g["count"][t][b, j]
            err = rel_err(g["O"][t][b, j][None], o_ref[None])
            assert err <= OUT_RTOL, f"{cfg.name} t={t} row={row}: {err}"
    del x, Q, K, V
    torch.cuda.empty_cache()


def test_llama_128k_16_layers_sampled():
    cfg = wl.config("llama32-1b-128k-16L")
    for layer in (0, 7, 15):
        sampled_check(cfg, layer, steps=[0, 16, 33, 63], rows=[0, 9, 22, 31])


def test_qwen_128k_sampled():
    cfg = wl.config("qwen25-1.5b-128k")
    sampled_check(cfg, 0, steps=[0, 31, 32, 63], rows=[0, 13, 30, 47])


def test_stress_batch16_sampled():
    cfg = wl.config("stress-b16-64k")
    sampled_check(cfg, 0, steps=[0, 63, 64, 127], rows=[0, 3 * 32 + 17, 15 * 32 + 31, 8 * 32 + 5])


# ------------------------------------------------------------------ edge cases

def _step(Q, K, V, N, tau, refresh):
    B, h_q, d = Q.shape
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    ws = saga.alloc_workspace(saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N))
    O = torch.empty(B, h_q, d, dtype=torch.float32, device="cuda")
    cnt = torch.empty(B, h_q, dtype=torch.int32, device="cuda")
    saga.saga_decode_step(Q, K, V, N, tau, refresh, O, cnt, ws)
    torch.cuda.synchronize()
    return O, cnt, ws


def test_stale_tau_extremes():
    x = wl.make_random(2, 8, 2, 4, 64, 2000, seed=11, device="cuda")
    Q, K, V = x["Q"][0], x["K"], x["V"]
    tau = torch.full((2, 8), 1e30, dtype=torch.float32, device="cuda")
    O, cnt, _ = _step(Q, K, V, 10, tau, False)
    assert (cnt == 0).all() and (O == 0).all()  # empty selection -> zero output
    tau.fill_(-1e30)
    O, cnt, _ = _step(Q, K, V, 10, tau, False)
    assert (cnt == 2000).all()
    Qh, Kh, Vh = bits(Q), bits(K), bits(V)
    ref = oracle.given_mask(Qh, Kh, Vh, 2, 4, np.ones((2, 8, 2000), np.uint8))[0]
    assert rel_err(O.cpu().numpy().astype(np.float64), ref) <= OUT_RTOL


def test_ties_at_threshold():
    """Duplicated key rows give exactly equal scores; all ties at tau are kept."""
    x = wl.make_random(1, 4, 1, 2, 64, 1024, seed=12, device="cuda")
    K = x["K"].clone()
    K[0, 0, 512:768] = K[0, 0, 256:512]   # every score in 256..767 appears twice
    K[0, 0, 100:110] = K[0, 0, 99]        # ten-way tie
    Q, V, N = x["Q"][0], x["V"], 7
    tau = torch.zeros(1, 4, dtype=torch.float32, device="cuda")
    O, cnt, ws = _step(Q, K, V, N, tau, True)
    S = read_scores(ws, (1, 4, 1, 2, 64, 1024), N)
    m = read_mask(ws, (1, 4, 1, 2, 64, 1024), N)
    for j in range(4):
        check_tau_bits(S[j], tau[0, j].item(), N, f"j={j}")
        assert np.array_equal(m[0, j].astype(bool), S[j] >= np.float32(tau[0, j].item()))
        assert cnt[0, j].item() == (S[j] >= np.float32(tau[0, j].item())).sum()
    assert np.array_equal(S[:, 512:768], S[:, 256:512])


def test_negative_zero_scores_canonical():
    """Key rows of -0.0 give score +0.0 (bit pattern 0), never -0.0."""
    x = wl.make_random(1, 4, 1, 2, 64, 256, seed=13, device="cuda")
    K = x["K"].clone()
    K[0, 0, :64] = -0.0
    tau = torch.zeros(1, 4, dtype=torch.float32, device="cuda")
    _, _, ws = _step(x["Q"][0], K, x["V"], 200, tau, True)
    S = read_scores(ws, (1, 4, 1, 2, 64, 256), 200)
    assert (S[:, :64].view(np.uint32) == 0).all()


def test_refresh_threshold_entry_point():
    x = wl.make_random(2, 12, 3, 6, 128, 6000, seed=14, device="cuda", planted=20)
    Q, K = x["Q"][0], x["K"]
    ws = saga.alloc_workspace(saga.saga_workspace_bytes(2, 12, 3, 3, 128, 6000, 300))
    tau = torch.zeros(2, 12, dtype=torch.float32, device="cuda")
    saga.saga_refresh_threshold(Q, K, 300, tau, ws)
    torch.cuda.synchronize()
    S = read_scores(ws, (2, 12, 3, 3, 128, 6000), 300)
    A = oracle.scores(bits(Q), bits(K), 3)
    for r in range(24):
        check_tau_bits(S[r], tau.view(-1)[r].item(), 300, f"row={r}")
        assert abs(tau.view(-1)[r].item() - oracle.nth_largest(A.reshape(24, -1)[r], 300)) < 1e-4


def test_deterministic_and_workspace_reuse():
    """Same inputs, same workspace, twice: bitwise identical tau, counts, output
    and selection (internal counters return to zero after every call)."""
    x = wl.make_random(1, 32, 4, 16, 64, 20000, seed=15, device="cuda", steps=6, planted=64)
    a = run_gpu_trajectory(x["Q"], x["K"], x["V"], 128, 3)
    b = run_gpu_trajectory(x["Q"], x["K"], x["V"], 128, 3)
    for t in range(6):
        assert np.array_equal(a["tau"][t].view(np.uint32), b["tau"][t].view(np.uint32))
        assert np.array_equal(a["count"][t], b["count"][t])
        assert np.array_equal(a["mask"][t], b["mask"][t])
        assert np.array_equal(a["O"][t], b["O"][t])


# ------------------------------------------------------------------ dense baseline

DENSE = [
    # B, h_q, h_kv, d, l_kv
    (1, 32, 8, 64, 5000),
    (2, 12, 2, 128, 3333),
    (1, 8, 8, 64, 100),
    (3, 6, 4, 128, 17),
    (1, 16, 1, 64, 2049),
]


def _dense(Q, K, V):
    B, h_q, d = Q.shape
    h_kv, l_kv = K.shape[1], K.shape[2]
    ws = torch.empty(saga.saga_dense_workspace_bytes(B, h_q, h_kv, d, l_kv), dtype=torch.uint8,
                     device="cuda")
    O = torch.empty(B, h_q, d, dtype=torch.float32, device="cuda")
    saga.saga_dense_gqa_baseline(Q, K, V, O, ws)
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", DENSE, ids=[str(c) for c in DENSE])
def test_dense_gqa_small(case):
    B, h_q, h_kv, d, l_kv = case
    x = wl.make_random(B, h_q, h_kv, h_kv, d, l_kv, seed=hash(case) % 9973, device="cuda",
                       planted=8)
    O = _dense(x["Q"][0], x["K"], x["V"])
    ref = oracle.dense(bits(x["Q"][0]), bits(x["K"]), bits(x["V"]))
    assert rel_err(O, ref) <= OUT_RTOL


FULL = [
    # B, h_q, h_k, h_v, d, l_kv
    (1, 32, 4, 16, 64, 3000),    # Llama-like: four value heads per key head
    (2, 12, 1, 4, 128, 2500),    # Qwen-like
    (1, 32, 2, 32, 128, 1500),   # sixteen value heads per key head: four subsets
    (2, 6, 4, 5, 64, 1001),      # non-integer head ratios, ragged tail
    (1, 8, 2, 2, 64, 700),       # h_k = h_v: dense GQA
    (1, 8, 2, 4, 64, 1234),      # two value heads per key head
    (1, 16, 2, 4, 64, 999),      # runs of four query heads per value head
    (1, 12, 4, 6, 64, 800),      # h_v divides h_q but h_k does not divide h_v
]


@pytest.mark.parametrize("case", FULL, ids=[str(c) for c in FULL])
def test_full_attention_small(case):
    """SAGA full attention (decoupled heads, no sparsity) against the oracle
    with every position selected."""
    B, h_q, h_k, h_v, d, l_kv = case
    x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=hash(case) % 7919, device="cuda",
                       planted=8)
    ws = torch.empty(saga.saga_full_attention_workspace_bytes(B, h_q, h_k, h_v, d, l_kv),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty(B, h_q, d, dtype=torch.float32, device="cuda")
    saga.saga_full_attention(x["Q"][0], x["K"], x["V"], O, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.given_mask(bits(x["Q"][0]), bits(x["K"]), bits(x["V"]), h_k, h_v,
                               np.ones((B, h_q, l_kv), np.uint8))
    assert rel_err(O.cpu().numpy().astype(np.float64), ref) <= OUT_RTOL


def test_full_attention_llama_128k():
    """SAGA full attention at the 128K Llama shape against the oracle."""
    cfg = wl.config("llama32-1b-128k-16L")
    x = wl.make_layer(cfg, 0, device="cuda", steps=1)
    B, h_q, h_k, h_v, d, l_kv = cfg.B, cfg.h_q, cfg.h_k, cfg.h_v, cfg.d, cfg.l_kv
    ws = torch.empty(saga.saga_full_attention_workspace_bytes(B, h_q, h_k, h_v, d, l_kv),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty(B, h_q, d, dtype=torch.float32, device="cuda")
    saga.saga_full_attention(x["Q"][0], x["K"], x["V"], O, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.given_mask(bits(x["Q"][0]), bits(x["K"]), bits(x["V"]), h_k, h_v,
                               np.ones((B, h_q, l_kv), np.uint8))
    assert rel_err(O.cpu().numpy().astype(np.float64), ref) <= OUT_RTOL


@pytest.mark.parametrize("name", ["llama32-1b-32k", "llama32-1b-128k-16L", "qwen25-1.5b-128k"])
def test_dense_gqa_full_size(name):
    cfg = wl.config(name)
    x = wl.make_dense_layer(cfg, 0, device="cuda")
    print(f"[parity] dense {cfg.name} h_kv={cfg.dense_h_kv}", flush=True)
    O = _dense(x["Q"], x["K"], x["V"])
    ref = oracle.dense(bits(x["Q"]), bits(x["K"]), bits(x["V"]))
    assert rel_err(O, ref) <= OUT_RTOL
    del x
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ HIP graphs

def test_graph_capture_replays_match_eager():
    """A captured decode step (refresh and non-refresh) replayed several times,
    with eager work and synchronisations in between, matches the eager result
    on every replay (no memset nodes; counters return to zero)."""
    x = wl.make_random(2, 12, 3, 6, 64, 9000, seed=21, device="cuda", steps=3, planted=32)
    Q, K, V = x["Q"], x["K"], x["V"]
    B, h_q, d = Q.shape[1:]
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    N = 77
    dev = Q.device
    ws = saga.alloc_workspace(saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N), dev)
    q = torch.empty_like(Q[0])
    tau = torch.zeros(B, h_q, dtype=torch.float32, device=dev)
    O = torch.empty(B, h_q, d, dtype=torch.float32, device=dev)
    cnt = torch.empty(B, h_q, dtype=torch.int32, device=dev)
    s = torch.cuda.Stream()
    ref = {}
    with torch.cuda.stream(s):
        for refresh, t in ((True, 0), (False, 1)):
            q.copy_(Q[t])
            saga.saga_decode_step(q, K, V, N, tau, refresh, O, cnt, ws)
            s.synchronize()
            ref[refresh] = (O.clone(), cnt.clone(), tau.clone())
        graphs = {}
        for refresh in (True, False):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                saga.saga_decode_step(q, K, V, N, tau, refresh, O, cnt, ws)
            graphs[refresh] = g
        for rep in range(3):
            for refresh, t in ((True, 0), (False, 1)):
                q.copy_(Q[t])
                O.fill_(float("nan"))
                cnt.fill_(-1)
                graphs[refresh].replay()
                s.synchronize()
                assert torch.equal(O, ref[refresh][0]), (rep, refresh)
                assert torch.equal(cnt, ref[refresh][1]), (rep, refresh)
                assert torch.equal(tau, ref[refresh][2]), (rep, refresh)
                # eager work on the same workspace between replays
                saga.saga_decode_step(q, K, V, N, tau, refresh, O, cnt, ws)
                s.synchronize()


def test_select_attend_halves_equal_decode_step():
    """saga_select followed by saga_attend is exactly saga_decode_step."""
    x = wl.make_random(1, 16, 2, 8, 128, 7000, seed=22, device="cuda", steps=2, planted=16)
    Q, K, V = x["Q"], x["K"], x["V"]
    B, h_q, d = Q.shape[1:]
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    N = 100
    ws = saga.alloc_workspace(saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N))
    outs = []
    for split in (False, True):
        tau = torch.zeros(B, h_q, dtype=torch.float32, device="cuda")
        O = torch.empty(B, h_q, d, dtype=torch.float32, device="cuda")
        cnt = torch.empty(B, h_q, dtype=torch.int32, device="cuda")
        res = []
        for t, refresh in ((0, True), (1, False)):
            if split:
                saga.saga_select(Q[t], K, h_v, N, tau, refresh, ws)
                saga.saga_attend(V, B, h_q, h_k, N, O, cnt, ws)
            else:
                saga.saga_decode_step(Q[t], K, V, N, tau, refresh, O, cnt, ws)
            torch.cuda.synchronize()
            res.append((O.clone(), cnt.clone(), tau.clone()))
        outs.append(res)
    for a, b in zip(*outs):
        for u, v in zip(a, b):
            assert torch.equal(u, v)


def test_attend_windows_and_long_records():
    """Far more than 256 survivors per wave (the attend kernel's wave-local
    LDS window of 256 entries is refilled many times) and segments far
    beyond the fifteen survivors a record's first 128 bytes hold: a stale
    tau of -inf selects every position.  The last two shapes take the
    streaming plan, whose upper waves flush survivors before the block ends
    and move them behind their segment's lower wave."""
    for (B, h_q, h_k, h_v, d, l_kv) in [(1, 8, 2, 4, 64, 10000), (2, 4, 1, 2, 128, 9001),
                                        (1, 8, 2, 4, 64, 40000), (1, 4, 1, 2, 128, 70001)]:
        x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=31 + d, device="cuda", planted=8)
        Q, K, V = x["Q"][0], x["K"], x["V"]
        tau = torch.full((B, h_q), float("-inf"), dtype=torch.float32, device="cuda")
        O, cnt, ws = _step(Q, K, V, 16, tau, False)
        assert (cnt == l_kv).all()
        ref, _ = oracle.given_mask(bits(Q), bits(K), bits(V), h_k, h_v,
                                   np.ones((B, h_q, l_kv), np.uint8))
        assert rel_err(O.cpu().numpy().astype(np.float64), ref) <= OUT_RTOL
        # a moderate stale threshold: about a third of each row survives
        A = oracle.scores(bits(Q), bits(K), h_k)
        t3 = np.quantile(A, 0.66, axis=-1).astype(np.float32)
        tau = torch.from_numpy(t3).cuda()
        O, cnt, ws = _step(Q, K, V, 16, tau, False)
        m = read_mask(ws, (B, h_q, h_k, h_v, d, l_kv), 16)
        for b in range(B):
            for j in range(h_q):
                check_selection(m[b, j], A[b, j], float(t3[b, j]), f"b={b} j={j}")
        Og, cg = oracle.given_mask(bits(Q), bits(K), bits(V), h_k, h_v, m)
        assert np.array_equal(cg, cnt.cpu().numpy())
        assert rel_err(O.cpu().numpy().astype(np.float64), Og) <= OUT_RTOL


def test_attend_mixed_counts_and_many_segments():
    """Rows of one launch with very different survivor counts (per-row stale
    thresholds: a few to half of the row), and rows with more than 256
    segments (one or two key heads over a long cache), match the oracle on
    the GPU's selection."""
    cases = [
        # B, h_q, h_k, h_v, d, l_kv, per-row quantiles of the stale threshold
        (2, 4, 1, 2, 64, 9001, [0.999, 0.66, 0.995, 0.5]),
        (2, 6, 2, 3, 128, 20000, [0.9995, 0.7, 0.998]),
        (1, 8, 1, 2, 64, 70001, [0.996]),
    ]
    for (B, h_q, h_k, h_v, d, l_kv, qs) in cases:
        x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=l_kv % 1009, device="cuda", planted=8)
        Q, K, V = x["Q"][0], x["K"], x["V"]
        A = oracle.scores(bits(Q), bits(K), h_k)
        t = np.empty((B, h_q), np.float32)
        for bb in range(B):
            for j in range(h_q):
                t[bb, j] = np.quantile(A[bb, j], qs[(bb * h_q + j) % len(qs)])
        tg = torch.from_numpy(t).cuda()
        O, cnt, ws = _step(Q, K, V, 16, tg, False)
        m = read_mask(ws, (B, h_q, h_k, h_v, d, l_kv), 16)
        for bb in range(B):
            for j in range(h_q):
                check_selection(m[bb, j], A[bb, j], float(t[bb, j]), f"b={bb} j={j}")
        Og, cg = oracle.given_mask(bits(Q), bits(K), bits(V), h_k, h_v, m)
        assert np.array_equal(cg, cnt.cpu().numpy())
        assert rel_err(O.cpu().numpy().astype(np.float64), Og) <= OUT_RTOL


def test_attend_row_per_block():
    """Launches whose column split would put two attend blocks or more on
    every compute unit (256 and 512 rows here) take the row-per-block attend
    kernel: every position selected (more than
    its 2048-survivor LDS window, so the window is refilled), about a third of
    each row, and per-row thresholds from a few survivors to half the row, all
    against the oracle on the GPU's selection; repeated calls are bitwise
    equal."""
    for (B, h_q, h_k, h_v, d, l_kv) in [(16, 32, 2, 32, 128, 3000), (8, 32, 4, 16, 64, 5001)]:
        print(f"[parity] attend rows B={B} h_q={h_q} h_k={h_k} h_v={h_v} d={d} l_kv={l_kv}",
              flush=True)
        x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=77 + d, device="cuda", planted=8)
        Q, K, V = x["Q"][0], x["K"], x["V"]
        A = oracle.scores(bits(Q), bits(K), h_k)
        qs = [0.999, 0.66, 0.995, 0.5]
        t_mixed = np.empty((B, h_q), np.float32)
        for bb in range(B):
            for j in range(h_q):
                t_mixed[bb, j] = np.quantile(A[bb, j], qs[(bb * h_q + j) % len(qs)])
        thresholds = [np.full((B, h_q), -np.inf, np.float32),
                      np.quantile(A, 0.66, axis=-1).astype(np.float32), t_mixed]
        for k, t in enumerate(thresholds):
            tau = torch.from_numpy(t).cuda()
            O, cnt, ws = _step(Q, K, V, 16, tau, False)
            m = read_mask(ws, (B, h_q, h_k, h_v, d, l_kv), 16)
            if k == 0:
                assert (cnt == l_kv).all()
            else:
                for bb in range(B):
                    for j in range(h_q):
                        check_selection(m[bb, j], A[bb, j], float(t[bb, j]), f"b={bb} j={j}")
            Og, cg = oracle.given_mask(bits(Q), bits(K), bits(V), h_k, h_v, m)
            assert np.array_equal(cg, cnt.cpu().numpy())
            assert rel_err(O.cpu().numpy().astype(np.float64), Og) <= OUT_RTOL, f"threshold {k}"
            O2 = torch.empty_like(O)
            c2 = torch.empty_like(cnt)
            saga.saga_attend(V, B, h_q, h_k, 16, O2, c2, ws)
            torch.cuda.synchronize()
            assert torch.equal(O, O2) and torch.equal(cnt, c2)


def test_read_probe_checksum():
    """The measurement probe reads every 16-byte item of its buffer exactly
    once: the XOR of its per-workgroup folds equals the XOR of all words."""
    g = torch.Generator().manual_seed(5)
    for nbytes in (16, 4096 + 48, (64 << 20) + 16 * 7):
        words = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64)
        host = words.to(torch.int32)
        buf = host.cuda()
        sink = torch.zeros(saga.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
        saga.saga_read_probe(buf, sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
        assert got == want, nbytes


@pytest.mark.parametrize("shape", [(256, 4, 8, True), (512, 4, 4, False), (1024, 4, 16, True),
                                   (256, 8, 8, False), (3, 8, 4, True)])
def test_read_probe_shape_checksum(shape):
    """The shaped read probe reads every 16-byte item exactly once in every
    launch shape: the XOR of the sink equals the XOR of the buffer's words."""
    blocks, waves, loads, chunked = shape
    g = torch.Generator().manual_seed(6)
    for nbytes in (16, 4096 + 48, (8 << 20) + 16 * 7):
        host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g,
                             dtype=torch.int64).to(torch.int32)
        sink = torch.zeros(saga.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
        saga.saga_read_probe_shape(host.cuda(), sink, blocks, waves, loads, chunked)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
        assert got == want, (shape, nbytes)


def ws_layout(B, h_q, h_k, h_v, d, l_kv, N):
    return saga.saga_workspace_layout(B, h_q, h_k, h_v, d, l_kv, N)


def record_order_keys(t, lay):
    """Rank of each position in the order the survivor records list them:
    chunk; segment s = group % 4; within the segment first the groups s, s+8,
    s+16, ... of the chunk, then s+4, s+12, ...; 16-row tile; then row % 4
    before row / 4 inside the tile."""
    t = np.asarray(t, np.int64)
    W = lay.n_seg // lay.n_chunk  # segments per chunk
    G = lay.chunk_len // lay.seg_group  # groups per chunk
    lo = -(-G // (2 * W))  # groups a segment lists before its second half
    c, o = t // lay.chunk_len, t % lay.chunk_len
    gi, i = o // lay.seg_group, o % lay.seg_group
    s, half, k = gi % W, (gi // W) % 2, gi // (2 * W)
    q = i % 16
    return (c * lay.chunk_len + s * lay.seg_cap + (half * lo + k) * lay.seg_group + (i - q)
            + (q % 4) * 4 + q // 4)


def _pivot_trajectory(Q, K, V, N, R, invalid_first=False):
    """Run the same steps with saga_decode_step (full refreshes) and with
    saga_decode_step_pivot (refresh 1 first, then refreshes from the pivot);
    return per-step (tau, O, counts, pivot-or-None, mask) of both."""
    T, B, h_q, d = Q.shape
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    shape = (B, h_q, h_k, h_v, d, l_kv)
    nb = saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N)
    ws_a, ws_b = saga.alloc_workspace(nb), saga.alloc_workspace(nb)
    tau_a = torch.zeros(B, h_q, device="cuda")
    tau_b = torch.zeros(B, h_q, device="cuda")
    piv = torch.full((B, h_q, N), -1, dtype=torch.int32, device="cuda")
    out_a, out_b = [], []
    for t in range(T):
        ref = t % R == 0
        O_a = torch.empty(B, h_q, d, device="cuda"); c_a = torch.empty(B, h_q, dtype=torch.int32, device="cuda")
        O_b = torch.empty_like(O_a); c_b = torch.empty_like(c_a)
        saga.saga_decode_step(Q[t], K, V, N, tau_a, ref, O_a, c_a, ws_a)
        mode = 0 if not ref else (2 if (t > 0 or invalid_first) else 1)
        saga.saga_decode_step_pivot(Q[t], K, V, N, tau_b, piv, mode, O_b, c_b, ws_b)
        torch.cuda.synchronize()
        out_a.append((tau_a.clone(), O_a, c_a, None, read_mask(ws_a, shape, N)))
        out_b.append((tau_b.clone(), O_b, c_b, piv.clone() if ref else None,
                      read_mask(ws_b, shape, N)))
    return out_a, out_b


PIVOT_CASES = [
    # B, h_q, h_k, h_v, d, l_kv, N, R, T, planted, drift
    (1, 32, 4, 16, 64, 32768, 256, 4, 9, 64, 0.05),
    (2, 12, 1, 4, 128, 20000, 100, 3, 7, 32, 0.05),
    (2, 6, 4, 5, 64, 3001, 37, 2, 5, 8, 0.05),
    (1, 8, 2, 4, 64, 30000, 64, 2, 5, 0, 3.0),   # the query changes a lot between refreshes
    (1, 32768, 512, 1024, 64, 300, 8, 2, 4, 0, 0.05),  # the largest head count
    (4, 32, 4, 16, 64, 20000, 256, 3, 7, 32, 0.05),   # 128 rows: a block per row in attend
    # 256 segments of 64 positions and N = 2048: the refine stages a thread per segment and
    # reads the entries past each record head (more than fifteen listed per segment)
    (1, 16, 4, 8, 64, 16384, 2048, 2, 5, 32, 0.05),
]


@pytest.mark.parametrize("case", PIVOT_CASES, ids=[str(c) for c in PIVOT_CASES])
def test_pivot_refresh_matches_full_refresh(case):
    """The refresh from a pivot gives the same tau bit for bit as the full
    refresh, hence the same selections, outputs (bitwise: same survivors in
    the same order) and counts; the recorded pivot rows are N increasing
    positions of the selection."""
    B, h_q, h_k, h_v, d, l_kv, N, R, T, P, drift = case
    x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=l_kv % 997, device="cuda", steps=T,
                       planted=P, drift=drift)
    out_a, out_b = _pivot_trajectory(x["Q"], x["K"], x["V"], N, R)
    for t, ((ta, Oa, ca, _, ma), (tb, Ob, cb, pv, mb)) in enumerate(zip(out_a, out_b)):
        assert torch.equal(ta.view(torch.int32), tb.view(torch.int32)), f"tau differs at step {t}"
        assert np.array_equal(ma, mb), f"selection differs at step {t}"
        assert torch.equal(ca, cb), f"counts differ at step {t}"
        assert torch.equal(Oa, Ob), f"outputs differ at step {t}"
        if pv is not None:
            p = pv.cpu().numpy()
            assert (p >= 0).all() and (p < l_kv).all()
            keys = record_order_keys(p, ws_layout(B, h_q, h_k, h_v, d, l_kv, N))
            assert (np.diff(keys, axis=-1) > 0).all(), "pivot not in record order"
            rows = np.take_along_axis(mb.reshape(B * h_q, l_kv), p.reshape(B * h_q, N), axis=1)
            assert (rows == 1).all(), f"pivot outside the selection at step {t}"


def test_pivot_refresh_with_unusable_pivot_is_exact():
    """A pivot row that is not N increasing positions (here all -1) gives the
    bound -inf: every score is listed and tau is still exact.  At l_kv = 20000
    the listing is longer than the refine kernel stages in LDS, and it stages
    the keys around rank N after one radix digit over the records; with
    N = 6000 even those do not fit, and it reads the records on every pass."""
    for (B, h_q, h_k, h_v, d, l_kv, N) in [(1, 8, 2, 4, 64, 20000, 50), (1, 4, 1, 2, 128, 5000, 5000),
                                           (1, 4, 1, 2, 64, 7000, 6000)]:
        x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=77, device="cuda", steps=2, planted=8)
        out_a, out_b = _pivot_trajectory(x["Q"], x["K"], x["V"], N, 1, invalid_first=True)
        for (ta, Oa, ca, _, ma), (tb, Ob, cb, pv, mb) in zip(out_a, out_b):
            assert torch.equal(ta.view(torch.int32), tb.view(torch.int32))
            assert np.array_equal(ma, mb) and torch.equal(ca, cb) and torch.equal(Oa, Ob)
            keys = record_order_keys(pv.cpu().numpy(), ws_layout(B, h_q, h_k, h_v, d, l_kv, N))
            assert (np.diff(keys, axis=-1) > 0).all()


CACHE_CASES = [
    # B, h_q, h_k, h_v, d, l0, T, N, R
    (1, 8, 2, 4, 64, 5000, 12, 64, 4),
    (1, 8, 2, 4, 64, 32760, 12, 128, 3),   # the chunking changes at 32768 positions
    (2, 12, 1, 4, 128, 3001, 9, 50, 4),
    (1, 32, 4, 16, 64, 32762, 10, 256, 4),  # Llama shape across the 32K select-plan change
    (4, 32, 4, 16, 64, 5000, 8, 64, 4),     # 128 rows: a block per row in attend
]


@pytest.mark.parametrize("case", CACHE_CASES, ids=[str(c) for c in CACHE_CASES])
def test_growing_context_matches_oracle(case):
    """KV append + decode over a growing prefix of caches with spare room, every
    step against the oracle's growing-cache trajectory (step t appends row
    l0 + t and attends over l0 + t + 1 rows; the new key meets the stale tau):
    on refresh steps tau bit-identical to a CPU sort of the GPU's fp32 scores
    of the prefix, selections within the band, counts exact, outputs within
    2e-3 of the oracle on the GPU's selection and of its own trajectory where
    the selections agree.  Each step also equals the contiguous path on a copy
    of the prefix bit for bit (the cache path refreshes from the pivot)."""
    B, h_q, h_k, h_v, d, l0, T, N, R = case
    cap = l0 + T
    print(f"[parity] growing B={B} h_q={h_q} h_k={h_k} h_v={h_v} d={d} l0={l0} T={T} N={N} R={R}",
          flush=True)
    x = wl.make_random(B, h_q, h_k, h_v, d, cap, seed=cap % 1013, device="cuda", steps=T,
                       planted=16)
    Kf, Vf, Q = x["K"], x["V"], x["Q"]
    Qh, Kh, Vh = bits(Q), bits(Kf), bits(Vf)
    ref_tr = oracle.trajectory_growing(Qh, Kh, Vh, h_k, h_v, l0, N, R, want_mask=True)
    K = torch.zeros_like(Kf)
    V = torch.zeros_like(Vf)
    K[:, :, :l0] = Kf[:, :, :l0]
    V[:, :, :l0] = Vf[:, :, :l0]
    ws_c = saga.alloc_workspace(saga.saga_cache_workspace_bytes(B, h_q, h_k, h_v, d, cap, N))
    tau_c = torch.zeros(B, h_q, device="cuda")
    tau_r = torch.zeros(B, h_q, device="cuda")
    piv = torch.full((B, h_q, N), -1, dtype=torch.int32, device="cuda")
    for t in range(T):
        pos = l0 + t
        saga.saga_append_kv(K, V, Kf[:, :, pos].contiguous(), Vf[:, :, pos].contiguous(), pos)
        length = pos + 1
        ref = t % R == 0
        mode = 0 if not ref else (1 if t == 0 else 2)
        O_c = torch.empty(B, h_q, d, device="cuda")
        c_c = torch.empty(B, h_q, dtype=torch.int32, device="cuda")
        saga.saga_decode_step_cache(Q[t], K, V, length, N, tau_c, piv, mode, O_c, c_c, ws_c)
        Kp, Vp = Kf[:, :, :length].contiguous(), Vf[:, :, :length].contiguous()
        O_r, c_r, ws_r = _step(Q[t], Kp, Vp, N, tau_r, ref)
        torch.cuda.synchronize()
        assert torch.equal(tau_c.view(torch.int32), tau_r.view(torch.int32)), f"tau at step {t}"
        assert torch.equal(c_c, c_r), f"counts at step {t}"
        assert torch.equal(O_c, O_r), f"outputs at step {t}"
        # against the oracle's growing trajectory
        shape = (B, h_q, h_k, h_v, d, length)
        m = read_mask(ws_c, shape, N)
        A = oracle.scores(Qh[t], np.ascontiguousarray(Kh[:, :, :length]), h_k)
        tc = tau_c.cpu().numpy()
        if ref:
            S = read_scores(ws_r, shape, N).reshape(B, h_q, length)
            for b in range(B):
                for j in range(h_q):
                    check_tau_bits(S[b, j], tc[b, j], N, f"growing t={t} b={b} j={j}")
        for b in range(B):
            for j in range(h_q):
                check_selection(m[b, j], A[b, j], ref_tr["tau"][t, b, j], f"growing t={t} b={b} j={j}")
        cc = c_c.cpu().numpy()
        assert np.array_equal(cc, m.sum(-1)), f"counts t={t}"
        Og, cg = oracle.given_mask(Qh[t], np.ascontiguousarray(Kh[:, :, :length]),
                                   np.ascontiguousarray(Vh[:, :, :length]), h_k, h_v, m)
        assert np.array_equal(cg, cc)
        Oc = O_c.cpu().numpy().astype(np.float64)
        assert rel_err(Oc, Og) <= OUT_RTOL, f"growing output t={t}: {rel_err(Oc, Og)}"
        agree = (m == ref_tr["mask"][t][..., :length]).all(-1)
        if agree.any():
            assert rel_err(Oc[agree], ref_tr["O"][t][agree]) <= OUT_RTOL
    assert torch.equal(K, Kf) and torch.equal(V, Vf)


# ------------------------------------------------------------------ the timed refresh path

def pivot_sampled_check(cfg, layer, steps, rows):
    """The refresh the benchmark times (saga_decode_step_pivot: an exact refresh
    recording the pivot at step 0, refreshes from the pivot at the later
    multiples of R, compares in between), in the benchmark's launch
    configuration, against (a) the full refresh of saga_decode_step bit for
    bit at every step (tau, counts, O; selections at the sampled steps) and
    (b) the oracle at the sampled rows and steps: tau bit-identical to a CPU
    sort of the GPU's fp32 scores, selection within the band, outputs within
    2e-3 of the oracle on the GPU's selection."""
    x = wl.make_layer(cfg, layer, device="cuda")
    Q, K, V = x["Q"], x["K"], x["V"]
    T, B, h_q, d = Q.shape
    h_k, l_kv, h_v = K.shape[1], K.shape[2], V.shape[1]
    N, R = cfg.N, cfg.R
    print(f"[parity] pivot {cfg.name} layer={layer} steps={steps} rows={rows}", flush=True)
    shape = (B, h_q, h_k, h_v, d, l_kv)
    nb = saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N)
    ws_a, ws_b = saga.alloc_workspace(nb), saga.alloc_workspace(nb)
    tau_a = torch.zeros(B, h_q, device="cuda")
    tau_b = torch.zeros(B, h_q, device="cuda")
    piv = torch.full((B, h_q, N), -1, dtype=torch.int32, device="cuda")
    O_a = torch.empty(B, h_q, d, device="cuda")
    O_b = torch.empty_like(O_a)
    c_a = torch.empty(B, h_q, dtype=torch.int32, device="cuda")
    c_b = torch.empty_like(c_a)
    Qh = bits(Q)
    Kr = {row: bits(K[row // h_q, ((row % h_q) * h_k) // h_q])[None, None] for row in rows}
    Vr = {row: bits(V[row // h_q, ((row % h_q) * h_v) // h_q]) for row in rows}
    modes = set()
    for t in range(T):
        ref = t % R == 0
        mode = 0 if not ref else (1 if t == 0 else 2)
        modes.add(mode)
        saga.saga_decode_step(Q[t], K, V, N, tau_a, ref, O_a, c_a, ws_a)
        saga.saga_decode_step_pivot(Q[t], K, V, N, tau_b, piv, mode, O_b, c_b, ws_b)
        torch.cuda.synchronize()
        assert torch.equal(tau_a.view(torch.int32), tau_b.view(torch.int32)), f"tau t={t}"
        assert torch.equal(c_a, c_b), f"counts t={t}"
        assert torch.equal(O_a, O_b), f"outputs t={t}"
        if t not in steps:
            continue
        m_b = read_mask(ws_b, shape, N)
        assert np.array_equal(m_b, read_mask(ws_a, shape, N)), f"selection t={t}"
        S = read_scores(ws_a, shape, N) if ref else None
        tb, cb = tau_b.cpu().numpy(), c_b.cpu().numpy()
        Ob = O_b.cpu().numpy().astype(np.float64)
        for row in rows:
            b, j = divmod(row, h_q)
            tr = R * (t // R)
            a_tr = oracle.scores(Qh[tr, b, j][None, None], Kr[row], 1)[0, 0]
            tau_ref = oracle.nth_largest(a_tr, N)
            a_t = oracle.scores(Qh[t, b, j][None, None], Kr[row], 1)[0, 0] if t != tr else a_tr
            if ref:
                assert np.abs(S[row] - a_t).max() <= 1e-5 * max(1.0, np.abs(a_t).max())
                check_tau_bits(S[row], tb[b, j], N, f"pivot {cfg.name} t={t} row={row}")
            check_selection(m_b[b, j], a_t, tau_ref, f"pivot {cfg.name} t={t} row={row}")
            assert cb[b, j] == m_b[b, j].sum()
            o_ref, c_ref = oracle.attend_row(a_t, m_b[b, j], Vr[row])
            assert c_ref == cb[b, j]
            err = rel_err(Ob[b, j][None], o_ref[None])
            assert err <= OUT_RTOL, f"pivot {cfg.name} t={t} row={row}: {err}"
    assert modes == {0, 1, 2}
    del x, Q, K, V, ws_a, ws_b
    torch.cuda.empty_cache()


def test_pivot_refresh_llama_128k_16_layers_sampled():
    cfg = wl.config("llama32-1b-128k-16L")
    for layer in (0, 7, 15):
        pivot_sampled_check(cfg, layer, steps=[0, 16, 33, 48, 63], rows=[0, 9, 22, 31])


def test_pivot_refresh_qwen_128k_sampled():
    cfg = wl.config("qwen25-1.5b-128k")
    pivot_sampled_check(cfg, 0, steps=[0, 31, 32, 63], rows=[0, 13, 30, 47])


def test_pivot_refresh_stress_batch16_sampled():
    cfg = wl.config("stress-b16-64k")
    pivot_sampled_check(cfg, 0, steps=[0, 63, 64, 127],
                        rows=[0, 3 * 32 + 17, 15 * 32 + 31, 8 * 32 + 5])


# ------------------------------------------------------------------ workspace robustness

def test_attend_on_fresh_workspace_is_empty():
    """saga_attend on a freshly initialised workspace (every record empty) gives
    O = 0 and counts = 0, with the column-split kernel (16 rows) and the
    row-per-block kernel (512 rows)."""
    for (B, h_q, h_k, h_v, d, l_kv, N) in [(2, 8, 2, 4, 64, 5000, 40),
                                           (16, 32, 2, 32, 128, 3000, 40)]:
        x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=3, device="cuda")
        ws = saga.alloc_workspace(saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N))
        O = torch.full((B, h_q, d), float("nan"), device="cuda")
        cnt = torch.full((B, h_q), -1, dtype=torch.int32, device="cuda")
        saga.saga_attend(x["V"], B, h_q, h_k, N, O, cnt, ws)
        torch.cuda.synchronize()
        assert (cnt == 0).all() and (O == 0).all()


def test_workspace_reused_for_larger_batch_refreshes_exactly():
    """One workspace (sized for the larger shape, initialised once) serves a
    refresh at B = 1 and then at B = 4, whose radix histograms and state sit
    where the first call's records were: tau stays bit-identical to a CPU sort
    of the GPU's own scores, and the selection matches the oracle."""
    h_q, h_k, h_v, d, l_kv, N = 12, 2, 4, 128, 9000, 70
    big = saga.saga_workspace_bytes(4, h_q, h_k, h_v, d, l_kv, N)
    ws = saga.alloc_workspace(big)
    for B in (1, 4, 2):
        x = wl.make_random(B, h_q, h_k, h_v, d, l_kv, seed=40 + B, device="cuda", planted=16)
        Q, K, V = x["Q"][0], x["K"], x["V"]
        tau = torch.zeros(B, h_q, device="cuda")
        O = torch.empty(B, h_q, d, device="cuda")
        cnt = torch.empty(B, h_q, dtype=torch.int32, device="cuda")
        saga.saga_decode_step(Q, K, V, N, tau, True, O, cnt, ws)
        torch.cuda.synchronize()
        shape = (B, h_q, h_k, h_v, d, l_kv)
        S = read_scores(ws, shape, N).reshape(B, h_q, l_kv)
        m = read_mask(ws, shape, N)
        A = oracle.scores(bits(Q), bits(K), h_k)
        tc = tau.cpu().numpy()
        for b in range(B):
            for j in range(h_q):
                check_tau_bits(S[b, j], tc[b, j], N, f"B={B} b={b} j={j}")
                check_selection(m[b, j], A[b, j], oracle.nth_largest(A[b, j], N), f"B={B}")
        Og, cg = oracle.given_mask(bits(Q), bits(K), bits(V), h_k, h_v, m)
        assert np.array_equal(cg, cnt.cpu().numpy())
        assert rel_err(O.cpu().numpy().astype(np.float64), Og) <= OUT_RTOL
