"""Checks that pin the fp64 oracle to things other than itself.

Each check takes an oracle library handle (so the mutation tests can run the
same checks against deliberately broken copies of the oracle) and raises
AssertionError when the oracle disagrees with:
  * closed forms (one-hot dot products, the two-entry softmax = logistic),
  * a library routine the definition reduces to (torch's scaled-dot-product
    attention in fp64 on the CPU for N = l_kv; numpy argsort for top-N),
  * invariants (counts at a refresh, permutation invariance, convex hull),
  * brute force on tiny inputs.
Sources: "More Value per Key" (picx.dev summary) eqs. 2-4, eq. 6,
Methodology > Atop-N Attention items 1-2 and eq. 7, SAGA Architecture.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

# ---------------------------------------------------------------- helpers


def bf16(x) -> np.ndarray:
    """Round a float array to bf16 (RNE, via torch) and return the bit patterns."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def widen(bits) -> np.ndarray:
    return oracle.bf16_bits_to_f64(bits)


def rand_case(rng, B, h_q, h_k, h_v, d, l_kv, T=1, scale=1.0):
    Q = bf16(rng.standard_normal((T, B, h_q, d)) * 2.0 * scale)
    K = bf16(rng.standard_normal((B, h_k, l_kv, d)))
    V = bf16(rng.standard_normal((B, h_v, l_kv, d)))
    return Q, K, V


def expand_heads(X: np.ndarray, h_q: int) -> np.ndarray:
    """[B][h][l][d] -> [B][h_q][l][d] with query head j reading head floor(j*h/h_q)."""
    h = X.shape[1]
    idx = [(j * h) // h_q for j in range(h_q)]
    return X[:, idx]


def sdpa_f64(Q64, K64, V64) -> np.ndarray:
    """torch scaled_dot_product_attention in fp64 on the CPU (the library routine
    dense softmax attention reduces to). Q [B][h][d]; K, V [B][h][l][d]."""
    q = torch.from_numpy(Q64)[:, :, None, :]
    k = torch.from_numpy(np.ascontiguousarray(K64))
    v = torch.from_numpy(np.ascontiguousarray(V64))
    with torch.no_grad():
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    return o[:, :, 0, :].numpy()


# ---------------------------------------------------------------- pins


def pin_scores_one_hot(lib):
    """Eq. 2 closed form: q = a*e_c, k_t = b_t*e_{c_t} -> A_t = a*b_t*[c == c_t]/sqrt(d).
    Also pins the key-head map floor(j*h_k/h_q) for a non-integer ratio."""
    d, l_kv, h_q, h_k = 8, 6, 6, 4
    Qf = np.zeros((1, h_q, d))
    for j in range(h_q):
        Qf[0, j, 1] = 2.0
    Kf = np.zeros((1, h_k, l_kv, d))
    for g in range(h_k):
        for t in range(l_kv):
            Kf[0, g, t, 1 if t % 2 == 0 else 3] = (g + 1) * (t + 1)
    A = oracle.scores(bf16(Qf), bf16(Kf), h_k, lib=lib)
    for j in range(h_q):
        g = (j * h_k) // h_q
        for t in range(l_kv):
            want = (2.0 * (g + 1) * (t + 1) / math.sqrt(d)) if t % 2 == 0 else 0.0
            assert A[0, j, t] == want, (j, t, A[0, j, t], want)


def pin_scores_sum_of_products(lib):
    """Eq. 2 with every coordinate contributing: q = (1..d), k_t = t*(1,..,1):
    A_t = t*d(d+1)/2 / sqrt(d) exactly (small integers are exact in bf16)."""
    d, l_kv = 16, 5
    Qf = np.arange(1, d + 1, dtype=np.float64)[None, None, :]
    Kf = np.stack([np.full(d, float(t)) for t in range(l_kv)])[None, None]
    Kf[0, 0, 2, 5] = -3.0  # row 2: coordinate 5 (q_5 = 6) changed from 2 to -3
    A = oracle.scores(bf16(Qf), bf16(Kf), 1, lib=lib)[0, 0]
    for t in range(l_kv):
        s = t * d * (d + 1) / 2.0
        if t == 2:
            s = s - 6 * 2.0 + 6 * (-3.0)
        assert A[t] == s / math.sqrt(d), (t, A[t], s / math.sqrt(d))


def pin_topn_argsort(lib, seed=0):
    """Eq. 6 + Atop-N item 1: with tau = exact N-th largest and no ties, the
    comparison set equals the brute-force top-N (numpy argsort)."""
    rng = np.random.default_rng(seed)
    for trial in range(20):
        n = int(rng.integers(5, 300))
        N = int(rng.integers(1, n + 1))
        a = rng.standard_normal(n) * 3.0
        tau = oracle.nth_largest(a, N, lib=lib)
        mask = np.zeros(n, np.uint8)
        cnt = lib.sao_select_row(np.ascontiguousarray(a), n, tau, mask)
        want = set(np.argsort(-a, kind="stable")[:N].tolist())
        got = set(np.nonzero(mask)[0].tolist())
        assert cnt == N and got == want, (trial, n, N)


def pin_nth_largest_ties(lib):
    """Ties at the threshold are all kept: count(a >= tau) >= N > count(a > tau)."""
    a = np.array([5.0, 1.0, 3.0, 3.0, 3.0, 0.5, 7.0, 3.0])
    for N in range(1, a.size + 1):
        tau = oracle.nth_largest(a, N, lib=lib)
        assert tau == sorted(a, reverse=True)[N - 1]
        assert (a >= tau).sum() >= N and (a > tau).sum() < N
    f = np.array([0.0, -0.0, 2.5, -1.0, 2.5], np.float32)
    assert oracle.nth_largest_f32(f, 1, lib=lib) == np.float32(2.5)
    assert oracle.nth_largest_f32(f, 3, lib=lib) == np.float32(0.0)
    assert oracle.nth_largest_f32(f, 5, lib=lib) == np.float32(-1.0)


def pin_dense_equals_sdpa(lib, seed=1):
    """N = l_kv selects everything, so Atop-N reduces to dense softmax attention
    (eqs. 2-4): compare with torch SDPA in fp64, heads expanded by the SAGA map
    (key head floor(j*h_k/h_q), value head floor(j*h_v/h_q))."""
    rng = np.random.default_rng(seed)
    for (B, h_q, h_k, h_v, d, l_kv) in [(2, 6, 2, 3, 16, 37), (1, 8, 3, 5, 8, 50),
                                        (1, 4, 4, 4, 32, 20)]:
        Q, K, V = rand_case(rng, B, h_q, h_k, h_v, d, l_kv, T=1)
        tr = oracle.trajectory(Q, K, V, h_k, h_v, N=l_kv, R=1, lib=lib)
        ref = sdpa_f64(widen(Q[0]), expand_heads(widen(K), h_q), expand_heads(widen(V), h_q))
        np.testing.assert_allclose(tr["O"][0], ref, rtol=1e-12, atol=1e-12)
        assert (tr["count"] == l_kv).all()


def pin_gqa_library(lib, seed=2):
    """h_k = h_v = h_kv is GQA: the dense oracle equals torch SDPA's own GQA
    grouping (enable_gqa); h_kv = h_q is MHA."""
    rng = np.random.default_rng(seed)
    for (B, h_q, h_kv, d, l_kv) in [(2, 8, 2, 16, 33), (1, 6, 6, 8, 19), (1, 12, 3, 32, 64)]:
        Q, K, V = rand_case(rng, B, h_q, h_kv, h_kv, d, l_kv, T=1)
        O = oracle.dense(Q[0], K, V, lib=lib)
        q = torch.from_numpy(widen(Q[0]))[:, :, None, :]
        with torch.no_grad():
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, torch.from_numpy(widen(K)), torch.from_numpy(widen(V)),
                enable_gqa=True)[:, :, 0, :].numpy()
        np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)
        tr = oracle.trajectory(Q, K, V, h_kv, h_kv, N=l_kv, R=1, lib=lib)
        np.testing.assert_allclose(tr["O"][0], ref, rtol=1e-12, atol=1e-12)


def pin_n1_argmax(lib, seed=3):
    """N = 1 without ties: softmax over one entry is 1, so O = V[argmax A] exactly."""
    rng = np.random.default_rng(seed)
    B, h_q, h_k, h_v, d, l_kv = 1, 4, 2, 4, 16, 40
    Q, K, V = rand_case(rng, B, h_q, h_k, h_v, d, l_kv, T=1)
    tr = oracle.trajectory(Q, K, V, h_k, h_v, N=1, R=1, lib=lib)
    Qw, Kw, Vw = widen(Q[0]), widen(K), widen(V)
    for j in range(h_q):
        g, v = (j * h_k) // h_q, (j * h_v) // h_q
        a = Kw[0, g] @ Qw[0, j]
        t = int(np.argmax(a))
        assert tr["count"][0, 0, j] == 1
        assert np.array_equal(tr["O"][0, 0, j], Vw[0, v, t]), j


def pin_two_entry_logistic(lib):
    """Two survivors: softmax of (a1, a2) is the logistic function, so
    O = s(a1-a2) v1 + s(a2-a1) v2 (closed form of eq. 7)."""
    d, l_kv = 4, 5
    # q = 2 e_0; rows score 2*k0/2 = k0 (sqrt(4)=2)
    Qf = np.zeros((1, 1, 1, d))
    Qf[..., 0] = 2.0
    k0 = [0.5, 3.0, -1.0, 2.0, -4.0]  # scores = k0; top-2 = t1 (3.0), t3 (2.0)
    Kf = np.zeros((1, 1, l_kv, d))
    Kf[0, 0, :, 0] = k0
    Vf = np.arange(l_kv * d, dtype=np.float64).reshape(1, 1, l_kv, d) / 8.0
    tr = oracle.trajectory(bf16(Qf), bf16(Kf), bf16(Vf), 1, 1, N=2, R=1, lib=lib)
    a1, a2 = 3.0, 2.0
    s = 1.0 / (1.0 + math.exp(-(a1 - a2)))
    want = s * Vf[0, 0, 1] + (1 - s) * Vf[0, 0, 3]
    assert tr["count"][0, 0, 0] == 2 and tr["tau"][0, 0, 0] == 2.0
    np.testing.assert_allclose(tr["O"][0, 0, 0], want, rtol=1e-14, atol=1e-14)


def pin_permutation_invariance(lib, seed=4):
    """Jointly permuting cache positions leaves tau, counts and O unchanged."""
    rng = np.random.default_rng(seed)
    B, h_q, h_k, h_v, d, l_kv, T = 1, 6, 2, 3, 16, 64, 4
    Q, K, V = rand_case(rng, B, h_q, h_k, h_v, d, l_kv, T=T)
    p = rng.permutation(l_kv)
    a = oracle.trajectory(Q, K, V, h_k, h_v, N=9, R=2, lib=lib)
    b = oracle.trajectory(Q, np.ascontiguousarray(K[:, :, p]), np.ascontiguousarray(V[:, :, p]),
                          h_k, h_v, N=9, R=2, lib=lib)
    assert np.array_equal(a["tau"], b["tau"]) and np.array_equal(a["count"], b["count"])
    np.testing.assert_allclose(a["O"], b["O"], rtol=1e-12, atol=1e-12)


def pin_convex_hull(lib, seed=5):
    """O is a convex combination of the selected value rows: every column lies
    within their min and max, and with all V rows equal, O equals that row."""
    rng = np.random.default_rng(seed)
    B, h_q, h_k, h_v, d, l_kv = 1, 4, 1, 2, 8, 50
    Q, K, V = rand_case(rng, B, h_q, h_k, h_v, d, l_kv, T=1)
    tr = oracle.trajectory(Q, K, V, h_k, h_v, N=7, R=1, want_mask=True, lib=lib)
    Vw = widen(V)
    for j in range(h_q):
        v = (j * h_v) // h_q
        sel = Vw[0, v][tr["mask"][0, 0, j].astype(bool)]
        o = tr["O"][0, 0, j]
        assert (o >= sel.min(0) - 1e-12).all() and (o <= sel.max(0) + 1e-12).all()
    Vc = np.broadcast_to(V[:, :, :1], V.shape).copy()
    tc = oracle.trajectory(Q, K, Vc, h_k, h_v, N=7, R=1, lib=lib)
    for j in range(h_q):
        v = (j * h_v) // h_q
        np.testing.assert_allclose(tc["O"][0, 0, j], widen(Vc)[0, v, 0], rtol=1e-14, atol=1e-14)


def pin_refresh_schedule(lib, seed=6):
    """Atop-N item 2: tau is recomputed exactly at steps t = 0, R, 2R, ... from
    that step's scores and reused in between; every step selects A_t >= tau."""
    rng = np.random.default_rng(seed)
    B, h_q, h_k, h_v, d, l_kv, T, N, R = 2, 4, 2, 2, 16, 80, 7, 6, 3
    Q, K, V = rand_case(rng, B, h_q, h_k, h_v, d, l_kv, T=T)
    tr = oracle.trajectory(Q, K, V, h_k, h_v, N=N, R=R, want_mask=True, lib=lib)
    Qw, Kw = widen(Q), widen(K)
    for t in range(T):
        tr_ = R * (t // R)
        for b in range(B):
            for j in range(h_q):
                g = (j * h_k) // h_q
                a_ref = Kw[b, g] @ Qw[tr_, b, j] / math.sqrt(d)
                tau = np.sort(a_ref)[::-1][N - 1]
                assert abs(tr["tau"][t, b, j] - tau) <= 1e-12 * max(1.0, abs(tau)), (t, b, j)
                a_t = Kw[b, g] @ Qw[t, b, j] / math.sqrt(d)
                tau_t = tr["tau"][t, b, j]
                want = a_t >= tau_t
                far = np.abs(a_t - tau_t) > 1e-12 * max(1.0, abs(tau_t))  # summation-order band
                assert np.array_equal(tr["mask"][t, b, j].astype(bool)[far], want[far]), (t, b, j)
                if t % R == 0:
                    assert tr["count"][t, b, j] >= N


def pin_empty_selection(lib):
    """A stale tau above every score selects nothing: O = 0 and count = 0.
    Step 0 scores are all positive (tau > 0); step 1 negates q, so every score
    at step 1 is negative and below the reused tau (R = 2)."""
    d, l_kv = 8, 12
    rng = np.random.default_rng(7)
    q = np.abs(rng.standard_normal(d)) + 0.5
    Qf = np.stack([q, -q])[:, None, None, :]
    Kf = (np.abs(rng.standard_normal((1, 1, l_kv, d))) + 0.1)
    Vf = rng.standard_normal((1, 1, l_kv, d))
    tr = oracle.trajectory(bf16(Qf), bf16(Kf), bf16(Vf), 1, 1, N=3, R=2, lib=lib)
    assert tr["count"][0, 0, 0] == 3 and tr["tau"][1, 0, 0] == tr["tau"][0, 0, 0] > 0
    assert tr["count"][1, 0, 0] == 0 and np.array_equal(tr["O"][1, 0, 0], np.zeros(d))


def pin_given_mask_consistent(lib, seed=8):
    """Given-mask mode with the trajectory's own selection reproduces its output;
    with an all-ones mask it equals the dense SDPA result."""
    rng = np.random.default_rng(seed)
    B, h_q, h_k, h_v, d, l_kv = 2, 6, 2, 3, 16, 45
    Q, K, V = rand_case(rng, B, h_q, h_k, h_v, d, l_kv, T=1)
    tr = oracle.trajectory(Q, K, V, h_k, h_v, N=5, R=1, want_mask=True, lib=lib)
    O, cnt = oracle.given_mask(Q[0], K, V, h_k, h_v, tr["mask"][0], lib=lib)
    np.testing.assert_allclose(O, tr["O"][0], rtol=1e-14, atol=1e-14)
    assert np.array_equal(cnt, tr["count"][0])
    O1, _ = oracle.given_mask(Q[0], K, V, h_k, h_v, np.ones((B, h_q, l_kv), np.uint8), lib=lib)
    ref = sdpa_f64(widen(Q[0]), expand_heads(widen(K), h_q), expand_heads(widen(V), h_q))
    np.testing.assert_allclose(O1, ref, rtol=1e-12, atol=1e-12)


def pin_brute_force_tiny(lib, seed=9):
    """Brute force on tiny inputs: enumerate every subset of size N of a row of 6,
    keep the one with the largest score sum (the top-N set when there are no
    ties), and compute its softmax-weighted value by direct summation."""
    import itertools

    rng = np.random.default_rng(seed)
    d, l_kv, N = 4, 6, 3
    for trial in range(10):
        Q, K, V = rand_case(rng, 1, 1, 1, 1, d, l_kv, T=1)
        a = widen(K)[0, 0] @ widen(Q)[0, 0, 0] / 2.0
        best = max(itertools.combinations(range(l_kv), N), key=lambda s: sum(a[i] for i in s))
        w = np.array([math.exp(a[i]) for i in best])
        w = w / w.sum()
        want = sum(w[k] * widen(V)[0, 0, i] for k, i in enumerate(best))
        tr = oracle.trajectory(Q, K, V, 1, 1, N=N, R=1, lib=lib)
        np.testing.assert_allclose(tr["O"][0, 0, 0], want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- growing cache
# The decode loop appends each token's key and value rows to the cache before
# the step attends (Introduction > Background: cached keys and values are
# reused); the threshold of the last refresh is reused for every position,
# the new ones included (Atop-N item 2).


def growing_case(rng, B, h_q, h_k, h_v, d, cap, T):
    return rand_case(rng, B, h_q, h_k, h_v, d, cap, T=T)


def pin_growing_brute_force(lib, seed=10):
    """Brute force on tiny inputs, written from the definition in numpy: step t
    scores the first l0 + t + 1 rows (matrix product in fp64), refreshes tau by a
    full sort at t mod R == 0, otherwise keeps the last refresh's tau, selects
    A >= tau and takes the softmax-weighted value rows."""
    rng = np.random.default_rng(seed)
    for (B, h_q, h_k, h_v, d, cap, l0, T, N, R) in [(2, 4, 2, 3, 8, 40, 20, 12, 5, 4),
                                                   (1, 6, 3, 6, 16, 30, 4, 9, 5, 3)]:
        Q, K, V = growing_case(rng, B, h_q, h_k, h_v, d, cap, T)
        tr = oracle.trajectory_growing(Q, K, V, h_k, h_v, l0, N, R, want_mask=True, lib=lib)
        Qw, Kw, Vw = widen(Q), widen(K), widen(V)
        tau = np.zeros((B, h_q))
        for t in range(T):
            n = l0 + t + 1
            for b in range(B):
                for j in range(h_q):
                    g, v = (j * h_k) // h_q, (j * h_v) // h_q
                    a = Kw[b, g, :n] @ Qw[t, b, j] / math.sqrt(d)
                    if t % R == 0:
                        tau[b, j] = np.sort(a)[::-1][N - 1]
                    sel = a >= tau[b, j]
                    o = np.zeros(d)  # an empty selection gives O = 0 (the reading for S empty)
                    if sel.any():
                        w = np.exp(a[sel] - a[sel].max())
                        o = (w[:, None] * Vw[b, v, :n][sel]).sum(0) / w.sum()
                    assert abs(tr["tau"][t, b, j] - tau[b, j]) <= 1e-12 * max(1, abs(tau[b, j]))
                    assert np.array_equal(tr["mask"][t, b, j, :n].astype(bool), sel), (t, b, j)
                    assert not tr["mask"][t, b, j, n:].any()
                    assert tr["count"][t, b, j] == sel.sum()
                    np.testing.assert_allclose(tr["O"][t, b, j], o, rtol=1e-12, atol=1e-12)


def pin_growing_new_keys_against_stale_tau(lib):
    """Closed-form counts: with a constant query and one refresh (R > T), each
    appended key joins S exactly when its score reaches the stale tau, so
    count_t = N + (appended keys so far above tau), and tau never changes.  The
    appended keys alternate between k = 4 q (far above every old score) and
    k = -q (far below); the last hot key is made dominant (k = 8 q), so the
    output equals its value row to within exp(-16).  (Step 0 refreshes over its
    own prefix, which already holds the first appended key.)"""
    rng = np.random.default_rng(11)
    d, l0, T, N = 16, 50, 8, 4
    cap = l0 + T
    q = np.sign(rng.standard_normal(d))                      # +-1 entries, |q|^2 = d
    Kf = rng.standard_normal((1, 1, cap, d)) * 0.25          # old scores |a| <~ 1
    for t in range(T):
        Kf[0, 0, l0 + t] = (4.0 * q if t % 2 == 0 else -q)
    Kf[0, 0, l0 + T - 2] = 8.0 * q                           # the last hot key dominates
    Vf = rng.standard_normal((1, 1, cap, d))
    Qf = np.broadcast_to(q, (T, 1, 1, d)).copy()
    tr = oracle.trajectory_growing(bf16(Qf), bf16(Kf), bf16(Vf), 1, 1, l0, N, R=T + 1,
                                   want_mask=True, lib=lib)
    hot = 0  # hot keys appended after the refresh at t = 0 (whose own key is among its top N)
    for t in range(T):
        hot += (t % 2 == 0 and t > 0)
        assert tr["tau"][t, 0, 0] == tr["tau"][0, 0, 0]
        assert tr["count"][t, 0, 0] == N + hot, (t, tr["count"][t, 0, 0])
        assert tr["mask"][t, 0, 0, l0 + t] == (t % 2 == 0)
    # scores of the two hot keys: 8d/4 = 32 and 4d/4 = 16 (exact in bf16), others <~ 1
    np.testing.assert_allclose(tr["O"][T - 1, 0, 0], widen(bf16(Vf))[0, 0, l0 + T - 2],
                               rtol=0, atol=1e-6)


def pin_growing_refresh_every_step_is_topn(lib, seed=12):
    """R = 1: every step is the exact top-N of its own prefix (numpy argsort on
    tie-free scores), and the step equals a static trajectory over that prefix."""
    rng = np.random.default_rng(seed)
    B, h_q, h_k, h_v, d, cap, l0, T, N = 1, 4, 2, 2, 16, 64, 40, 10, 7
    Q, K, V = growing_case(rng, B, h_q, h_k, h_v, d, cap, T)
    tr = oracle.trajectory_growing(Q, K, V, h_k, h_v, l0, N, 1, want_mask=True, lib=lib)
    Qw, Kw = widen(Q), widen(K)
    for t in range(T):
        n = l0 + t + 1
        st = oracle.trajectory(Q[t:t + 1], np.ascontiguousarray(K[:, :, :n]),
                               np.ascontiguousarray(V[:, :, :n]), h_k, h_v, N, 1, want_mask=True,
                               lib=lib)
        np.testing.assert_array_equal(st["mask"][0], tr["mask"][t][..., :n])
        np.testing.assert_allclose(st["O"][0], tr["O"][t], rtol=1e-14, atol=1e-14)
        for j in range(h_q):
            g = (j * h_k) // h_q
            a = Kw[0, g, :n] @ Qw[t, 0, j]
            want = set(np.argsort(-a, kind="stable")[:N].tolist())
            assert set(np.nonzero(tr["mask"][t, 0, j])[0].tolist()) == want, (t, j)


ALL_PINS = [
    pin_scores_one_hot,
    pin_scores_sum_of_products,
    pin_topn_argsort,
    pin_nth_largest_ties,
    pin_dense_equals_sdpa,
    pin_gqa_library,
    pin_n1_argmax,
    pin_two_entry_logistic,
    pin_permutation_invariance,
    pin_convex_hull,
    pin_refresh_schedule,
    pin_empty_selection,
    pin_given_mask_consistent,
    pin_brute_force_tiny,
    pin_growing_brute_force,
    pin_growing_new_keys_against_stale_tau,
    pin_growing_refresh_every_step_is_topn,
]
