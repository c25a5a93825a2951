"""Checks that pin the key-merge oracle (oracle/key_merge.py) to things other than itself.

Each check takes the oracle module (so the mutation tests can run the same
checks against deliberately broken copies) and raises AssertionError when the
oracle disagrees with:
  * an independent least-squares solve of the eq. 13 objective, set up as an
    explicit linear system in the entries of M (numpy lstsq);
  * closed forms (isotropic query statistics: the merge is the mean of the two
    projections and the loss is g c / 2 ||X (W_a - W_b)||^2);
  * brute-force scalar loops over tokens and channels for eq. 13;
  * first-order optimality of the merge (central differences);
  * exhaustive minimisation over all permutations sigma of eq. 14, and the
    count (h-1)!! of perfect matchings;
  * planted structure (identical head pairs, an unqueried group, a null
    direction of the query statistics).
Source: "More Value per Key" (picx.dev summary), GQA-to-SAGA Conversion,
Stage 1: eqs. 13-15, Lemma 4.1, Theorem 4.2.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def _case(rng, n, dm, d, h_q, h_kt):
    X = rng.standard_normal((n, dm))
    Q = rng.standard_normal((n, h_q, d))
    W = rng.standard_normal((h_kt, dm, d)) / math.sqrt(dm)
    return X, Q, W


def _design(km, X, Q, W, a, b):
    """eq. 13 as || A vec(M) - y ||^2: A's columns are the logits of unit matrices."""
    n, h_q, d = Q.shape
    dm = X.shape[1]
    h_kt = W.shape[0]
    heads = [(r, j) for r in (a, b) for j in km.query_heads(r, h_q, h_kt)]
    cols = []
    for p in range(dm):
        for c in range(d):
            E = np.zeros((dm, d))
            E[p, c] = 1.0
            cols.append(np.concatenate([(Q[:, j, :] @ (X @ E).T).ravel() for _, j in heads]))
    A = np.stack(cols, axis=1)
    y = np.concatenate([(Q[:, j, :] @ (X @ W[r]).T).ravel() for r, j in heads])
    return A, y


def pin_merge_is_least_squares_minimiser(km):
    """Eq. 15 equals the unique minimiser of eq. 13 found by a generic lstsq."""
    rng = np.random.default_rng(11)
    X, Q, W = _case(rng, n=7, dm=5, d=3, h_q=4, h_kt=2)
    A, y = _design(km, X, Q, W, 0, 1)
    m, *_ = np.linalg.lstsq(A, y, rcond=None)
    M_ls = m.reshape(5, 3)
    S = [km.second_moment(Q, r, 2) for r in range(2)]
    M = km.merged_key(W[0], W[1], S[0], S[1])
    assert np.allclose(M, M_ls, rtol=1e-9, atol=1e-11), np.abs(M - M_ls).max()
    w, merged = km.pair_weights(X, Q, W)
    best = float(np.sum((A @ m - y) ** 2))
    assert math.isclose(w[0, 1], best, rel_tol=1e-9), (w[0, 1], best)


def pin_isotropic_queries(km):
    """S_a = S_b = g c I: the merge is (W_a + W_b)/2, the loss g c/2 ||X (W_a - W_b)||^2."""
    rng = np.random.default_rng(12)
    n, dm, d, h_q, h_kt, c = 9, 6, 4, 6, 2, 2.5
    X = rng.standard_normal((n, dm))
    W = rng.standard_normal((h_kt, dm, d))
    Q = np.zeros((n, h_q, d))
    for j in range(h_q):
        U, _ = np.linalg.qr(rng.standard_normal((n, d)))
        Q[:, j, :] = math.sqrt(c) * U
    g = h_q // h_kt
    w, merged = km.pair_weights(X, Q, W)
    assert np.allclose(merged[(0, 1)], (W[0] + W[1]) / 2, atol=1e-12)
    want = g * c / 2 * float(np.sum((X @ (W[0] - W[1])) ** 2))
    assert math.isclose(w[0, 1], want, rel_tol=1e-10), (w[0, 1], want)


def pin_loss_brute_force(km):
    """Eq. 13 by scalar loops over query heads, tokens and channels."""
    rng = np.random.default_rng(13)
    n, dm, d, h_q, h_kt = 3, 2, 2, 4, 2
    X, Q, W = _case(rng, n, dm, d, h_q, h_kt)
    M = rng.standard_normal((dm, d))
    for a, b in ((0, 1), (1, 0)):
        want = 0.0
        for r in (a, b):
            for j in range(h_q):
                if (j * h_kt) // h_q != r:
                    continue
                for t in range(n):
                    for u in range(n):
                        diff = 0.0
                        for ch in range(d):
                            kh = sum(X[u, p] * M[p, ch] for p in range(dm))
                            kr = sum(X[u, p] * W[r, p, ch] for p in range(dm))
                            diff += Q[t, j, ch] * (kh - kr)
                        want += diff * diff
        got = km.pair_loss(X, Q, W, a, b, M)
        assert math.isclose(got, want, rel_tol=1e-12), (got, want)


def pin_merge_first_order_optimal(km):
    """At eq. 15 the central difference of eq. 13 vanishes and every step costs."""
    rng = np.random.default_rng(14)
    X, Q, W = _case(rng, n=12, dm=6, d=4, h_q=8, h_kt=4)
    S = [km.second_moment(Q, r, 4) for r in range(4)]
    for a, b in ((0, 2), (1, 3)):
        M = km.merged_key(W[a], W[b], S[a], S[b])
        L0 = km.pair_loss(X, Q, W, a, b, M)
        for _ in range(4):
            D = rng.standard_normal(M.shape)
            eps = 1e-3
            Lp = km.pair_loss(X, Q, W, a, b, M + eps * D)
            Lm = km.pair_loss(X, Q, W, a, b, M - eps * D)
            curv = (Lp + Lm - 2 * L0) / eps ** 2
            slope = (Lp - Lm) / (2 * eps)
            assert curv > 0 and Lp > L0 and Lm > L0
            assert abs(slope) <= 1e-6 * curv, (slope, curv)


def pin_rank_deficient_statistics(km):
    """Singular S_a + S_b (4 query vectors in 6 channels): eq. 15 still attains the
    least-squares minimum, and the merged key is zero along every direction that no
    query reads (the pseudoinverse's range)."""
    rng = np.random.default_rng(15)
    n, dm, d, h_q, h_kt = 2, 5, 6, 2, 2
    X, Q, W = _case(rng, n, dm, d, h_q, h_kt)
    A, y = _design(km, X, Q, W, 0, 1)
    m, *_ = np.linalg.lstsq(A, y, rcond=1e-12)
    best = float(np.sum((A @ m - y) ** 2))
    S = [km.second_moment(Q, r, h_kt) for r in range(h_kt)]
    M = km.merged_key(W[0], W[1], S[0], S[1])
    got = km.pair_loss(X, Q, W, 0, 1, M)
    scale = float(np.sum(y ** 2))
    assert abs(got - best) <= 1e-10 * scale, (got, best)
    rows = Q.reshape(n * h_q, d)
    _, sv, Vt = np.linalg.svd(rows)
    null = Vt[int(np.sum(sv > 1e-12 * sv[0])):]
    assert null.shape[0] == d - n * h_q
    assert np.abs(M @ null.T).max() <= 1e-10 * np.abs(M).max(), np.abs(M @ null.T).max()


def pin_identical_heads_merge_free(km):
    """W_a == W_b: the merge returns that projection and costs nothing."""
    rng = np.random.default_rng(16)
    X, Q, W = _case(rng, n=10, dm=6, d=4, h_q=4, h_kt=2)
    W[1] = W[0]
    w, merged = km.pair_weights(X, Q, W)
    assert np.allclose(merged[(0, 1)], W[0], atol=1e-12)
    assert abs(w[0, 1]) <= 1e-20 * float(np.sum((X @ W[0]) ** 2))


def pin_unqueried_group_merges_free(km):
    """A key head whose query heads are all zero can merge with any head at no cost."""
    rng = np.random.default_rng(17)
    X, Q, W = _case(rng, n=8, dm=5, d=3, h_q=8, h_kt=4)
    for j in km.query_heads(2, 8, 4):
        Q[:, j, :] = 0.0
    w, _ = km.pair_weights(X, Q, W)
    assert np.all(np.abs(w[2]) <= 1e-20), w[2]
    assert w[0, 1] > 0 and w[1, 3] > 0


def pin_query_groups(km):
    """Q_r is the GQA group: floor(j h_kt / h_q) == r, and S_r sums exactly those heads."""
    assert km.query_heads(3, 32, 8) == [12, 13, 14, 15]
    assert km.query_heads(0, 12, 2) == [0, 1, 2, 3, 4, 5]
    assert [km.group_of(j, 6, 4) for j in range(6)] == [0, 0, 1, 2, 2, 3]
    n, h_q, d = 5, 8, 3
    Q = np.zeros((n, h_q, d))
    for j in range(h_q):
        Q[:, j, 0] = j + 1.0
    for r in range(4):
        S = km.second_moment(Q, r, 4)
        assert S[0, 0] == n * sum((j + 1.0) ** 2 for j in (2 * r, 2 * r + 1)), (r, S[0, 0])
        assert np.count_nonzero(S) == 1


def pin_matching_exhaustive(km):
    """Eq. 14 minimised over every permutation sigma equals the matching optimum,
    and there are (h-1)!! distinct perfect matchings."""
    rng = np.random.default_rng(18)
    for h in (2, 4, 6, 8):
        ms = list(km.perfect_matchings(range(h)))
        want = math.prod(range(h - 1, 0, -2))
        assert len(ms) == want, (h, len(ms))
        canon = {tuple(sorted(tuple(sorted(p)) for p in m)) for m in ms}
        assert len(canon) == want
        assert all(sorted(x for p in m for x in p) == list(range(h)) for m in ms)
    for trial in range(5):
        h = 6
        A = rng.random((h, h))
        w = A + A.T
        np.fill_diagonal(w, 0.0)
        brute = min(sum(w[s[2 * i], s[2 * i + 1]] for i in range(h // 2))
                    for s in itertools.permutations(range(h)))
        pairs, total = km.best_pairing(w)
        assert math.isclose(total, brute, rel_tol=1e-12), (total, brute)
        assert math.isclose(sum(w[a, b] for a, b in pairs), total, rel_tol=1e-12)


def pin_planted_pairs(km):
    """Four planted pairs of identical key heads: the conversion finds exactly them
    with zero total loss, and the merged keys are the shared projections."""
    rng = np.random.default_rng(19)
    n, dm, d, h_q, h_kt = 16, 8, 4, 16, 8
    X, Q, W = _case(rng, n, dm, d, h_q, h_kt)
    perm = rng.permutation(h_kt)
    planted = sorted((min(perm[2 * i], perm[2 * i + 1]), max(perm[2 * i], perm[2 * i + 1]))
                     for i in range(h_kt // 2))
    for a, b in planted:
        W[b] = W[a]
    out = km.convert(X, Q, W)
    assert out["pairs"] == [tuple(map(int, p)) for p in planted], (out["pairs"], planted)
    assert out["total"] <= 1e-20 * float(np.sum(X ** 2))
    for i, (a, b) in enumerate(planted):
        assert np.allclose(out["W_merged"][i], W[a], atol=1e-12)
    forced = [(planted[0][0], planted[1][0]), (planted[0][1], planted[1][1])] + planted[2:]
    out2 = km.convert(X, Q, W, pairs=forced)
    assert out2["total"] > 0
    assert math.isclose(out2["total"], sum(out["w"][a, b] for a, b in forced), rel_tol=1e-12)


ALL_PINS = [
    pin_merge_is_least_squares_minimiser,
    pin_isotropic_queries,
    pin_loss_brute_force,
    pin_merge_first_order_optimal,
    pin_rank_deficient_statistics,
    pin_identical_heads_merge_free,
    pin_unqueried_group_merges_free,
    pin_query_groups,
    pin_matching_exhaustive,
    pin_planted_pairs,
]
