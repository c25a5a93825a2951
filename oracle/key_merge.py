"""fp64 CPU oracle for the GQA -> SAGA key-head merge -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark may import this module.  The product path (the HIP library and its
Python binding) never does, and this module imports nothing from it.

Source: "More Value per Key: Asymmetric Sparse Attention for Faster LLM
Decoding" (picx.dev summary), GQA-to-SAGA Conversion, Stage 1 (Closed-Form
Initialization): eq. 13 (pairwise squared-logit loss), eq. 14 (objective over
pairings), eq. 15 with Lemma 4.1 (closed-form merged key projection,
S_r = sum over the query heads j of group r of Q^j^T Q^j) and Theorem 4.2 (the
best pairing is a minimum-weight perfect matching on the complete graph whose
edge weights are the eq. 13 losses at eq. 15).

Everything is written in the pages' orientation and notation:
  * X    [n][d_model]       calibration inputs of the layer;
  * Q    [n][h_q][d]        calibration queries, Q^j = Q[:, j, :];
  * W    [h_kt][d_model][d] key projections, W_K^a = W[a], keys X W_K^a;
  * group r (the pages' Q_r) = query heads j with floor(j*h_kt/h_q) == r,
    the query-to-key-head map of a GQA teacher (reading: contiguous groups).
The pages pair key heads (h_k^T = 2 h_k^S, sigma_{2i-1} with sigma_{2i});
only that ratio is defined here.

Readings (the pages leave these open):
  * the pseudoinverse of the symmetric positive semi-definite S_a + S_b is
    taken from its eigendecomposition, with eigenvalues at or below
    ``RTOL`` times the largest one counted as zero;
  * ties between pairings go to the first pairing in the enumeration order of
    ``perfect_matchings`` (lowest free head paired with each higher head in
    increasing order);
  * a pairing is reported canonically: pairs (a, b) with a < b, sorted by a.

Cost: eq. 13 is evaluated as written (n x n logit matrices), so keep n small
(hundreds of tokens).
"""
from __future__ import annotations

import numpy as np

RTOL = 1e-9


def group_of(j: int, h_q: int, h_kt: int) -> int:
    """Key head of the teacher that query head j reads (GQA grouping)."""
    return (j * h_kt) // h_q


def query_heads(r: int, h_q: int, h_kt: int) -> list[int]:
    """The pages' Q_r: the query heads attached to key head r."""
    return [j for j in range(h_q) if group_of(j, h_q, h_kt) == r]


def second_moment(Q: np.ndarray, r: int, h_kt: int) -> np.ndarray:
    """S_r = sum over j in Q_r of (Q^j)^T Q^j  (d x d), the matrix under eq. 15."""
    n, h_q, d = Q.shape
    S = np.zeros((d, d))
    for j in query_heads(r, h_q, h_kt):
        Qj = Q[:, j, :]
        S += Qj.T @ Qj
    return S


def pinv_psd(S: np.ndarray, rtol: float = RTOL) -> np.ndarray:
    """Moore-Penrose pseudoinverse of a symmetric PSD matrix via eigh."""
    lam, V = np.linalg.eigh(S)
    top = lam.max() if lam.size else 0.0
    inv = np.zeros_like(lam)
    keep = lam > rtol * top
    inv[keep] = 1.0 / lam[keep]
    return (V * inv) @ V.T


def merged_key(Wa: np.ndarray, Wb: np.ndarray, Sa: np.ndarray, Sb: np.ndarray,
               rtol: float = RTOL) -> np.ndarray:
    """Eq. 15 (Lemma 4.1): (W_K^a S_a + W_K^b S_b)(S_a + S_b)^+  (d_model x d)."""
    return (Wa @ Sa + Wb @ Sb) @ pinv_psd(Sa + Sb, rtol)


def pair_loss(X: np.ndarray, Q: np.ndarray, W: np.ndarray, a: int, b: int, M: np.ndarray) -> float:
    """Eq. 13: logit reconstruction error of both groups when heads a and b share key M."""
    n, h_q, d = Q.shape
    h_kt = W.shape[0]
    KM = X @ M
    total = 0.0
    for r in (a, b):
        Kr = X @ W[r]
        for j in query_heads(r, h_q, h_kt):
            Qj = Q[:, j, :]
            total += float(np.sum((Qj @ KM.T - Qj @ Kr.T) ** 2))
    return total


def pair_weights(X: np.ndarray, Q: np.ndarray, W: np.ndarray, rtol: float = RTOL):
    """Edge weights of Theorem 4.2: w(a, b) = eq. 13 at the eq. 15 merge, for all a != b.

    Returns (w, merged) with w symmetric (zero diagonal) and merged[(a, b)] the
    eq. 15 projection for a < b."""
    h_kt = W.shape[0]
    S = [second_moment(Q, r, h_kt) for r in range(h_kt)]
    w = np.zeros((h_kt, h_kt))
    merged = {}
    for a in range(h_kt):
        for b in range(a + 1, h_kt):
            M = merged_key(W[a], W[b], S[a], S[b], rtol)
            w[a, b] = w[b, a] = pair_loss(X, Q, W, a, b, M)
            merged[(a, b)] = M
    return w, merged


def perfect_matchings(heads):
    """Every way to split ``heads`` into unordered pairs (lowest free head first)."""
    heads = list(heads)
    if not heads:
        yield []
        return
    first = heads[0]
    for k in range(1, len(heads)):
        rest = heads[1:k] + heads[k + 1:]
        for tail in perfect_matchings(rest):
            yield [(first, heads[k])] + tail


def best_pairing(w: np.ndarray):
    """Eq. 14 / Theorem 4.2: the perfect matching of minimum total weight, by enumeration."""
    h = w.shape[0]
    best, best_cost = None, np.inf
    for m in perfect_matchings(range(h)):
        cost = sum(w[a, b] for a, b in m)
        if cost < best_cost:
            best, best_cost = m, cost
    return best, float(best_cost)


def convert(X: np.ndarray, Q: np.ndarray, W: np.ndarray, pairs=None, rtol: float = RTOL) -> dict:
    """Stage 1 of the conversion: weights, pairing (optimal unless given) and merged keys.

    Returns {"w": [h_kt][h_kt], "pairs": [(a, b), ...] canonical, "total": float,
             "W_merged": [h_kt/2][d_model][d]} -- merged head i serves the query
    heads of teacher groups pairs[i][0] and pairs[i][1]."""
    h_kt = W.shape[0]
    if h_kt % 2:
        raise ValueError("the pages merge key heads in pairs: h_kt must be even")
    w, merged = pair_weights(X, Q, W, rtol)
    if pairs is None:
        pairs, total = best_pairing(w)
    else:
        pairs = sorted((min(a, b), max(a, b)) for a, b in pairs)
        if sorted(x for p in pairs for x in p) != list(range(h_kt)):
            raise ValueError("pairs must cover every key head exactly once")
        total = float(sum(w[a, b] for a, b in pairs))
    W_merged = np.stack([merged[(a, b)] for a, b in pairs])
    return {"w": w, "pairs": [tuple(map(int, p)) for p in pairs], "total": total,
            "W_merged": W_merged}
