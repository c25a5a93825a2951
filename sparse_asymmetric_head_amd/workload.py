"""Seeded synthetic decode workloads for SAGA + Atop-N.

This module only draws random inputs.  It holds none of the method's
arithmetic (no scores, no thresholds, no softmax) and imports neither the HIP
binding nor the oracle, so both sides can consume the same tensors.

Recipe (the pages measure on Llama 3.2-1B and Qwen2.5-1.5B decode at up to
128K context; no weights or datasets are used, these tensors stand in for
that attention shape):
  * K and V caches: i.i.d. N(0, 1) in fp32, rounded to bf16.
  * q_0: 2 * N(0, 1) rounded to bf16.
  * planted keys: per (batch, key head g), P positions drawn uniformly without
    replacement; each is  k = mean_{j in group g} fp32(q_0[b, j]) + 0.3 z,
    or, for the heavy-tailed stress workload, |T| * mean + 0.3 z with T drawn
    from a Student-t with 3 degrees of freedom per planted key.  The group of
    key head g is the query heads j with floor(j*h_k/h_q) == g.
  * query drift: q_t = bf16(fp32(q_{t-1}) + sigma * z_t).
  * a layer's tensors come from one generator seeded with 1000*i + layer,
    where i is the workload's index in ``CONFIGS``.
The dense-GQA baseline cache (h_kv heads for both K and V) follows the same
recipe with h_k = h_v = h_kv, from seed 1000*i + layer + 500.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class SagaConfig:
    name: str
    B: int
    h_q: int
    h_k: int
    h_v: int
    d: int
    l_kv: int
    N: int
    R: int
    steps: int
    layers: int = 1
    planted: int = 16
    q_scale: float = 2.0
    drift: float = 0.05
    heavy_tail: bool = False
    dense_h_kv: int | None = None

    def with_(self, **kw) -> "SagaConfig":
        return replace(self, **kw)


CONFIGS = [
    SagaConfig("tiny", B=1, h_q=4, h_k=1, h_v=2, d=64, l_kv=1024, N=64, R=1, steps=8, planted=16),
    SagaConfig("llama32-1b-32k", B=1, h_q=32, h_k=4, h_v=16, d=64, l_kv=32768, N=256, R=16,
               steps=64, planted=64, dense_h_kv=8),
    SagaConfig("llama32-1b-128k-16L", B=1, h_q=32, h_k=4, h_v=16, d=64, l_kv=131072, N=512, R=16,
               steps=64, layers=16, planted=128, dense_h_kv=8),
    SagaConfig("qwen25-1.5b-128k", B=4, h_q=12, h_k=1, h_v=4, d=128, l_kv=131072, N=512, R=32,
               steps=64, planted=128, dense_h_kv=2),
    SagaConfig("stress-b16-64k", B=16, h_q=32, h_k=2, h_v=32, d=128, l_kv=65536, N=1024, R=64,
               steps=128, planted=256, drift=0.1, heavy_tail=True),
]


def config(name: str) -> SagaConfig:
    """The decode workload of that name."""
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def config_index(cfg: SagaConfig) -> int:
    for i, c in enumerate(CONFIGS):
        if c.name == cfg.name:
            return i
    return 0


def layer_seed(cfg_index: int, layer: int) -> int:
    return 1000 * cfg_index + layer


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def group_members(j_count: int, h_k: int, g: int) -> list[int]:
    """Query heads j with floor(j*h_k/h_q) == g (recipe's 'row group')."""
    return [j for j in range(j_count) if (j * h_k) // j_count == g]


def make_cache(B: int, h_q: int, h_k: int, h_v: int, d: int, l_kv: int, q0: torch.Tensor,
               planted: int, heavy_tail: bool, g: torch.Generator, device):
    """K [B][h_k][l_kv][d], V [B][h_v][l_kv][d] (bf16) with planted keys near
    each key head's query-group mean."""
    K = _normal((B, h_k, l_kv, d), g, device)
    V = _normal((B, h_v, l_kv, d), g, device)
    P = min(int(planted), l_kv)
    if P > 0:
        q32 = q0.to(torch.float32)
        for b in range(B):
            for kh in range(h_k):
                members = group_members(h_q, h_k, kh)
                qbar = q32[b, members].mean(dim=0)
                pos = torch.randperm(l_kv, generator=g, device=device)[:P]
                z = _normal((P, d), g, device)
                if heavy_tail:
                    # Student-t, 3 dof: Z / sqrt(chi2_3 / 3)
                    zt = _normal((P,), g, device)
                    chi = (_normal((P, 3), g, device) ** 2).sum(dim=1)
                    t3 = zt / torch.sqrt(chi / 3.0)
                    rows = t3.abs()[:, None] * qbar[None, :] + 0.3 * z
                else:
                    rows = qbar[None, :] + 0.3 * z
                K[b, kh, pos] = rows
    return K.to(torch.bfloat16).contiguous(), V.to(torch.bfloat16).contiguous()


def make_queries(B: int, h_q: int, d: int, steps: int, q_scale: float, drift: float,
                 g: torch.Generator, device) -> torch.Tensor:
    """Q [steps][B][h_q][d] bf16: q_0 = bf16(q_scale * z), q_t = bf16(fp32(q_{t-1}) + drift * z)."""
    q = (q_scale * _normal((B, h_q, d), g, device)).to(torch.bfloat16)
    out = [q]
    for _ in range(1, steps):
        q = (q.to(torch.float32) + drift * _normal((B, h_q, d), g, device)).to(torch.bfloat16)
        out.append(q)
    return torch.stack(out).contiguous()


def make_layer(cfg: SagaConfig, layer: int = 0, device="cpu", cfg_index: int | None = None,
               steps: int | None = None):
    """One layer's seeded inputs: dict(Q [T][B][h_q][d], K, V) in bf16."""
    ci = config_index(cfg) if cfg_index is None else cfg_index
    g = _gen(layer_seed(ci, layer), device)
    T = cfg.steps if steps is None else steps
    Q = make_queries(cfg.B, cfg.h_q, cfg.d, T, cfg.q_scale, cfg.drift, g, device)
    K, V = make_cache(cfg.B, cfg.h_q, cfg.h_k, cfg.h_v, cfg.d, cfg.l_kv, Q[0], cfg.planted,
                      cfg.heavy_tail, g, device)
    return {"Q": Q, "K": K, "V": V}


def make_dense_layer(cfg: SagaConfig, layer: int = 0, device="cpu", cfg_index: int | None = None,
                     h_kv: int | None = None):
    """Dense-GQA baseline cache with h_kv heads for both K and V (same recipe)."""
    ci = config_index(cfg) if cfg_index is None else cfg_index
    hk = int(h_kv or cfg.dense_h_kv or cfg.h_k)
    g = _gen(layer_seed(ci, layer) + 500, device)
    q0 = (cfg.q_scale * _normal((cfg.B, cfg.h_q, cfg.d), g, device)).to(torch.bfloat16)
    K, V = make_cache(cfg.B, cfg.h_q, hk, hk, cfg.d, cfg.l_kv, q0, cfg.planted, cfg.heavy_tail,
                      g, device)
    return {"Q": q0.contiguous(), "K": K, "V": V}


def make_random(B: int, h_q: int, h_k: int, h_v: int, d: int, l_kv: int, seed: int, device="cpu",
                steps: int = 1, planted: int = 0, drift: float = 0.05, q_scale: float = 2.0,
                heavy_tail: bool = False):
    """Generic seeded case for tests (arbitrary shapes)."""
    g = _gen(seed, device)
    Q = make_queries(B, h_q, d, steps, q_scale, drift, g, device)
    K, V = make_cache(B, h_q, h_k, h_v, d, l_kv, Q[0], planted, heavy_tail, g, device)
    return {"Q": Q, "K": K, "V": V}


# ------------------------------------------------------ key-merge (conversion)
#
# Recipe for the GQA -> SAGA key-merge inputs (the pages convert pretrained
# Llama/Qwen GQA models with calibration data; no weights or data are used, these
# tensors stand in for one attention layer of that shape):
#   * X [n][d_model]: i.i.d. N(0, 1), rounded to bf16 (normalised hidden states);
#   * teacher key heads come in h_kt/2 hidden families assigned by a seeded
#     permutation: W_K^r = B_family(r) + spread * E_r with B, E i.i.d.
#     N(0, 1/d_model), so some pairs are much closer than others and the best
#     pairing is not the identity;
#   * queries Q_j = X W_Q^j with W_Q^j i.i.d. N(0, 1/d_model) scaled by
#     exp(-c/decay) on channel c (anisotropic query statistics, condition
#     number about exp(2 d/decay) over the channels), rounded to bf16;
#   * the planted variant makes the two heads of every family identical.
# The generator holds none of the conversion's arithmetic.


@dataclass(frozen=True)
class MergeConfig:
    name: str
    n: int
    h_q: int
    h_kt: int
    d: int
    d_model: int
    spread: float = 0.5
    decay: float = 32.0

    def with_(self, **kw) -> "MergeConfig":
        return replace(self, **kw)


MERGE_CONFIGS = [
    MergeConfig("merge-tiny", n=300, h_q=32, h_kt=8, d=64, d_model=256),
    MergeConfig("merge-llama32-1b-16k", n=16384, h_q=32, h_kt=8, d=64, d_model=2048),
    MergeConfig("merge-qwen25-1.5b-16k", n=16384, h_q=12, h_kt=2, d=128, d_model=1536, decay=64.0),
]
# the layer shapes the key merge is benchmarked on (16384 calibration tokens)
MERGE_BENCH = ("merge-llama32-1b-16k", "merge-qwen25-1.5b-16k")


def merge_config(name: str) -> MergeConfig:
    """The key-merge workload of that name."""
    for c in MERGE_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def make_merge_inputs(cfg: MergeConfig, seed: int, device="cpu", planted: bool = False):
    """(X [n][d_model], Q [n][h_q][d], W_K [h_kt*d][d_model]) in bf16.  The random
    draws come from one CPU generator (identical on every host); the query
    projection runs on ``device``."""
    g = _gen(seed, "cpu")
    n, dm, d, h_kt, h_q = cfg.n, cfg.d_model, cfg.d, cfg.h_kt, cfg.h_q
    X = _normal((n, dm), g, "cpu").to(torch.bfloat16)
    fam = torch.randperm(h_kt, generator=g) // 2
    base = _normal((h_kt // 2, d, dm), g, "cpu") / dm ** 0.5
    dev = _normal((h_kt, d, dm), g, "cpu") / dm ** 0.5
    W = base[fam] + (0.0 if planted else cfg.spread) * dev
    scale = torch.exp(-torch.arange(d, dtype=torch.float32) / cfg.decay)
    WQ = _normal((h_q, d, dm), g, "cpu") / dm ** 0.5 * scale[None, :, None]
    Xd = X.to(device)
    Q = (Xd.to(torch.float32) @ WQ.reshape(h_q * d, dm).to(device).t()).reshape(n, h_q, d)
    return (Xd.contiguous(), Q.to(torch.bfloat16).contiguous(),
            W.reshape(h_kt * d, dm).to(torch.bfloat16).to(device).contiguous())
