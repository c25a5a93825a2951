"""The numeric statements the pages make that a test can check
(tests/golden/page_facts.json, each with its citation)."""
import json
import os

import numpy as np
import torch

import oracle
from sparse_asymmetric_head_amd import workload as wl

FACTS = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "page_facts.json")))


def _kv_bytes(h_k, h_v, h_q=8, d=64, l_kv=256):
    g = torch.Generator().manual_seed(3)
    q0 = (2 * torch.randn(1, h_q, d, generator=g)).to(torch.bfloat16)
    K, V = wl.make_cache(1, h_q, h_k, h_v, d, l_kv, q0, planted=8, heavy_tail=False, g=g,
                         device="cpu")
    return K.numel() * K.element_size() + V.numel() * V.element_size()


def test_kv_footprint_of_saga_1_8_against_8_8():
    """(h_k, h_v) = (1, 8) keeps a little over half the KV cache of (8, 8): the
    generator's caches at the two head counts, byte for byte."""
    f = FACTS["kv_footprint_saga_1_8_vs_8_8"]
    ratio = _kv_bytes(*f["h_k_h_v_saga"]) / _kv_bytes(*f["h_k_h_v_base"])
    assert f["ratio_lower_exclusive"] < ratio < f["ratio_upper_exclusive"]
    assert ratio == (1 + 8) / (8 + 8)


def test_value_rows_read_scale_with_n_not_l_kv():
    """Eq. 7: at a refresh step (tie-free scores) the oracle's output reads exactly
    N value rows per query head whatever the context length."""
    rng = np.random.default_rng(5)
    N = 13
    for l_kv in (64, 1024, 8192):
        q = torch.as_tensor(rng.standard_normal((1, 1, 4, 16)) * 2).to(torch.bfloat16)
        k = torch.as_tensor(rng.standard_normal((1, 1, l_kv, 16))).to(torch.bfloat16)
        v = torch.as_tensor(rng.standard_normal((1, 2, l_kv, 16))).to(torch.bfloat16)
        tr = oracle.trajectory(q, k, v, 1, 2, N, 1)
        assert (tr["count"] == N).all(), (l_kv, tr["count"])
