"""Stored fixtures: the oracle's own regression value and the ratios the pages print."""
import json
import os

import numpy as np

import oracle.cca as O
from synth import make_prefill, shape_from_dict, workload

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_prefill_regression():
    g = json.load(open(os.path.join(GOLD, "tiny_prefill_oracle.json")))
    s = shape_from_dict(g["shape"])
    P = make_prefill(s, 0)
    y = O.prefill(P.x, P.weights.f64(), s)
    np.testing.assert_allclose(y, np.array(g["y"]), rtol=1e-13, atol=1e-15)


def test_workloads_reproduce_page_ratios():
    g = json.load(open(os.path.join(GOLD, "page_ratios.json")))
    # latent KV cache per token is 2 * e_kv values against 2 * E for MHA
    for name in ("ccgqa_prefill_t8192", "ccgqa_decode_b64_l32768"):
        s = workload(name)
        assert (2 * s.d_model) / (2 * s.e_kv) == g["kv_cache_compression_vs_mha"]
        # a GQA/MLA cache at the same query compression keeps e_q-wide k and v
        assert s.e_kv / s.e_q <= g["ccgqa_cache_vs_gqa_mla"]
    # attention FLOPs scale with the latent query width e_q instead of E
    ratios = sorted({workload(n).d_model // workload(n).e_q
                     for n in ("cca_prefill_b4_t2048", "ccgqa_prefill_t16384")})
    assert ratios == g["flop_reduction_examples"]
