"""The FLOP model against the numbers the pages print."""

import json
import os

from shifted_sparse_attention_amd import flops as F


def test_table7_attention_shares(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "table7_attention_flops.json")))
    for c in fx["cases"]:
        share = 100.0 * F.llama2_7b_attention_share(c["L"], c["keys_per_query"])
        assert round(share, 1) == c["share_percent"], (c, share)


def test_quadratic_law(golden_dir):
    law = json.load(open(os.path.join(golden_dir, "table7_attention_flops.json")))["quadratic_law"]
    a = F.fwd_flops(1, law["L_large"], 32, 128, law["L_large"])   # full attention: G = L
    b = F.fwd_flops(1, law["L_small"], 32, 128, law["L_small"])
    assert a / b == law["ratio"]


def test_counted_flops_headline():
    # Llama2-7B heads, L = 32768, G = 8192: 7 * B * Hq * L * G * d
    assert F.fwd_bwd_flops(1, 32768, 32, 128, 8192) == 7 * 32 * 32768 * 8192 * 128
    assert abs(F.fwd_bwd_flops(1, 32768, 32, 128, 8192) - 7.697e12) / 7.697e12 < 1e-3


def test_counted_flops_match_pair_count():
    # 4d FLOPs per allowed (query, key) pair, with G^2/2 pairs per group
    B, L, Hq, d, G = 2, 64, 4, 16, 16
    pairs = B * Hq * (L // G) * G * G / 2
    assert F.fwd_flops(B, L, Hq, d, G) == 4 * d * pairs
