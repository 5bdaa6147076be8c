"""s2attn_bwd_noalloc (row term in the library's device array) against
s2attn_bwd (row term in the caller's delta_ws): the same kernels, so the
gradients must agree bit for bit.  Two calls in a row, the second smaller,
so the second reuses the array the first filled; the smaller one is also
checked against the oracle."""

import numpy as np
import pytest
import torch

import shifted_sparse_attention_amd as s2
from oracle import s2attn as O
from seeded_inputs.gen import bf16_round
from tests.gpu_util import BF16_MAX_ABS, BF16_REL_F, bf16_store_tol, check, host, say

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _inputs(seed, B, L, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    shapes = ((B, L, Hq, d), (B, L, Hkv, d), (B, L, Hkv, d), (B, L, Hq, d))
    return [bf16_round(rng.standard_normal(s, dtype=np.float32)) for s in shapes]


def _both(x, B, L, Hq, Hkv, d, G, sh):
    tq, tk, tv, tdo = (torch.from_numpy(a).to(BF).cuda() for a in x)
    o, lse = s2.forward(tq, tk, tv, G, sh)

    def nan(t):
        return torch.full_like(t, float("nan"))

    ref = [nan(t) for t in (tq, tk, tv)]
    delta = torch.full((B * Hq * L,), float("nan"), dtype=torch.float32, device="cuda")
    s2.s2attn_bwd(tq, tk, tv, o, lse, tdo, *ref, delta, B, L, Hq, Hkv, d, G, sh)
    got = [nan(t) for t in (tq, tk, tv)]
    s2.s2attn_bwd_noalloc(tq, tk, tv, o, lse, tdo, *got, B, L, Hq, Hkv, d, G, sh)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert bool(torch.isfinite(a.float()).all()), name
        assert torch.equal(a, b), f"{name}: s2attn_bwd_noalloc differs from s2attn_bwd"
    return got


def test_noalloc_backward_equals_plain_backward_twice():
    # first call: the 32k training shape (2^20 row-term floats)
    B, L, Hq, Hkv, d, G, sh = 1, 32768, 32, 32, 128, 8192, 16
    say(f"[noalloc] call 1: B{B} L{L} H{Hq}/{Hkv} d{d} G{G} shifted {sh}")
    _both(_inputs(71, B, L, Hq, Hkv, d), B, L, Hq, Hkv, d, G, sh)
    # second call, smaller (GQA, d = 64): bitwise the plain backward, and the oracle
    B, L, Hq, Hkv, d, G, sh = 2, 1024, 4, 2, 64, 256, 2
    say(f"[noalloc] call 2: B{B} L{L} H{Hq}/{Hkv} d{d} G{G} shifted {sh}")
    x = _inputs(72, B, L, Hq, Hkv, d)
    got = _both(x, B, L, Hq, Hkv, d, G, sh)
    rdq, rdk, rdv, _, _ = O.backward(*x, G, sh)
    for name, a, ref in zip(("dq", "dk", "dv"), got, (rdq, rdk, rdv)):
        check(name + "(bf16)", host(a), ref, BF16_REL_F, bf16_store_tol(ref))


def test_noalloc_rejects_sizes_past_its_array():
    B, L, Hq, Hkv, d, G = 2, 1 << 22, 2, 2, 64, 1 << 22   # B Hq L = 2^24 > 2^23
    assert B * Hq * L > s2.S2ATTN_NOALLOC_MAX_ROWS
    fake = 1 << 16
    with pytest.raises(s2.S2AttnError) as e:
        s2.s2attn_bwd_noalloc(*([fake] * 9), B, L, Hq, Hkv, d, G, 0)
    assert e.value.status == s2.S2ATTN_ERR_WORKSPACE
    assert BF16_MAX_ABS > 0
