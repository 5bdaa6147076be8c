"""GPU parity: libs2attn's HIP kernels against the CPU oracle on seeded inputs.

Small shapes (several tiles, ragged tails, GQA, RoPE, degenerate groups) are
compared element by element over whole tensors.  The workloads run at full
size on the GPU into NaN-filled outputs.  The 32k training workload is
compared over whole tensors (the oracle runs every unit in worker
processes); the 100k and grouped-query workloads on units (one KV head and
group, with all its query heads) that include unshifted groups and the
shifted group that wraps; dense causal attention (one group spanning the
context) on sampled rows; plus properties that hold at any size over every
group.

Tolerances: bf16 outputs and gradients rel-Frobenius <= 5e-3 and max-abs <=
2e-2; fp32 path <= 1e-5 for both.  Gradients are compared as the kernels
produce them, stored in fp32 (`grad_dtype` float32; only the final store
differs from the bf16 path).  A bf16-stored gradient additionally carries
its store's rounding, half a bf16 ulp of its value, which alone passes 2e-2
once |x| >= 8 (dK, dV of the grouped-query workload reach ~12): those are
held to 2e-2 plus that half ulp at the reference's largest magnitude.
"""

import dataclasses

import numpy as np
import pytest
import torch

import shifted_sparse_attention_amd as s2
from oracle import s2attn as O
from seeded_inputs import CONFIGS, make_inputs
from seeded_inputs.gen import bf16_round
from tests.gpu_util import (BF16_MAX_ABS, BF16_REL_F, F32_TOL, bf16_store_tol, check, dev,
                            host, say)

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def rand_inputs(seed, B, L, Hq, Hkv, d, bf16=True):
    rng = np.random.default_rng(seed)
    out = []
    for shp in ((B, L, Hq, d), (B, L, Hkv, d), (B, L, Hkv, d), (B, L, Hq, d)):
        x = rng.standard_normal(shp, dtype=np.float32)
        out.append(bf16_round(x) if bf16 else x)
    return out


# ---------------------------------------------------------------------------
# Small shapes, whole tensors.
# ---------------------------------------------------------------------------

SMALL = [
    # B, L, Hq, Hkv, d, G, shifted, rope
    (1, 256, 4, 4, 64, 64, 2, None),
    (2, 640, 4, 2, 128, 320, 2, None),       # q tiles 128+128+64 (ragged), GQA r=2, B=2
    (1, 600, 2, 1, 128, 200, 2, None),       # G not a multiple of 64, MQA
    (1, 512, 4, 4, 128, 512, 0, None),       # G = L, no shift: full causal attention
    (1, 1024, 8, 1, 64, 256, 8, None),       # every head shifted, r=8
    (1, 64, 2, 2, 128, 2, 2, None),          # tiny groups
    (1, 64, 2, 2, 64, 1, 0, None),           # G = 1: o = v
    (1, 1536, 2, 2, 128, 768, 1, (10000.0, 256)),  # RoPE with position interpolation
    (1, 768, 4, 2, 64, 384, 2, (500.0, 64)),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}L{c[1]}H{c[2]}/{c[3]}d{c[4]}G{c[5]}s{c[6]}"
                                             f"{'rope' if c[7] else ''}" for c in SMALL])
def test_small_bf16_fwd_bwd(case):
    B, L, Hq, Hkv, d, G, sh, rope = case
    say(f"[small bf16] {case}")
    q, k, v, do = rand_inputs(1000 + L + G, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh, rope=rope)
    g32 = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, rope=rope, grad_dtype=torch.float32)
    g16 = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, rope=rope)
    torch.cuda.synchronize()
    rdq, rdk, rdv, ro, rlse = O.backward(q, k, v, do, G, sh, rope=rope)
    check("o", host(o), ro, BF16_REL_F, BF16_MAX_ABS)
    check("lse", host(lse), rlse, BF16_REL_F, BF16_MAX_ABS)
    for name, a, b, ref in zip(("dq", "dk", "dv"), g32, g16, (rdq, rdk, rdv)):
        check(name, host(a), ref, BF16_REL_F, BF16_MAX_ABS)
        check(name + "(bf16)", host(b), ref, BF16_REL_F, bf16_store_tol(ref))


def _random_cases(n, seed):
    """Seeded small shapes over the library's options: batch, query and KV
    heads (GQA ratio 1, 2 or 4), d = 64 or 128, group sizes with ragged 32-
    and 64-row tiles, 1-4 groups per sequence, shifted-head counts the
    backward accepts (a multiple of Hq / Hkv; G even when any head shifts),
    RoPE on or off, a softmax scale of its own, dS kept or recomputed, and
    fp32- or bf16-stored gradients."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        r = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.integers(1, 3))
        Hq = Hkv * r
        sh = r * int(rng.integers(0, Hkv + 1))
        G = int(rng.integers(1, 700))
        if sh and G % 2:
            G += 1
        n_g = int(rng.integers(1, 5))
        L = G * n_g
        if L > 2048:
            continue
        B = int(rng.integers(1, 3))
        rope = (float(rng.choice([500.0, 10000.0])), int(rng.choice([64, 256]))) if rng.random() < 0.3 else None
        scale = float(rng.uniform(0.05, 0.15)) if rng.random() < 0.25 else None
        ds = 0 if rng.random() < 0.3 else None
        gd = torch.float32 if rng.random() < 0.5 else BF
        cases.append((B, L, Hq, Hkv, d, G, sh, rope, scale, ds, gd))
    return cases


RANDOM = _random_cases(64, 20261203)


@pytest.mark.parametrize("case", RANDOM, ids=[
    f"B{c[0]}L{c[1]}H{c[2]}/{c[3]}d{c[4]}G{c[5]}s{c[6]}{'rope' if c[7] else ''}"
    f"{'scale' if c[8] else ''}{'ds0' if c[9] == 0 else ''}{'f32' if c[10] == torch.float32 else 'bf16'}"
    for c in RANDOM])
def test_random_small_shapes(case):
    """Whole tensors against the oracle over a seeded sweep of shapes and
    options, at the same bounds as the fixed small cases (fp32-stored
    gradients and O at 2e-2 flat; bf16-stored gradients plus their store's
    half ulp)."""
    B, L, Hq, Hkv, d, G, sh, rope, scale, ds, gd = case
    say(f"[random small] {case}")
    q, k, v, do = rand_inputs(3000 + L + G + d, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh, scale=scale, rope=rope)
    g = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, scale=scale, rope=rope, grad_dtype=gd,
                    ds_max_mib=ds)
    torch.cuda.synchronize()
    rdq, rdk, rdv, ro, rlse = O.backward(q, k, v, do, G, sh, scale=scale, rope=rope)
    check("o", host(o), ro, BF16_REL_F, BF16_MAX_ABS)
    check("lse", host(lse), rlse, BF16_REL_F, BF16_MAX_ABS)
    for name, a, ref in zip(("dq", "dk", "dv"), g, (rdq, rdk, rdv)):
        tol = BF16_MAX_ABS if gd == torch.float32 else bf16_store_tol(ref)
        check(name, host(a), ref, BF16_REL_F, tol)


F32_CASES = [
    (1, 256, 4, 2, 64, 64, 2),
    (1, 192, 2, 2, 128, 96, 1),
    (2, 120, 2, 1, 64, 40, 0),
]


@pytest.mark.parametrize("case", F32_CASES)
def test_small_f32_fwd_bwd(case):
    B, L, Hq, Hkv, d, G, sh = case
    say(f"[small f32] {case}")
    q, k, v, do = rand_inputs(2000 + L, B, L, Hq, Hkv, d, bf16=False)
    tq, tk, tv, tdo = (dev(x, torch.float32) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh)
    dq, dk, dv = s2.backward(tq, tk, tv, o, lse, tdo, G, sh)
    torch.cuda.synchronize()
    rdq, rdk, rdv, ro, rlse = O.backward(q, k, v, do, G, sh)
    for name, x, r in (("o", o, ro), ("lse", lse, rlse), ("dq", dq, rdq), ("dk", dk, rdk),
                       ("dv", dv, rdv)):
        check(name, host(x), r, F32_TOL, F32_TOL)


def test_many_small_units():
    """L = 65536 cut into 1024 groups of 64: 4096 (head, group) units, one
    query tile each, so the grid is tens of thousands of workgroups spread
    over the XCDs by the unit map; whole tensors against the oracle.  Every
    row sits near the start of its group, where a query sees few keys and P
    is large: the residual split (on by default here, G < 4096) takes nearly
    every dK/dV tile, and switched off the bf16 rounding of P and dS shows in
    dV and dK (about 1.4e-2 and 2.3e-2 max-abs)."""
    B, L, Hq, Hkv, d, G, sh = 1, 65536, 4, 2, 64, 64, 2
    say("[small units] L65536 G64")
    q, k, v, do = rand_inputs(65, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh)
    g32 = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, grad_dtype=torch.float32)
    off = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, grad_dtype=torch.float32,
                      residual_split=False)
    torch.cuda.synchronize()
    rdq, rdk, rdv, ro, rlse = O.backward(q, k, v, do, G, sh)
    check("o", host(o), ro, BF16_REL_F, BF16_MAX_ABS)
    check("lse", host(lse), rlse, BF16_REL_F, BF16_MAX_ABS)
    for name, a, ref in zip(("dq", "dk", "dv"), g32, (rdq, rdk, rdv)):
        check(name, host(a), ref, BF16_REL_F, BF16_MAX_ABS)
    # dQ does not take the split; dV's error is P's rounding alone
    assert torch.equal(g32[0], off[0])
    _, dv_on = check("dv, split", host(g32[2]), rdv, BF16_REL_F, 1e-4)
    _, dv_off = check("dv, no split", host(off[2]), rdv, BF16_REL_F, 1e-1)
    _, dk_off = check("dk, no split", host(off[1]), rdk, BF16_REL_F, 1e-1)
    assert dv_off > 100 * dv_on


def test_growing_scores_move_the_reference_max():
    """Scores that climb along the keys: q_i and k_j lie near one direction u,
    k_j scaled by its in-group position, so a row's running maximum rises by
    about 85 raw units per 128-key tile, past the forward's lazy threshold
    (8 / (scale log2 e), 62.7 at d = 128) in nearly every tile.  O and l are
    then rescaled mid-row again and again; outputs and gradients must still
    match the oracle (the shifted head adds a wrap where the scores fall)."""
    B, L, Hq, Hkv, d, G, sh = 1, 2048, 2, 2, 128, 1024, 1
    say("[edge] growing scores")
    rng = np.random.default_rng(77)
    u = rng.standard_normal(d).astype(np.float32)
    pos = (np.arange(L) % G).astype(np.float32)
    q = u[None, None, None, :] + 0.3 * rng.standard_normal((B, L, Hq, d), dtype=np.float32)
    k = (u[None, None, None, :] * (0.005 * pos)[None, :, None, None]
         + 0.3 * rng.standard_normal((B, L, Hkv, d), dtype=np.float32))
    v = rng.standard_normal((B, L, Hkv, d), dtype=np.float32)
    do = rng.standard_normal((B, L, Hq, d), dtype=np.float32)
    q, k, v, do = (bf16_round(x.astype(np.float32)) for x in (q, k, v, do))
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh)
    g32 = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    rdq, rdk, rdv, ro, rlse = O.backward(q, k, v, do, G, sh)
    assert float(np.max(rlse)) > 60.0   # the scores really do climb
    check("o", host(o), ro, BF16_REL_F, BF16_MAX_ABS)
    check("lse", host(lse), rlse, BF16_REL_F, BF16_MAX_ABS)
    for name, a, ref in zip(("dk", "dv"), g32[1:], (rdk, rdv)):
        check(name, host(a), ref, BF16_REL_F, BF16_MAX_ABS)
    # dQ = scale sum_j dS_ij k_j takes dS rounded to bf16, and delta_i from
    # the bf16-stored O, as any bf16 attention backward does.  Here the k_j
    # share a large component along u and sum_j dS_ij = 0, so the sum cancels
    # down to |dq| < 0.7 while its terms reach |dS| |k| ~ 10^2: those two
    # roundings bound the error, not the size of dq.  (A model of the kernels'
    # arithmetic in fp64 puts nearly all of it on delta: with delta from the
    # exact O the same bf16 dS gives dq within 4e-5.)  First-order bound per
    # element, with 2^-8 (twice the bf16 rounding) per rounded value:
    #   scale 2^-8 (sum_j |dS_ij| |k_jc| + sum_c' |dO_ic' O_ic'| sum_j P_ij |k_jc|)
    # (P, dS from the oracle's lse and O), plus the usual 2e-2.
    gdq = host(g32[0])
    scale = 1.0 / np.sqrt(d)
    for h in range(Hq):
        m = O.allowed_mask(L, G, O.head_shift(h, Hq, G, sh))
        qh, kh, vh, dh = (x[0, :, h].astype(np.float64) for x in (q, k, v, do))
        oh = ro[0, :, h]
        P = np.where(m, np.exp(scale * qh @ kh.T - rlse[0, h][:, None]), 0.0)
        dS = P * (dh @ vh.T - (dh * oh).sum(1)[:, None])
        from_ds = np.abs(dS) @ np.abs(kh)
        from_delta = np.abs(dh * oh).sum(1)[:, None] * (P @ np.abs(kh))
        bound = scale * (from_ds + from_delta) * 2.0 ** -8 + BF16_MAX_ABS
        err = np.abs(gdq[0, :, h] - rdq[0, :, h])
        say(f"  dq[h{h}]    max_abs={err.max():.3e}, worst err/bound={float((err / bound).max()):.3f}")
        assert (err <= bound).all(), f"dq of head {h} outside the bf16-dS rounding bound"


# ---------------------------------------------------------------------------
# The five workloads at full size.
# ---------------------------------------------------------------------------

def test_workload_fwd_f32_L256():
    wl = CONFIGS["fwd_f32_L256"]
    say(f"[workload] {wl.name}")
    x = make_inputs(wl)
    tq, tk, tv = (dev(x[n], torch.float32) for n in ("q", "k", "v"))
    o, lse = s2.forward(tq, tk, tv, wl.G, wl.shifted_heads)
    torch.cuda.synchronize()
    ro, rlse = O.forward(x["q"], x["k"], x["v"], wl.G, wl.shifted_heads)
    check("o", host(o), ro, F32_TOL, F32_TOL)
    check("lse", host(lse), rlse, F32_TOL, F32_TOL)


def test_workload_fwd_bf16_L8k():
    wl = CONFIGS["fwd_bf16_L8k"]
    say(f"[workload] {wl.name}")
    x = make_inputs(wl)
    tq, tk, tv = (dev(x[n], BF) for n in ("q", "k", "v"))
    o, lse = s2.forward(tq, tk, tv, wl.G, wl.shifted_heads)
    torch.cuda.synchronize()
    ro, rlse = O.forward(x["q"], x["k"], x["v"], wl.G, wl.shifted_heads)
    check("o", host(o), ro, BF16_REL_F, BF16_MAX_ABS)
    check("lse", host(lse), rlse, BF16_REL_F, BF16_MAX_ABS)


def _group_sums_hold(wl, tdo, dk, dv, rope):
    """Over every KV head and group: sum_j dV_j = sum over its query heads of sum_i dO_i,
    and (without RoPE) sum_j dK_j = 0."""
    B, L, Hq, Hkv, G, r = wl.B, wl.L, wl.Hq, wl.Hkv, wl.G, wl.r
    worst_v, worst_k = 0.0, 0.0
    do64, dv64, dk64 = tdo.double(), dv.double(), dk.double()
    for hk in range(Hkv):
        s = O.head_shift(hk * r, Hq, G, wl.shifted_heads)
        for g in range(L // G):
            rows = torch.from_numpy(O.group_members(L, G, s, g)).cuda()
            want = do64[:, rows, hk * r:(hk + 1) * r].sum(dim=(1, 2))
            got = dv64[:, rows, hk].sum(dim=1)
            worst_v = max(worst_v, float((got - want).abs().max() / (want.abs().max() + 1)))
            if not rope:
                worst_k = max(worst_k, float(dk64[:, rows, hk].sum(dim=1).abs().max()))
    say(f"  group sums: dV vs dO rel {worst_v:.2e}; |sum dK| {worst_k:.2e}")
    assert worst_v < 2e-2
    if not rope:
        assert worst_k < 0.5   # a sum of G bf16 values of size ~1 that cancels exactly


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def _run_fwdbwd(wl, x, grad_dtype=BF, ds_max_mib=None, residual_split=None):
    """Forward and backward at full size into NaN-filled outputs (every
    element must be written); `ds_max_mib` bounds the dS tiles kept (None:
    the library default)."""
    rope = (wl.rope_base, wl.rope_orig_len) if wl.rope else None
    tq, tk, tv, tdo = (dev(x[n], BF) for n in ("q", "k", "v", "do"))
    B, L, Hq, Hkv, d = wl.B, wl.L, wl.Hq, wl.Hkv, wl.d
    o, lse = _nan(tq.shape, BF), _nan((B, Hq, L), torch.float32)
    fo = s2.make_opts(BF, rope=rope)
    nf = s2.s2attn_workspace_size(0, B, L, Hq, Hkv, d, wl.G, fo)
    wsf = torch.empty(nf, dtype=torch.uint8, device="cuda") if nf else None
    s2.s2attn_fwd_ex(tq, tk, tv, o, lse, B, L, Hq, Hkv, d, wl.G, wl.shifted_heads, fo, wsf, nf)
    del wsf
    bo = s2.make_opts(BF, grad_dtype=grad_dtype, rope=rope, ds_max_mib=ds_max_mib,
                      residual_split=residual_split)
    nb = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, wl.G, bo)
    wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dq = _nan(tq.shape, grad_dtype)
    dk, dv = _nan(tk.shape, grad_dtype), _nan(tv.shape, grad_dtype)
    s2.s2attn_bwd_ex(tq, tk, tv, o, lse, tdo, dq, dk, dv, B, L, Hq, Hkv, d, wl.G,
                     wl.shifted_heads, bo, wsb, nb)
    torch.cuda.synchronize()
    n0 = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, wl.G,
                                  s2.make_opts(BF, grad_dtype=grad_dtype, rope=rope, ds_max_mib=0))
    say(f"  workspace {nb / 2**30:.1f} GiB (dS tiles {'kept' if nb > n0 else 'not kept'})")
    del wsb
    return (tq, tk, tv, tdo), (o, lse, dq, dk, dv)


@pytest.mark.timeout(900)
def test_workload_fwdbwd_bf16_L32k():
    """The 32k training workload over whole tensors: O, LSE and fp32-stored
    dQ, dK, dV against the oracle run over all 128 (head, group) units; then
    the bf16-stored gradients, whose store rounding is within 2e-2 here
    (|dK|, |dV| < 8); then fp32-stored gradients again with the residual
    split forced on (off by default at this shape)."""
    from tests import oracle_pool
    wl = CONFIGS["fwdbwd_bf16_L32k"]
    say(f"[workload] {wl.name}, whole tensors")
    x = make_inputs(wl)
    ins, outs = _run_fwdbwd(wl, x, grad_dtype=torch.float32)
    outs = [host(t) for t in outs]
    say(f"  oracle over every unit ({oracle_pool.workers()} processes)")
    ro, rlse, rdq, rdk, rdv = oracle_pool.full_backward(x, wl.G, wl.shifted_heads)
    say(" gradients stored in fp32")
    for name, got, ref in zip(("o", "lse", "dq", "dk", "dv"), outs, (ro, rlse, rdq, rdk, rdv)):
        check(name, got, ref, BF16_REL_F, BF16_MAX_ABS)
    del outs
    _, outs16 = _run_fwdbwd(wl, x, grad_dtype=BF)
    say(" gradients stored in bf16")
    for name, got, ref in zip(("dq", "dk", "dv"), outs16[2:], (rdq, rdk, rdv)):
        check(name + "(bf16)", host(got), ref, BF16_REL_F, bf16_store_tol(ref))
    _group_sums_hold(wl, ins[3], outs16[3], outs16[4], rope=False)
    del outs16
    _, outs_s = _run_fwdbwd(wl, x, grad_dtype=torch.float32, residual_split=True)
    say(" gradients stored in fp32, residual split forced on")
    for name, got, ref in zip(("dq", "dk", "dv"), outs_s[2:], (rdq, rdk, rdv)):
        check(name, host(got), ref, BF16_REL_F, BF16_MAX_ABS)


def _unit_parity(wl, x, outs, units, grads_f32, o_lse=True):
    """Compare the outputs of whole KV units (all their query heads) with the oracle."""
    from tests import oracle_pool
    o, lse, dq, dk, dv = outs
    rope = (wl.rope_base, wl.rope_orig_len) if wl.rope else None
    res = oracle_pool.kv_units(x, wl.G, wl.shifted_heads, units, rope)
    for (b, hk, g) in units:
        r = res[(b, hk, g)]
        rows = torch.from_numpy(r["rows"]).cuda()
        heads = list(range(hk * wl.r, (hk + 1) * wl.r))
        say(f" unit b={b} kv_head={hk} group={g}")
        if o_lse:
            check("o", np.stack([host(o[b, rows, h]) for h in heads]), r["o"], BF16_REL_F, BF16_MAX_ABS)
            check("lse", np.stack([host(lse[b, h, rows]) for h in heads]), r["lse"], BF16_REL_F,
                  BF16_MAX_ABS)
        gdq = np.stack([host(dq[b, rows, h]) for h in heads])
        for name, got, ref in (("dq", gdq, r["dq"]), ("dk", host(dk[b, rows, hk]), r["dk"]),
                               ("dv", host(dv[b, rows, hk]), r["dv"])):
            if grads_f32:
                check(name, got, ref, BF16_REL_F, BF16_MAX_ABS)
            else:
                check(name + "(bf16)", got, ref, BF16_REL_F, bf16_store_tol(ref))


@pytest.mark.timeout(900)
def test_workload_fwdbwd_bf16_L100k_rope():
    """100k tokens with RoPE-PI: four units (an unshifted first group, two
    shifted groups, the shifted group that wraps), fp32-stored gradients with
    the dS tiles kept (85 GB, bound raised to 96 GiB), then bf16-stored with
    the default bound (dQ recomputes); group sums over every unit."""
    wl = CONFIGS["fwdbwd_bf16_L100k_rope"]
    say(f"[workload] {wl.name}")
    x = make_inputs(wl)
    units = [(0, 0, 0), (0, 16, 1), (0, 31, 3), (0, 9, 2)]
    ins, outs = _run_fwdbwd(wl, x, grad_dtype=torch.float32, ds_max_mib=96 << 10)
    _group_sums_hold(wl, ins[3], outs[3], outs[4], rope=True)
    say(" gradients stored in fp32, dS kept")
    _unit_parity(wl, x, outs, units, grads_f32=True)
    del outs
    _, outs16 = _run_fwdbwd(wl, x, grad_dtype=BF)
    say(" gradients stored in bf16, dQ recomputed")
    _unit_parity(wl, x, outs16, units[2:], grads_f32=False, o_lse=False)


@pytest.mark.timeout(600)
def test_workload_fwdbwd_bf16_L32k_gqa():
    """The grouped-query 32k workload: every KV head (8 units of 8 query
    heads; KV heads 4-7 serve the shifted query heads, KV head 7 in the group
    that wraps), fp32-stored gradients with the dS tiles kept (16.5 GiB, bound
    raised), then bf16-stored with the default bound (dQ recomputes)."""
    wl = CONFIGS["fwdbwd_bf16_L32k_gqa"]
    say(f"[workload] {wl.name}")
    x = make_inputs(wl)
    units = [(0, hk, hk % wl.n_groups) for hk in range(wl.Hkv)]
    ins, outs = _run_fwdbwd(wl, x, grad_dtype=torch.float32, ds_max_mib=32 << 10)
    _group_sums_hold(wl, ins[3], outs[3], outs[4], rope=False)
    say(" gradients stored in fp32, dS kept")
    _unit_parity(wl, x, outs, units, grads_f32=True)
    del outs
    _, outs16 = _run_fwdbwd(wl, x, grad_dtype=BF)
    say(" gradients stored in bf16, dQ recomputed")
    _unit_parity(wl, x, outs16, units[3:], grads_f32=False, o_lse=False)


def _causal_rows(G):
    """In-group rows to sample: the first, tile edges (32 / 64 / 128 / 256) on
    both sides, the middle, and the last rows of the group."""
    edges = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257}
    return sorted(edges | {G // 2 - 1, G // 2, G - 257, G - 256, G - 129, G - 128, G - 2, G - 1})


@pytest.mark.timeout(600)
def test_plane_at_the_32bit_offset_limit():
    """The kernels address a tile row as a (batch, head) plane base plus a
    32-bit byte offset, so the host accepts planes L H d 2 below 2^31 bytes.
    Here a plane is 2^31 - 2^24 bytes: L = 520192, 16 heads, d = 128, G = 4096,
    the longest L the host accepts at this head count and group size (one
    more group reaches 2^31), with half the heads shifted.  The dS tiles are
    kept (about 36 GB of workspace, past 2^32 bytes), and the fp32 gradients
    are 4.3 GB per tensor.  The inputs are standard normals rounded to bf16,
    drawn on the device by a seeded torch generator (no period, so an offset
    that wrapped would read different values).  Units with rows at the
    plane's far end, the wrap group of a shifted head (rows at both ends)
    and the first and a middle unit match the oracle, rows gathered with the
    oracle's own row map."""
    import math
    from tests import oracle_pool
    B, L, Hq, Hkv, d, G, sh = 1, 520192, 16, 16, 128, 4096, 8
    assert L * Hq * d * 2 == 2**31 - 2**24 and (L + G) * Hq * d * 2 == 2**31
    say("[plane limit] L=520192 H=16 d=128 G=4096")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(52)
    tq, tk, tv, tdo = (torch.randn((B, L, H, d), generator=gen, device="cuda").to(BF)
                       for H in (Hq, Hkv, Hkv, Hq))
    ds_mib = 48 << 10
    opts = s2.make_opts(BF, grad_dtype=torch.float32, ds_max_mib=ds_mib)
    assert s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts) > 2**32   # dS tiles kept
    o, lse = s2.forward(tq, tk, tv, G, sh)
    dq, dk, dv = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, grad_dtype=torch.float32,
                             ds_max_mib=ds_mib)
    torch.cuda.synchronize()
    n_g = L // G
    units = [(0, 7, n_g - 1), (0, 15, n_g - 1), (0, 15, 0), (0, 0, n_g // 2)]
    scale = 1.0 / math.sqrt(d)
    f64 = lambda t: t.double().cpu().numpy()
    tasks, rows_of = [], {}
    for b, h, g in units:
        rows = O.unit_rows(L, G, Hq, sh, h, g)
        idx = torch.as_tensor(rows, device="cuda")
        rows_of[(b, h, g)] = idx
        tasks.append(((b, h, g), f64(tq[b, idx, h])[None], f64(tk[b, idx, h]), f64(tv[b, idx, h]),
                      f64(tdo[b, idx, h])[None], scale, None))
    ref = oracle_pool.kv_units_gathered(tasks)
    for (b, h, g), idx in rows_of.items():
        u = ref[(b, h, g)]
        tag = f"unit ({b},{h},{g})"
        check("o " + tag, f64(o[b, idx, h]), u["o"][0], BF16_REL_F, BF16_MAX_ABS)
        check("lse " + tag, f64(lse[b, h, idx]), u["lse"][0], BF16_REL_F, BF16_MAX_ABS)
        check("dq " + tag, f64(dq[b, idx, h]), u["dq"][0], BF16_REL_F, BF16_MAX_ABS)
        check("dk " + tag, f64(dk[b, idx, h]), u["dk"], BF16_REL_F, BF16_MAX_ABS)
        check("dv " + tag, f64(dv[b, idx, h]), u["dv"], BF16_REL_F, BF16_MAX_ABS)


def test_token_row_at_the_24bit_limit():
    """Row offsets are formed as a 24-bit by 24-bit product of row index and
    row bytes, so the host accepts token rows H d 2 below 2^24 bytes.  Here
    65535 heads of d = 128 make a row of 2^24 - 256 bytes (one head more
    reaches 2^24), with L = 64, G = 32 and half the heads shifted.  The
    131070 units are not a multiple of the 8 XCDs, so the work decode takes
    its unaligned form.  Units of the last heads (the largest offsets inside a
    row), a shifted head's wrap group and the first unit match the oracle."""
    import math
    from tests import oracle_pool
    B, L, Hq, Hkv, d, G, sh = 1, 64, 65535, 65535, 128, 32, 32768
    assert Hq * d * 2 == 2**24 - 256 and (Hq + 1) * d * 2 == 2**24
    say("[row limit] H=65535 d=128 L=64 G=32")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(53)
    tq, tk, tv, tdo = (torch.randn((B, L, H, d), generator=gen, device="cuda").to(BF)
                       for H in (Hq, Hkv, Hkv, Hq))
    o, lse = s2.forward(tq, tk, tv, G, sh)
    dq, dk, dv = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    units = [(0, Hq - 1, 1), (0, Hq - 1, 0), (0, Hq - sh - 1, 1), (0, 0, 0)]
    scale = 1.0 / math.sqrt(d)
    f64 = lambda t: t.double().cpu().numpy()
    tasks, rows_of = [], {}
    for b, h, g in units:
        idx = torch.as_tensor(O.unit_rows(L, G, Hq, sh, h, g), device="cuda")
        rows_of[(b, h, g)] = idx
        tasks.append(((b, h, g), f64(tq[b, idx, h])[None], f64(tk[b, idx, h]), f64(tv[b, idx, h]),
                      f64(tdo[b, idx, h])[None], scale, None))
    ref = oracle_pool.kv_units_gathered(tasks)
    for (b, h, g), idx in rows_of.items():
        u = ref[(b, h, g)]
        tag = f"unit ({b},{h},{g})"
        check("o " + tag, f64(o[b, idx, h]), u["o"][0], BF16_REL_F, BF16_MAX_ABS)
        check("lse " + tag, f64(lse[b, h, idx]), u["lse"][0], BF16_REL_F, BF16_MAX_ABS)
        check("dq " + tag, f64(dq[b, idx, h]), u["dq"][0], BF16_REL_F, BF16_MAX_ABS)
        check("dk " + tag, f64(dk[b, idx, h]), u["dk"], BF16_REL_F, BF16_MAX_ABS)
        check("dv " + tag, f64(dv[b, idx, h]), u["dv"], BF16_REL_F, BF16_MAX_ABS)


@pytest.mark.parametrize("name", ["fwd_bf16_causal_L32k", "fwd_bf16_causal_L100k"])
def test_workload_dense_causal(name):
    """Dense causal attention (one group spanning the context, no shift), the
    inference pass: sampled rows of several heads against the oracle, row by
    row, and every output finite."""
    wl = CONFIGS[name]
    say(f"[workload] {wl.name}")
    x = make_inputs(wl)
    tq, tk, tv = (dev(x[n], BF) for n in ("q", "k", "v"))
    o, lse = s2.forward(tq, tk, tv, wl.G, wl.shifted_heads)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    # query 0 sees only itself: o = v exactly
    assert torch.equal(o[:, 0], tv[:, 0].repeat_interleave(wl.r, dim=1))
    rows = _causal_rows(wl.G)
    for h in (0, 13, wl.Hq - 1):
        toks, ro, rl = O.sampled_rows_forward(x["q"], x["k"], x["v"], wl.G, wl.shifted_heads,
                                              0, h, 0, rows)
        tt = torch.from_numpy(toks).cuda()
        say(f" head {h}: {len(rows)} rows")
        check("o", host(o[0, tt, h]), ro, BF16_REL_F, BF16_MAX_ABS)
        check("lse", host(lse[0, h, tt]), rl, BF16_REL_F, BF16_MAX_ABS)


@pytest.mark.parametrize("sh", [0, 32])
def test_shift_counts_full_size(sh):
    """The 32k training shape with no shifted head (plain short attention) and
    with every head shifted: sampled units and group sums."""
    wl = CONFIGS["fwdbwd_bf16_L32k"]
    say(f"[shift count] {wl.name} shifted_heads={sh}")
    x = make_inputs(wl)
    wl2 = dataclasses.replace(wl, shifted_heads=sh, name=f"{wl.name}_sh{sh}")
    ins, outs = _run_fwdbwd(wl2, x, grad_dtype=torch.float32)
    _group_sums_hold(wl2, ins[3], outs[3], outs[4], rope=False)
    _unit_parity(wl2, x, outs, [(0, 5, 3), (0, 30, 0)], grads_f32=True)


def test_d64_gqa_rope_full_size():
    """d = 64 at a training length: L 32768, G 8192, 16 query / 4 KV heads
    (8 shifted), RoPE-PI.  The d = 64 instantiations of every kernel (forward,
    dK/dV with the dS tiles, dQ from them, the RoPE pre-pass and epilogues) at
    full size: sampled units, one unshifted and the shifted last group that
    wraps, and the group sums over every unit."""
    wl = dataclasses.replace(CONFIGS["fwdbwd_bf16_L32k"], name="fwdbwd_bf16_L32k_d64_gqa_rope",
                             Hq=16, Hkv=4, d=64, shifted_heads=8, seed=33, rope=True)
    say(f"[d64] {wl.name}")
    x = make_inputs(wl)
    ins, outs = _run_fwdbwd(wl, x, grad_dtype=torch.float32)
    _group_sums_hold(wl, ins[3], outs[3], outs[4], rope=True)
    _unit_parity(wl, x, outs, [(0, 0, 1), (0, 3, 3)], grads_f32=True)


def test_dispatch_bands_with_a_partial_last_band():
    """40 (head, group) units of one 32768-token group each at d = 64: 5 units
    per XCD.  The forward, dK/dV and the recomputing dQ re-read 8 MiB per unit,
    so they dispatch in bands of 4 units and the last band holds one; dQ from
    the stored dS re-reads 4 MiB and takes all 5 in one band.  Every output is
    written (NaN-filled buffers come back finite), sampled rows of heads in
    both bands match the oracle, the group sums hold over every unit, dK and
    dV agree bitwise with and without stored dS, and the two dQ agree."""
    B, L, Hq, Hkv, d, G, sh = 1, 32768, 40, 40, 64, 32768, 20
    say("[bands] L32768 G32768 H40 d64")
    q, k, v, do = rand_inputs(4040, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))

    def nan(shape, dtype):
        return torch.full(shape, float("nan"), dtype=dtype, device="cuda")

    o, lse = nan(tq.shape, BF), nan((B, Hq, L), torch.float32)
    s2.s2attn_fwd_ex(tq, tk, tv, o, lse, B, L, Hq, Hkv, d, G, sh, s2.make_opts(BF), None, 0)
    grads = {}
    for ds_max in (64 << 10, 0):   # dS tiles kept (43 GB), then not kept
        opts = s2.make_opts(BF, grad_dtype=torch.float32, ds_max_mib=ds_max)
        wsb = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
        assert (wsb > 40e9) == (ds_max > 0)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        g = tuple(nan(t.shape, torch.float32) for t in (tq, tk, tv))
        s2.s2attn_bwd_ex(tq, tk, tv, o, lse, tdo, *g, B, L, Hq, Hkv, d, G, sh, opts, ws, wsb)
        torch.cuda.synchronize()
        del ws
        grads[ds_max > 0] = g
    for t in (o, lse) + grads[True] + grads[False]:
        assert bool(torch.isfinite(t).all())
    assert torch.equal(grads[True][1], grads[False][1]) and torch.equal(grads[True][2], grads[False][2])
    check("dq (stored dS vs recomputed)", host(grads[True][0]), host(grads[False][0]),
          BF16_REL_F, BF16_MAX_ABS)
    wl = dataclasses.replace(CONFIGS["fwdbwd_bf16_L32k"], name="bands", Hq=Hq, Hkv=Hkv, d=d, G=G,
                             shifted_heads=sh)
    _group_sums_hold(wl, tdo, grads[False][1], grads[False][2], rope=False)
    rows = _causal_rows(G)
    for h in (3, 19, 20, 35, 39):   # units 32..39 form the partial band
        toks, ro, rl = O.sampled_rows_forward(q, k, v, G, sh, 0, h, 0, rows)
        tt = torch.from_numpy(toks).cuda()
        say(f" head {h}: {len(rows)} rows")
        check("o", host(o[0, tt, h]), ro, BF16_REL_F, BF16_MAX_ABS)
        check("lse", host(lse[0, h, tt]), rl, BF16_REL_F, BF16_MAX_ABS)


# ---------------------------------------------------------------------------
# Kernel-level invariants.
# ---------------------------------------------------------------------------

INV_SHAPE = dict(B=1, L=2048, Hq=4, Hkv=4, d=128, G=512, sh=2)


def _inv_inputs(seed=7):
    s = INV_SHAPE
    return rand_inputs(seed, s["B"], s["L"], s["Hq"], s["Hkv"], s["d"])


def _all_outputs(q, k, v, do, grad_dtype=BF):
    s = INV_SHAPE
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, s["G"], s["sh"])
    dq, dk, dv = s2.backward(tq, tk, tv, o, lse, tdo, s["G"], s["sh"], grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o, lse, dq, dk, dv)]


def test_run_to_run_bit_determinism():
    say("[invariant] determinism")
    x = _inv_inputs()
    a, b = _all_outputs(*x), _all_outputs(*x)
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_group_independence_bitwise():
    say("[invariant] group independence")
    s = INV_SHAPE
    q, k, v, do = _inv_inputs(8)
    base = _all_outputs(q, k, v, do)
    h, g = 3, 1   # a shifted head
    rows = O.unit_rows(s["L"], s["G"], s["Hq"], s["sh"], h, g)
    rng = np.random.default_rng(9)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[0, rows, h] = bf16_round(rng.standard_normal((len(rows), s["d"]), dtype=np.float32))
    pert = _all_outputs(q2, k2, v2, do2)
    other = torch.from_numpy(np.setdiff1d(np.arange(s["L"]), rows))
    rows_t = torch.from_numpy(rows)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), base, pert):
        if name == "lse":
            assert torch.equal(a[0, h, other], b[0, h, other]), name
            assert not torch.equal(a[0, h, rows_t], b[0, h, rows_t]), name
            assert torch.equal(a[0, :h], b[0, :h]), name
        else:
            assert torch.equal(a[0, other, h], b[0, other, h]), name
            assert not torch.equal(a[0, rows_t, h], b[0, rows_t, h]), name
            assert torch.equal(a[0, :, :h], b[0, :, :h]), name


def test_roll_by_group_equivariance_bitwise():
    say("[invariant] roll by G")
    s = INV_SHAPE
    x = _inv_inputs(10)
    a = _all_outputs(*x)
    b = _all_outputs(*(np.roll(t, s["G"], axis=1) for t in x))
    for name, u, w in zip(("o", "lse", "dq", "dk", "dv"), a, b):
        ax = 2 if name == "lse" else 1
        assert torch.equal(torch.roll(u, s["G"], dims=ax), w), name


def test_every_output_written_and_no_stray_writes():
    """Outputs pre-filled with NaN come back finite; sentinels around every
    output buffer are untouched."""
    say("[invariant] nan-fill and redzones")
    s = INV_SHAPE
    q, k, v, do = _inv_inputs(11)
    B, L, Hq, Hkv, d, G, sh = s["B"], s["L"], s["Hq"], s["Hkv"], s["d"], s["G"], s["sh"]
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    pad = 4096
    SENT = -1024.0   # exact in bf16 and fp32

    def padded(n, dtype):
        buf = torch.full((n + 2 * pad,), SENT, dtype=dtype, device="cuda")
        body = buf[pad:pad + n]
        body.fill_(float("nan"))
        return buf, body

    nq, nk, nl = B * L * Hq * d, B * L * Hkv * d, B * Hq * L
    ob, o = padded(nq, BF)
    lb, lse = padded(nl, torch.float32)
    s2.s2attn_fwd(tq, tk, tv, o, lse, B, L, Hq, Hkv, d, G, sh)
    dqb, dq = padded(nq, BF)
    dkb, dk = padded(nk, BF)
    dvb, dv = padded(nk, BF)
    deb, de = padded(nl, torch.float32)       # the row term, [B, Hq, L]
    s2.s2attn_bwd(tq, tk, tv, o, lse, tdo, dq, dk, dv, de, B, L, Hq, Hkv, d, G, sh)
    torch.cuda.synchronize()
    for buf, body in ((ob, o), (lb, lse), (dqb, dq), (dkb, dk), (dvb, dv), (deb, de)):
        assert torch.isfinite(body.float()).all()
        assert (buf[:pad].float() == SENT).all() and (buf[-pad:].float() == SENT).all()
    # and the values are right
    rdq, rdk, rdv, ro, rl = O.backward(q, k, v, do, G, sh)
    check("o", host(o.view(B, L, Hq, d)), ro, BF16_REL_F, BF16_MAX_ABS)
    check("dk", host(dk.view(B, L, Hkv, d)), rdk, BF16_REL_F, BF16_MAX_ABS)


@pytest.mark.parametrize("rope", [None, (10000.0, 64)])
def test_workspace_writes_stay_inside(rope):
    """The _ex backward writes only inside its workspace (delta, rotated q/k,
    the dS tiles of a ragged group: G = 200 leaves an 8-query last tile),
    and the stored-dS dQ path agrees with the recomputing one, reached both
    through s2attn_bwd and through opts.ds_max_mib = 0."""
    B, L, Hq, Hkv, d, G, sh = 1, 600, 4, 2, 128, 200, 2
    say(f"[invariant] workspace redzones rope={rope}")
    q, k, v, do = rand_inputs(31, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh, rope=rope)
    opts = s2.make_opts(BF, rope=rope)
    n = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
    NB = ((G + 31) // 32 + 7) // 8
    assert n >= B * Hq * (L // G) * 32 * NB * (NB + 1) * 2048
    pad = 1 << 16
    SENT = 0x5A
    buf = torch.full((n + 2 * pad,), SENT, dtype=torch.uint8, device="cuda")
    ws = buf[pad:pad + n]
    dq, dk, dv = (torch.empty_like(x) for x in (tq, tk, tv))
    s2.s2attn_bwd_ex(tq, tk, tv, o, lse, tdo, dq, dk, dv, B, L, Hq, Hkv, d, G, sh, opts, ws, n)
    torch.cuda.synchronize()
    assert (buf[:pad] == SENT).all() and (buf[-pad:] == SENT).all()
    rdq, rdk, rdv, _, _ = O.backward(q, k, v, do, G, sh, rope=rope)
    for name, a, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        check(name, host(a), ref, BF16_REL_F, bf16_store_tol(ref))
    if rope is None:
        pq = torch.empty_like(tq)
        pk, pv = torch.empty_like(tk), torch.empty_like(tv)
        de = torch.empty(B * Hq * L, dtype=torch.float32, device="cuda")
        s2.s2attn_bwd(tq, tk, tv, o, lse, tdo, pq, pk, pv, de, B, L, Hq, Hkv, d, G, sh)
        torch.cuda.synchronize()
        check("dq (recompute path)", host(pq), rdq, BF16_REL_F, bf16_store_tol(rdq))
        assert torch.equal(pk, dk) and torch.equal(pv, dv)   # same dK/dV kernel
    # ds_max_mib = 0: a smaller workspace without dS tiles, and dQ recomputes
    n0 = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, s2.make_opts(BF, rope=rope, ds_max_mib=0))
    assert n0 < n
    zq, zk, zv = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, rope=rope, ds_max_mib=0)
    torch.cuda.synchronize()
    check("dq (ds_max_mib=0)", host(zq), rdq, BF16_REL_F, bf16_store_tol(rdq))
    assert torch.equal(zk, dk) and torch.equal(zv, dv)
    if rope is None:
        assert torch.equal(zq, pq)   # the same recomputing kernel as s2attn_bwd


@pytest.mark.parametrize("rope", [None, (10000.0, 64)])
def test_backward_stages_equal_one_call(rope):
    """PRE, DKDV, DQ through s2attn_bwd_stage_ex, in that order on one stream,
    give bitwise the gradients of one s2attn_bwd_ex call (the DQ stage reads
    the dS tiles DKDV left in the workspace)."""
    B, L, Hq, Hkv, d, G, sh = 1, 600, 4, 2, 128, 200, 2
    say(f"[stages] rope={rope}")
    q, k, v, do = rand_inputs(41, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh, rope=rope)
    ref = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, rope=rope)
    opts = s2.make_opts(BF, rope=rope)
    n = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (tq, tk, tv))
    for stage in (s2.S2ATTN_BWD_STAGE_PRE, s2.S2ATTN_BWD_STAGE_DKDV, s2.S2ATTN_BWD_STAGE_DQ):
        s2.s2attn_bwd_stage_ex(stage, tq, tk, tv, o, lse, tdo, dq, dk, dv, B, L, Hq, Hkv, d, G, sh,
                               opts, ws, n)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("rope", [None, (10000.0, 64)])
def test_backward_stages_on_two_streams_without_ds(rope):
    """Without dS tiles in the workspace (ds_max_mib = 0), DKDV and DQ read
    only PRE's results and the inputs, so they may run concurrently: PRE on
    one stream, then DKDV and DQ on two others that wait for it.  The
    gradients equal one recomputing s2attn_bwd_ex call bit for bit."""
    B, L, Hq, Hkv, d, G, sh = 1, 600, 4, 2, 128, 200, 2
    say(f"[stages, two streams] rope={rope}")
    q, k, v, do = rand_inputs(43, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh, rope=rope)
    ref = s2.backward(tq, tk, tv, o, lse, tdo, G, sh, rope=rope, ds_max_mib=0)
    opts = s2.make_opts(BF, rope=rope, ds_max_mib=0)
    n = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (tq, tk, tv))
    torch.cuda.synchronize()
    s_pre, s_kv, s_q = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    args = (tq, tk, tv, o, lse, tdo, dq, dk, dv, B, L, Hq, Hkv, d, G, sh, opts, ws, n)
    s2.s2attn_bwd_stage_ex(s2.S2ATTN_BWD_STAGE_PRE, *args, stream=s_pre)
    done = torch.cuda.Event()
    done.record(s_pre)
    s_kv.wait_event(done)
    s_q.wait_event(done)
    s2.s2attn_bwd_stage_ex(s2.S2ATTN_BWD_STAGE_DKDV, *args, stream=s_kv)
    s2.s2attn_bwd_stage_ex(s2.S2ATTN_BWD_STAGE_DQ, *args, stream=s_q)
    torch.cuda.synchronize()
    for name, a, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert torch.equal(a, want), name


@pytest.mark.parametrize("d,Hkv", [(128, 2), (64, 4)])
def test_fused_query_rotation_equals_the_prepass(d, Hkv):
    """With RoPE the forward rotates its query fragments in registers, while the
    backward's pre-pass writes rotated q~ and k~ to its workspace (after the row
    term, each part 256-byte aligned, as the header lays it out).  Both call one
    rotation, so a forward without RoPE on those q~ and k~ reproduces the fused
    forward's o and lse bit for bit (rows of wrapped, shifted and ragged groups
    included: L = 600, G = 200)."""
    B, L, Hq, G, sh = 1, 600, 4, 200, 2
    rope = (10000.0, 64)
    say(f"[fused rotation] d={d} Hkv={Hkv}")
    q, k, v, do = rand_inputs(47, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    o, lse = s2.forward(tq, tk, tv, G, sh, rope=rope)
    opts = s2.make_opts(BF, rope=rope)
    n = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (tq, tk, tv))
    s2.s2attn_bwd_stage_ex(s2.S2ATTN_BWD_STAGE_PRE, tq, tk, tv, o, lse, tdo, dq, dk, dv,
                           B, L, Hq, Hkv, d, G, sh, opts, ws, n)
    torch.cuda.synchronize()
    r256 = lambda x: (x + 255) // 256 * 256
    nq, nk = B * L * Hq * d * 2, B * L * Hkv * d * 2
    off_q = r256(B * Hq * L * 4)
    off_k = off_q + r256(nq)
    assert off_k + nk <= n
    qr = ws[off_q:off_q + nq].view(BF).view(B, L, Hq, d).clone()
    kr = ws[off_k:off_k + nk].view(BF).view(B, L, Hkv, d).clone()
    assert not torch.equal(qr, tq) and not torch.equal(kr, tk)   # rotated
    o2, lse2 = s2.forward(qr, kr, tv, G, sh)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(lse, lse2)


def test_graph_capture_replays_bitwise():
    """The forward and backward enqueue only kernel launches on the caller's
    stream (no allocation, copy, memset or synchronisation), so a caller can
    capture them in a HIP graph.  Captured once with RoPE on (rotation
    pre-passes, forward, row term, dK/dV, dQ from stored dS) and replayed three
    times, with other eager work and a synchronisation between replays, every
    replay reproduces the eager results bit for bit."""
    B, L, Hq, Hkv, d, G, sh = 1, 1024, 4, 2, 128, 256, 2
    rope = (10000.0, 256)
    say("[graph] capture and replay")
    q, k, v, do = rand_inputs(91, B, L, Hq, Hkv, d)
    tq, tk, tv, tdo = (dev(x, BF) for x in (q, k, v, do))
    opts = s2.make_opts(BF, rope=rope)
    nf = s2.s2attn_workspace_size(0, B, L, Hq, Hkv, d, G, opts)
    nb = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
    wsf = torch.empty(nf, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(tq)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x) for x in (tq, tk, tv))
    outs = (o, lse, dq, dk, dv)

    def run():
        s2.s2attn_fwd_ex(tq, tk, tv, o, lse, B, L, Hq, Hkv, d, G, sh, opts, wsf, nf)
        s2.s2attn_bwd_ex(tq, tk, tv, o, lse, tdo, dq, dk, dv, B, L, Hq, Hkv, d, G, sh, opts, wsb, nb)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    a = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        a = torch.tanh(a @ a.T)          # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager run"
