"""Pins for the CPU oracle: facts fixed by the pages and by the mathematics.

Each test ties the oracle to something other than itself: the blog's worked
shift example, a library routine (torch scaled_dot_product_attention and
autograd in float64), closed forms, invariants the method implies, and
central finite differences.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import s2attn as O

RNG = np.random.default_rng(12345)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def qkv(B, L, Hq, Hkv, d, rng=RNG, grad=False):
    q, k, v = rand(B, L, Hq, d, rng=rng), rand(B, L, Hkv, d, rng=rng), rand(B, L, Hkv, d, rng=rng)
    if grad:
        return q, k, v, rand(B, L, Hq, d, rng=rng)
    return q, k, v


# --------------------------------------------------------------------------
# Index map: the blog's worked example (section 3.3).
# --------------------------------------------------------------------------

def test_blog_shift_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "shift_example_blog_s33.json")))
    L, G, s = ex["L"], ex["G"], ex["shift"]
    for g, want in enumerate(ex["unshifted_groups_1based"]):
        assert list(O.group_members(L, G, 0, g) + 1) == want
    for g, printed in enumerate(ex["shifted_groups_1based_as_printed"]):
        want = [((p - 1) % L) + 1 for p in printed]  # cyclic reading of 13, 14
        assert list(O.group_members(L, G, s, g) + 1) == want
    # the shift of a shifted head is half a group
    assert O.head_shift(3, 4, G, 2) == s and O.head_shift(0, 4, G, 2) == 0


def test_brute_force_loops_on_the_blog_example(golden_dir):
    """Plain Python loops, no numpy algebra, on the blog's 12-token, 4-token
    group example: each head's groups are read off the golden fixture (the
    shifted head's as printed, with the cyclic reading of 13 and 14); query t
    attends to the members of its group up to and including itself, in group
    order.  O, LSE and all three gradients from those loops (dS = P (dP - D),
    D = dO . O) must equal the oracle's group form."""
    ex = json.load(open(os.path.join(golden_dir, "shift_example_blog_s33.json")))
    L, G = ex["L"], ex["G"]
    groups = {0: [[t - 1 for t in grp] for grp in ex["unshifted_groups_1based"]],
              1: [[(t - 1) % L for t in grp] for grp in ex["shifted_groups_1based_as_printed"]]}
    Hq, d = 2, 3
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal((1, L, Hq, d)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    o = [[[0.0] * d for _ in range(Hq)] for _ in range(L)]
    lse = [[0.0] * L for _ in range(Hq)]
    dq, dk, dv = ([[[0.0] * d for _ in range(Hq)] for _ in range(L)] for _ in range(3))
    for h in range(Hq):
        for grp in groups[h]:
            for a, t in enumerate(grp):
                keys = grp[:a + 1]
                sc = [scale * sum(q[0, t, h, c] * k[0, j, h, c] for c in range(d)) for j in keys]
                mx = max(sc)
                z = sum(math.exp(x - mx) for x in sc)
                P = [math.exp(x - mx) / z for x in sc]
                lse[h][t] = mx + math.log(z)
                for c in range(d):
                    o[t][h][c] = sum(P[n] * v[0, j, h, c] for n, j in enumerate(keys))
                D = sum(do[0, t, h, c] * o[t][h][c] for c in range(d))
                for n, j in enumerate(keys):
                    dP = sum(do[0, t, h, c] * v[0, j, h, c] for c in range(d))
                    dS = P[n] * (dP - D)
                    for c in range(d):
                        dq[t][h][c] += scale * dS * k[0, j, h, c]
                        dk[j][h][c] += scale * dS * q[0, t, h, c]
                        dv[j][h][c] += P[n] * do[0, t, h, c]
    rdq, rdk, rdv, ro, rl = O.backward(q, k, v, do, G, 1)
    np.testing.assert_allclose(ro[0], np.array(o), atol=1e-12)
    np.testing.assert_allclose(rl[0], np.array(lse), atol=1e-12)
    np.testing.assert_allclose(rdq[0], np.array(dq), atol=1e-12)
    np.testing.assert_allclose(rdk[0], np.array(dk), atol=1e-12)
    np.testing.assert_allclose(rdv[0], np.array(dv), atol=1e-12)


def test_index_maps_inverse():
    for L, s in [(12, 2), (16, 4), (24, 3)]:
        t = np.arange(L)
        assert np.array_equal(O.rolled_to_original(O.original_to_rolled(t, L, s), L, s), t)


def test_allowed_mask_structure():
    L, G = 16, 4
    for s in (0, 2):
        M = O.allowed_mask(L, G, s)
        assert M.diagonal().all()                       # no empty row
        assert M.sum() == (L // G) * G * (G + 1) // 2   # G(G+1)/2 pairs per group
        for g in range(L // G):
            rows = O.group_members(L, G, s, g)
            sub = M[np.ix_(rows, rows)]
            assert np.array_equal(sub, np.tril(np.ones((G, G), bool)))


# --------------------------------------------------------------------------
# Group form (gather / dense causal / scatter) vs explicit-mask form.
# --------------------------------------------------------------------------

def _sweep():
    for L, G in [(8, 2), (8, 4), (8, 8), (12, 4), (12, 6), (16, 4), (16, 8), (24, 6), (24, 8)]:
        for Hq, Hkv in [(2, 1), (2, 2), (4, 1), (4, 2), (4, 4)]:
            for d in (4, 8):
                for sh in sorted({0, Hq // 2, Hq}):
                    yield L, G, Hq, Hkv, d, sh


@pytest.mark.parametrize("rope", [None, (10000.0, 4)])
def test_group_form_matches_explicit_mask(rope):
    rng = np.random.default_rng(7)
    worst = 0.0
    for i, (L, G, Hq, Hkv, d, sh) in enumerate(_sweep()):
        B = 1 + (i % 2)
        q, k, v, do = qkv(B, L, Hq, Hkv, d, rng=rng, grad=True)
        o1, l1 = O.forward(q, k, v, G, sh, rope=rope)
        o2, l2 = O.forward_dense(q, k, v, G, sh, rope=rope)
        g1 = O.backward(q, k, v, do, G, sh, rope=rope)[:3]
        g2 = O.backward_dense(q, k, v, do, G, sh, rope=rope)
        for a, b in [(o1, o2), (l1, l2)] + list(zip(g1, g2)):
            worst = max(worst, float(np.max(np.abs(a - b))))
    assert worst <= 1e-12, worst


# --------------------------------------------------------------------------
# Against torch's SDPA and autograd (float64, CPU) with the explicit mask.
# --------------------------------------------------------------------------

def _torch_masked(q, k, v, G, sh, scale=None):
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    tq = torch.tensor(q).permute(0, 2, 1, 3).contiguous().requires_grad_()
    tk = torch.tensor(k).permute(0, 2, 1, 3).contiguous().requires_grad_()
    tv = torch.tensor(v).permute(0, 2, 1, 3).contiguous().requires_grad_()
    masks = torch.stack([torch.tensor(O.allowed_mask(L, G, O.head_shift(h, Hq, G, sh)))
                         for h in range(Hq)])[None]
    ke = tk.repeat_interleave(r, dim=1)
    ve = tv.repeat_interleave(r, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, attn_mask=masks, scale=scale)
    sc = (tq @ ke.transpose(-1, -2)) * (scale if scale is not None else 1 / math.sqrt(d))
    lse = torch.logsumexp(sc.masked_fill(~masks, -math.inf), dim=-1)
    return tq, tk, tv, out, lse


@pytest.mark.parametrize("L,G,Hq,Hkv,d,sh", [
    (16, 4, 4, 4, 8, 2), (12, 6, 2, 1, 4, 2), (24, 8, 4, 2, 8, 2), (16, 16, 2, 2, 4, 1),
    (32, 8, 8, 2, 16, 4)])
def test_explicit_mask_matches_torch_sdpa_and_autograd(L, G, Hq, Hkv, d, sh):
    rng = np.random.default_rng(L * 100 + G)
    q, k, v, do = qkv(2, L, Hq, Hkv, d, rng=rng, grad=True)
    tq, tk, tv, out, lse = _torch_masked(q, k, v, G, sh)
    o_ref, l_ref = O.forward_dense(q, k, v, G, sh)
    assert np.allclose(out.detach().permute(0, 2, 1, 3).numpy(), o_ref, atol=1e-12, rtol=0)
    assert np.allclose(lse.detach().numpy(), l_ref, atol=1e-12, rtol=0)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    dq, dk, dv = O.backward_dense(q, k, v, do, G, sh)
    dq1, dk1, dv1 = O.backward(q, k, v, do, G, sh)[:3]
    for t, a, b in [(tq, dq, dq1), (tk, dk, dk1), (tv, dv, dv1)]:
        ref = t.grad.permute(0, 2, 1, 3).numpy()
        assert np.allclose(a, ref, atol=1e-11, rtol=0)
        assert np.allclose(b, ref, atol=1e-11, rtol=0)


def test_nondefault_scale_matches_torch():
    rng = np.random.default_rng(3)
    q, k, v = qkv(1, 16, 2, 2, 8, rng=rng)
    _, _, _, out, lse = _torch_masked(q, k, v, 4, 1, scale=0.3)
    o, l = O.forward(q, k, v, 4, 1, scale=0.3)
    assert np.allclose(out.detach().permute(0, 2, 1, 3).numpy(), o, atol=1e-12)
    assert np.allclose(lse.detach().numpy(), l, atol=1e-12)


# --------------------------------------------------------------------------
# Special cases and invariants of the method.
# --------------------------------------------------------------------------

def test_full_attention_special_case():
    """G = L with no shift is ordinary causal attention (the inference mode:
    model card, features list, and blog section 3.1 use full attention there)."""
    rng = np.random.default_rng(11)
    q, k, v, do = qkv(2, 24, 4, 4, 8, rng=rng, grad=True)
    o, _ = O.forward(q, k, v, 24, 0)
    tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_()
    tk = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_()
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    assert np.allclose(out.detach().permute(0, 2, 1, 3).numpy(), o, atol=1e-12)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    dq, dk, dv = O.backward(q, k, v, do, 24, 0)[:3]
    assert np.allclose(tq.grad.permute(0, 2, 1, 3).numpy(), dq, atol=1e-11)
    assert np.allclose(tk.grad.permute(0, 2, 1, 3).numpy(), dk, atol=1e-11)
    assert np.allclose(tv.grad.permute(0, 2, 1, 3).numpy(), dv, atol=1e-11)


def test_shifted_head_is_grouped_attention_on_rolled_sequence():
    """A shifted head equals unshifted grouped attention on the rolled inputs,
    rolled back (nearauto.com article: shift, then regroup into the batch)."""
    rng = np.random.default_rng(5)
    L, G, Hq, d = 24, 8, 4, 8
    q, k, v, do = qkv(1, L, Hq, Hq, d, rng=rng, grad=True)
    o, lse = O.forward_dense(q, k, v, G, Hq)          # all heads shifted, mask form
    dq, dk, dv = O.backward_dense(q, k, v, do, G, Hq)
    s = G // 2
    roll = lambda x: np.roll(x, -s, axis=1)           # rolled[p] = x[p + s]
    unroll = lambda x: np.roll(x, s, axis=1)
    o0, l0 = O.forward(roll(q), roll(k), roll(v), G, 0)
    g0 = O.backward(roll(q), roll(k), roll(v), roll(do), G, 0)[:3]
    assert np.allclose(unroll(o0), o, atol=1e-12)
    assert np.allclose(np.roll(l0, s, axis=2), lse, atol=1e-12)
    for a, b in zip(g0, (dq, dk, dv)):
        assert np.allclose(unroll(a), b, atol=1e-12)


@pytest.mark.parametrize("sh", [0, 2, 4])
def test_group_independence(sh):
    """Perturbing one group's inputs leaves every other group bit-identical."""
    rng = np.random.default_rng(21 + sh)
    L, G, Hq, d = 32, 8, 4, 8
    q, k, v, do = qkv(1, L, Hq, Hq, d, rng=rng, grad=True)
    base = O.backward(q, k, v, do, G, sh)
    h = Hq - 1
    rows = O.unit_rows(L, G, Hq, sh, h, 1)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[0, rows, h] += rng.standard_normal((G, d))
    pert = O.backward(q2, k2, v2, do2, G, sh)
    other = np.setdiff1d(np.arange(L), rows)
    for a, b in zip(base[:4], pert[:4]):        # dq, dk, dv, o
        assert np.array_equal(a[0, other, h], b[0, other, h])
        assert not np.array_equal(a[0, rows, h], b[0, rows, h])
        assert np.array_equal(a[0, :, :h], b[0, :, :h])   # other heads untouched
    assert np.array_equal(base[4][0, h, other], pert[4][0, h, other])


@pytest.mark.parametrize("sh", [0, 2, 4])
def test_roll_by_group_equivariance(sh):
    """Rolling every input by G rolls every output by G (groups permute)."""
    rng = np.random.default_rng(31 + sh)
    L, G, Hq, d = 32, 8, 4, 8
    q, k, v, do = qkv(1, L, Hq, 2, d, rng=rng, grad=True)
    R = lambda x, ax=1: np.roll(x, G, axis=ax)
    a = O.backward(q, k, v, do, G, sh)
    b = O.backward(R(q), R(k), R(v), R(do), G, sh)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(R(x), y)
    assert np.array_equal(R(a[4], 2), b[4])


def test_closed_forms():
    rng = np.random.default_rng(41)
    L, G, Hq, d, sh = 24, 6, 4, 8, 2
    q, k, v = qkv(1, L, Hq, Hq, d, rng=rng)
    # V constant -> O constant
    o, _ = O.forward(q, k, np.full_like(v, 0.75), G, sh)
    assert np.allclose(o, 0.75, atol=1e-14)
    # Q = 0 -> O_i = mean of allowed v_j, lse_i = ln |A(i)|
    o, lse = O.forward(np.zeros_like(q), k, v, G, sh)
    for h in range(Hq):
        M = O.allowed_mask(L, G, O.head_shift(h, Hq, G, sh))
        assert np.allclose(o[0, :, h], (M @ v[0, :, h]) / M.sum(1)[:, None], atol=1e-13)
        assert np.allclose(lse[0, h], np.log(M.sum(1)), atol=1e-13)
    # G = 1, no shift -> O = V and lse_i = scale q_i . k_i
    o, lse = O.forward(q, k, v, 1, 0)
    assert np.allclose(o, v, atol=1e-14)
    assert np.allclose(lse[0], np.einsum("lhd,lhd->hl", q[0], k[0]) / math.sqrt(d), atol=1e-13)
    # k + c (same c for all keys) -> O unchanged, lse shifted by scale q_i . c
    c = rng.standard_normal(d)
    o1, l1 = O.forward(q, k, v, G, sh)
    o2, l2 = O.forward(q, k + c, v, G, sh)
    assert np.allclose(o1, o2, atol=1e-12)
    assert np.allclose(l2 - l1, np.einsum("lhd,d->hl", q[0], c)[None] / math.sqrt(d), atol=1e-12)


def test_gradient_identities():
    """Per KV head and group: sum_j dV_j = sum_i dO_i, and sum_j dK_j = 0 (no RoPE)."""
    rng = np.random.default_rng(51)
    L, G, Hq, Hkv, d, sh = 32, 8, 4, 2, 8, 2
    q, k, v, do = qkv(1, L, Hq, Hkv, d, rng=rng, grad=True)
    dq, dk, dv, _, _ = O.backward(q, k, v, do, G, sh)
    r = Hq // Hkv
    for hk in range(Hkv):
        s = O.head_shift(hk * r, Hq, G, sh)
        for g in range(L // G):
            rows = O.group_members(L, G, s, g)
            sum_do = sum(do[0, rows, h].sum(0) for h in range(hk * r, (hk + 1) * r))
            assert np.allclose(dv[0, rows, hk].sum(0), sum_do, atol=1e-12)
            assert np.allclose(dk[0, rows, hk].sum(0), 0.0, atol=1e-12)


@pytest.mark.parametrize("rope", [None, (100.0, 3)])
def test_finite_differences(rope):
    """Central differences of Phi = sum(dO * O) agree with the analytic grads."""
    rng = np.random.default_rng(61)
    L, G, Hq, Hkv, d, sh = 8, 4, 2, 1, 4, 2
    q, k, v, do = qkv(1, L, Hq, Hkv, d, rng=rng, grad=True)
    dq, dk, dv, _, _ = O.backward(q, k, v, do, G, sh, rope=rope)
    eps = 1e-6

    def phi(q_, k_, v_):
        return float(np.sum(do * O.forward(q_, k_, v_, G, sh, rope=rope)[0]))

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, k, v]
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num[idx] = (phi(*ap) - phi(*am)) / (2 * eps)
        err = np.max(np.abs(num - grad)) / np.max(np.abs(grad))
        assert err < 1e-6, (which, err)


def test_gqa_equals_repeated_heads():
    """Sharing a KV head among r query heads is the same as repeating it r times;
    the shared head's gradient is the sum over the repeats."""
    rng = np.random.default_rng(71)
    L, G, Hq, Hkv, d, sh = 16, 4, 4, 2, 8, 2
    q, k, v, do = qkv(1, L, Hq, Hkv, d, rng=rng, grad=True)
    r = Hq // Hkv
    ke, ve = np.repeat(k, r, axis=2), np.repeat(v, r, axis=2)
    a = O.backward(q, k, v, do, G, sh)
    b = O.backward(q, ke, ve, do, G, sh)
    assert np.allclose(a[3], b[3], atol=1e-14)   # o
    assert np.allclose(a[0], b[0], atol=1e-13)   # dq
    assert np.allclose(a[1], b[1].reshape(1, L, Hkv, r, d).sum(3), atol=1e-13)
    assert np.allclose(a[2], b[2].reshape(1, L, Hkv, r, d).sum(3), atol=1e-13)


# --------------------------------------------------------------------------
# RoPE with position interpolation (blog section 3.4).
# --------------------------------------------------------------------------

def test_rope_properties():
    rng = np.random.default_rng(81)
    B, L, H, d = 1, 32, 2, 16
    x = rng.standard_normal((B, L, H, d))
    th = O.rope_angles(L, d, 10000.0, 8)
    y = O.rope_rotate(x, th)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-13)
    assert np.array_equal(y[:, 0], x[:, 0])                       # position 0: identity
    assert np.allclose(O.rope_rotate_transpose(y, th), x, atol=1e-13)
    # position interpolation: positions scaled by L0/L, i.e. th at L equals
    # plain RoPE (L0 = L) evaluated at t * L0 / L
    plain = O.rope_angles(L, d, 10000.0, L)
    assert np.allclose(th, plain * (8 / L), atol=0)


def test_rope_is_complex_rotation():
    """Half-split RoPE with L0 = L equals multiplying x_c + i x_{c+d/2} by exp(i t w_c)."""
    rng = np.random.default_rng(82)
    L, d = 20, 8
    x = rng.standard_normal((1, L, 1, d))
    y = O.rope_rotate(x, O.rope_angles(L, d, 10000.0, L))
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    t = np.arange(L)[:, None]
    w = 10000.0 ** (-np.arange(0, d, 2) / d)[None, :]
    zr = z * np.exp(1j * t * w)[None, :, None, :]
    assert np.allclose(y[..., : d // 2], zr.real, atol=1e-13)
    assert np.allclose(y[..., d // 2:], zr.imag, atol=1e-13)


def test_rope_relative_position():
    """Unshifted head, G = L: scores depend on position differences only, so
    offsetting every position leaves O unchanged."""
    rng = np.random.default_rng(83)
    L, H, d = 16, 2, 8
    q, k, v = qkv(1, L, H, H, d, rng=rng)
    th = O.rope_angles(L, d, 10000.0, L)
    o_a, _ = O.forward(O.rope_rotate(q, th), O.rope_rotate(k, th), v, L, 0)
    o_b, _ = O.forward(O.rope_rotate(q, th + 5 * th[1]), O.rope_rotate(k, th + 5 * th[1]), v, L, 0)
    assert np.allclose(o_a, o_b, atol=1e-12)
    o_c, _ = O.forward(q, k, v, L, 0, rope=(10000.0, L))
    assert np.allclose(o_a, o_c, atol=1e-14)


def test_sampled_units_match_full():
    rng = np.random.default_rng(91)
    L, G, Hq, Hkv, d, sh = 32, 8, 4, 2, 8, 2
    q, k, v, do = qkv(2, L, Hq, Hkv, d, rng=rng, grad=True)
    for rope in (None, (10000.0, 8)):
        dq, dk, dv, o, lse = O.backward(q, k, v, do, G, sh, rope=rope)
        fw = O.sampled_forward(q, k, v, G, sh, [(1, 3, 2), (0, 0, 0)], rope=rope)
        for (b, h, g), (rows, og, lg) in fw.items():
            assert np.allclose(o[b, rows, h], og, atol=1e-13)
            assert np.allclose(lse[b, h, rows], lg, atol=1e-13)
        bw = O.sampled_kv_backward(q, k, v, do, G, sh, [(1, 1, 3), (0, 0, 1)], rope=rope)
        for (b, hk, g), res in bw.items():
            rows = res["rows"]
            assert np.allclose(dk[b, rows, hk], res["dk"], atol=1e-12)
            assert np.allclose(dv[b, rows, hk], res["dv"], atol=1e-12)
            for h, x in res["dq"].items():
                assert np.allclose(dq[b, rows, h], x, atol=1e-12)


def test_sampled_rows_match_explicit_mask():
    """Row-at-a-time forward (used where a unit spans a whole long context)
    against the explicit-mask form, including the diagonal row and rows of a
    shifted head whose group wraps around the sequence end."""
    rng = np.random.default_rng(93)
    for (L, G, Hq, Hkv, d, sh, rope) in ((24, 24, 2, 1, 8, 0, None), (32, 8, 4, 2, 8, 2, None),
                                         (32, 32, 2, 2, 8, 0, (100.0, 8)), (24, 8, 2, 2, 4, 1, (50.0, 6))):
        q, k, v = qkv(1, L, Hq, Hkv, d, rng=rng)
        o, lse = O.forward_dense(q, k, v, G, sh, rope=rope)
        for h in range(Hq):
            for g in range(L // G):
                rows_in = [0, 1, G // 2, G - 1]
                toks, og, lg = O.sampled_rows_forward(q, k, v, G, sh, 0, h, g, rows_in, rope=rope)
                assert np.allclose(og, o[0, toks, h], atol=1e-12), (L, G, sh, h, g)
                assert np.allclose(lg, lse[0, h, toks], atol=1e-12), (L, G, sh, h, g)


def test_invalid_arguments():
    q, k, v = qkv(1, 12, 2, 2, 4)
    with pytest.raises(ValueError):
        O.forward(q, k, v, 5, 0)          # L % G != 0
    with pytest.raises(ValueError):
        O.forward(q, k, v, 3, 1)          # odd G with a shift
    with pytest.raises(ValueError):
        O.forward(q, k[:, :, :1].repeat(3, 2), v[:, :, :1].repeat(3, 2), 4, 0)  # Hq % Hkv
    with pytest.raises(ValueError):
        O.head_shift(0, 2, 4, 3)


def test_pooled_units_equal_the_oracle():
    """The worker-pool driver the full-size GPU parity tests use returns the
    oracle's own values: every KV unit through `kv_unit_backward` in worker
    processes, scattered back, equals `backward` bit for bit, and every unit
    through `unit_forward` equals `forward` (GQA, shifted heads, B = 2, with
    and without RoPE)."""
    from tests import oracle_pool
    rng = np.random.default_rng(12)
    B, L, Hq, Hkv, d, G, sh = 2, 192, 4, 2, 16, 48, 2
    x = {n: rng.standard_normal(s) for n, s in (("q", (B, L, Hq, d)), ("k", (B, L, Hkv, d)),
                                                 ("v", (B, L, Hkv, d)), ("do", (B, L, Hq, d)))}
    started_here = oracle_pool._POOL is None
    try:
        for rope in (None, (100.0, 64)):
            dq, dk, dv, o, lse = O.backward(x["q"], x["k"], x["v"], x["do"], G, sh, rope=rope)
            po, plse, pdq, pdk, pdv = oracle_pool.full_backward(x, G, sh, rope)
            for a, b in ((po, o), (plse, lse), (pdq, dq), (pdk, dk), (pdv, dv)):
                assert np.array_equal(a, b)
            fo, flse = oracle_pool.full_forward(x["q"], x["k"], x["v"], G, sh, rope)
            ro, rlse = O.forward(x["q"], x["k"], x["v"], G, sh, rope=rope)
            assert np.array_equal(fo, ro) and np.array_equal(flse, rlse)
    finally:
        if started_here:
            oracle_pool.stop()
