"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutation below edits one expression of the oracle's source; the pins
from test_oracle_pins.py are then run against the mutated oracle and at least
one of them must fail.  This shows the pins constrain each part of the oracle
(index map, mask, softmax, each gradient term, RoPE, KV-head sharing).
"""

import inspect

import pytest

from oracle import s2attn as O
from tests import test_oracle_pins as P


def _pins(golden_dir):
    return [
        lambda: P.test_blog_shift_example(golden_dir),
        lambda: P.test_brute_force_loops_on_the_blog_example(golden_dir),
        P.test_allowed_mask_structure,
        lambda: P.test_group_form_matches_explicit_mask(None),
        lambda: P.test_explicit_mask_matches_torch_sdpa_and_autograd(16, 4, 4, 4, 8, 2),
        lambda: P.test_explicit_mask_matches_torch_sdpa_and_autograd(24, 8, 4, 2, 8, 2),
        P.test_full_attention_special_case,
        P.test_shifted_head_is_grouped_attention_on_rolled_sequence,
        lambda: P.test_finite_differences(None),
        lambda: P.test_finite_differences((100.0, 3)),
        P.test_gqa_equals_repeated_heads,
        P.test_rope_properties,
        P.test_rope_is_complex_rotation,
        P.test_closed_forms,
        P.test_gradient_identities,
        P.test_sampled_rows_match_explicit_mask,
    ]


# (function name, original text, mutated text)
MUTATIONS = [
    ("rolled_to_original", "(np.asarray(p) + s) % L", "(np.asarray(p) - s) % L"),
    ("head_shift", "return G // 2 if h >= Hq - shifted_heads else 0",
     "return G // 2 if h < shifted_heads else 0"),
    ("head_shift", "return G // 2 if", "return G // 4 if"),
    ("allowed_mask", "idx[None, :] <= idx[:, None]", "idx[None, :] < idx[:, None] + 2"),
    ("_masked_scores", "s[cols > rows] = -np.inf", "s[cols >= rows + 2] = -np.inf"),
    ("_masked_scores", "s = scale * (qb @ k[:i1].T)", "s = (qb @ k[:i1].T)"),
    ("unit_forward", "lse[i0:i1] = m + np.log(l)", "lse[i0:i1] = m + np.log(l) * 0.5"),
    ("unit_backward", "ds = p * (dp - D[:, None])", "ds = p * (dp + D[:, None])"),
    ("unit_backward", "dq[i0:i1] = scale * (ds @ kg[:i1])", "dq[i0:i1] = (ds @ kg[:i1])"),
    ("unit_backward", "dk[:i1] += scale * (ds.T @ qg[i0:i1])", "dk[:i1] += scale * (ds.T @ dog[i0:i1])"),
    ("unit_backward", "dv[:i1] += p.T @ dog[i0:i1]", "dv[:i1] += ds.T @ dog[i0:i1]"),
    ("unit_backward", "D = np.sum(dog[i0:i1] * o[i0:i1], axis=1)", "D = np.sum(dog[i0:i1] * o[i0:i1], axis=1) * 0"),
    ("backward_dense", "dv[b, :, hk] += p.T @ do[b, :, h]", "dv[b, :, hk] = p.T @ do[b, :, h]"),
    ("forward", "k[b, rows, h // r], v[b, rows, h // r]", "k[b, rows, h % k.shape[2]], v[b, rows, h % k.shape[2]]"),
    ("rope_rotate", "x1 * c - x2 * s, x1 * s + x2 * c", "x1 * c + x2 * s, x1 * s + x2 * c"),
    ("rope_rotate_transpose", "g1 * c + g2 * s, -g1 * s + g2 * c", "g1 * c - g2 * s, g1 * s + g2 * c"),
    ("rope_angles", "pos = np.arange(L, dtype=np.float64) * (float(orig_len) / float(L))",
     "pos = np.arange(L, dtype=np.float64)"),
    ("sampled_rows_forward", "keys = members[:i + 1]", "keys = members[:i + 2]"),
    ("sampled_rows_forward", "s = scale * (kk @ qi)", "s = kk @ qi"),
    ("sampled_rows_forward", "kk = rope_rotate(kk[None, :, None, :], theta[keys])[0, :, 0, :]",
     "kk = rope_rotate(kk[None, :, None, :], theta[keys][::-1])[0, :, 0, :]"),
    ("rope_angles", "(-2.0 * np.arange(d // 2, dtype=np.float64) / d)",
     "(-1.0 * np.arange(d // 2, dtype=np.float64) / d)"),
]


@pytest.mark.parametrize("fname,orig,mut", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_mutation_is_caught(fname, orig, mut, monkeypatch, golden_dir):
    src = inspect.getsource(getattr(O, fname))
    assert orig in src, f"mutation text not found in {fname}"
    ns = dict(vars(O))
    exec(src.replace(orig, mut), ns)
    monkeypatch.setattr(O, fname, ns[fname])
    caught = []
    for pin in _pins(golden_dir):
        try:
            pin()
        except (AssertionError, ValueError):
            caught.append(pin)
            break
    assert caught, f"no pin caught the mutation in {fname}: {mut!r}"


# Mutations of the attention-block oracle, against its own pins.
from oracle import block as OB  # noqa: E402
from tests import test_block_oracle as BP  # noqa: E402

BLOCK_PINS = [
    lambda: BP.test_block_matches_torch_autograd(1, 24, 4, 2, 8, 8, 2, 3),
    BP.test_lora_merges_into_weight,
    BP.test_zero_up_projection_has_zero_down_gradient,
    BP.test_finite_differences_with_rope,
    BP.test_sampled_tokens_match_full_forward,
]

BLOCK_MUTATIONS = [
    ("lora_proj", "s * ((X @ A.T) @ Bm.T)", "((X @ A.T) @ Bm.T)"),
    ("lora_proj_backward", "dX = dY @ W + s * (t @ A)", "dX = dY @ W"),
    ("lora_proj_backward", "dA = s * (t.T @ X)", "dA = s * (t.T @ dY[:, :X.shape[1]])"),
    ("lora_proj_backward", "dB = s * (dY.T @ (X @ A.T))", "dB = dY.T @ (X @ A.T)"),
    ("backward", "dx += dX", "dx = dX"),
    ("forward", 'k = lora_proj(X, p["wk"], p["ak"], p["bk"], s)', 'k = lora_proj(X, p["wk"], p["aq"][:, :], p["bk"], s)'),
    ("sampled_forward_tokens", "attn[n, sq] = (e / e.sum()) @ vg[:i + 1]", "attn[n, sq] = (e / e.sum()) @ vg[:i + 1] * 1.0001"),
]


@pytest.mark.parametrize("fname,orig,mut", BLOCK_MUTATIONS,
                         ids=[f"block.{m[0]}:{i}" for i, m in enumerate(BLOCK_MUTATIONS)])
def test_block_mutation_is_caught(fname, orig, mut, monkeypatch):
    src = inspect.getsource(getattr(OB, fname))
    assert orig in src, f"mutation text not found in {fname}"
    ns = dict(vars(OB))
    exec(src.replace(orig, mut), ns)
    monkeypatch.setattr(OB, fname, ns[fname])
    caught = False
    for pin in BLOCK_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            caught = True
            break
    assert caught, f"no pin caught the mutation in {fname}: {mut!r}"
