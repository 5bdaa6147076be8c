"""Attention block oracle in float64 numpy.  TEST INFRASTRUCTURE ONLY.

One Llama-style attention block as LongLoRA fine-tunes it (LongLoRA blog,
smallflyingpig.github.io, section 3.2: LoRA adapters on the Q, K, V and O
projections with the base weights frozen; section 3.4: RoPE with position
interpolation; section 3.3: shift short attention).  A LoRA-adapted
projection of rows X is

    X W^T + s (X A^T) B^T,

with W [out, in] frozen, A [r, in] (down) and B [out, r] (up) trainable and
s the LoRA scale.  The block is

    q, k, v = proj_q(x), proj_k(x), proj_v(x)       ([B, L, H, d] views)
    attn    = S2-Attn(q, k, v)                       (oracle.s2attn, RoPE inside)
    y       = proj_o(attn)

and its backward returns dx and the gradients of every A and B (W is frozen).
The attention parts call the S2-Attn oracle; the projections are written out
here.  Nothing is shared with the HIP path.
"""

import numpy as np

from . import s2attn as S

NAMES = ("q", "k", "v", "o")


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def lora_proj(X, W, A, Bm, s):
    """X W^T + s (X A^T) B^T for rows X [n, in]."""
    X, W, A, Bm = _f64(X), _f64(W), _f64(A), _f64(Bm)
    return X @ W.T + s * ((X @ A.T) @ Bm.T)


def lora_proj_backward(X, W, A, Bm, s, dY):
    """Gradients of lora_proj: (dX, dA, dB)."""
    X, W, A, Bm, dY = _f64(X), _f64(W), _f64(A), _f64(Bm), _f64(dY)
    t = dY @ Bm                      # [n, r]
    dX = dY @ W + s * (t @ A)
    dA = s * (t.T @ X)               # [r, in]
    dB = s * (dY.T @ (X @ A.T))      # [out, r]
    return dX, dA, dB


def forward(x, p, G, shifted_heads, Hq, Hkv, d, s, rope=None):
    """x [B, L, Dm]; p: dict of W*, A*, B* arrays.  Returns (y, cache)."""
    B, L, Dm = x.shape
    X = _f64(x).reshape(B * L, Dm)
    q = lora_proj(X, p["wq"], p["aq"], p["bq"], s).reshape(B, L, Hq, d)
    k = lora_proj(X, p["wk"], p["ak"], p["bk"], s).reshape(B, L, Hkv, d)
    v = lora_proj(X, p["wv"], p["av"], p["bv"], s).reshape(B, L, Hkv, d)
    attn, lse = S.forward(q, k, v, G, shifted_heads, rope=rope)
    y = lora_proj(attn.reshape(B * L, Hq * d), p["wo"], p["ao"], p["bo"], s).reshape(B, L, Dm)
    return y, dict(q=q, k=k, v=v, attn=attn, lse=lse)


def backward(x, p, dy, G, shifted_heads, Hq, Hkv, d, s, rope=None):
    """Returns (y, grads) with grads dx and dA*, dB* for * in q, k, v, o."""
    B, L, Dm = x.shape
    y, c = forward(x, p, G, shifted_heads, Hq, Hkv, d, s, rope=rope)
    X = _f64(x).reshape(B * L, Dm)
    dY = _f64(dy).reshape(B * L, Dm)
    g = {}
    dattn, g["dao"], g["dbo"] = lora_proj_backward(c["attn"].reshape(B * L, Hq * d), p["wo"],
                                                   p["ao"], p["bo"], s, dY)
    dq, dk, dv, _, _ = S.backward(c["q"], c["k"], c["v"], dattn.reshape(B, L, Hq, d), G,
                                  shifted_heads, rope=rope)
    dx = np.zeros_like(X)
    for name, dz in (("q", dq), ("k", dk), ("v", dv)):
        dX, g["da" + name], g["db" + name] = lora_proj_backward(
            X, p["w" + name], p["a" + name], p["b" + name], s, dz.reshape(B * L, -1))
        dx += dX
    g["dx"] = dx.reshape(B, L, Dm)
    return y, g


def sampled_forward_tokens(x, p, G, shifted_heads, Hq, Hkv, d, s, b, tokens, rope=None):
    """y at chosen original token positions of batch row b, for a full-size input.

    y at token t needs every head's attention output at t.  For head h, t sits
    at in-group index i of one group under that head's shift; by causality
    only the group's rows 0 .. i enter, so just those rows are projected (the
    head's slice of each projection), rotated when RoPE is on, and row i is
    attended to from the definition.  Returns y rows [len(tokens), Dm].
    """
    B, L, Dm = x.shape
    r = Hq // Hkv
    scale = 1.0 / np.sqrt(d)
    theta = S.rope_angles(L, d, *rope) if rope is not None else None
    attn = np.zeros((len(tokens), Hq * d))
    for h in range(Hq):
        shift = S.head_shift(h, Hq, G, shifted_heads)
        hk = h // r
        sq, skv = slice(h * d, (h + 1) * d), slice(hk * d, (hk + 1) * d)
        by_group = {}
        for n, t in enumerate(tokens):
            pr = int(S.original_to_rolled(t, L, shift))
            by_group.setdefault(pr // G, []).append((n, pr % G))
        for g, items in by_group.items():
            rows = S.group_members(L, G, shift, g)[:max(i for _, i in items) + 1]
            Xg = _f64(x[b, rows])
            qg = lora_proj(Xg, p["wq"][sq], p["aq"], p["bq"][sq], s)
            kg = lora_proj(Xg, p["wk"][skv], p["ak"], p["bk"][skv], s)
            vg = lora_proj(Xg, p["wv"][skv], p["av"], p["bv"][skv], s)
            if theta is not None:
                qg = S.rope_rotate(qg[None, :, None, :], theta[rows])[0, :, 0, :]
                kg = S.rope_rotate(kg[None, :, None, :], theta[rows])[0, :, 0, :]
            for n, i in items:
                sc = scale * (kg[:i + 1] @ qg[i])
                e = np.exp(sc - sc.max())
                attn[n, sq] = (e / e.sum()) @ vg[:i + 1]
    return lora_proj(attn, p["wo"], p["ao"], p["bo"], s)
