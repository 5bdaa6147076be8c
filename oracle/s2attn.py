"""S2-Attn oracle in float64 numpy.  TEST INFRASTRUCTURE ONLY (see package doc).

Notation (one layer, batch index b):
  L  sequence length, G group size, n_g = L / G groups
  Hq query heads, Hkv key/value heads, r = Hq / Hkv, KV head of query head h is h // r
  s_h  shift of head h: G/2 for the last `shifted_heads` heads, else 0
  rolled sequence of head h:  rolled[p] = x[(p + s_h) mod L]      (a left roll)
  group of rolled position p:  p // G,  in-group index p mod G

Each query attends, with softmax, to the keys of its own group whose in-group
index is not after its own (causal inside the group, rolled order); the
outputs are returned at the tokens' original positions.

Readings of points the pages leave open (each also recorded in the design
notes): the shift is a cyclic roll, so the last shifted group is the last G/2
tokens followed by the first G/2 (the blog's worked example prints positions
past the end of its 12-token sequence); the shifted heads are the last
`shifted_heads` heads of a layer; the softmax scale defaults to 1/sqrt(d); LSE
is the natural-log log-sum-exp of the scaled scores, indexed [b, h, t] by
original position t; RoPE pairs channel c with c + d/2 and rotates position t
(original index) by angle t * (L0 / L) * base^(-2c/d).
"""

import math

import numpy as np

# ---------------------------------------------------------------------------
# Index maps.  LongLoRA blog (smallflyingpig.github.io), section 3.3, worked
# shift example: with groups of 4 over 12 tokens, the shifted grouping starts
# at token 3 (1-based), i.e. every shifted group begins half a group later.
# ---------------------------------------------------------------------------


def head_shift(h, Hq, G, shifted_heads):
    """Shift of query head h: half a group for the last `shifted_heads` heads.

    python88.com article (section on reducing computation): heads are split
    into two sets and one set is shifted; nearauto.com article (shift short
    attention section): step 1 shifts the tokens in half of the heads.
    """
    if not 0 <= shifted_heads <= Hq:
        raise ValueError("shifted_heads out of range")
    return G // 2 if h >= Hq - shifted_heads else 0


def rolled_to_original(p, L, s):
    """Original token index held at rolled position p (left roll by s)."""
    return (np.asarray(p) + s) % L


def original_to_rolled(t, L, s):
    """Rolled position of original token t."""
    return (np.asarray(t) - s) % L


def group_members(L, G, s, g):
    """Original token indices of group g, listed in rolled (in-group) order."""
    return rolled_to_original(g * G + np.arange(G), L, s)


def allowed_mask(L, G, s):
    """Explicit L x L mask: allowed[i, j] iff query token i may see key token j.

    Both are original indices.  Same group of the rolled sequence and key's
    in-group index <= query's in-group index.
    """
    rho = original_to_rolled(np.arange(L), L, s)
    grp = rho // G
    idx = rho % G
    return (grp[:, None] == grp[None, :]) & (idx[None, :] <= idx[:, None])


# ---------------------------------------------------------------------------
# RoPE with position interpolation.  LongLoRA blog, section 3.4: the target
# length L is squeezed onto the pretrained length L0 by scaling positions by
# L0 / L.  Pairing (c, c + d/2) is the half-split convention.
# ---------------------------------------------------------------------------


def rope_angles(L, d, base, orig_len):
    """theta[t, c] = t * (orig_len / L) * base^(-2c/d), float64, shape [L, d/2]."""
    pos = np.arange(L, dtype=np.float64) * (float(orig_len) / float(L))
    omega = float(base) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    return pos[:, None] * omega[None, :]


def rope_rotate(x, theta):
    """Rotate pairs (x_c, x_{c+d/2}) of x [B, L, H, d] by theta [L, d/2]."""
    half = x.shape[-1] // 2
    c = np.cos(theta)[None, :, None, :]
    s = np.sin(theta)[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_rotate_transpose(g, theta):
    """Apply the transposed (inverse) rotation: gradient w.r.t. the pre-RoPE input."""
    half = g.shape[-1] // 2
    c = np.cos(theta)[None, :, None, :]
    s = np.sin(theta)[None, :, None, :]
    g1, g2 = g[..., :half], g[..., half:]
    return np.concatenate([g1 * c + g2 * s, -g1 * s + g2 * c], axis=-1)


# ---------------------------------------------------------------------------
# One group of one head: dense causal softmax attention on G rows given in
# rolled order.  Query rows are processed in blocks only to bound memory;
# every row is computed on its own from the definition, and a block of rows
# < i1 needs only keys < i1 (the rest are outside every row's allowed set).
# ---------------------------------------------------------------------------

_BLOCK_ELEMS = 1 << 25  # score elements per row block (256 MB of float64)


def _row_blocks(G):
    nb = max(1, min(G, _BLOCK_ELEMS // max(G, 1)))
    for i0 in range(0, G, nb):
        yield i0, min(G, i0 + nb)


def _masked_scores(qb, k, i0, i1, scale):
    """Scores of rows i0..i1-1 against keys 0..i1-1, -inf where key > row."""
    s = scale * (qb @ k[:i1].T)
    rows = np.arange(i0, i1)[:, None]
    cols = np.arange(i1)[None, :]
    s[cols > rows] = -np.inf
    return s


def unit_forward(qg, kg, vg, scale):
    """Causal attention on one group: returns (o [G, d], lse [G])."""
    G = qg.shape[0]
    o = np.empty((G, vg.shape[1]), dtype=np.float64)
    lse = np.empty(G, dtype=np.float64)
    for i0, i1 in _row_blocks(G):
        s = _masked_scores(qg[i0:i1], kg, i0, i1, scale)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        lse[i0:i1] = m + np.log(l)
        p = e / l[:, None]
        o[i0:i1] = p @ vg[:i1]
    return o, lse


def unit_backward(qg, kg, vg, dog, scale):
    """Gradients of one group's causal attention, from its inputs alone.

    The forward is recomputed here (O and LSE are never taken from outside).
    With P the probabilities and D_i = dO_i . O_i:
      dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
      dK = scale dS^T Q,  dV = P^T dO.
    Returns (dq, dk, dv, o, lse).
    """
    o, lse = unit_forward(qg, kg, vg, scale)
    G = qg.shape[0]
    dq = np.zeros_like(qg, dtype=np.float64)
    dk = np.zeros_like(kg, dtype=np.float64)
    dv = np.zeros_like(vg, dtype=np.float64)
    for i0, i1 in _row_blocks(G):
        s = _masked_scores(qg[i0:i1], kg, i0, i1, scale)
        p = np.exp(s - lse[i0:i1, None])
        dp = dog[i0:i1] @ vg[:i1].T
        D = np.sum(dog[i0:i1] * o[i0:i1], axis=1)
        ds = p * (dp - D[:, None])
        dq[i0:i1] = scale * (ds @ kg[:i1])
        dk[:i1] += scale * (ds.T @ qg[i0:i1])
        dv[:i1] += p.T @ dog[i0:i1]
    return dq, dk, dv, o, lse


# ---------------------------------------------------------------------------
# Whole-tensor drivers, group form.  nearauto.com article, shift short
# attention section: shift half the heads, then treat each group as its own
# sequence; the gather below is that regrouping, the scatter undoes it.
# ---------------------------------------------------------------------------


def _prep(q, k, v, G, shifted_heads, scale, rope):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, L, Hkv, d) or v.shape != k.shape:
        raise ValueError("k, v must be [B, L, Hkv, d] matching q")
    if Hq % Hkv or L % G or (shifted_heads and G % 2):
        raise ValueError("need Hq % Hkv == 0, L % G == 0 and even G when shifting")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    theta = None
    if rope is not None:
        base, orig_len = rope
        theta = rope_angles(L, d, base, orig_len)
        q = rope_rotate(q, theta)
        k = rope_rotate(k, theta)
    return q, k, v, scale, theta


def units(B, Hq, L, G):
    """All (b, h, g) work units."""
    return [(b, h, g) for b in range(B) for h in range(Hq) for g in range(L // G)]


def forward(q, k, v, G, shifted_heads, scale=None, rope=None):
    """Group-form S2-Attn forward.  Returns (o [B, L, Hq, d], lse [B, Hq, L]).

    `rope` is None or (base, orig_len); q and k are then rotated at their
    original positions before attention.
    """
    q, k, v, scale, _ = _prep(q, k, v, G, shifted_heads, scale, rope)
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    o = np.zeros((B, L, Hq, d), dtype=np.float64)
    lse = np.zeros((B, Hq, L), dtype=np.float64)
    for b, h, g in units(B, Hq, L, G):
        rows = group_members(L, G, head_shift(h, Hq, G, shifted_heads), g)
        og, lg = unit_forward(q[b, rows, h], k[b, rows, h // r], v[b, rows, h // r], scale)
        o[b, rows, h] = og
        lse[b, h, rows] = lg
    return o, lse


def backward(q, k, v, do, G, shifted_heads, scale=None, rope=None):
    """Group-form S2-Attn backward.  Returns (dq, dk, dv, o, lse).

    Gradients are taken w.r.t. the pre-RoPE q and k when `rope` is given.
    dk and dv sum the contributions of the r query heads sharing a KV head.
    """
    q, k, v, scale, theta = _prep(q, k, v, G, shifted_heads, scale, rope)
    do = np.asarray(do, dtype=np.float64)
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, L), dtype=np.float64)
    for b, h, g in units(B, Hq, L, G):
        rows = group_members(L, G, head_shift(h, Hq, G, shifted_heads), g)
        hk = h // r
        dqg, dkg, dvg, og, lg = unit_backward(
            q[b, rows, h], k[b, rows, hk], v[b, rows, hk], do[b, rows, h], scale)
        dq[b, rows, h] = dqg
        dk[b, rows, hk] += dkg
        dv[b, rows, hk] += dvg
        o[b, rows, h] = og
        lse[b, h, rows] = lg
    if theta is not None:
        dq = rope_rotate_transpose(dq, theta)
        dk = rope_rotate_transpose(dk, theta)
    return dq, dk, dv, o, lse


# ---------------------------------------------------------------------------
# Sampled evaluation at full size: the outputs of a chosen set of units.
# ---------------------------------------------------------------------------


def unit_rows(L, G, Hq, shifted_heads, h, g):
    """Original token indices of unit (h, g), in rolled order."""
    return group_members(L, G, head_shift(h, Hq, G, shifted_heads), g)


def sampled_forward(q, k, v, G, shifted_heads, unit_list, scale=None, rope=None):
    """Forward of selected (b, h, g) units only: {unit: (rows, o [G,d], lse [G])}."""
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    theta = rope_angles(L, d, *rope) if rope is not None else None
    out = {}
    for b, h, g in unit_list:
        rows = unit_rows(L, G, Hq, shifted_heads, h, g)
        qg, kg, vg = (np.asarray(x[b, rows, hh], dtype=np.float64)
                      for x, hh in ((q, h), (k, h // r), (v, h // r)))
        if theta is not None:
            qg = rope_rotate(qg[None, :, None, :], theta[rows])[0, :, 0, :]
            kg = rope_rotate(kg[None, :, None, :], theta[rows])[0, :, 0, :]
        og, lg = unit_forward(qg, kg, vg, scale)
        out[(b, h, g)] = (rows, og, lg)
    return out


def sampled_rows_forward(q, k, v, G, shifted_heads, b, h, g, rows_in_group, scale=None, rope=None):
    """Forward of chosen query rows of unit (b, h, g), each on its own.

    Row i (in-group index, rolled order) attends to the keys of in-group
    index 0 .. i of its group: the plain definition, one row at a time, for
    units too long to run whole (a dense causal pass with G = L).  Returns
    (original token indices of the rows, o [n, d], lse [n]).
    """
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    members = unit_rows(L, G, Hq, shifted_heads, h, g)
    theta = rope_angles(L, d, *rope) if rope is not None else None
    toks, os_, lses = [], [], []
    for i in rows_in_group:
        keys = members[:i + 1]
        qi = np.asarray(q[b, members[i], h], dtype=np.float64)
        kk = np.asarray(k[b, keys, h // r], dtype=np.float64)
        vv = np.asarray(v[b, keys, h // r], dtype=np.float64)
        if theta is not None:
            qi = rope_rotate(qi[None, None, None, :], theta[members[i]][None])[0, 0, 0]
            kk = rope_rotate(kk[None, :, None, :], theta[keys])[0, :, 0, :]
        s = scale * (kk @ qi)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        toks.append(members[i])
        lses.append(m + np.log(l))
        os_.append((e / l) @ vv)
    return np.array(toks), np.array(os_), np.array(lses)


def kv_unit_backward(qs, kg, vg, dos, scale, theta=None):
    """Gradients of one (b, KV head, group) unit from its gathered rows.

    qs, dos: [r, G, d], the r query heads sharing the KV head, rows in rolled
    (in-group) order; kg, vg: [G, d] the KV head's rows in the same order;
    theta: RoPE angles [G, d/2] of those rows at their original positions, or
    None.  Each query head runs `unit_backward`; dk and dv sum over the r
    heads.  With RoPE, q and k are rotated first and dq, dk rotated back.
    Returns dict(dk [G,d], dv [G,d], dq [r,G,d], o [r,G,d], lse [r,G]).
    """

    def rot(x):
        return x if theta is None else rope_rotate(x[None, :, None, :], theta)[0, :, 0, :]

    def rot_t(x):
        return x if theta is None else rope_rotate_transpose(x[None, :, None, :], theta)[0, :, 0, :]

    r, G, d = np.shape(qs)
    kg = rot(np.asarray(kg, dtype=np.float64))
    vg = np.asarray(vg, dtype=np.float64)
    dk = np.zeros((G, d))
    dv = np.zeros((G, d))
    dq = np.zeros((r, G, d))
    o = np.zeros((r, G, d))
    lse = np.zeros((r, G))
    for j in range(r):
        qg = rot(np.asarray(qs[j], dtype=np.float64))
        dog = np.asarray(dos[j], dtype=np.float64)
        dqg, dkg, dvg, og, lg = unit_backward(qg, kg, vg, dog, scale)
        dk += dkg
        dv += dvg
        dq[j] = rot_t(dqg)
        o[j] = og
        lse[j] = lg
    return dict(dk=rot_t(dk), dv=dv, dq=dq, o=o, lse=lse)


def kv_unit_inputs(q, k, v, do, G, shifted_heads, unit, rope=None):
    """The gathered rows `kv_unit_backward` takes for unit (b, hk, g).

    Returns (rows, qs, kg, vg, dos, theta): rows are the group's original
    token indices in rolled order; theta is None without RoPE.  Requires the
    r query heads of the KV head to share one shift.
    """
    b, hk, g = unit
    B, L, Hq, d = np.shape(q)
    r = Hq // np.shape(k)[2]
    heads = list(range(hk * r, (hk + 1) * r))
    shifts = {head_shift(h, Hq, G, shifted_heads) for h in heads}
    if len(shifts) != 1:
        raise ValueError("query heads of one KV head have different shifts")
    rows = group_members(L, G, shifts.pop(), g)
    theta = rope_angles(L, d, *rope)[rows] if rope is not None else None
    qs = np.stack([q[b, rows, h] for h in heads])
    dos = np.stack([do[b, rows, h] for h in heads])
    return rows, qs, k[b, rows, hk], v[b, rows, hk], dos, theta


def sampled_kv_backward(q, k, v, do, G, shifted_heads, kv_units, scale=None, rope=None):
    """Gradients for selected (b, kv_head, g) units, whose r query heads share a shift.

    Returns {(b, hk, g): dict(rows, dk [G,d], dv [G,d], dq {h: [G,d]}, o {h: ..}, lse {h: ..})}.
    dq of every query head of the KV head is included (rows of the same group).
    Requires all r query heads of the KV head to have the same shift, so that
    their groups cover the same rows.
    """
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    res = {}
    for b, hk, g in kv_units:
        rows, qs, kg, vg, dos, theta = kv_unit_inputs(q, k, v, do, G, shifted_heads, (b, hk, g), rope)
        u = kv_unit_backward(qs, kg, vg, dos, scale, theta)
        heads = range(hk * r, (hk + 1) * r)
        res[(b, hk, g)] = dict(rows=rows, dk=u["dk"], dv=u["dv"],
                               dq={h: u["dq"][j] for j, h in enumerate(heads)},
                               o={h: u["o"][j] for j, h in enumerate(heads)},
                               lse={h: u["lse"][j] for j, h in enumerate(heads)})
    return res


# ---------------------------------------------------------------------------
# Explicit-mask form (tiny inputs only): full L x L scores, the mask from
# `allowed_mask`, no rolling and no regrouping.
# ---------------------------------------------------------------------------


def forward_dense(q, k, v, G, shifted_heads, scale=None, rope=None):
    """Explicit-mask S2-Attn forward.  Returns (o, lse)."""
    q, k, v, scale, _ = _prep(q, k, v, G, shifted_heads, scale, rope)
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    o = np.zeros((B, L, Hq, d))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            M = allowed_mask(L, G, head_shift(h, Hq, G, shifted_heads))
            s = scale * (q[b, :, h] @ k[b, :, h // r].T)
            s = np.where(M, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            l = np.exp(s - m).sum(axis=1, keepdims=True)
            lse[b, h] = (m + np.log(l))[:, 0]
            p = np.exp(s - lse[b, h][:, None])
            o[b, :, h] = p @ v[b, :, h // r]
    return o, lse


def backward_dense(q, k, v, do, G, shifted_heads, scale=None, rope=None):
    """Explicit-mask S2-Attn backward.  Returns (dq, dk, dv)."""
    q, k, v, scale, theta = _prep(q, k, v, G, shifted_heads, scale, rope)
    do = np.asarray(do, dtype=np.float64)
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // r
            M = allowed_mask(L, G, head_shift(h, Hq, G, shifted_heads))
            s = np.where(M, scale * (q[b, :, h] @ k[b, :, hk].T), -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, :, hk]
            dp = do[b, :, h] @ v[b, :, hk].T
            ds = p * (dp - np.sum(do[b, :, h] * o, axis=1, keepdims=True))
            dq[b, :, h] = scale * ds @ k[b, :, hk]
            dk[b, :, hk] += scale * ds.T @ q[b, :, h]
            dv[b, :, hk] += p.T @ do[b, :, h]
    if theta is not None:
        dq = rope_rotate_transpose(dq, theta)
        dk = rope_rotate_transpose(dk, theta)
    return dq, dk, dv
