"""FLOP and byte accounting for S2-Attn.

Counted FLOPs follow group-local causal attention: a group of G queries sees
G^2 / 2 (query, key) pairs, each costing 2d FLOPs for a score and 2d for its
share of P.V, so the forward is 4 * B * Hq * n_g * (G^2/2) * d = 2 * B * Hq * L * G * d.
The backward recomputes nothing in this count: dV, dP, dQ, dK and the score
recompute give 5 products against the forward's 2, i.e. 2.5x the forward.

The nearauto.com LongLoRA article, ablation section, Table 7, reports the
share of Llama2-7B FLOPs spent in attention; it counts the matrix products of
attention non-causally, 4 * N * d_model per token per layer where N is the
number of keys a query sees (L for full attention, the group size G for
S2-Attn).  `llama2_7b_attention_share` reproduces those shares.
"""


def fwd_flops(B, L, Hq, d, G):
    """Counted forward FLOPs: 2 * B * Hq * L * G * d."""
    return 2.0 * B * Hq * L * G * d


def bwd_flops(B, L, Hq, d, G):
    """Counted backward FLOPs: 2.5x the forward."""
    return 2.5 * fwd_flops(B, L, Hq, d, G)


def fwd_bwd_flops(B, L, Hq, d, G):
    return fwd_flops(B, L, Hq, d, G) + bwd_flops(B, L, Hq, d, G)


def fwd_bytes(B, L, Hq, Hkv, d, elem=2):
    """Algorithmic HBM bytes of the forward: read q, k, v; write o and lse (fp32)."""
    return elem * B * L * d * (2 * Hq + 2 * Hkv) + 4 * B * Hq * L


def bwd_bytes(B, L, Hq, Hkv, d, elem=2, grad_elem=2):
    """Algorithmic HBM bytes of the backward.

    Reads q, k, v, o, dO and lse; writes and re-reads the fp32 row term
    D = rowsum(dO * O); writes dq, dk, dv.
    """
    reads = elem * B * L * d * (3 * Hq + 2 * Hkv) + 4 * B * Hq * L
    delta = 2 * 4 * B * Hq * L
    writes = grad_elem * B * L * d * (Hq + 2 * Hkv)
    return reads + delta + writes


# Llama2-7B dimensions for the Table 7 reproduction.  Hidden size 4096 (32
# heads of 128) and vocabulary 32000 agree with the pages (the python88.com
# article puts the embedding at 1.94% of the 7B parameters); 32 layers and
# the FFN width 11008 are the published Llama2-7B architecture, not on the pages.
LLAMA2_7B = dict(layers=32, hidden=4096, ffn=11008, vocab=32000)


def llama2_7b_attention_share(L, keys_per_query, dims=LLAMA2_7B):
    """Fraction of per-token FLOPs spent in attention products (Table 7 convention).

    Linear layers per token: 2 * (layers * (4 h^2 + 3 h f) + h * vocab).
    Attention per token: layers * 4 * N * h with N = keys_per_query.
    """
    h, f, nl, V = dims["hidden"], dims["ffn"], dims["layers"], dims["vocab"]
    linear = 2.0 * (nl * (4 * h * h + 3 * h * f) + h * V)
    attn = nl * 4.0 * keys_per_query * h
    return attn / (attn + linear)


def block_flops(B, L, Hq, Hkv, d, G, r):
    """Counted FLOPs of one attention block (LoRA Q/K/V/O, frozen W) forward and backward.

    Each product is 2 * rows * fan_in * fan_out.  Forward: the projections
    x W^T (Q, K, V) and attn Wo^T, the LoRA down (x A^T, attn Ao^T) and up
    (u B^T) products, and S2-Attn.  Backward: dattn = dy Wo and dx = sum dz W
    (no dW: W is frozen), the LoRA factor gradients and the LoRA terms of
    dattn and dx, and the S2-Attn backward.  Returns (forward, backward).
    """
    M, Dm, Nq, Nkv = float(B) * L, Hq * d, Hq * d, Hkv * d
    n_qkv = Nq + 2 * Nkv
    fwd = (2 * M * Dm * n_qkv + 2 * M * Nq * Dm          # x W^T, attn Wo^T
           + 2 * M * r * (3 * Dm + Nq)                   # x A^T (q, k, v), attn Ao^T
           + 2 * M * r * (n_qkv + Dm)                    # u B^T
           + fwd_flops(B, L, Hq, d, G))
    bwd = (2 * M * Nq * Dm + 2 * M * Dm * n_qkv          # dy Wo, dz W
           + 2 * M * r * (Dm + n_qkv)                    # t = dz B
           + 2 * M * r * (Dm + n_qkv)                    # dB = dz^T u
           + 2 * M * r * (Nq + 3 * Dm)                   # dA = t^T (attn | x)
           + 2 * M * r * (Nq + 3 * Dm)                   # t A into dattn, dx
           + bwd_flops(B, L, Hq, d, G))
    return fwd, bwd
