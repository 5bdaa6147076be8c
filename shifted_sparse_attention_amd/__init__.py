"""libs2attn: S2-Attn (LongLoRA's shift short attention) forward and backward on MI355X.

The C entry points are re-exported under their own names (`s2attn_fwd`,
`s2attn_bwd`, `s2attn_fwd_ex`, `s2attn_bwd_ex`, `s2attn_workspace_size`, ...).
`forward` and `backward` allocate outputs with torch and call them.

Tensors are [B, L, H, d] contiguous (q, o, dout: H = Hq; k, v: H = Hkv); LSE
is [B, Hq, L] float32.  The last `shifted_heads` query heads attend within
groups shifted by G/2 tokens.
"""

import math

import torch

from . import flops  # noqa: F401
from ._lib import (  # noqa: F401
    LIB_PATH, S2ATTN_BF16, S2ATTN_BWD_STAGE_DKDV, S2ATTN_BWD_STAGE_DQ, S2ATTN_BWD_STAGE_PRE,
    S2ATTN_ERR_HIP, S2ATTN_ERR_INVALID_ARG, S2ATTN_ERR_UNSUPPORTED, S2ATTN_ERR_WORKSPACE,
    S2ATTN_F32, S2ATTN_OK, S2AttnError, lib, s2attn_bwd, s2attn_bwd_ex, s2attn_bwd_noalloc, s2attn_bwd_stage_ex,
    S2ATTN_NOALLOC_MAX_ROWS,
    s2attn_fwd, s2attn_fwd_ex, s2attn_opts, s2attn_opts_init, s2attn_status_string,
    s2attn_version, s2attn_workspace_size, s2block_bwd, s2block_config, s2block_config_init,
    s2block_fwd, s2block_grads, s2block_params, s2block_saved, s2block_workspace_size)
from . import block  # noqa: F401,E402

_DT = {torch.bfloat16: S2ATTN_BF16, torch.float32: S2ATTN_F32}


def _on_one_gpu(named):
    """Every tensor contiguous and on one CUDA device (checked before any
    library call: a strided view or a host pointer would be read as a dense
    device buffer)."""
    for name, t in named:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (strides {tuple(t.stride())})")
    dev = None
    for name, t in named:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} like the other tensors")


def _shapes(q, k, v, placed=True):
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, L, Hq, d]; k and v [B, L, Hkv, d]")
    B, L, Hq, d = q.shape
    if k.shape[0] != B or k.shape[1] != L or k.shape[3] != d:
        raise ValueError("k, v must match q in B, L and d")
    if q.dtype not in _DT:
        raise ValueError("q, k, v must be torch.bfloat16 or torch.float32")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
    if placed:
        _on_one_gpu((("q", q), ("k", k), ("v", v)))
    return B, L, Hq, k.shape[2], d


def make_opts(dtype, grad_dtype=None, scale=None, rope=None, ds_max_mib=None,
              residual_split=None):
    """Build s2attn_opts.  `rope` is None or (base, orig_len); `ds_max_mib`
    bounds the dS tiles the backward keeps in its workspace (None: the
    library default, 0: never); `residual_split` True / False forces the
    bf16 backward's residual products of P and dS on or off (None: by shape)."""
    gd = grad_dtype if grad_dtype is not None else dtype
    if dtype not in _DT or gd not in _DT:
        raise ValueError("dtypes must be torch.bfloat16 or torch.float32")
    o = s2attn_opts_init()
    o.dtype = _DT[dtype]
    o.grad_dtype = _DT[gd]
    o.softmax_scale = 0.0 if scale is None else float(scale)
    if rope is not None:
        o.rope = 1
        o.rope_base = float(rope[0])
        o.rope_orig_len = int(rope[1])
    if ds_max_mib is not None:
        o.ds_max_mib = int(ds_max_mib)
    if residual_split is not None:
        o.residual_split = 1 if residual_split else 0
    return o


def forward(q, k, v, G, shifted_heads, *, scale=None, rope=None, stream=None):
    """S2-Attn forward.  Returns (o, lse)."""
    B, L, Hq, Hkv, d = _shapes(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    opts = make_opts(q.dtype, scale=scale, rope=rope)
    ws_bytes = s2attn_workspace_size(0, B, L, Hq, Hkv, d, G, opts)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    s2attn_fwd_ex(q, k, v, o, lse, B, L, Hq, Hkv, d, G, shifted_heads, opts, ws, ws_bytes, stream)
    return o, lse


def backward(q, k, v, o, lse, dout, G, shifted_heads, *, scale=None, rope=None,
             grad_dtype=None, ds_max_mib=None, residual_split=None, stream=None):
    """S2-Attn backward.  Returns (dq, dk, dv) in `grad_dtype` (default: q's dtype).

    The workspace it allocates holds the dS tiles (about B Hq L G bytes) unless
    they exceed `ds_max_mib` MiB (default 16 GiB; 0: dQ recomputes instead).
    """
    B, L, Hq, Hkv, d = _shapes(q, k, v, placed=False)
    if dout.shape != q.shape or o.shape != q.shape or lse.shape != (B, Hq, L):
        raise ValueError("o and dout must match q; lse must be [B, Hq, L]")
    for name, t in (("o", o), ("dout", dout)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
    if lse.dtype != torch.float32:
        raise ValueError(f"lse must be torch.float32, got {lse.dtype}")
    _on_one_gpu((("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)))
    gd = grad_dtype if grad_dtype is not None else q.dtype
    dq = torch.empty(q.shape, dtype=gd, device=q.device)
    dk = torch.empty(k.shape, dtype=gd, device=q.device)
    dv = torch.empty(v.shape, dtype=gd, device=q.device)
    opts = make_opts(q.dtype, grad_dtype=gd, scale=scale, rope=rope, ds_max_mib=ds_max_mib,
                     residual_split=residual_split)
    ws_bytes = s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    s2attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, L, Hq, Hkv, d, G, shifted_heads,
                  opts, ws, ws_bytes, stream)
    return dq, dk, dv


def default_scale(d):
    return 1.0 / math.sqrt(d)
