"""The attention block around S2-Attn (s2block.h), with torch-allocated buffers.

`Block` holds a configuration; `forward` returns y and the activations the
backward needs, `backward` returns dx and the LoRA gradients.  Every step
runs in libs2attn (hipBLASLt projections, S2-Attn kernels).
"""

import torch

from . import _lib

PARAM_NAMES = ("wq", "wk", "wv", "wo", "aq", "ak", "av", "ao", "bq", "bk", "bv", "bo")


def param_shapes(Hq, Hkv, d, r):
    """Shapes of the frozen projections W and the LoRA factors A (down) and B (up)."""
    Dm, Nq, Nkv = Hq * d, Hq * d, Hkv * d
    return {"wq": (Nq, Dm), "wk": (Nkv, Dm), "wv": (Nkv, Dm), "wo": (Dm, Nq),
            "aq": (r, Dm), "ak": (r, Dm), "av": (r, Dm), "ao": (r, Nq),
            "bq": (Nq, r), "bk": (Nkv, r), "bv": (Nkv, r), "bo": (Dm, r)}


class Block:
    def __init__(self, B, L, Hq, Hkv, d, G, shifted_heads, lora_rank=8, lora_scale=2.0,
                 rope=None):
        c = _lib.s2block_config_init()
        c.B, c.L, c.Hq, c.Hkv, c.d, c.G, c.shifted_heads = B, L, Hq, Hkv, d, G, shifted_heads
        c.lora_rank, c.lora_scale = lora_rank, float(lora_scale)
        if rope is not None:
            c.rope, c.rope_base, c.rope_orig_len = 1, float(rope[0]), int(rope[1])
        self.cfg = c
        self.shape = (B, L, Hq, Hkv, d)
        self.r = lora_rank

    def workspace(self, is_bwd, device):
        n = _lib.s2block_workspace_size(is_bwd, self.cfg)
        if n == 0:
            raise ValueError("invalid block configuration")
        return torch.empty(n, dtype=torch.uint8, device=device), n

    def alloc_saved(self, device):
        B, L, Hq, Hkv, d = self.shape
        bf = torch.bfloat16
        return {"q": torch.empty(B, L, Hq, d, dtype=bf, device=device),
                "k": torch.empty(B, L, Hkv, d, dtype=bf, device=device),
                "v": torch.empty(B, L, Hkv, d, dtype=bf, device=device),
                "attn": torch.empty(B, L, Hq, d, dtype=bf, device=device),
                "lse": torch.empty(B, Hq, L, dtype=torch.float32, device=device),
                "u": torch.empty(B * L, 4 * self.r, dtype=bf, device=device)}

    def _check(self, x, params, saved=None, dy=None):
        """Shapes, dtypes and placement of every tensor, before any library call."""
        B, L, Hq, Hkv, d = self.shape
        named = [("x", x)]
        if tuple(x.shape) != (B, L, Hq * d) or x.dtype != torch.bfloat16:
            raise ValueError(f"x must be bfloat16 [{B}, {L}, {Hq * d}], got {x.dtype} {tuple(x.shape)}")
        shapes = param_shapes(Hq, Hkv, d, self.r)
        for name in PARAM_NAMES:
            t = params.get(name)
            if t is None or tuple(t.shape) != shapes[name] or t.dtype != torch.bfloat16:
                got = None if t is None else (t.dtype, tuple(t.shape))
                raise ValueError(f"params[{name!r}] must be bfloat16 {shapes[name]}, got {got}")
            named.append((name, t))
        if saved is not None:
            want = {k: (tuple(t.shape), t.dtype) for k, t in self.alloc_saved("meta").items()}
            for name, (shp, dt) in want.items():
                t = saved.get(name)
                if t is None or tuple(t.shape) != shp or t.dtype != dt:
                    got = None if t is None else (t.dtype, tuple(t.shape))
                    raise ValueError(f"saved[{name!r}] must be {dt} {shp}, got {got}")
                named.append(("saved " + name, t))
        if dy is not None:
            if dy.shape != x.shape or dy.dtype != x.dtype:
                raise ValueError("dy must match x in shape and dtype")
            named.append(("dy", dy))
        from . import _on_one_gpu
        _on_one_gpu(named)

    def forward(self, x, params, stream=None, ws=None):
        self._check(x, params)
        saved = self.alloc_saved(x.device)
        y = torch.empty_like(x)
        ws, n = ws if ws is not None else self.workspace(0, x.device)
        _lib.s2block_fwd(self.cfg, x, params, y, saved, ws, n, stream)
        return y, saved

    def backward(self, x, params, saved, dy, stream=None, ws=None):
        self._check(x, params, saved, dy)
        B, L, Hq, Hkv, d = self.shape
        grads = {"dx": torch.empty_like(x)}
        for name, shp in param_shapes(Hq, Hkv, d, self.r).items():
            if name[0] in "ab":
                grads["d" + name] = torch.empty(shp, dtype=torch.float32, device=x.device)
        ws, n = ws if ws is not None else self.workspace(1, x.device)
        _lib.s2block_bwd(self.cfg, x, params, saved, dy, grads, ws, n, stream)
        return grads
