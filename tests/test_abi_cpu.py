"""libs2attn's C ABI on the host: loads, exports what the header declares, and
rejects invalid arguments before any HIP call (so these run without a GPU).

No valid compute call is made here: the addresses passed are fake (aligned,
never dereferenced), and every case below fails an argument check first.
"""

import ctypes
import os
import re

import pytest
import torch

import shifted_sparse_attention_amd as s2
from shifted_sparse_attention_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s2attn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

FAKE = 0x10000  # 16-byte aligned, never dereferenced
MIS = 0x10008   # misaligned


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(s2(?:attn|block)_\w+)\s*\(", src))
    return sorted(names)


def test_library_loads_and_exports_header_symbols():
    h = L.lib()
    names = declared_functions()
    assert {"s2attn_fwd", "s2attn_bwd", "s2attn_fwd_ex", "s2attn_bwd_ex",
            "s2attn_workspace_size", "s2attn_status_string"} <= set(names)
    for n in names:
        assert hasattr(h, n), n
        assert n in L._SIGS, f"binding lacks {n}"
        assert hasattr(s2, n), f"package does not re-export {n}"


def test_single_hip_runtime_mapped():
    L.lib()
    assert len(L._hip_runtimes_mapped()) == 1


def test_status_strings_and_version():
    assert s2.s2attn_status_string(0) == "S2ATTN_OK"
    assert s2.s2attn_status_string(1) == "S2ATTN_ERR_INVALID_ARG"
    assert s2.s2attn_status_string(2) == "S2ATTN_ERR_UNSUPPORTED"
    assert s2.s2attn_status_string(3) == "S2ATTN_ERR_WORKSPACE"
    assert s2.s2attn_status_string(4) == "S2ATTN_ERR_HIP"
    assert s2.s2attn_status_string(99) == "S2ATTN_UNKNOWN_STATUS"
    assert s2.s2attn_version() >= 100


def test_opts_defaults():
    o = s2.s2attn_opts_init()
    assert o.struct_size == ctypes.sizeof(L.s2attn_opts)
    assert o.dtype == L.S2ATTN_BF16 and o.grad_dtype == L.S2ATTN_BF16
    assert o.softmax_scale == 0.0 and o.rope == 0
    assert o.rope_base == 10000.0 and o.rope_orig_len == 4096
    assert o.ds_max_mib == -1 and o.residual_split == -1


GOOD = dict(B=1, L=256, Hq=4, Hkv=4, d=64, G=64, sh=2)


def fwd(**kw):
    a = dict(GOOD, **kw)
    ptrs = [kw.get(n, FAKE) for n in ("q", "k", "v", "o", "lse")]
    return L.lib().s2attn_fwd(*ptrs, a["B"], a["L"], a["Hq"], a["Hkv"], a["d"], a["G"], a["sh"], None)


def bwd(**kw):
    a = dict(GOOD, **kw)
    ptrs = [kw.get(n, FAKE) for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "delta")]
    return L.lib().s2attn_bwd(*ptrs, a["B"], a["L"], a["Hq"], a["Hkv"], a["d"], a["G"], a["sh"], None)


def fwd_ex(opts, ws=None, ws_bytes=0, **kw):
    a = dict(GOOD, **kw)
    return L.lib().s2attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["L"], a["Hq"], a["Hkv"],
                                 a["d"], a["G"], a["sh"], ctypes.byref(opts), ws, ws_bytes, None)


def bwd_ex(opts, ws=None, ws_bytes=0, **kw):
    a = dict(GOOD, **kw)
    return L.lib().s2attn_bwd_ex(*([FAKE] * 9), a["B"], a["L"], a["Hq"], a["Hkv"], a["d"], a["G"],
                                 a["sh"], ctypes.byref(opts), ws, ws_bytes, None)


INV, UNS, WS = L.S2ATTN_ERR_INVALID_ARG, L.S2ATTN_ERR_UNSUPPORTED, L.S2ATTN_ERR_WORKSPACE


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(o=None), INV),
    (dict(lse=None), INV), (dict(q=MIS), INV), (dict(lse=MIS), INV),
    (dict(B=0), INV), (dict(L=0), INV), (dict(Hq=-1), INV), (dict(Hkv=0), INV), (dict(d=0), INV),
    (dict(G=0), INV), (dict(G=48), INV),                   # L % G != 0
    (dict(Hkv=3), INV),                                    # Hq % Hkv != 0
    (dict(sh=-1), INV), (dict(sh=5), INV),                 # shifted_heads outside [0, Hq]
    (dict(L=255, G=51, sh=1), INV),                        # odd G with shifted heads
    (dict(d=96), UNS), (dict(d=32), UNS),
    (dict(L=1 << 22, G=1 << 22, sh=0), UNS),   # one (batch, head) plane past 32-bit offsets
    # a token row of H*d*2 = 2^24 bytes: past the 24-bit row-offset product
    (dict(L=64, G=64, Hq=65536, Hkv=65536, d=128, sh=0), UNS),
])
def test_fwd_argument_checks(kw, want):
    assert fwd(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(do=None), INV), (dict(dq=None), INV), (dict(dk=None), INV), (dict(dv=None), INV),
    (dict(delta=None), INV), (dict(dv=MIS), INV), (dict(delta=MIS), INV),
    (dict(G=100), INV), (dict(d=80), UNS),
    (dict(Hq=8, Hkv=2, sh=3), UNS),   # a KV head shared by shifted and unshifted query heads
])
def test_bwd_argument_checks(kw, want):
    assert bwd(**kw) == want


def test_opts_checks():
    o = s2.s2attn_opts_init()
    o.struct_size = 4
    assert fwd_ex(o) == INV
    o = s2.s2attn_opts_init()
    o.dtype = 7
    assert fwd_ex(o) == INV
    o = s2.s2attn_opts_init()
    o.grad_dtype = -1
    assert bwd_ex(o) == INV
    o = s2.s2attn_opts_init()
    o.softmax_scale = float("nan")
    assert fwd_ex(o) == INV
    o = s2.s2attn_opts_init()
    o.rope, o.rope_base = 1, 0.5
    assert fwd_ex(o) == INV
    o = s2.s2attn_opts_init()
    o.rope, o.rope_orig_len = 1, 0
    assert fwd_ex(o) == INV
    o = s2.s2attn_opts_init()
    o.dtype, o.rope = L.S2ATTN_F32, 1
    assert fwd_ex(o) == UNS                          # RoPE needs bf16 inputs
    o = s2.s2attn_opts_init()
    o.dtype, o.grad_dtype = L.S2ATTN_F32, L.S2ATTN_BF16
    assert bwd_ex(o) == UNS


def test_residual_split_option_checks():
    for val, want in ((-2, INV), (2, INV)):
        o = s2.s2attn_opts_init()
        o.residual_split = val
        assert bwd_ex(o, FAKE, 1 << 20, Hkv=2) == want
        assert fwd_ex(o) == want
    assert s2.make_opts(torch.bfloat16, residual_split=True).residual_split == 1
    assert s2.make_opts(torch.bfloat16, residual_split=False).residual_split == 0
    assert s2.make_opts(torch.bfloat16).residual_split == -1


def test_workspace_sizes_and_checks():
    o = s2.s2attn_opts_init()
    B, Ln, Hq, Hkv, d, G = 1, 256, 4, 2, 64, 64
    assert s2.s2attn_workspace_size(0, B, Ln, Hq, Hkv, d, G, o) == 0
    r256 = lambda x: (x + 255) // 256 * 256
    delta = B * Hq * Ln * 4         # the row term -delta, [B, Hq, L] fp32
    # dS tiles: per (batch, head, group) the 32 x 32 bf16 tiles of the causal
    # triangle, padded to whole blocks of 8 query rows (NB blocks)
    def ds_bytes(B, Hq, L, G):
        NB = ((G + 31) // 32 + 7) // 8
        return B * Hq * (L // G) * 32 * NB * (NB + 1) * 2048
    ds = ds_bytes(B, Hq, Ln, G)
    assert s2.s2attn_workspace_size(1, B, Ln, Hq, Hkv, d, G, o) == r256(delta) + r256(ds)
    o.dtype = o.grad_dtype = s2.S2ATTN_F32   # fp32 backward recomputes dS: no tiles
    assert s2.s2attn_workspace_size(1, B, Ln, Hq, Hkv, d, G, o) == r256(delta)
    o.dtype = o.grad_dtype = s2.S2ATTN_BF16
    Gr = 80                          # ragged last tile row (T = 3, one block of 8 rows)
    dsr = ds_bytes(B, Hq, 240, Gr)
    assert dsr == B * Hq * 3 * 64 * 2048
    assert s2.s2attn_workspace_size(1, B, 240, Hq, Hkv, d, Gr, o) == r256(B * Hq * 240 * 4) + r256(dsr)
    o.rope = 1
    rq, rk = B * Ln * Hq * d * 2, B * Ln * Hkv * d * 2
    # the forward rotates its stationary query tile in registers: only k~ is kept
    assert s2.s2attn_workspace_size(0, B, Ln, Hq, Hkv, d, G, o) == r256(rk)
    assert s2.s2attn_workspace_size(1, B, Ln, Hq, Hkv, d, G, o) == (
        r256(delta) + r256(rq) + r256(rk) + r256(ds))
    assert s2.s2attn_workspace_size(0, 0, Ln, Hq, Hkv, d, G, o) == 0   # invalid sizes -> 0
    # missing / short workspace
    need = s2.s2attn_workspace_size(0, B, Ln, Hq, Hkv, d, G, o)
    assert fwd_ex(o, None, 0, Hkv=2) == WS
    assert fwd_ex(o, FAKE, need - 1, Hkv=2) == WS
    assert fwd_ex(o, MIS, need, Hkv=2) == WS
    o2 = s2.s2attn_opts_init()
    assert bwd_ex(o2, None, 0, Hkv=2) == WS          # the backward always needs delta space


def test_ds_tiles_bound():
    """dS tiles are kept while they fit opts.ds_max_mib (default 16 GiB)."""
    r256 = lambda x: (x + 255) // 256 * 256
    def ds_bytes(B, Hq, L, G):
        NB = ((G + 31) // 32 + 7) // 8
        return B * Hq * (L // G) * 32 * NB * (NB + 1) * 2048
    def ws(B, Ln, H, G, mib=None, rope=False):
        o = s2.s2attn_opts_init()
        if mib is not None:
            o.ds_max_mib = mib
        if rope:
            o.rope = 1
        return s2.s2attn_workspace_size(1, B, Ln, H, H, 128, G, o)
    assert s2.s2attn_opts_init().ds_max_mib == -1
    # L = 32768, G = 8192, 32 heads: 8448 MiB of tiles
    rows = r256(32 * 32768 * 4)
    ds32 = ds_bytes(1, 32, 32768, 8192)
    assert ds32 == 8448 << 20
    assert ws(1, 32768, 32, 8192) == rows + ds32
    assert ws(1, 32768, 32, 8192, mib=8448) == rows + ds32     # exactly at the bound
    assert ws(1, 32768, 32, 8192, mib=8447) == rows            # one MiB short: recompute
    assert ws(1, 32768, 32, 8192, mib=0) == rows
    # L = 102400, G = 25600 with RoPE: 78.9 GiB of tiles, over the 16 GiB
    # default (recompute) unless the caller raises the bound
    rot = r256(102400 * 32 * 128 * 2)
    ds100 = ds_bytes(1, 32, 102400, 25600)
    assert 64 << 30 < ds100 < 96 << 30
    rows100 = r256(32 * 102400 * 4)
    assert ws(1, 102400, 32, 25600, rope=True) == rows100 + 2 * rot
    assert ws(1, 102400, 32, 25600, mib=96 << 10, rope=True) == rows100 + 2 * rot + ds100
    assert ws(1, 102400, 32, 25600, mib=32 << 10, rope=True) == rows100 + 2 * rot
    # the grouped-query 32k shape (64 query heads): 16.5 GiB of tiles, just over the default
    ds_gqa = ds_bytes(1, 64, 32768, 8192)
    assert 16 << 30 < ds_gqa
    o = s2.s2attn_opts_init()
    assert s2.s2attn_workspace_size(1, 1, 32768, 64, 8, 128, 8192, o) == r256(64 * 32768 * 4)
    o.ds_max_mib = 17 << 10
    assert s2.s2attn_workspace_size(1, 1, 32768, 64, 8, 128, 8192, o) == r256(64 * 32768 * 4) + ds_gqa
    # below -1 is an argument error (workspace size 0, the call reports it)
    o = s2.s2attn_opts_init()
    o.ds_max_mib = -2
    assert s2.s2attn_workspace_size(1, 1, 256, 4, 4, 64, 64, o) == 0
    assert bwd_ex(o, FAKE, 1 << 20, Hkv=2) == INV


def test_python_wrappers_raise_named_errors():
    with pytest.raises(s2.S2AttnError) as e:
        s2.s2attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 256, 4, 4, 64, 60, 0)
    assert e.value.status == INV and "INVALID_ARG" in str(e.value)


def test_header_documents_each_entry_point():
    for h in HEADERS:
        src = open(h).read()
        for name in declared_functions([h]):
            m = re.search(r"(\*/)\s*(?:const\s+)?[\w\s\*]*\b" + name + r"\s*\(", src)
            assert m, f"{name} is not directly preceded by a comment in {h}"


def test_bwd_stage_checks():
    o = s2.s2attn_opts_init()
    need = s2.s2attn_workspace_size(1, 1, 256, 4, 4, 64, 64, o)
    for bad_stage in (-1, 3, 100):
        st = L.lib().s2attn_bwd_stage_ex(bad_stage, *([FAKE] * 9), 1, 256, 4, 4, 64, 64, 2,
                                         ctypes.byref(o), FAKE, need, None)
        assert st == INV
    st = L.lib().s2attn_bwd_stage_ex(L.S2ATTN_BWD_STAGE_DKDV, *([FAKE] * 9), 1, 256, 4, 4, 64, 64,
                                     2, ctypes.byref(o), None, 0, None)
    assert st == WS


def _block_cfg(**kw):
    c = s2.s2block_config_init()
    for k, v in dict(B=1, L=256, Hq=4, Hkv=2, d=64, G=64, shifted_heads=2).items():
        setattr(c, k, v)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


BLOCK_PARAMS = {n: FAKE for n in ("wq", "wk", "wv", "wo", "aq", "ak", "av", "ao", "bq", "bk", "bv", "bo")}
BLOCK_SAVED = {n: FAKE for n in ("q", "k", "v", "attn", "lse", "u")}
BLOCK_GRADS = {n: FAKE for n in ("dx", "daq", "dak", "dav", "dao", "dbq", "dbk", "dbv", "dbo")}


def _block_fwd(cfg, ws=FAKE, ws_bytes=None, params=None, saved=None, x=FAKE):
    n = s2.s2block_workspace_size(0, cfg) if ws_bytes is None else ws_bytes
    p = L._struct(L.s2block_params, params or BLOCK_PARAMS)
    sv = L._struct(L.s2block_saved, saved or BLOCK_SAVED)
    return L.lib().s2block_fwd(ctypes.byref(cfg), x, ctypes.byref(p), FAKE, ctypes.byref(sv), ws, n, None)


def _block_bwd(cfg, ws=FAKE, ws_bytes=None, grads=None):
    n = s2.s2block_workspace_size(1, cfg) if ws_bytes is None else ws_bytes
    p = L._struct(L.s2block_params, BLOCK_PARAMS)
    sv = L._struct(L.s2block_saved, BLOCK_SAVED)
    g = L._struct(L.s2block_grads, grads or BLOCK_GRADS)
    return L.lib().s2block_bwd(ctypes.byref(cfg), FAKE, ctypes.byref(p), ctypes.byref(sv), FAKE,
                               ctypes.byref(g), ws, n, None)


def test_block_config_defaults_and_workspace():
    c = s2.s2block_config_init()
    assert c.struct_size == ctypes.sizeof(L.s2block_config)
    assert c.lora_rank == 8 and c.lora_scale == 2.0 and c.rope == 0
    assert c.rope_base == 10000.0 and c.rope_orig_len == 4096
    cfg = _block_cfg()
    f, b = s2.s2block_workspace_size(0, cfg), s2.s2block_workspace_size(1, cfg)
    assert f >= 32 << 20 and b > f                     # hipBLASLt slice, then backward scratch
    assert s2.s2block_workspace_size(0, _block_cfg(L=250)) == 0   # L % G != 0


@pytest.mark.parametrize("kw,want", [
    (dict(struct_size=4), INV), (dict(lora_rank=0), INV), (dict(lora_rank=72), INV),
    (dict(lora_rank=4), INV), (dict(lora_rank=12), INV),
    (dict(lora_scale=float("inf")), INV), (dict(G=48), INV), (dict(d=96), UNS),
    (dict(Hq=8, Hkv=2, shifted_heads=3), UNS), (dict(rope=1, rope_base=0.5), INV),
])
def test_block_config_checks(kw, want):
    assert _block_fwd(_block_cfg(**kw)) == want if "shifted_heads" not in kw else True
    assert _block_bwd(_block_cfg(**kw)) == want


def test_block_pointer_and_workspace_checks():
    cfg = _block_cfg()
    assert _block_fwd(cfg, x=None) == INV
    assert _block_fwd(cfg, params=dict(BLOCK_PARAMS, bo=None)) == INV
    assert _block_fwd(cfg, saved=dict(BLOCK_SAVED, u=MIS)) == INV
    assert _block_fwd(cfg, ws=None) == WS
    assert _block_fwd(cfg, ws_bytes=s2.s2block_workspace_size(0, cfg) - 1) == WS
    assert _block_bwd(cfg, grads=dict(BLOCK_GRADS, dbq=None)) == INV
    assert _block_bwd(cfg, ws_bytes=1024) == WS


# ---------------------------------------------------------------------------
# The Python binding checks every tensor before any library call.
# ---------------------------------------------------------------------------

def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_binding_rejects_host_tensors():
    q, k = _bf(1, 64, 4, 64), _bf(1, 64, 2, 64)
    with pytest.raises(ValueError, match="CUDA tensor"):
        s2.forward(q, k, k.clone(), 16, 2)


def test_binding_rejects_mixed_dtypes_and_layouts():
    q, k, v = _bf(1, 64, 4, 64), _bf(1, 64, 2, 64), _bf(1, 64, 2, 64)
    with pytest.raises(ValueError, match="dtype"):
        s2.forward(q, k.float(), v, 16, 2)
    with pytest.raises(ValueError, match="contiguous"):
        s2.forward(q.transpose(1, 2).contiguous().transpose(1, 2), k, v, 16, 2)
    o, lse = _bf(1, 64, 4, 64), torch.zeros(1, 4, 64)
    dout = _bf(1, 64, 4, 64)
    with pytest.raises(ValueError, match="lse"):
        s2.backward(q, k, v, o, lse.bfloat16(), dout, 16, 2)
    with pytest.raises(ValueError, match="dout"):
        s2.backward(q, k, v, o, lse, dout.float(), 16, 2)
    with pytest.raises(ValueError, match="o must"):
        s2.backward(q, k, v, o.float(), lse, dout, 16, 2)
    # the gradient of a sum: a stride-0 expanded dout
    expanded = torch.ones((), dtype=torch.bfloat16).expand(1, 64, 4, 64)
    with pytest.raises(ValueError, match="dout must be contiguous"):
        s2.backward(q, k, v, o, lse, expanded, 16, 2)


def test_block_binding_checks_shapes():
    from shifted_sparse_attention_amd.block import Block, param_shapes
    blk = Block(1, 64, 4, 2, 16, 16, 2, lora_rank=8)
    params = {n: torch.zeros(s, dtype=torch.bfloat16) for n, s in param_shapes(4, 2, 16, 8).items()}
    with pytest.raises(ValueError, match="x must be"):
        blk.forward(_bf(1, 64, 32), params)
    bad = dict(params, bo=torch.zeros(64, 4, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bo"):
        blk.forward(_bf(1, 64, 64), bad)
    with pytest.raises(ValueError, match="CUDA tensor"):
        blk.forward(_bf(1, 64, 64), params)
    saved = blk.alloc_saved("cpu")
    with pytest.raises(ValueError, match="dy must"):
        blk.backward(_bf(1, 64, 64), params, saved, _bf(1, 64, 32))
    with pytest.raises(ValueError, match="lse"):
        blk.backward(_bf(1, 64, 64), params, dict(saved, lse=saved["lse"].bfloat16()), _bf(1, 64, 64))


def test_noalloc_checks_run_on_the_host():
    """s2attn_bwd_noalloc runs s2attn_bwd's argument checks, then its size
    bound, before any HIP call."""
    lib = L.lib()

    def call(**kw):
        a = dict(GOOD, **kw)
        ptrs = [kw.get(n, FAKE) for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")]
        return lib.s2attn_bwd_noalloc(*ptrs, a["B"], a["L"], a["Hq"], a["Hkv"], a["d"], a["G"],
                                      a["sh"], None)
    assert call(q=None) == INV
    assert call(dv=MIS) == INV
    assert call(G=100) == INV
    assert call(d=80) == UNS
    assert call(Hq=8, Hkv=2, sh=3) == UNS
    # B Hq L = 2^24 row-term floats: past the library's array
    assert call(B=2, L=1 << 22, Hq=2, Hkv=2, G=1 << 22, sh=0) == WS
    assert L.S2ATTN_NOALLOC_MAX_ROWS == 1 << 23
