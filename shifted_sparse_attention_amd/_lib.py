"""ctypes binding to libs2attn.so: the C entry points under the same names.

Argument marshalling only: tensors become device pointers, streams become
hipStream_t handles, a nonzero status becomes an exception.  All computation
happens in the library's HIP kernels.  A missing library is an error; there is
no fallback of any kind.
"""

import ctypes
import os

import torch  # loads torch's HIP runtime first; libs2attn links against the same one

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libs2attn.so")

S2ATTN_OK = 0
S2ATTN_ERR_INVALID_ARG = 1
S2ATTN_ERR_UNSUPPORTED = 2
S2ATTN_ERR_WORKSPACE = 3
S2ATTN_ERR_HIP = 4

S2ATTN_BF16 = 0
S2ATTN_F32 = 1

S2ATTN_BWD_STAGE_PRE = 0
S2ATTN_BWD_STAGE_DKDV = 1
S2ATTN_BWD_STAGE_DQ = 2


class S2AttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_name(status)} ({status})")


class s2attn_opts(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("rope", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("rope_orig_len", ctypes.c_int32),
        ("ds_max_mib", ctypes.c_int32),
        ("residual_split", ctypes.c_int32),
    ]


class s2block_config(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("L", ctypes.c_int32), ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("G", ctypes.c_int32), ("shifted_heads", ctypes.c_int32),
        ("lora_rank", ctypes.c_int32),
        ("lora_scale", ctypes.c_float),
        ("rope", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("rope_orig_len", ctypes.c_int32),
    ]


class s2block_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("wq", "wk", "wv", "wo", "aq", "ak", "av", "ao", "bq", "bk", "bv", "bo")]


class s2block_saved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v", "attn", "lse", "u")]


class s2block_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "daq", "dak", "dav", "dao", "dbq", "dbk", "dbv", "dbo")]


_lib = None

_vp, _ci, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "s2attn_opts_init": (None, [ctypes.POINTER(s2attn_opts)]),
    "s2attn_fwd": (_ci, [_vp, _vp, _vp, _vp, _vp] + [_ci] * 7 + [_vp]),
    "s2attn_bwd": (_ci, [_vp] * 10 + [_ci] * 7 + [_vp]),
    "s2attn_bwd_noalloc": (_ci, [_vp] * 9 + [_ci] * 7 + [_vp]),
    "s2attn_workspace_size": (_sz, [_ci] * 7 + [ctypes.POINTER(s2attn_opts)]),
    "s2attn_fwd_ex": (_ci, [_vp] * 5 + [_ci] * 7 + [ctypes.POINTER(s2attn_opts), _vp, _sz, _vp]),
    "s2attn_bwd_ex": (_ci, [_vp] * 9 + [_ci] * 7 + [ctypes.POINTER(s2attn_opts), _vp, _sz, _vp]),
    "s2attn_bwd_stage_ex": (_ci, [_ci] + [_vp] * 9 + [_ci] * 7
                            + [ctypes.POINTER(s2attn_opts), _vp, _sz, _vp]),
    "s2attn_status_string": (ctypes.c_char_p, [_ci]),
    "s2attn_version": (_ci, []),
    "s2block_config_init": (s2block_config, []),
    "s2block_workspace_size": (_sz, [_ci, ctypes.POINTER(s2block_config)]),
    "s2block_fwd": (_ci, [ctypes.POINTER(s2block_config), _vp, ctypes.POINTER(s2block_params), _vp,
                          ctypes.POINTER(s2block_saved), _vp, _sz, _vp]),
    "s2block_bwd": (_ci, [ctypes.POINTER(s2block_config), _vp, ctypes.POINTER(s2block_params),
                          ctypes.POINTER(s2block_saved), _vp, ctypes.POINTER(s2block_grads), _vp,
                          _sz, _vp]),
}


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def lib():
    """Load libs2attn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m shifted_sparse_attention_amd.build`")
    h = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped in this process: {runtimes}")
    _lib = h
    return h


def status_name(status):
    return lib().s2attn_status_string(int(status)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    raise TypeError(f"expected a tensor, an int address or None, got {type(x)}")


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    raise TypeError("stream must be None, an int handle or a torch.cuda.Stream")


def _opts_ptr(opts):
    return None if opts is None else ctypes.byref(opts)


def _check(status, what):
    if status != S2ATTN_OK:
        raise S2AttnError(status, what)


def s2attn_opts_init():
    o = s2attn_opts()
    lib().s2attn_opts_init(ctypes.byref(o))
    return o


def s2attn_fwd(q, k, v, o, lse, B, L, Hq, Hkv, d, G, shifted_heads, stream=None):
    _check(lib().s2attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                            B, L, Hq, Hkv, d, G, shifted_heads, _stream(stream)), "s2attn_fwd")


def s2attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, L, Hq, Hkv, d, G, shifted_heads,
               stream=None):
    _check(lib().s2attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta_ws),
                            B, L, Hq, Hkv, d, G, shifted_heads, _stream(stream)), "s2attn_bwd")


S2ATTN_NOALLOC_MAX_ROWS = 1 << 23


def s2attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, L, Hq, Hkv, d, G, shifted_heads,
                       stream=None):
    _check(lib().s2attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                    _ptr(dq), _ptr(dk), _ptr(dv), B, L, Hq, Hkv, d, G,
                                    shifted_heads, _stream(stream)), "s2attn_bwd_noalloc")


def s2attn_workspace_size(is_bwd, B, L, Hq, Hkv, d, G, opts=None):
    return int(lib().s2attn_workspace_size(int(is_bwd), B, L, Hq, Hkv, d, G, _opts_ptr(opts)))


def s2attn_fwd_ex(q, k, v, o, lse, B, L, Hq, Hkv, d, G, shifted_heads, opts, ws, ws_bytes,
                  stream=None):
    _check(lib().s2attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               B, L, Hq, Hkv, d, G, shifted_heads, _opts_ptr(opts), _ptr(ws),
                               int(ws_bytes), _stream(stream)), "s2attn_fwd_ex")


def s2attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, L, Hq, Hkv, d, G, shifted_heads, opts,
                  ws, ws_bytes, stream=None):
    _check(lib().s2attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, L, Hq, Hkv, d, G, shifted_heads,
                               _opts_ptr(opts), _ptr(ws), int(ws_bytes), _stream(stream)),
           "s2attn_bwd_ex")


def s2attn_bwd_stage_ex(stage, q, k, v, o, lse, dout, dq, dk, dv, B, L, Hq, Hkv, d, G,
                        shifted_heads, opts, ws, ws_bytes, stream=None):
    _check(lib().s2attn_bwd_stage_ex(int(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, L, Hq, Hkv, d,
                                     G, shifted_heads, _opts_ptr(opts), _ptr(ws), int(ws_bytes),
                                     _stream(stream)), f"s2attn_bwd_stage_ex({stage})")


def s2attn_status_string(status):
    return status_name(status)


def s2attn_version():
    return int(lib().s2attn_version())


def s2block_config_init():
    return lib().s2block_config_init()


def s2block_workspace_size(is_bwd, cfg):
    return int(lib().s2block_workspace_size(int(is_bwd), ctypes.byref(cfg)))


def _struct(cls, d):
    return cls(**{name: _ptr(d[name]) for name, _ in cls._fields_})


def s2block_fwd(cfg, x, params, y, saved, ws, ws_bytes, stream=None):
    """params / saved: dicts of tensors keyed by the struct field names."""
    p, sv = _struct(s2block_params, params), _struct(s2block_saved, saved)
    _check(lib().s2block_fwd(ctypes.byref(cfg), _ptr(x), ctypes.byref(p), _ptr(y), ctypes.byref(sv),
                             _ptr(ws), int(ws_bytes), _stream(stream)), "s2block_fwd")


def s2block_bwd(cfg, x, params, saved, dy, grads, ws, ws_bytes, stream=None):
    p, sv = _struct(s2block_params, params), _struct(s2block_saved, saved)
    g = _struct(s2block_grads, grads)
    _check(lib().s2block_bwd(ctypes.byref(cfg), _ptr(x), ctypes.byref(p), ctypes.byref(sv), _ptr(dy),
                             ctypes.byref(g), _ptr(ws), int(ws_bytes), _stream(stream)),
           "s2block_bwd")
