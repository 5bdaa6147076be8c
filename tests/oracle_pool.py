"""Run the oracle's per-unit backward over many units in worker processes.

Test infrastructure: the workers call `oracle.s2attn.kv_unit_backward` on the
rows the parent gathers with `oracle.s2attn.kv_unit_inputs`, one KV unit per
task, with one BLAS thread each.  The pool is forked once at the start of a
test session, before any test touches the GPU, so the workers inherit no
device state; they run numpy only.
"""

import math
import multiprocessing as mp
import os

import numpy as np

from oracle import s2attn as O

_POOL = None


def _init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def workers():
    """Worker count: the host cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def start():
    global _POOL
    if _POOL is None:
        _POOL = mp.get_context("fork").Pool(workers(), initializer=_init_worker)
    return _POOL


def stop():
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None


def _task(args):
    key, qs, kg, vg, dos, scale, theta = args
    return key, O.kv_unit_backward(qs, kg, vg, dos, scale, theta)


def kv_units(x, G, shifted_heads, units, rope=None, scale=None):
    """{(b, hk, g): dict(rows, dk, dv, dq [r,G,d], o [r,G,d], lse [r,G])} for `units`."""
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    d = q.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows_of, tasks = {}, []
    for u in units:
        rows, qs, kg, vg, dos, theta = O.kv_unit_inputs(q, k, v, do, G, shifted_heads, u, rope)
        rows_of[u] = rows
        tasks.append((u, qs, kg, vg, dos, scale, theta))
    pool = _POOL if _POOL is not None else start()
    out = {}
    for key, res in pool.imap_unordered(_task, tasks):
        res["rows"] = rows_of[key]
        out[key] = res
    return out


def kv_units_gathered(tasks):
    """{key: kv_unit_backward result} for tasks already gathered by the caller:
    (key, qs [r, G, d], kg [G, d], vg [G, d], dos [r, G, d], scale, theta)."""
    pool = _POOL if _POOL is not None else start()
    return dict(pool.imap_unordered(_task, tasks))


def full_backward(x, G, shifted_heads, rope=None):
    """Whole reference tensors (o, lse, dq, dk, dv) in float64 from every KV unit."""
    q, k = x["q"], x["k"]
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    r = Hq // Hkv
    units = [(b, hk, g) for b in range(B) for hk in range(Hkv) for g in range(L // G)]
    res = kv_units(x, G, shifted_heads, units, rope)
    o = np.empty((B, L, Hq, d))
    dq = np.empty((B, L, Hq, d))
    lse = np.empty((B, Hq, L))
    dk = np.empty((B, L, Hkv, d))
    dv = np.empty((B, L, Hkv, d))
    for (b, hk, g), u in res.items():
        rows = u["rows"]
        for j in range(r):
            h = hk * r + j
            o[b, rows, h] = u["o"][j]
            dq[b, rows, h] = u["dq"][j]
            lse[b, h, rows] = u["lse"][j]
        dk[b, rows, hk] = u["dk"]
        dv[b, rows, hk] = u["dv"]
    return o, lse, dq, dk, dv


def _fwd_task(args):
    key, qg, kg, vg, scale = args
    return key, O.unit_forward(qg, kg, vg, scale)


def full_forward(q, k, v, G, shifted_heads, rope=None, scale=None):
    """Whole (o, lse) in float64 from every (b, h, g) unit's `unit_forward`,
    q and k rotated first (oracle.s2attn.rope_rotate) when `rope` is given."""
    B, L, Hq, d = q.shape
    r = Hq // k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    theta = O.rope_angles(L, d, *rope) if rope is not None else None
    rows_of, tasks = {}, []
    for b, h, g in O.units(B, Hq, L, G):
        rows = O.unit_rows(L, G, Hq, shifted_heads, h, g)
        qg = np.asarray(q[b, rows, h], dtype=np.float64)
        kg = np.asarray(k[b, rows, h // r], dtype=np.float64)
        if theta is not None:
            qg = O.rope_rotate(qg[None, :, None, :], theta[rows])[0, :, 0, :]
            kg = O.rope_rotate(kg[None, :, None, :], theta[rows])[0, :, 0, :]
        rows_of[(b, h, g)] = rows
        tasks.append(((b, h, g), qg, kg, np.asarray(v[b, rows, h // r], dtype=np.float64), scale))
    pool = _POOL if _POOL is not None else start()
    o = np.empty((B, L, Hq, d))
    lse = np.empty((B, Hq, L))
    for (b, h, g), (og, lg) in pool.imap_unordered(_fwd_task, tasks):
        rows = rows_of[(b, h, g)]
        o[b, rows, h] = og
        lse[b, h, rows] = lg
    return o, lse
