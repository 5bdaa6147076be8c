"""Throughput of S2-Attn forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

With --workload, any bf16 workload of seeded_inputs.CONFIGS (forward-only
ones time the forward alone) or of seeded_inputs.BLOCK_CONFIGS (the attention
block around S2-Attn: LoRA Q/K/V/O projections, RoPE-PI, forward+backward).

A step is one pass of the whole path over one batch of synthetic inputs
already resident in HBM: the forward (O, LSE) and the backward (row term,
dK/dV, dQ).  The default workload is Llama2-7B heads at 32k context
(B=1, Hq=Hkv=32, d=128, L=32768, G=8192, 16 heads shifted), seeded N(0, 1)
inputs rounded to bf16.  Throughput counts group-local causal FLOPs
(forward 2*B*Hq*L*G*d, backward 2.5x that).

Printed: one JSON line with the throughput, the roofline of the dominant
kernel (its average duration from HIP events recorded on its launch stream
inside the timed region) and the CPU oracle timed on a bounded sample.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "S²-Attn fwd+bwd TFLOP/s and % of bf16 MFMA peak, Llama2-7B heads, L=32k"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwdbwd_bf16_L32k.json")


# The sources that define the attention kernels the stored counters describe.
KERNEL_SOURCES = ("s2_device.h", "s2_params.h", "s2attn_fwd.hip", "s2attn_bwd.hip")


def kernel_source_sha():
    """Hash of the attention kernels' sources, to tell whether stored counters are current."""
    csrc = os.path.join(ROOT, "shifted_sparse_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


class ClockSampler:
    """Samples the shader clock the amdgpu kernel driver reports (pp_dpm_sclk, the level
    marked '*') every few milliseconds while the timed region runs."""

    def __init__(self, period_s=0.004):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for line in open(self.path).read().splitlines():
            if line.rstrip().endswith("*"):
                return float(line.split(":")[1].strip().split("M")[0].split("m")[0])
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except (OSError, ValueError, IndexError):
                v = None
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        xs = self.samples
        return {"mean": round(sum(xs) / len(xs), 1), "min": min(xs), "max": max(xs), "samples": len(xs),
                "source": self.path}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--flush-mb", type=int, default=0,
                    help="overwrite a scratch buffer of this many MiB before each timed step (cold caches); "
                         "value and ms_per_step then come from the per-step spans, which exclude the flush")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--ds-max-mib", type=int, default=96 << 10,
                    help="bound on the dS tiles the backward keeps in its workspace (MiB; the "
                         "library default is 16 GiB; 0: dQ recomputes the scores)")
    ap.add_argument("--two-step-sdpa", action="store_true",
                    help="also time the method in its two-step PyTorch form (torch.roll, groups folded "
                         "into the batch, torch SDPA's flash kernel) on the same inputs, as context")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on one GPU; units are independent, so several GPUs would "
              "split heads or batch with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import shifted_sparse_attention_amd as s2
    from seeded_inputs import BLOCK_CONFIGS, CONFIGS, make_inputs
    from seeded_inputs.configs import HEADLINE
    from shifted_sparse_attention_amd import flops as F

    if args.workload in BLOCK_CONFIGS:
        return bench_block(args, BLOCK_CONFIGS[args.workload])
    wl = CONFIGS[args.workload or HEADLINE]
    if wl.dtype != "bf16":
        raise SystemExit("bench.py times bf16 workloads")
    B, L, Hq, Hkv, d, G, sh = wl.B, wl.L, wl.Hq, wl.Hkv, wl.d, wl.G, wl.shifted_heads
    rope = (wl.rope_base, wl.rope_orig_len) if wl.rope else None

    t0 = time.time()
    x = make_inputs(wl)
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v"))
    tdo = torch.from_numpy(x["do"]).to(torch.bfloat16).to(dev) if wl.backward else torch.empty_like(tq)
    print(f"# inputs ready in {time.time() - t0:.1f}s: {wl.name}", file=sys.stderr, flush=True)

    o = torch.empty_like(tq)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    opts = s2.make_opts(torch.bfloat16, rope=rope, ds_max_mib=args.ds_max_mib)
    fws = s2.s2attn_workspace_size(0, B, L, Hq, Hkv, d, G, opts)
    bws = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G, opts)
    bws0 = s2.s2attn_workspace_size(1, B, L, Hq, Hkv, d, G,
                                    s2.make_opts(torch.bfloat16, rope=rope, ds_max_mib=0))
    ws = torch.empty(max(fws, bws, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sargs = (tq, tk, tv, o, lse, tdo, dq, dk, dv, B, L, Hq, Hkv, d, G, sh, opts, ws, bws, stream)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        s2.s2attn_fwd_ex(tq, tk, tv, o, lse, B, L, Hq, Hkv, d, G, sh, opts, ws, fws, stream)
        if ev is not None:
            ev[1].record(stream)
        if not wl.backward:
            return
        s2.s2attn_bwd_stage_ex(s2.S2ATTN_BWD_STAGE_PRE, *sargs)
        if ev is not None:
            ev[2].record(stream)
        s2.s2attn_bwd_stage_ex(s2.S2ATTN_BWD_STAGE_DKDV, *sargs)
        if ev is not None:
            ev[3].record(stream)
        s2.s2attn_bwd_stage_ex(s2.S2ATTN_BWD_STAGE_DQ, *sargs)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    n_ev = 5 if wl.backward else 2
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush = (torch.empty(args.flush_mb << 20, dtype=torch.uint8, device=dev)
             if args.flush_mb > 0 else None)
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        start.record(stream)
        for i in range(args.steps):
            if flush is not None:
                flush.fill_(i & 255)   # evicts L2 and the last-level cache before the step
            step(evs[i])
        end.record(stream)
        torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    names = ["fwd", "bwd_pre", "bwd_dkdv", "bwd_dq"][:n_ev - 1]
    kms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    # Per-step spans (events on the launch stream): forward, backward, both.
    spans = {"fwd": [e[0].elapsed_time(e[1]) for e in evs]}
    if wl.backward:
        spans["bwd"] = [e[1].elapsed_time(e[n_ev - 1]) for e in evs]
        spans["fwd_bwd"] = [e[0].elapsed_time(e[n_ev - 1]) for e in evs]
    span_stats = {k: {"median": round(float(np.median(v)), 4), "min": round(float(np.min(v)), 4)}
                  for k, v in spans.items()}
    if flush is not None:   # the flush sits between the steps: time the steps alone
        ms_step = float(np.mean(spans["fwd_bwd" if wl.backward else "fwd"]))

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        b.copy_(a)
        torch.cuda.synchronize()

    fl = F.fwd_bwd_flops(B, L, Hq, d, G) if wl.backward else F.fwd_flops(B, L, Hq, d, G)
    tflops = fl / (ms_step * 1e-3) / 1e12
    unit = float(B) * Hq * L * G * d     # one product over all group-local causal pairs
    alg_flops = {"fwd": 2 * unit, "bwd_dkdv": 4 * unit, "bwd_dq": 1 * unit}
    alg_flops = {k: v for k, v in alg_flops.items() if k in kms}
    dom = max(alg_flops, key=lambda n: kms[n])
    achieved = alg_flops[dom] / (kms[dom] * 1e-3) / 1e12

    traffic = None
    if wl.name == HEADLINE and os.path.exists(TRAFFIC_FILE):   # counters were taken on that workload
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("source_sha") == kernel_source_sha() and dom in tr.get("kernels", {}):
            traffic = tr["kernels"][dom]["hbm_bytes_per_launch"]

    metric = METRIC if wl.name == HEADLINE else f"S²-Attn {'fwd+bwd' if wl.backward else 'fwd'} TFLOP/s, {wl.name}"
    out = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "L": L, "Hq": Hq, "Hkv": Hkv, "d": d, "G": G,
                   "shifted_heads": sh, "rope": bool(wl.rope), "seed": wl.seed,
                   "parallelism": "single GPU",
                   "ds_max_mib": args.ds_max_mib,
                   "dq_from": ("stored dS" if bws > bws0 else "recomputed scores") if wl.backward else None,
                   "caches": f"flushed ({args.flush_mb} MiB written before each step)" if flush is not None else "warm"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {k: round(v, 4) for k, v in kms.items()},
        "step_spans_ms": span_stats,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": alg_flops[dom],
        },
        "clock_mhz": clk.summary(),
        "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
    }

    if args.two_step_sdpa:
        out["two_step_sdpa"] = time_two_step_sdpa(wl, tq, tk, tv, tdo, (o, dq, dk, dv), args.steps,
                                                  args.warmup, fl)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def _roll_heads(x, shifted_heads, shift):
    """The last `shifted_heads` heads of x [B, L, H, d] rolled by `shift` along L (a copy)."""
    import torch
    if shifted_heads == 0:
        return x
    H = x.shape[2]
    return torch.cat([x[:, :, :H - shifted_heads], x[:, :, H - shifted_heads:].roll(shift, dims=1)], dim=2)


def _fold(x, G, shifted_heads):
    """[B, L, H, d] -> [B * L / G, H, G, d]: shifted heads rolled by -G/2, groups folded into
    the batch (a strided view of the rolled tensor)."""
    B, L, H, d = x.shape
    return _roll_heads(x, shifted_heads, -(G // 2)).reshape(B * (L // G), G, H, d).transpose(1, 2)


def _unfold(y, L, G, shifted_heads):
    """Inverse of _fold."""
    N, H, _, d = y.shape
    return _roll_heads(y.transpose(1, 2).reshape(N * G // L, L, H, d), shifted_heads, G // 2)


def two_step_form(q, k, v, G, shifted_heads):
    """S2-Attn the way the LongLoRA pages implement it in PyTorch (blog section 3.3;
    nearauto.com article, shift-short-attention section): the last `shifted_heads` heads
    are rolled by -G/2 along the sequence (torch.roll, a copy), the groups are folded into
    the batch (a view), causal attention runs per group (torch's scaled_dot_product_attention,
    whichever backend the caller enables), and the output is unfolded and rolled back.
    q, k, v: [B, L, H, d] with one KV head per query head.  Differentiable through autograd."""
    import torch.nn.functional as Fn
    y = Fn.scaled_dot_product_attention(_fold(q, G, shifted_heads), _fold(k, G, shifted_heads),
                                        _fold(v, G, shifted_heads), is_causal=True)
    return _unfold(y, q.shape[1], G, shifted_heads)


def time_two_step_sdpa(wl, tq, tk, tv, tdo, ours, steps, warmup, counted_flops):
    """two_step_form on this GPU (forward, and backward for fwd+bwd workloads) with torch SDPA
    restricted to its flash kernel (no fallback to the math path), timed like the main steps;
    outputs compared with this library's (`ours` = o, dq, dk, dv of the same inputs).
    Context, not a target: it measures torch's kernels and copies."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    if wl.Hq != wl.Hkv or wl.rope:
        return {"skipped": "multi-head workloads without RoPE only"}
    q, k, v = (t.detach().clone().requires_grad_(wl.backward) for t in (tq, tk, tv))

    def step():
        q.grad = k.grad = v.grad = None
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]), torch.set_grad_enabled(wl.backward):
            y = two_step_form(q, k, v, wl.G, wl.shifted_heads)
            if wl.backward:
                y.backward(tdo)
        return y

    try:
        y = step()
    except RuntimeError as e:   # no flash kernel for this shape or device
        return {"skipped": f"torch SDPA flash kernel unavailable: {str(e).splitlines()[0][:200]}"}
    torch.cuda.synchronize()

    def rel_f(a, b):
        a, b = a.double(), b.double()
        return float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))

    got = (y.detach(), q.grad, k.grad, v.grad) if wl.backward else (y,)
    agree = {n: round(rel_f(a, b), 6) for n, a, b in zip(("o", "dq", "dk", "dv"), got, ours)}
    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    ms = timed(step)
    # The attention kernels alone: inputs already rolled and folded into contiguous
    # [B * L / G, H, G, d] tensors, so no roll or layout copy is timed.
    qf, kf, vf = (_fold(t, wl.G, wl.shifted_heads).contiguous().requires_grad_(wl.backward)
                  for t in (tq, tk, tv))
    dof = _fold(tdo, wl.G, wl.shifted_heads).contiguous() if wl.backward else None

    def step_attention():
        qf.grad = kf.grad = vf.grad = None
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]), torch.set_grad_enabled(wl.backward):
            yf = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, is_causal=True)
            if wl.backward:
                yf.backward(dof)

    ms_attn = timed(step_attention)
    return {"ms_per_step": round(ms, 4), "tflops": round(counted_flops / (ms * 1e-3) / 1e12, 2),
            "attention_only_ms": round(ms_attn, 4),
            "attention_only_tflops": round(counted_flops / (ms_attn * 1e-3) / 1e12, 2),
            "backend": "torch SDPA, flash kernel only (AOTriton on ROCm)",
            "rel_frobenius_vs_libs2attn": agree, "torch": torch.__version__}


def bench_block(args, wl):
    """The attention block (LoRA Q/K/V/O on hipBLASLt, RoPE-PI, S2-Attn): one
    step is its forward and backward."""
    import numpy as np
    import torch

    import shifted_sparse_attention_amd as s2
    from seeded_inputs import make_block_inputs
    from shifted_sparse_attention_amd import flops as F

    t0 = time.time()
    inp = make_block_inputs(wl)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)

    x, dy = up(inp["x"]), up(inp["dy"])
    params = {k: up(v) for k, v in inp["params"].items()}
    print(f"# inputs ready in {time.time() - t0:.1f}s: {wl.name}", file=sys.stderr, flush=True)
    rope = (wl.rope_base, wl.rope_orig_len) if wl.rope else None
    blk = s2.block.Block(wl.B, wl.L, wl.Hq, wl.Hkv, wl.d, wl.G, wl.shifted_heads, wl.lora_rank,
                         wl.lora_scale, rope=rope)
    wsb = blk.workspace(1, dev)          # the backward's workspace covers the forward's
    stream = torch.cuda.current_stream()
    saved = blk.alloc_saved(dev)
    y = torch.empty_like(x)
    grads = {"dx": torch.empty_like(x)}
    for name, shp in s2.block.param_shapes(wl.Hq, wl.Hkv, wl.d, wl.lora_rank).items():
        if name[0] in "ab":
            grads["d" + name] = torch.empty(shp, dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        s2.s2block_fwd(blk.cfg, x, params, y, saved, wsb[0], wsb[1], stream)
        if ev is not None:
            ev[1].record(stream)
        s2.s2block_bwd(blk.cfg, x, params, saved, dy, grads, wsb[0], wsb[1], stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clk:
        start.record(stream)
        for i in range(args.steps):
            step(evs[i])
        end.record(stream)
        torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    kms = {"block_fwd": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
           "block_bwd": float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))}
    spans = {"fwd": [e[0].elapsed_time(e[1]) for e in evs], "bwd": [e[1].elapsed_time(e[2]) for e in evs],
             "fwd_bwd": [e[0].elapsed_time(e[2]) for e in evs]}
    span_stats = {k: {"median": round(float(np.median(v)), 4), "min": round(float(np.min(v)), 4)}
                  for k, v in spans.items()}
    ffl, bfl = F.block_flops(wl.B, wl.L, wl.Hq, wl.Hkv, wl.d, wl.G, wl.lora_rank)
    att = F.fwd_bwd_flops(wl.B, wl.L, wl.Hq, wl.d, wl.G)
    tflops = (ffl + bfl) / (ms_step * 1e-3) / 1e12
    dom = max(kms, key=kms.get)
    dom_fl = ffl if dom == "block_fwd" else bfl
    achieved = dom_fl / (kms[dom] * 1e-3) / 1e12
    out = {
        "metric": f"Attention block (LoRA Q/K/V/O + RoPE-PI + S²-Attn) fwd+bwd TFLOP/s, {wl.name}",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights)",
        "config": {"workload": wl.name, "B": wl.B, "L": wl.L, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d,
                   "G": wl.G, "shifted_heads": wl.shifted_heads, "lora_rank": wl.lora_rank,
                   "rope": bool(wl.rope), "seed": wl.seed, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {k: round(v, 4) for k, v in kms.items()},
        "step_spans_ms": span_stats,
        "attention_flop_share": round(att / (ffl + bfl), 4),
        # The block's launches sit inside one C call each; the dominant unit
        # timed with events on its stream is the forward or the backward call.
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": dom_fl},
        "clock_mhz": clk.summary(),
        "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block(wl, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def host_info():
    """The host the CPU baseline ran on: CPU model, numpy and BLAS library."""
    import platform

    import numpy as np
    from threadpoolctl import threadpool_info

    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
            if i.get("user_api") == "blas"]
    return {"cpu_model": model, "numpy": np.__version__, "blas": ", ".join(blas)}


def cpu_baseline_block(wl, inp, seconds):
    """The block oracle (fp64 numpy) on the same workload: y at a few tokens at
    a time, each from the definition (every head's projections of the causal
    prefix of its group, attention, the output projection), until about
    `seconds` of CPU time.  FLOPs are those the oracle performs."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import block as OB
    from oracle import s2attn as O

    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    rng = np.random.default_rng(0)
    Dm, d, r = wl.Hq * wl.d, wl.d, wl.lora_rank
    rope = (wl.rope_base, wl.rope_orig_len) if wl.rope else None
    fl, done, t0 = 0.0, 0, time.time()
    while time.time() - t0 < seconds:
        toks = [int(t) for t in rng.integers(0, wl.L, 2)]
        OB.sampled_forward_tokens(inp["x"], inp["params"], wl.G, wl.shifted_heads, wl.Hq, wl.Hkv,
                                  wl.d, wl.lora_scale, 0, toks, rope=rope)
        for h in range(wl.Hq):
            s = O.head_shift(h, wl.Hq, wl.G, wl.shifted_heads)
            rows = max(int(O.original_to_rolled(t, wl.L, s)) % wl.G for t in toks) + 1
            fl += 2.0 * rows * Dm * 3 * (d + r) + 2.0 * rows * r * 3 * d   # q, k, v slices + LoRA
            fl += sum(4.0 * d * (int(O.original_to_rolled(t, wl.L, s)) % wl.G + 1) for t in toks)
        fl += len(toks) * (2.0 * Dm * Dm + 2.0 * r * (2 * Dm))            # output projection
        done += len(toks)
    dt = time.time() - t0
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"block output y at {done} tokens of the same workload, fp64, each from its "
                      f"heads' causal group prefixes ({dt:.1f} s); forward only",
            "seconds": round(dt, 2), **host_info()}


def cpu_baseline(wl, x, seconds):
    """The oracle (fp64 numpy, as it stands) on whole (head, group) units of the
    same workload, forward + backward, until about `seconds` of CPU time.
    Forward-only workloads run the oracle's row-at-a-time forward on rows
    spread over the group instead (a unit there can span the whole context)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import s2attn as O
    from shifted_sparse_attention_amd import flops as F

    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    if not wl.backward:
        rng = np.random.default_rng(0)
        done_rows, fl, t0 = 0, 0.0, time.time()
        while time.time() - t0 < seconds:
            rows = sorted(int(i) for i in rng.integers(0, wl.G, 8))
            h = int(rng.integers(0, wl.Hq))
            O.sampled_rows_forward(x["q"], x["k"], x["v"], wl.G, wl.shifted_heads, 0, h, 0, rows)
            fl += sum(4.0 * wl.d * (i + 1) for i in rows)   # 2d per key for Q.K and for P.V
            done_rows += len(rows)
        dt = time.time() - t0
        return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{done_rows} query rows drawn uniformly over the group, forward in fp64 row by row "
                          f"({dt:.1f} s); counted FLOPs 4*d per attended key",
                "seconds": round(dt, 2), **host_info()}

    scale = 1.0 / np.sqrt(wl.d)
    heads = [h for h in dict.fromkeys((0, wl.Hq - 1, wl.Hq // 2, 1, wl.Hq // 4, 3 * wl.Hq // 4, 2,
                                       wl.Hq - 2)) if 0 <= h < wl.Hq]
    units = [(0, h, g) for h in heads for g in range(wl.n_groups)]
    done, t0 = 0, time.time()
    for b, h, g in units:
        rows = O.unit_rows(wl.L, wl.G, wl.Hq, wl.shifted_heads, h, g)
        hk = h // wl.r
        O.unit_backward(x["q"][b, rows, h].astype(np.float64), x["k"][b, rows, hk].astype(np.float64),
                        x["v"][b, rows, hk].astype(np.float64), x["do"][b, rows, h].astype(np.float64),
                        scale)
        done += 1
        if time.time() - t0 >= seconds:
            break
    dt = time.time() - t0
    fl = done * F.fwd_bwd_flops(1, wl.G, 1, wl.d, wl.G)   # one unit = one head, one group
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} (head, group) units of G={wl.G} rows, forward+backward in fp64 "
                      f"({dt:.1f} s); counted FLOPs as for the GPU",
            "seconds": round(dt, 2), **host_info()}


if __name__ == "__main__":
    main()
