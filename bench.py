"""Benchmark of the differential-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
per-head lambda for both workloads, the fused V1 prefill (with the per-head
RMS-norm epilogue) of the long multi-needle workload (B=1, 32 heads,
N=65536, d=64, dv=128, layer 12), and the V2 split-KV decode of the GQA
workload (B=32, 32 query heads over 8 KV heads, D=128, lengths uniform in
[4096, 65536]).  Inputs are generated on the GPU and resident in HBM before
the timed region.

Prints one JSON line: whole-step algorithmic TFLOP/s as `value`, the prefill
kernel against the bf16 matrix-core roofline, the decode kernels against the
HBM roofline, and the CPU oracle timed on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import contextlib
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "diff-attn prefill TFLOP/s & decode HBM GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E peak


def prefill_flops(case) -> float:
    """Algorithmic flops: per visible (query, key) pair, two d-long dot
    products and one dv-wide weighted accumulation: 4d + 2dv."""
    return float(case.pairs()) * (4 * case.d + 2 * case.dv)


def executed_prefill_flops(case) -> float:
    """Matrix-core flops the fused kernel executes: per visible pair, both
    d-long score dots and one dv-wide accumulation per map."""
    return float(case.pairs()) * (4 * case.d + 4 * case.dv)


def decode_bytes(case, lens) -> float:
    """Algorithmic HBM bytes: every visible K and V row once (bf16), plus q,
    lambda, lengths and the fp32 output."""
    kv = float(sum(int(x) for x in lens)) * case.Hkv * 2 * case.D * 2
    return kv + case.B * case.Hq * case.D * 2 + (case.Hq // 2) * 4 + case.B * 4 + \
        case.B * (case.Hq // 2) * case.D * 4


def decode_flops(case, lens) -> float:
    """Per visible key and pair: two D-long dots and one D-wide accumulation."""
    return float(sum(int(x) for x in lens)) * (case.Hq // 2) * 6 * case.D


PROFILE = os.path.join(ROOT, "profiles", "bench_multineedle64k_v2decode_trace_and_bytes.md")


def profiled_traffic(kernel: str):
    """HBM bytes per launch recorded by the rocprofv3 byte-counter runs in
    profiles/, or None if the kernel source changed since they were taken."""
    import hashlib
    srcs = {"prefill": ("prefill_pp.hip", "bf16_tile.h"), "decode": ("decode.hip",)}[kernel]
    try:
        h = hashlib.sha256()
        for src in srcs:
            h.update(open(os.path.join(ROOT, "differential_attention_prefill_amd", "csrc", src), "rb").read())
        sha = h.hexdigest()[:16]
        fields = dict(line.split(": ", 1) for line in open(PROFILE).read().splitlines()
                      if line.startswith(kernel + "_"))
    except (OSError, ValueError):
        return None
    if fields.get(kernel + "_source_sha256_16", "").strip() != sha:
        return None
    return float(fields[kernel + "_traffic_bytes_per_launch"])


class Ranges:
    """roctx ranges around the bench's phases, from the ROCm profiler SDK's
    roctx library: `rocprofv3 --marker-trace` shows them beside the kernels.
    The ranges mark host-side enqueue intervals (launches are asynchronous).
    Where the library is absent the ranges do nothing."""

    def __init__(self):
        self._lib = None
        path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib",
                            "librocprofiler-sdk-roctx.so.1")
        try:
            lib = ctypes.CDLL(path)
            lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            lib.roctxRangePushA.restype = ctypes.c_int
            lib.roctxRangePop.argtypes = []
            lib.roctxRangePop.restype = ctypes.c_int
            self._lib = lib
        except (OSError, AttributeError):
            pass

    @contextlib.contextmanager
    def __call__(self, name: str):
        if self._lib is not None:
            self._lib.roctxRangePushA(name.encode())
        try:
            yield
        finally:
            if self._lib is not None:
                self._lib.roctxRangePop()


RANGE = Ranges()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill", default="multineedle_64k",
                    choices=["multineedle_64k", "needle_32k", "v1_norm"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the layouts measured beside the step (V2 prefill, ...)")
    ap.add_argument("--only-extras", default="",
                    help="comma-separated subset of the extras to run (%s)" % ", ".join(EXTRAS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, copy this many MiB device-to-device once: "
                         "a plain copy of known size that calibrates HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU; sharding across GPUs is a design only, with no "
              "launch path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    dev = "cuda:0"
    torch.cuda.set_device(0)
    api.load_library()
    pcase = {"multineedle_64k": W.MULTI_NEEDLE_64K, "needle_32k": W.NEEDLE_32K,
             "v1_norm": W.V1_NORM}[args.prefill]
    dcase = W.V2_DECODE
    print("# generating inputs: %s + %s" % (pcase.name, dcase.name), file=sys.stderr, flush=True)
    pin = W.make_prefill(pcase, device=dev)
    din = W.make_decode(dcase, device=dev)
    d = pcase.d
    q1, q2 = pin["q"][..., :d], pin["q"][..., d:]
    k1, k2 = pin["k"][..., :d], pin["k"][..., d:]
    v = pin["v"]
    plam_in = [pin[k].contiguous() for k in ("lq1", "lk1", "lq2", "lk2")]
    dlam_in = [din[k].contiguous() for k in ("lq1", "lk1", "lq2", "lk2")]
    plam = torch.empty(pcase.H, dtype=torch.float32, device=dev)
    dlam = torch.empty(dcase.Hq // 2, dtype=torch.float32, device=dev)
    pout = torch.empty((pcase.B, pcase.H, pcase.N, pcase.dv), dtype=torch.float32, device=dev)
    dout = torch.empty((dcase.B, dcase.Hq // 2, dcase.D), dtype=torch.float32, device=dev)
    ws = torch.empty(api.diffattn_decode_workspace_bytes(dcase.B, dcase.Hq, dcase.Hkv, dcase.D,
                                                         dcase.Lmax), dtype=torch.uint8, device=dev)
    norm_scale = (1.0 - api.diffattn_lambda_init(pcase.layer)) if pcase.rmsnorm else 1.0
    lens = din["seq_lens"].cpu().tolist()
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(record):
        if record:
            ev[0].record()
        with RANGE("lambda"):
            api.diffattn_lambda(*plam_in, layer=pcase.layer, out=plam)
            api.diffattn_lambda(*dlam_in, layer=dcase.layer, out=dlam)
        if record:
            ev[1].record()
        with RANGE("prefill"):
            api.diffattn_prefill(q1, q2, k1, k2, v, plam, causal=pcase.causal,
                                 rmsnorm=pcase.rmsnorm, eps=pcase.eps, norm_scale=norm_scale,
                                 out=pout)
        if record:
            ev[2].record()
        with RANGE("decode"):
            api.diffattn_decode(din["q"], din["k_cache"], din["v_cache"], din["seq_lens"], dlam,
                                workspace=ws, out=dout)
        if record:
            ev[3].record()

    with RANGE("warmup"):
        for i in range(args.warmup):
            step(False)
            print("# warmup step %d done" % i, file=sys.stderr, flush=True)
        torch.cuda.synchronize()

    t_lam, t_pre, t_dec = [], [], []
    with RANGE("timed steps"):
        t0 = time.perf_counter()
        for i in range(args.steps):
            with RANGE("step %d" % i):
                step(True)
                torch.cuda.synchronize()   # per-step sync keeps the event pairs readable
            t_lam.append(ev[0].elapsed_time(ev[1]))
            t_pre.append(ev[1].elapsed_time(ev[2]))
            t_dec.append(ev[2].elapsed_time(ev[3]))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    print("# timed %d steps in %.3f s" % (args.steps, wall), file=sys.stderr, flush=True)

    ms_step = 1e3 * wall / args.steps
    fp = prefill_flops(pcase)
    fd = decode_flops(dcase, lens)
    bd = decode_bytes(dcase, lens)
    pre_ms = float(np.mean(t_pre))
    dec_ms = float(np.mean(t_dec))
    pre_tflops = fp / (pre_ms * 1e-3) / 1e12
    dec_gbps = bd / (dec_ms * 1e-3) / 1e9
    value = (fp + fd) / (ms_step * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 3),
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
        "config": {
            "workload": "%s prefill + %s decode" % (pcase.name, dcase.name),
            "prefill": {"B": pcase.B, "H": pcase.H, "N": pcase.N, "d": pcase.d, "dv": pcase.dv,
                        "causal": pcase.causal, "rmsnorm": pcase.rmsnorm, "layer": pcase.layer},
            "decode": {"B": dcase.B, "Hq": dcase.Hq, "Hkv": dcase.Hkv, "D": dcase.D,
                       "max_len": dcase.Lmax, "sum_len": int(sum(lens))},
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_pp_kernel<64,128>",
            "achieved": round(pre_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": profiled_traffic("prefill"),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
            "algorithmic_flops_per_launch": fp,
            "avg_launch_ms": round(pre_ms, 4),
            # The exact single pass keeps one accumulator per map, so the
            # matrix cores execute 2d + 2d + dv + dv = 4d + 4dv flop per pair
            # (1.5x the algorithmic count at d = 64, dv = 128): the matrix-core
            # utilisation beside the algorithmic fraction.
            "executed_mfma_flops_per_launch": executed_prefill_flops(pcase),
            "executed_mfma_frac": round(executed_prefill_flops(pcase) / (pre_ms * 1e-3) / 1e12
                                        / PEAK_BF16_TFLOPS, 4),
        },
        "decode": {
            "bound": "hbm",
            "achieved": round(dec_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes_per_launch": bd,
            "traffic": profiled_traffic("decode"),
            "avg_launch_ms": round(dec_ms, 4),
        },
        "lambda_avg_ms": round(float(np.mean(t_lam)), 4),
    }

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = n
        del src, dst

    if not args.no_extras:
        del pin, din, q1, q2, k1, k2, v, pout, dout, ws
        torch.cuda.empty_cache()
        only = [x for x in args.only_extras.split(",") if x]
        for x in only:
            if x not in EXTRAS:
                raise SystemExit("unknown extra %r (choose from %s)" % (x, ", ".join(EXTRAS)))
        with RANGE("extras"):
            result["extras"] = measure_extras(dev, max(3, args.steps), set(only or EXTRAS))
        pin = din = None

    if not args.no_cpu_baseline:
        if pin is None:
            pin = W.make_prefill(pcase, device=dev)
            din = W.make_decode(dcase, device=dev)
        with RANGE("cpu baseline"):
            result["cpu_baseline"] = cpu_baseline(pcase, pin, dcase, din, plam, dlam, norm_scale,
                                                  args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _time_launches(fn, reps):
    """Average duration of fn() in ms over `reps` launches, HIP events on the
    current stream, after one untimed launch."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


EXTRAS = ("prefill_workloads", "prefill_length_sweep", "v2_prefill", "unfused_vs_fused",
          "v1_decode", "baseline_decode", "snr_sweep")


def measure_extras(dev, reps, which=frozenset(EXTRAS)):
    """Layouts measured beside the step, each on its own synthetic workload."""
    extras = {}
    runs = (("prefill_workloads", _extra_prefill_workloads),
            ("prefill_length_sweep", _extra_prefill_length_sweep), ("v2_prefill", _extra_v2_prefill),
            ("unfused_vs_fused", _extra_unfused), ("v1_decode", _extra_v1_decode),
            ("baseline_decode", _extra_baseline_decode))
    for name, fn in runs:
        if name in which:
            with RANGE("extras: " + name):
                extras[name] = fn(dev, reps)
    if "snr_sweep" in which:
        with RANGE("extras: snr_sweep"):
            extras.update(_extra_snr(dev))
    return extras


def _extra_prefill_workloads(dev, reps):
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    # The other prefill workloads the operator is specified on, each timed on
    # its own: the tiny fp32 case (vector-ALU path, launch-bound: no roofline
    # claim), the V1 norm workload at N = 2048 and the 32k needle workload
    # (bf16 matrix-core roofline), the latter with the last query's SNR
    # towards its needle read off the kernel (probe values).
    from differential_attention_prefill_amd import snr
    per_cfg = {}
    for c in (W.TINY_FP32, W.V1_NORM, W.NEEDLE_32K):
        print("# extras: %s" % c.name, file=sys.stderr, flush=True)
        inp = W.make_prefill(c, device=dev)
        lam = api.diffattn_lambda(*(inp[x].contiguous() for x in ("lq1", "lk1", "lq2", "lk2")),
                                  layer=c.layer)
        scale = (1.0 - api.diffattn_lambda_init(c.layer)) if c.rmsnorm else 1.0
        out = torch.empty((c.B, c.H, c.N, c.dv), dtype=torch.float32, device=dev)
        ms = _time_launches(lambda: api.diffattn_prefill_packed(
            inp["q"], inp["k"], inp["v"], lam, causal=c.causal, rmsnorm=c.rmsnorm, eps=c.eps,
            norm_scale=scale, out=out), max(reps, 20))
        f = prefill_flops(c)
        rec = {"dtype": c.dtype, "avg_launch_ms": round(ms, 4), "algorithmic_flops_per_launch": f,
               "achieved_tflops": round(f / (ms * 1e-3) / 1e12, 2)}
        if c.dtype == "bf16":
            rec["frac_of_bf16_peak"] = round(f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if c.n_needles:
            # At d = 64 the 5x needle scores about 40 above the noise, so the
            # noise weight of the last query sits far below fp32 resolution:
            # the kernel reads the signal's share of the row weight; the SNRs
            # themselves come from the fp64 oracle.
            r = snr.noise_sweep_point(inp["q"], inp["k"], lam, inp["needles"][:, 0],
                                      causal=c.causal)
            rec["last_query_signal_share_mean"] = {"plain": round(float(r["plain_signal"].mean()), 6),
                                                   "diff": round(float(r["diff_signal"].mean()), 6)}
        per_cfg[c.name] = rec
        del inp, out
        torch.cuda.empty_cache()
    return per_cfg


def _extra_prefill_length_sweep(dev, reps):
    """The fused V1 prefill (the step's kernel and norm) at other lengths,
    4k to 128k, on plain unit-variance inputs: its rate against N."""
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    per_len = {}
    for c in W.V1_LENGTH_SWEEP:
        print("# extras: %s" % c.name, file=sys.stderr, flush=True)
        inp = W.make_prefill(c, device=dev)
        lam = api.diffattn_lambda(*(inp[x].contiguous() for x in ("lq1", "lk1", "lq2", "lk2")),
                                  layer=c.layer)
        scale = 1.0 - api.diffattn_lambda_init(c.layer)
        out = torch.empty((c.B, c.H, c.N, c.dv), dtype=torch.float32, device=dev)
        n = max(reps, 20) if c.N <= 16384 else max(3, reps // 2)
        ms = _time_launches(lambda: api.diffattn_prefill_packed(
            inp["q"], inp["k"], inp["v"], lam, causal=c.causal, rmsnorm=c.rmsnorm, eps=c.eps,
            norm_scale=scale, out=out), n)
        f = prefill_flops(c)
        per_len[c.name] = {"N": c.N, "H": c.H, "avg_launch_ms": round(ms, 4),
                           "algorithmic_flops_per_launch": f,
                           "achieved_tflops": round(f / (ms * 1e-3) / 1e12, 2),
                           "frac_of_bf16_peak": round(f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del inp, out
        torch.cuda.empty_cache()
    return per_len


def _extra_v2_prefill(dev, reps):
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    # V2 prefill: doubled query heads over shared K/V heads, D = 128 for both maps.
    c = W.V2_PREFILL_32K
    print("# extras: %s" % c.name, file=sys.stderr, flush=True)
    inp = W.make_prefill_v2(c, device=dev)
    lam = api.diffattn_lambda(*(inp[k].contiguous() for k in ("lq1", "lk1", "lq2", "lk2")),
                              layer=c.layer)
    out = torch.empty((c.B, c.Hq // 2, c.N, c.D), dtype=torch.float32, device=dev)
    ms = _time_launches(lambda: api.diffattn_prefill_v2(inp["q"], inp["k"], inp["v"], lam,
                                                        causal=c.causal, out=out), reps)
    f = float(c.pairs()) * (4 * c.D + 2 * c.D)
    rec = {"workload": c.name, "avg_launch_ms": round(ms, 4),
           "algorithmic_flops_per_launch": f,
           "achieved_tflops": round(f / (ms * 1e-3) / 1e12, 2),
           "frac_of_bf16_peak": round(f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del inp, out
    torch.cuda.empty_cache()
    return rec


def _extra_unfused(dev, reps):
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    # Unfused two-pass path on the step's prefill workload: single-map
    # attention for each map (V read twice, two fp32 intermediates), then the
    # combine pass; beside the fused kernel on the same inputs.  The device
    # memory each path needs beyond its inputs is read from torch's allocator
    # (the library allocates nothing): the fused call holds only its output,
    # the same as a plain attention of this width would.
    c = W.MULTI_NEEDLE_64K
    print("# extras: unfused vs fused, %s" % c.name, file=sys.stderr, flush=True)
    inp = W.make_prefill(c, device=dev)
    d = c.d
    q, k, v = inp["q"], inp["k"], inp["v"]
    lam = api.diffattn_lambda(*(inp[x].contiguous() for x in ("lq1", "lk1", "lq2", "lk2")),
                              layer=c.layer)
    scale = 1.0 - api.diffattn_lambda_init(c.layer)
    shape = (c.B, c.H, c.N, c.dv)
    torch.cuda.synchronize()
    inputs_bytes = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    def fused_call(out):
        api.diffattn_prefill(q[..., :d], q[..., d:], k[..., :d], k[..., d:], v, lam, causal=True,
                             rmsnorm=c.rmsnorm, eps=c.eps, norm_scale=scale, out=out)

    out = torch.empty(shape, dtype=torch.float32, device=dev)
    fused_call(out)
    torch.cuda.synchronize()
    fused_peak = torch.cuda.max_memory_allocated() - inputs_bytes
    del out
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    o1 = torch.empty(shape, dtype=torch.float32, device=dev)
    o2 = torch.empty(shape, dtype=torch.float32, device=dev)
    out = torch.empty(shape, dtype=torch.float32, device=dev)
    api.diffattn_attention(q[..., :d], k[..., :d], v, out=o1)
    api.diffattn_attention(q[..., d:], k[..., d:], v, out=o2)
    api.diffattn_combine(o1, o2, lam, rmsnorm=c.rmsnorm, eps=c.eps, norm_scale=scale, out=out)
    torch.cuda.synchronize()
    unfused_peak = torch.cuda.max_memory_allocated() - inputs_bytes

    fused_ms = _time_launches(lambda: fused_call(out), reps)
    att_ms = _time_launches(lambda: (api.diffattn_attention(q[..., :d], k[..., :d], v, out=o1),
                                     api.diffattn_attention(q[..., d:], k[..., d:], v, out=o2)),
                            reps)
    cmb_ms = _time_launches(lambda: api.diffattn_combine(o1, o2, lam, rmsnorm=c.rmsnorm, eps=c.eps,
                                                         norm_scale=scale, out=out), reps)
    rows = c.B * c.H * c.N
    in_bytes = rows * (2 * (2 * d) * 2 + c.dv * 2)          # q and k (both halves), v
    out_bytes = rows * c.dv * 4
    inter = 2 * rows * c.dv * 4                              # o1 and o2
    rec = {
        "workload": c.name, "fused_ms": round(fused_ms, 4),
        "unfused_ms": round(att_ms + cmb_ms, 4), "unfused_attention_ms": round(att_ms, 4),
        "unfused_combine_ms": round(cmb_ms, 4),
        "fused_speedup": round((att_ms + cmb_ms) / fused_ms, 3),
        "fused_hbm_bytes_model": in_bytes + out_bytes,
        "unfused_hbm_bytes_model": in_bytes + rows * c.dv * 2 + 2 * inter + out_bytes,
        "inputs_device_bytes": int(inputs_bytes),
        "fused_device_bytes_beyond_inputs": int(fused_peak),
        "unfused_device_bytes_beyond_inputs": int(unfused_peak),
        "fused_footprint_vs_unfused": round((inputs_bytes + fused_peak) / (inputs_bytes + unfused_peak), 4),
    }
    del inp, q, k, v, o1, o2, out
    torch.cuda.empty_cache()
    return rec


def _extra_v1_decode(dev, reps):
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    # V1-layout decode: half-width maps over per-head K1|K2 and V caches, RMS norm.
    c = W.V1_DECODE
    print("# extras: %s" % c.name, file=sys.stderr, flush=True)
    inp = W.make_decode_v1(c, device=dev)
    lam = api.diffattn_lambda(*(inp[x].contiguous() for x in ("lq1", "lk1", "lq2", "lk2")),
                              layer=c.layer)
    ws = torch.empty(api.diffattn_decode_v1_workspace_bytes(c.B, c.H, c.Lmax), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((c.B, c.H, c.dv), dtype=torch.float32, device=dev)
    scale = 1.0 - api.diffattn_lambda_init(c.layer)
    ms = _time_launches(lambda: api.diffattn_decode_v1(
        inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam, rmsnorm=True, eps=c.eps,
        norm_scale=scale, workspace=ws, out=out), max(reps, 20))
    lens = inp["seq_lens"].cpu().tolist()
    nbytes = float(sum(int(x) for x in lens)) * c.H * (2 * c.d + c.dv) * 2 + \
        c.B * c.H * (2 * c.d * 2 + c.dv * 4) + c.H * 4 + c.B * 4
    rec = {"workload": c.name, "avg_launch_ms": round(ms, 4),
           "algorithmic_bytes_per_launch": nbytes,
           "achieved_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    del inp, ws, out
    torch.cuda.empty_cache()
    return rec


def _extra_baseline_decode(dev, reps):
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    # The decode the V2 layout is compared with: a baseline model whose heads
    # are single softmax maps, with half the query heads (16) over the same
    # 8 KV heads and the same cache, timed beside the V2 differential decode
    # (32 query heads = 16 pairs) on that cache.
    c = W.V2_DECODE
    print("# extras: baseline decode vs V2 decode, %s" % c.name, file=sys.stderr, flush=True)
    inp = W.make_decode(c, device=dev)
    lam = api.diffattn_lambda(*(inp[x].contiguous() for x in ("lq1", "lk1", "lq2", "lk2")),
                              layer=c.layer)
    hb = c.Hq // 2
    qb = inp["q"][:, 0::2].contiguous()          # one query per baseline head
    ws = torch.empty(api.diffattn_decode_workspace_bytes(c.B, c.Hq, c.Hkv, c.D, c.Lmax),
                     dtype=torch.uint8, device=dev)
    out2 = torch.empty((c.B, c.Hq // 2, c.D), dtype=torch.float32, device=dev)
    outb = torch.empty((c.B, hb, c.D), dtype=torch.float32, device=dev)
    v2_ms = _time_launches(lambda: api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"],
                                                       inp["seq_lens"], lam, workspace=ws, out=out2),
                           max(reps, 20))
    base_ms = _time_launches(lambda: api.diffattn_attention_decode(
        qb, inp["k_cache"], inp["v_cache"], inp["seq_lens"], workspace=ws, out=outb), max(reps, 20))
    lens = inp["seq_lens"].cpu().tolist()
    kv = float(sum(int(x) for x in lens)) * c.Hkv * 2 * c.D * 2
    rec = {"workload": c.name, "v2_query_heads": c.Hq, "baseline_query_heads": hb,
           "kv_heads": c.Hkv, "v2_ms": round(v2_ms, 4), "baseline_ms": round(base_ms, 4),
           "v2_over_baseline": round(v2_ms / base_ms, 4), "kv_cache_bytes_read": kv,
           "v2_gbps": round(kv / (v2_ms * 1e-3) / 1e9, 1),
           "baseline_gbps": round(kv / (base_ms * 1e-3) / 1e9, 1)}
    del inp, ws, out2, outb, qb
    torch.cuda.empty_cache()
    return rec


def _extra_snr(dev):
    import torch

    from differential_attention_prefill_amd import api
    from differential_attention_prefill_amd import workloads as W

    extras = {}
    # Signal-to-noise of the last query towards a planted needle, plain vs
    # differential, as the context grows (kernel run with probe values).
    from differential_attention_prefill_amd import snr
    # The needle key is scaled so that its score sits 10 above zero (the mean
    # noise score) in every head, a fixed signal strength across lengths.
    sweep = []
    for n in (1024, 4096, 16384, 65536, 262144):
        c = W.scaled_prefill(W.NEEDLE_32K, N=n, H=16, dv=64, needle_score=10.0)
        print("# extras: noise floor N=%d" % n, file=sys.stderr, flush=True)
        inp = W.make_prefill(c, device=dev)
        lam = api.diffattn_lambda(*(inp[x].contiguous() for x in ("lq1", "lk1", "lq2", "lk2")),
                                  layer=c.layer)
        r = snr.noise_sweep_point(inp["q"], inp["k"], lam, inp["needles"][:, 0])
        pt = {"N": n, "heads": c.H}
        for key in ("plain_signal", "plain_noise", "diff_signal", "diff_noise"):
            pt[key + "_mean"] = round(float(r[key].mean()), 5)
        for key in ("plain_snr", "diff_snr"):
            pt[key + "_median"] = round(float(r[key].median()), 2)
        sweep.append(pt)
        del inp
    extras["snr_sweep"] = sweep
    c = W.scaled_prefill(W.MULTI_NEEDLE_64K, H=4, dv=64)
    inp = W.make_prefill(c, device=dev)
    lam = api.diffattn_lambda(*(inp[x].contiguous() for x in ("lq1", "lk1", "lq2", "lk2")),
                              layer=c.layer)
    m = snr.needle_mass(inp["q"], inp["k"], lam, inp["needles"])
    extras["needle_mass_64k"] = {"workload": c.name, "needles": c.n_needles, "heads": c.H,
                                 "plain_mean": round(float(m["plain"].mean()), 5),
                                 "diff_mean": round(float(m["diff"].mean()), 5)}
    del inp
    torch.cuda.empty_cache()
    return extras


def cpu_model() -> str:
    """The host CPU's model name (first /proc/cpuinfo entry), for the record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pcase, pin, dcase, din, plam, dlam, norm_scale, target_s):
    """The CPU oracle, as it stands, on a bounded sample of the same step:
    uniformly drawn prefill query rows, plus the decode of a few sequences."""
    import numpy as np

    import oracle

    d = pcase.d
    q, k, v = (pin[x].cpu() for x in ("q", "k", "v"))
    q1, q2 = q[..., :d].contiguous(), q[..., d:].contiguous()
    k1, k2 = k[..., :d].contiguous(), k[..., d:].contiguous()
    v = v.contiguous()
    lam = plam.cpu().numpy()
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)
    total_rows = pcase.B * pcase.H * pcase.N
    per_pair = 4 * pcase.d + 2 * pcase.dv

    def run_rows(n):
        rows = rng.integers(0, total_rows, size=n).astype(np.int64)
        flops = float(((rows % pcase.N) + 1).sum()) * per_pair
        t = time.perf_counter()
        oracle.prefill(q1, q2, k1, k2, v, lam, causal=True, rmsnorm=pcase.rmsnorm, eps=pcase.eps,
                       norm_scale=norm_scale, rows=rows, nthreads=threads)
        return flops, time.perf_counter() - t

    f0, t0 = run_rows(4 * threads)                 # calibration
    rate = f0 / max(t0, 1e-6)
    n = max(threads, int(0.8 * target_s * rate / (pcase.N / 2.0 * per_pair)))
    f1, t1 = run_rows(n)
    # Decode: the first two sequences, all pairs.
    nb = 2
    t = time.perf_counter()
    oracle.decode(din["q"][:nb].cpu(), din["k_cache"][:nb].cpu(), din["v_cache"][:nb].cpu(),
                  din["seq_lens"][:nb].cpu(), dlam.cpu().numpy(), nthreads=threads)
    t2 = time.perf_counter() - t
    f2 = float(din["seq_lens"][:nb].sum().item()) * (dcase.Hq // 2) * 6 * dcase.D
    value = (f0 + f1 + f2) / (t0 + t1 + t2) / 1e12
    return {"value": round(value, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "seconds": round(t0 + t1 + t2, 2),
            "sample": "%d uniformly drawn query rows of the %d prefill rows (all their visible "
                      "keys, with the norm epilogue) + the decode of the first %d sequences; "
                      "fp64 C oracle, %d threads" % (4 * threads + n, total_rows, nb, threads)}


if __name__ == "__main__":
    main()
