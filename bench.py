"""Throughput of the attention hot path on one MI355X.

A step is one pass of the whole path over the multi-head causal workload
(B=4, H=16, N=2048, D=128, bf16 Q/K/V iid N(0,1), scale 1/sqrt(128)): the
forward (O and lse) followed by the backward (dQ, dK, dV from the forward's O
and lse, deterministic variant). `value` is the step's algorithmic TFLOP/s:
forward 4*B*H*N^2*D plus backward 10*B*H*N^2*D, both halved for causal.

Also reported, each timed on its own with HIP events on the launch stream:
every other workload's headline pass (the float32 single head, the D=256
forward, the causal backward, the long-context FP8 forward), the roofline of
the dominant kernel, and the float64 oracle timed on the host cores on a
sample of the same workload.

The dominant kernel is the backward's key-tile pass (dK, dV); it is timed
alone through fa_bwd_dkdv (preprocess + key-tile kernel) and credited with
the four contractions it performs (S, dP, dV, dK): 8*B*H*N^2*D flops, halved
for causal. Its HBM traffic comes from rocprofv3 FETCH_SIZE / WRITE_SIZE
counters recorded in profiles/traffic_bwd_dkdv.json, scaled by the same
counters' reading for a plain copy kernel of known size (--calibrate-copy);
it is reported only while the kernel sources still hash to the recorded value.

The defaults (W = K = 200, about 0.15 s of GPU work) let the GPU reach its
sustained clock before the timed steps: with 5 warm-up steps the first timed
steps ran at a lower clock and the step read about 15% slower.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-breakdown] [--breakdown-only]
       python bench.py --calibrate-copy    (plain 512 MiB device copy, for counter calibration)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "f32": 157.3}  # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--breakdown-only", action="store_true",
                    help="time each workload's headline pass alone and print that JSON (no step line)")
    return ap.parse_args()


KERNEL_SOURCES = ("tiled_online_softmax_amd/csrc/bwd.hip", "tiled_online_softmax_amd/csrc/common.hpp")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_bwd_dkdv.json")
MFMA_RECORD = os.path.join(ROOT, "profiles", "mfma_util_step.json")


def _hash_files(paths, root=ROOT):
    """sha256 of the files' code: `//` comments, trailing blanks and blank lines removed."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in paths:
        with open(os.path.join(root, f)) as fh:
            text = re.sub(r"//[^\n]*", "", fh.read())
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()


def sources_sha256():
    """Hash of the dominant kernel's sources with comments and blank lines removed (code changes only)."""
    return _hash_files(KERNEL_SOURCES)


def step_sources_sha256():
    """Hash of every kernel source (comments and blank lines removed): the step's kernels' code."""
    d = os.path.join(ROOT, "tiled_online_softmax_amd", "csrc")
    return _hash_files(sorted(os.path.join("tiled_online_softmax_amd", "csrc", f) for f in os.listdir(d)))


def recorded_mfma():
    """Per-kernel MFMA utilisation (%) and HBM GB/s of the step from the committed counter record, or None if stale."""
    try:
        with open(MFMA_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != step_sources_sha256():
        return None
    out = {}
    for k, v in rec["kernels"].items():
        key = next((n for n in ("fwd_pipe_kernel", "fwd_pp_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel",
                                "bwd_pre_kernel") if n in k), k)
        out[key] = {"mfma_util_pct": round(v["mfma_util_pct"], 1), "hbm_gbps": round(v["hbm_gbps"] or 0.0, 1)}
    return {"kernels": out, "source": "profiles/mfma_util_mh_causal_b4h16n2048d128.md"}


def recorded_traffic():
    """HBM bytes per launch of the dK/dV pass from the committed counter record, or None if stale."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sources_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_copy():
    """A plain device copy of known size; its FETCH/WRITE counters calibrate the traffic figures."""
    import torch

    n = 512 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_inputs(w, with_grad, shape=None):
    import torch

    from tiled_online_softmax_amd import inputs

    d = inputs.make(w, with_grad=with_grad, shape=shape)
    out = {}
    for n in ("q", "k", "v", "do"):
        if n not in d:
            continue
        if w.dtype == "f32":
            out[n] = torch.from_numpy(d[n]).to("cuda:0")
        elif w.dtype == "bf16":
            out[n] = torch.from_numpy(d[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
        else:
            out[n] = torch.from_numpy(d[n]).to("cuda:0")  # fp32 draws, quantised on the GPU
    return out


def time_fn(fn, iters, warmup=3, warm_ms=50.0):
    """Average milliseconds per call of `fn` (launches on torch's current stream), by HIP events.

    Untimed calls first: at least `warmup` of them and at least `warm_ms` of wall time, so that a
    GPU left idle by host work (input generation, the CPU baseline) is back at its sustained clock.
    """
    import torch

    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def breakdown():
    """Each workload's headline pass, timed alone."""
    import torch

    from tiled_online_softmax_amd import fa, inputs

    res = {}
    for name, w in inputs.WORKLOADS.items():
        t0 = time.time()
        x = device_inputs(w, with_grad=(w.passes != "fwd"))
        legs = []  # (label, pass, fn, flops, peak, iters)
        if w.lengths is not None:  # packed sequences
            cu = torch.from_numpy(w.cu_seqlens()).to("cuda:0")
            mx = max(w.lengths)
            o, lse = fa.fwd_varlen(x["q"], x["k"], x["v"], cu, cu, mx, mx, causal=w.causal)
            ws = torch.empty(fa.bwd_workspace_size(1, w.H, w.shape[0], w.D, fa.FA_BWD_DETERMINISTIC),
                             dtype=torch.uint8, device="cuda:0")
            g = [torch.empty_like(x[n]) for n in ("q", "k", "v")]
            legs.append((name + ":fwd", "fwd", lambda: fa.fwd_varlen(x["q"], x["k"], x["v"], cu, cu, mx, mx,
                                                                   causal=w.causal, out=o, lse=lse),
                         w.fwd_flops(), PEAK_TFLOPS["bf16"], 50))
            legs.append((name + ":bwd", "bwd", lambda: fa.bwd_varlen(x["q"], x["k"], x["v"], o, x["do"], lse, cu, cu,
                                                                   mx, mx, causal=w.causal,
                                                                   variant=fa.FA_BWD_DETERMINISTIC, workspace=ws,
                                                                   dq=g[0], dk=g[1], dv=g[2]),
                         w.bwd_flops(), PEAK_TFLOPS["bf16"], 20))
        elif w.block_pattern is not None:  # block-sparse; the lists are built once, outside the timed calls
            mask = torch.from_numpy(w.block_mask()).to("cuda:0").expand(w.B, w.H, -1, -1)
            bl = fa.block_lists(mask, w.N, w.N, w.causal, w.window)
            o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, window=w.window, block_lists=bl)
            ws = torch.empty(fa.bwd_workspace_size(w.B, w.H, w.N, w.D, fa.FA_BWD_DETERMINISTIC), dtype=torch.uint8,
                             device="cuda:0")
            legs.append((name + ":fwd", "fwd", lambda: fa.fwd(x["q"], x["k"], x["v"], causal=w.causal,
                                                            window=w.window, block_lists=bl, out=o, lse=lse),
                         w.fwd_flops(), PEAK_TFLOPS["bf16"], 50))
            legs.append((name + ":bwd", "bwd", lambda: fa.bwd(x["q"], x["k"], x["v"], o, x["do"], lse,
                                                            causal=w.causal, window=w.window,
                                                            variant=fa.FA_BWD_DETERMINISTIC, workspace=ws,
                                                            block_lists=bl),
                         w.bwd_flops(), PEAK_TFLOPS["bf16"], 20))
        elif w.dtype == "fp8":
            qc, qd = fa.quantize_fp8(x["q"])
            kc, kd = fa.quantize_fp8(x["k"])
            vc, vd = fa.quantize_fp8(x["v"])
            del x
            fn = lambda: fa.fwd_fp8(qc, kc, vc, causal=w.causal, q_descale=qd, k_descale=kd, v_descale=vd)
            legs.append((name, "fwd", fn, w.fwd_flops(), PEAK_TFLOPS["fp8"], 10))
        if w.passes in ("fwd", "fwd+bwd") and w.dtype != "fp8" and w.lengths is None and w.block_pattern is None:
            fn = lambda: fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, window=w.window)
            peak = PEAK_TFLOPS["f32" if w.dtype == "f32" else "bf16"]
            legs.append((name if w.passes == "fwd" else name + ":fwd", "fwd", fn, w.fwd_flops(), peak,
                         200 if w.N <= 2048 else 30))
        if w.passes in ("bwd", "fwd+bwd") and w.lengths is None and w.block_pattern is None:
            o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, window=w.window)
            ws = torch.empty(fa.bwd_workspace_size(w.B, w.H, w.N, w.D, fa.FA_BWD_DETERMINISTIC), dtype=torch.uint8,
                             device="cuda:0")
            fn = lambda: fa.bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=w.causal,
                                variant=fa.FA_BWD_DETERMINISTIC, workspace=ws, window=w.window)
            legs.append((name if w.passes == "bwd" else name + ":bwd", "bwd", fn, w.bwd_flops(), PEAK_TFLOPS["bf16"],
                         50))
        for label, pss, fn, flops, peak, iters in legs:
            try:
                ms = time_fn(fn, iters)
            except Exception as e:  # report, do not hide
                res[label] = {"error": str(e)}
                continue
            tf = flops / (ms * 1e-3) / 1e12
            res[label] = {"pass": pss, "dtype": w.dtype, "ms": round(ms, 4), "tflops": round(tf, 2),
                          "pct_of_peak": round(100 * tf / peak, 2), "peak_tflops": peak}
            log(f"[breakdown] {label}: {ms:.4f} ms  {tf:.1f} TFLOP/s  ({100 * tf / peak:.1f}% of {peak})"
                f"  [{time.time() - t0:.1f}s]")
        torch.cuda.empty_cache()
    return res


def cpu_baseline(w, step_flops, heads=None):
    """The float64 oracle on a sample of the step workload (forward + backward of `heads` heads), in TFLOP/s."""
    from oracle import attention, codecs
    from tiled_online_softmax_amd import inputs

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    heads = w.B * w.H if heads is None else heads
    d = inputs.make(w, with_grad=True, shape=(1, heads, w.N, w.D))
    q, k, v, do = (codecs.bf16_to_f64(d[n + "_bits"]) for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    attention.forward(q, k, v, w.causal, w.scale)
    attention.backward(q, k, v, do, w.causal, w.scale)
    dt = time.perf_counter() - t0
    frac = heads / (w.B * w.H)
    tf = step_flops * frac / dt / 1e12
    return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} (b,h) heads of the step workload, forward + backward, float64 "
                      f"numpy oracle, {dt:.2f} s"}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from tiled_online_softmax_amd import fa, inputs

    fa.lib()
    if args.breakdown_only:
        print(json.dumps({"workloads": breakdown()}), flush=True)
        return
    w = inputs.WORKLOADS["mh_causal_bf16"]
    x = device_inputs(w, with_grad=True)
    variant = fa.FA_BWD_DETERMINISTIC
    ws = torch.empty(fa.bwd_workspace_size(w.B, w.H, w.N, w.D, variant), dtype=torch.uint8, device="cuda:0")
    o = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))

    def fwd():
        fa.fwd(x["q"], x["k"], x["v"], causal=w.causal, out=o, lse=lse)

    def bwd():
        fa.bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=w.causal, variant=variant, workspace=ws,
               dq=dq, dk=dk, dv=dv)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    step_flops = w.fwd_flops() + w.bwd_flops()
    value = step_flops / (ms * 1e-3) / 1e12
    log(f"[step] {ms:.4f} ms/step, {value:.1f} TFLOP/s")

    # forward and backward passes separately, and the dominant kernel (the backward's
    # key-tile pass: preprocess + dK/dV kernel) alone through fa_bwd_dkdv
    ms_f = time_fn(fwd, 100)
    ms_b = time_fn(bwd, 100)
    fwd_tf = w.fwd_flops() / (ms_f * 1e-3) / 1e12
    bwd_tf = w.bwd_flops() / (ms_b * 1e-3) / 1e12
    dk2, dv2 = torch.empty_like(x["q"]), torch.empty_like(x["q"])
    ws_d = torch.empty(fa.bwd_workspace_size(w.B, w.H, w.N, w.D, fa.FA_BWD_DETERMINISTIC), dtype=torch.uint8,
                       device="cuda:0")

    def dkdv():
        fa.bwd_dkdv(x["q"], x["k"], x["v"], o, x["do"], lse, causal=w.causal, workspace=ws_d, dk=dk2, dv=dv2)

    ms_k = time_fn(dkdv, 100)
    kflops = 8.0 * w.B * w.H * w.N * w.N * w.D / (2 if w.causal else 1)
    k_tf = kflops / (ms_k * 1e-3) / 1e12
    log(f"[fwd] {ms_f:.4f} ms {fwd_tf:.1f} TF/s   [bwd] {ms_b:.4f} ms {bwd_tf:.1f} TF/s   "
        f"[dK/dV pass] {ms_k:.4f} ms {k_tf:.1f} TF/s")
    roofline = {"bound": "mfma", "achieved": round(k_tf, 2), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": round(k_tf / PEAK_TFLOPS["bf16"], 4), "traffic": recorded_traffic(),
                "kernel": "backward key-tile pass (bwd_pre_kernel + bwd_dkdv_kernel, via fa_bwd_dkdv)",
                "avg_launch_ms": round(ms_k, 5), "algorithmic_flops_per_launch": kflops,
                "traffic_unit": "HBM bytes per launch"}

    out = {"metric": "attention fwd/bwd TFLOP/s on 1 MI355X + % of bf16/fp8 MFMA peak", "value": round(value, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "multi-head causal attention forward + backward", "B": w.B, "H": w.H, "N": w.N,
                      "D": w.D, "causal": True, "inputs": "bf16 iid N(0,1)", "scale": "1/sqrt(128)",
                      "bwd_variant": "deterministic"},
           "pct_of_bf16_peak": round(100 * value / PEAK_TFLOPS["bf16"], 2),
           "fwd": {"ms": round(ms_f, 5), "tflops": round(fwd_tf, 2)},
           "bwd": {"ms": round(ms_b, 5), "tflops": round(bwd_tf, 2)},
           "roofline": roofline,
           "rocprof": recorded_mfma()}
    del x
    torch.cuda.empty_cache()
    if not args.no_breakdown:
        out["workloads"] = breakdown()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, step_flops)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
