"""Throughput of the joint-sequence attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload pro-clip]
                    [--no-cpu-baseline] [--no-kernels] [--no-long-video]

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM:
  joint_concat_permute(Q segments, RoPE on video)  -> q [B,H,S,D]
  joint_concat_permute(K segments, RoPE on video)  -> k
  joint_concat_permute(V segments)                 -> v
  attn_fwd(q, k, v, scale, kv_chunk)               -> out, lse
(the chunked online softmax and the explicit log-sum-exp merge run inside
attn_fwd).  `value` is attention TFLOP/s over the whole step, counting
4*B*H*Sq*Skv*D flops per step.  The standalone rope3d_apply and lse_merge
entry points are timed after the step loop on the same workload shapes and
reported under "kernels", with the shard-shape proxies, attn_fwd on the
tiny (fp32), lite-clip and image-dit workloads (their own seeded inputs and
kv_chunk) and
on the long-video workload (GPU-drawn inputs with its outlier keys).

roofline.achieved is 4*B*H*Sq*Skv*D over the mean duration of the timed
r3d_attn_fwd calls, measured with HIP events on the launch stream; a call is
two dispatches, the head-statistics pre-pass (reads K and V once) and the
attention kernel, so the call time is a slight over-estimate of the attention
kernel's own.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
MI355X_FP32_PEAK_TFLOPS = 157.3    # fp32 (the tiny workload's path runs in fp32)
MI355X_HBM_GBPS = 8000.0
METRIC = "attention TFLOP/s (4·B·H·Sq·Skv·D) + % bf16 MFMA peak; ms/call at 52k tokens"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_pro-clip_traffic.md")
MFMA_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_pro-clip_mfma_util.md")
POWER_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_pro-clip_power.md")
ATTN_SRC = os.path.join(ROOT, "long_sequence_attention_rope3d_amd", "csrc", "attn_fwd_bf16.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_code_sha256(path: str) -> str:
    """sha256 of a source file's code: '//' comments, trailing blanks and empty
    lines removed, so that editing a comment does not count as a kernel change."""
    lines = []
    for line in open(path, encoding="utf-8").read().splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line:
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def _profile_values(path: str, keys):
    """{key: float} read from a committed rocprofv3 summary, or None if the file or
    a key is missing or the attention kernel's code changed since it was taken."""
    try:
        text = open(path).read()
        src_hash = kernel_code_sha256(ATTN_SRC)
    except OSError:
        return None
    m_hash = re.search(r"kernel_code_sha256:\s*([0-9a-f]{64})", text)
    if not m_hash or m_hash.group(1) != src_hash:
        return None
    vals = {}
    for key in keys:
        m = re.search(key + r":\s*([0-9.eE+]+)", text)
        if not m:
            return None
        vals[key] = float(m.group(1))
    return vals


def _traffic_for_current_kernel():
    """HBM bytes per attn_fwd launch from the committed rocprofv3 --pmc summary,
    or None if there is none or the kernel code changed since it was taken."""
    vals = _profile_values(TRAFFIC_FILE, ["hbm_bytes_per_launch"])
    return None if vals is None else vals["hbm_bytes_per_launch"]


def _mfma_counters_for_current_kernel():
    """Matrix-core busy fraction and the clock the attention kernel ran at, from
    the committed rocprofv3 --pmc summary (SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE), or None if the kernel code changed since."""
    vals = _profile_values(MFMA_FILE, ["mfma_busy_frac", "sclk_ghz_under_load"])
    if vals is None:
        return None
    vals["source"] = os.path.relpath(MFMA_FILE, ROOT)
    # Board power under the same kernel (SMI samples beside the bench loop), if recorded.
    power = _profile_values(POWER_FILE, ["package_power_w_under_load", "power_cap_w"])
    if power is not None:
        vals.update(power)
        vals["power_source"] = os.path.relpath(POWER_FILE, ROOT)
    return vals


def power_cap_watts():
    """The board's power cap (W) from a read-only SMI query, or None: the attention kernel
    runs at the clock this cap allows, so boxes with different caps differ in ms per call."""
    try:
        out = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", out)
    return float(m.group(1)) if m else None


def cpu_baseline(w, inp, n_rows: int):
    """The fp64 oracle, as it is, on a bounded sample: RoPE of all of Q and K,
    the re-layout, then attention for n_rows query rows spread over every
    head.  Reported in the metric's unit (attention TFLOP/s of the sampled
    rows over the whole oracle time)."""
    import numpy as np
    import oracle
    from workloads.inputs import to_f64
    rng = np.random.default_rng(w.seed + 7)
    rows = np.sort(rng.choice(w.B * w.H * w.S, size=n_rows, replace=False))
    t0 = time.perf_counter()
    q, k, v = oracle.prepare_qkv([to_f64(s) for s in inp["q"]], [to_f64(s) for s in inp["k"]],
                                 [to_f64(s) for s in inp["v"]], w.grid, w.split, w.theta,
                                 "bf16" if w.dtype == "bf16" else "f32")
    oracle.attention_rows(q, k, v, rows, w.scale)
    dt = time.perf_counter() - t0
    flops = 4.0 * n_rows * w.S * w.D
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_rows} query rows of {w.B * w.H * w.S} ({w.name}), with the fp64 RoPE "
                      f"and re-layout of the full Q/K/V; {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="pro-clip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--no-kernels", action="store_true")
    ap.add_argument("--no-long-video", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note, not part of this library).", file=sys.stderr)
        sys.exit(2)

    # The board's power cap, read before this process touches the GPU (the query runs
    # as a child process).
    power_cap = power_cap_watts()

    import torch
    import long_sequence_attention_rope3d_amd as r3d
    from workloads import by_name, make_inputs

    w = by_name(args.workload)
    dev = torch.device("cuda", 0)
    props = torch.cuda.get_device_properties(dev)
    log(f"workload {w.name}: B={w.B} H={w.H} S={w.S} D={w.D} kv_chunk={w.kv_chunk} {w.dtype}")
    t0 = time.perf_counter()
    inp = make_inputs(w)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    segs = {n: [s.to(dev) for s in inp[n]] for n in "qkv"}
    rope = r3d.Rope3D(w.grid, w.split, w.theta)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.empty((w.B, w.H, w.S, w.D), dtype=tdt, device=dev)
    k, v, out = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, r3d.attn_fwd_workspace_size(w.B, w.H, w.S, w.S, w.D, w.kv_chunk, tdt)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        r3d.joint_concat_permute(segs["q"], rope, out=q)
        r3d.joint_concat_permute(segs["k"], rope, out=k)
        r3d.joint_concat_permute(segs["v"], None, out=v)
        if ev is not None:
            ev[0].record(stream)
        r3d.attn_fwd(q, k, v, scale=w.scale, kv_chunk=w.kv_chunk, out=out, lse=lse, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = [a.elapsed_time(b) for a, b in events]
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    ms_per_step = wall * 1e3 / args.steps
    flops = float(w.attn_flops)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (attn_avg_ms * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms, attn_fwd {attn_avg_ms:.3f} ms (min {min(attn_ms):.3f}) "
        f"= {achieved:.1f} TFLOP/s ({100 * achieved / MI355X_BF16_PEAK_TFLOPS:.1f}% of bf16 peak)")
    assert torch.isfinite(out.float()).all().item()

    kernels = {}
    if not args.no_kernels:
        kernels = time_side_kernels(torch, r3d, w, segs, q, k, v, lse, rope, dev, stream)
        if w.name == "pro-clip":
            for other in ("tiny", "lite-clip", "image-dit"):
                kernels["attn_fwd_" + other.replace("-", "_")] = time_attn_workload(torch, r3d, other, dev, stream)
            if not args.no_long_video:
                kernels["attn_fwd_long_video"] = time_long_video(torch, r3d, dev, stream)

    traffic_bytes = _traffic_for_current_kernel()
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MI355X_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_bytes,
                "kernel": "r3d_attn_fwd call (head_stats_kernel<128> + attn_bf16_kernel<128>)",
                "counters": _mfma_counters_for_current_kernel()}

    cpu = None
    if not args.no_cpu_baseline:
        del segs
        torch.cuda.synchronize()
        log(f"cpu baseline: oracle on {args.cpu_rows} rows ...")
        cpu = cpu_baseline(w, inp, args.cpu_rows)
        log(f"cpu baseline {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V shaped like the workload; no datasets)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Sq": w.S, "Skv": w.S, "D": w.D,
                   "video_grid": list(w.grid), "joint": dict(w.joint), "kv_chunk": w.kv_chunk,
                   "n_chunks": w.n_chunks, "parallelism": "single-gpu"},
        "attn_ms_per_call": round(attn_avg_ms, 4),
        "attn_ms_median": round(statistics.median(attn_ms), 4),
        "attn_ms_min": round(min(attn_ms), 4),
        "device": {"name": props.name, "compute_units": props.multi_processor_count,
                   "power_cap_w": power_cap},
        "attn_tflops": round(achieved, 2),
        "pct_bf16_peak": round(100 * achieved / MI355X_BF16_PEAK_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(rec), flush=True)


def time_side_kernels(torch, r3d, w, segs, q, k, v, lse, rope, dev, stream, reps: int = 5):
    """HBM-bound entry points on this workload's shapes, as GB/s of
    algorithmic bytes (each input read once, each output written once)."""
    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    res = {}
    es = 2 if w.dtype == "bf16" else 4
    n_all = w.B * w.H * w.S * w.D
    n_vid = w.B * w.H * w.Nv * w.D
    # fused RoPE + joint concat + re-layout of one tensor (Q)
    ms = timed(lambda: r3d.joint_concat_permute(segs["q"], rope, out=q))
    res["joint_concat_permute_rope"] = {"ms": round(ms, 4), "bytes": 2 * n_all * es,
                                        "GBps": round(2 * n_all * es / ms / 1e6, 1)}
    ms = timed(lambda: r3d.joint_concat_permute(segs["v"], None, out=q))
    res["joint_concat_permute"] = {"ms": round(ms, 4), "bytes": 2 * n_all * es,
                                   "GBps": round(2 * n_all * es / ms / 1e6, 1)}
    # QK-norm fused ahead of RoPE and the re-layout (weights for every segment)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 11)
    wts = [1.0 + 0.1 * torch.randn(w.H * w.D, device=dev, generator=g) for _ in segs["q"]]
    ms = timed(lambda: r3d.joint_concat_permute(segs["q"], rope, out=q, norm=wts))
    res["joint_concat_permute_qknorm_rope"] = {"ms": round(ms, 4), "bytes": 2 * n_all * es,
                                               "GBps": round(2 * n_all * es / ms / 1e6, 1)}
    del wts
    x = segs["q"][0]
    y = torch.empty_like(x)
    ms = timed(lambda: r3d.rope3d_apply(x, w.grid, w.split, w.theta, out=y))
    res["rope3d_apply"] = {"ms": round(ms, 4), "bytes": 2 * n_vid * es,
                           "GBps": round(2 * n_vid * es / ms / 1e6, 1)}
    del y
    # ring-form combine: one fp32 partial per kv_chunk
    n = w.n_chunks
    parts = torch.empty((n, w.B, w.H, w.S, w.D), dtype=torch.float32, device=dev).normal_()
    lparts = torch.empty((n, w.B, w.H, w.S), dtype=torch.float32, device=dev).normal_()
    mout = torch.empty((w.B, w.H, w.S, w.D), dtype=q.dtype, device=dev)
    nbytes = n * w.B * w.H * w.S * (w.D * 4 + 4) + w.B * w.H * w.S * (w.D * es + 4)
    ms = timed(lambda: r3d.lse_merge(parts, lparts, out=mout, lse_out=lse))
    res["lse_merge"] = {"ms": round(ms, 4), "n_parts": n, "bytes": nbytes,
                        "GBps": round(nbytes / ms / 1e6, 1)}
    del parts, lparts, mout
    for kname, r in res.items():
        r["frac_hbm_peak"] = round(r["GBps"] / MI355X_HBM_GBPS, 4)
        log(f"{kname}: {r['ms']:.3f} ms, {r['GBps']:.0f} GB/s")
    # attn_fwd writing its output token-major ([B,S,H,D], the inverse re-layout
    # fused into the epilogue); same flops as the timed step's attn_fwd.
    r3d.joint_concat_permute(segs["q"], rope, out=q)
    obshd = torch.empty((w.B, w.S, w.H, w.D), dtype=q.dtype, device=dev)
    ms = timed(lambda: r3d.attn_fwd(q, k, v, scale=w.scale, kv_chunk=w.kv_chunk, out=obshd, lse=lse,
                                    out_layout="bshd"))
    res["attn_fwd_bshd"] = {"ms": round(ms, 4), "TFLOPs": round(w.attn_flops / (ms * 1e-3) / 1e12, 2)}
    log(f"attn_fwd_bshd: {ms:.3f} ms, {res['attn_fwd_bshd']['TFLOPs']:.1f} TFLOP/s")
    # the constant-max variant (Cauchy-Schwarz row bound; key-norm pre-pass included)
    if w.dtype == "bf16":
        ws = torch.empty(r3d.attn_fwd_constmax_workspace_size(w.B, w.H, w.S, w.S, w.D, q.dtype),
                         dtype=torch.uint8, device=dev)
        ms = timed(lambda: r3d.attn_fwd_constmax(q, k, v, scale=w.scale, out=obshd.view(q.shape), lse=lse,
                                                 workspace=ws))
        res["attn_fwd_constmax"] = {"ms": round(ms, 4),
                                    "TFLOPs": round(w.attn_flops / (ms * 1e-3) / 1e12, 2)}
        log(f"attn_fwd_constmax: {ms:.3f} ms, {res['attn_fwd_constmax']['TFLOPs']:.1f} TFLOP/s")
        del ws
    del obshd
    # One rank's share of the sharded forms (P = 8), on this GPU: a Ulysses rank's H/P heads at
    # the full sequence, and a CP/ring rank's S/P query rows against all keys with one kv_chunk
    # per ring round.
    P = 8
    if w.H % P == 0 and w.S % P == 0:
        hp, sp = w.H // P, w.S // P
        qh, kh, vh = (t[:, :hp].contiguous() for t in (q, k, v))
        ms = timed(lambda: r3d.attn_fwd(qh, kh, vh, scale=w.scale, kv_chunk=w.kv_chunk))
        fl = 4.0 * w.B * hp * w.S * w.S * w.D
        res["attn_fwd_ulysses_shard"] = {"ms": round(ms, 4), "H": hp, "S": w.S,
                                         "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2)}
        del qh, kh, vh
        qs = q[:, :, :sp].contiguous()
        ms = timed(lambda: r3d.attn_fwd(qs, k, v, scale=w.scale, kv_chunk=sp))
        fl = 4.0 * w.B * w.H * sp * w.S * w.D
        res["attn_fwd_cp_shard"] = {"ms": round(ms, 4), "Sq": sp, "Skv": w.S, "kv_chunk": sp,
                                    "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2)}
        del qs
        for kname in ("attn_fwd_ulysses_shard", "attn_fwd_cp_shard"):
            log(f"{kname}: {res[kname]['ms']:.3f} ms, {res[kname]['TFLOPs']:.1f} TFLOP/s")
    return res


def time_attn_workload(torch, r3d, name, dev, stream, reps: int = 20):
    """attn_fwd alone on another workload's full shape (its seeded host inputs, RoPE and
    re-layout by joint_concat_permute, its kv_chunk).  "ms": mean per call over `reps`
    calls issued back to back between two HIP events (the host stays ahead of the GPU, as
    in a model's stream of layers); "ms_event_median" / "ms_min": the same calls each
    bracketed by its own events (a call the host issues late also counts the GPU's wait
    for it); "ms_graph": the same calls replayed from one captured HIP graph (no host issue
    time per call).  TFLOP/s and the fraction of the peak are from "ms"."""
    from workloads import by_name, make_inputs
    w = by_name(name)
    inp = make_inputs(w)
    rope = r3d.Rope3D(w.grid, w.split, w.theta)
    q = r3d.joint_concat_permute([s.to(dev) for s in inp["q"]], rope)
    k = r3d.joint_concat_permute([s.to(dev) for s in inp["k"]], rope)
    v = r3d.joint_concat_permute([s.to(dev) for s in inp["v"]], None)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, r3d.attn_fwd_workspace_size(w.B, w.H, w.S, w.S, w.D, w.kv_chunk, q.dtype)),
                     dtype=torch.uint8, device=dev)
    call = lambda: r3d.attn_fwd(q, k, v, scale=w.scale, kv_chunk=w.kv_chunk, out=out, lse=lse,  # noqa: E731
                                workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    per_call = a.elapsed_time(b) / reps
    # The same calls captured in one HIP graph and replayed: the GPU-side rate without the
    # host's issue time per call, which bounds a back-to-back loop of calls this small.
    # (A capture that fails leaves this figure null; the others stand.)
    per_call_graph = None
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            call()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                call()
        graph.replay()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(5):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per_call_graph = a.elapsed_time(b) / (5 * reps)
    except RuntimeError as e:
        log(f"attn_fwd_{w.name}: graph timing skipped ({e})")
        torch.cuda.synchronize()
    tf = w.attn_flops / (per_call * 1e-3) / 1e12
    log(f"attn_fwd_{w.name}: {per_call:.4f} ms per call back to back (each call between its own "
        f"events: median {med:.4f}, min {ms[0]:.4f}; replayed from a graph "
        f"{'-' if per_call_graph is None else f'{per_call_graph:.4f}'}), "
        f"{tf:.1f} TFLOP/s")
    res = {"ms": round(per_call, 4), "ms_event_median": round(med, 4), "ms_min": round(ms[0], 4),
           "ms_graph": None if per_call_graph is None else round(per_call_graph, 4), "S": w.S, "H": w.H, "kv_chunk": w.kv_chunk,
           "TFLOPs": round(tf, 3)}
    if w.dtype == "bf16":
        res["frac_bf16_peak"] = round(tf / MI355X_BF16_PEAK_TFLOPS, 4)
    else:
        res["dtype"] = w.dtype
        res["frac_fp32_peak"] = round(tf / MI355X_FP32_PEAK_TFLOPS, 5)
    return res


def time_long_video(torch, r3d, dev, stream, reps: int = 3):
    """attn_fwd on the long-video workload (119056 tokens, 1% of key tokens at 8x):
    Q/K/V drawn N(0,1) on the GPU (seeded) in the per-segment layout, the outlier
    keys scaled as the workload recipe does, RoPE + re-layout by joint_concat_permute,
    then attn_fwd timed.  Timing only (the parity tests use the host-generated inputs);
    here the outlier keys make each row's Cauchy-Schwarz bound loose, so the gated row
    max is formed on every step."""
    from workloads import by_name
    w = by_name("long-video")
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    segs = {n: [torch.randn((w.B, L, w.H, w.D), device=dev, generator=g).to(torch.bfloat16)
                for L in w.seg_lens] for n in "qkv"}
    idx = torch.randperm(w.S, device=dev, generator=g)[: int(w.outlier_frac * w.S)]
    off = 0
    for seg in segs["k"]:
        L = seg.shape[1]
        sel = idx[(idx >= off) & (idx < off + L)] - off
        seg[:, sel] *= w.outlier_mult
        off += L
    rope = r3d.Rope3D(w.grid, w.split, w.theta)
    q = r3d.joint_concat_permute(segs["q"], rope)
    k = r3d.joint_concat_permute(segs["k"], rope)
    v = r3d.joint_concat_permute(segs["v"], None)
    del segs
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    r3d.attn_fwd(q, k, v, scale=w.scale, kv_chunk=w.kv_chunk, out=out, lse=lse)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        r3d.attn_fwd(q, k, v, scale=w.scale, kv_chunk=w.kv_chunk, out=out, lse=lse)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del q, k, v, out, lse
    tf = w.attn_flops / (ms * 1e-3) / 1e12
    log(f"attn_fwd_long_video: {ms:.3f} ms, {tf:.1f} TFLOP/s")
    return {"ms": round(ms, 3), "S": w.S, "kv_chunk": w.kv_chunk, "TFLOPs": round(tf, 2),
            "data": "N(0,1) drawn on the GPU, 1% of key tokens x8"}


if __name__ == "__main__":
    main()
