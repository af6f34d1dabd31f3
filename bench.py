"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one forward pass (attn_fwd) over the long-context workload
B=4, H=32, N=4096, D=128, bf16, non-causal (the headline "attention fwd
TFLOP/s" workload); `value` is its throughput in TFLOP/s with the pages' flop
convention 4 B H Nq Nkv D (x0.5 causal, x3 for the fused JVP forward).  The
same run also times the fused JVP forward (B=4, H=16, N=2048, D=64) -- the
"+ JVP fwd TFLOP/s" half of the metric -- the causal variants, the causal
D=64 workload and the jagged workload, and reports them under `extra`.

Timing: inputs are resident in HBM before the timed region; W untimed steps,
then exactly K steps between two device synchronisations; per-launch HIP
events on the launch stream give the kernel's average duration for the
`roofline` object.  Each entry of `extra` also reports the median and minimum
launch and a cold-cache median (a 512 MiB buffer is rewritten before every
launch, outside the events, which evicts L2 and the Infinity Cache), each
median over at least 50 launches.  `roofline` and `jvp_roofline` give the
headline forward's and the JVP forward's kernel rate (average launch from the
events) against the bf16 MFMA peak.  `cpu_baseline` and `cpu_baseline_jvp`
time the fp64 CPU oracle on bounded samples of those two workloads (whole
(batch, head) slices) on this host's cores; `cpu_oracle_configs` gives the
oracle's seconds on the other workloads (fp32 tiny, causal D=64, jagged),
with the GPU/CPU ratio.

Profiling modes (for rocprofv3 runs): --only {fwd,fwd_causal,jvp,jvp_causal,
causal_d64,jagged,tiny_fp32,bwd,bwd_causal,fwd_fp16,fwd_bias,fwd_mask,bwd_bias,jagged_bwd} runs just that workload K times; --copy-calibration runs a
plain device copy of known size (the scale for FETCH_SIZE / WRITE_SIZE).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# sources of the headline kernel (attn_fwd_bf16_kernel and its tile mapping): the
# stored HBM traffic figure is valid only while they are unchanged
KERNEL_SOURCES = ["attn_common.h", "attn_fwd_bf16.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_forward_online_attn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dense_flops(B, H, Nq, Nkv, D, causal, jvp=False):
    f = 4.0 * B * H * Nq * Nkv * D
    if causal:
        f *= 0.5
    if jvp:
        f *= 3.0
    return f


def jagged_flops(lengths, H, D, causal=False):
    s = sum(int(x) * int(x) for x in lengths)
    return 4.0 * H * D * s * (0.5 if causal else 1.0)


class Case:
    """One workload bound to resident device inputs."""

    def __init__(self, name, run, flops, bytes_, desc):
        self.name, self.run, self.flops, self.bytes, self.desc = name, run, flops, bytes_, desc


def make_cases(torch, attn, wl, only=None):
    """Workloads bound to resident device inputs.  With `only`, just that
    case is built, and nothing but what it needs (its inputs, and the forward
    pass that produces a backward's O and LSE) is launched before it runs, so
    a profile of `--only X` holds X's kernels alone."""
    dev = torch.device("cuda:0")
    memo = {}

    def shared(key, fn):  # inputs several cases use, built once
        if key not in memo:
            memo[key] = fn()
        return memo[key]

    w, w2, w4, w5 = (wl.WORKLOADS[n] for n in ("long_d128", "causal_d64", "jvp_d64", "jagged_d128"))
    head = lambda: shared("head", lambda: [t.to(dev) for t in wl.dense_inputs(w.B, w.H, w.N, w.N, w.D, "bf16", 0)])
    io_bytes = 4 * w.B * w.H * w.N * w.D * 2 + w.B * w.H * w.N * 4
    bwd_io = 8 * w.B * w.H * w.N * w.D * 2 + w.B * w.H * w.N * 4
    # the headline shape with a score operand (bias page): a per-head additive
    # bias shared by the batch, and a per-batch boolean mask shared by the heads
    bias = lambda: shared("bias", lambda: wl.score_bias((1, w.H, w.N, w.N), "bf16", 0).to(dev))
    mask = lambda: shared("mask", lambda: wl.score_mask((w.B, 1, w.N, w.N), 0.75, 0).to(dev))
    grad = lambda: shared("do", lambda: wl.grad_output((w.B, w.H, w.N, w.D), "bf16", 0).to(dev))
    lengths = wl.jagged_lengths(w5.num_seqs, w5.max_len, 0)
    jag = lambda: shared("jag", lambda: [t.to(dev) for t in wl.jagged_inputs(lengths, w5.H, w5.D, "bf16", 0)])

    def fwd_case(causal):
        q, k, v = head()
        return Case("fwd_causal" if causal else "fwd", lambda: attn.fwd(q, k, v, causal=causal, sm_scale=w.sm_scale),
                    dense_flops(w.B, w.H, w.N, w.N, w.D, causal), io_bytes,
                    f"{w.name}: B={w.B} H={w.H} N={w.N} D={w.D} bf16 causal={causal}")

    def fp16_case():  # the headline shape with fp16 inputs (same 16-bit MFMA peak)
        qh, kh, vh = (t.to(dev) for t in wl.dense_inputs(w.B, w.H, w.N, w.N, w.D, "fp16", 0))
        return Case("fwd_fp16", lambda: attn.fwd(qh, kh, vh, causal=False, sm_scale=w.sm_scale),
                    dense_flops(w.B, w.H, w.N, w.N, w.D, False), io_bytes,
                    f"{w.name}: B={w.B} H={w.H} N={w.N} D={w.D} fp16 causal=False")

    def bias_case():
        q, k, v = head()
        b = bias()
        return Case("fwd_bias", lambda: attn.fwd_bias(q, k, v, bias=b, sm_scale=w.sm_scale),
                    dense_flops(w.B, w.H, w.N, w.N, w.D, False), io_bytes + b.numel() * 2,
                    f"{w.name}: B={w.B} H={w.H} N={w.N} D={w.D} bf16 + bias [1,{w.H},{w.N},{w.N}] bf16")

    def mask_case():
        q, k, v = head()
        m = mask()
        return Case("fwd_mask", lambda: attn.fwd_bias(q, k, v, mask=m, sm_scale=w.sm_scale),
                    dense_flops(w.B, w.H, w.N, w.N, w.D, False), io_bytes + m.numel(),
                    f"{w.name}: B={w.B} H={w.H} N={w.N} D={w.D} bf16 + mask [{w.B},1,{w.N},{w.N}] bool")

    def jvp_case(causal):
        ts = shared("jvp", lambda: [t.to(dev) for t in wl.dense_inputs(w4.B, w4.H, w4.N, w4.N, w4.D, "bf16", 0,
                                                                        tangents=True)])
        return Case("jvp_causal" if causal else "jvp", lambda: attn.fwd_jvp(*ts, causal=causal, sm_scale=w4.sm_scale),
                    dense_flops(w4.B, w4.H, w4.N, w4.N, w4.D, causal, jvp=True),
                    8 * w4.B * w4.H * w4.N * w4.D * 2 + w4.B * w4.H * w4.N * 4,
                    f"{w4.name}: B={w4.B} H={w4.H} N={w4.N} D={w4.D} bf16 causal={causal} (O, tO, LSE)")

    def tiny_case():  # the small fp32 correctness workload (launch-latency bound)
        t = wl.WORKLOADS["tiny_fp32"]
        q1, k1, v1 = (x.to(dev) for x in wl.dense_inputs(t.B, t.H, t.N, t.N, t.D, "fp32", 0))
        return Case("tiny_fp32", lambda: attn.fwd(q1, k1, v1, causal=False, sm_scale=t.sm_scale),
                    dense_flops(t.B, t.H, t.N, t.N, t.D, False), 4 * q1.numel() * 4 + t.B * t.H * t.N * 4,
                    f"{t.name}: B={t.B} H={t.H} N={t.N} D={t.D} fp32 causal=False")

    def causal_d64_case():
        q2, k2, v2 = (t.to(dev) for t in wl.dense_inputs(w2.B, w2.H, w2.N, w2.N, w2.D, "bf16", 0))
        return Case("causal_d64", lambda: attn.fwd(q2, k2, v2, causal=True, sm_scale=w2.sm_scale),
                    dense_flops(w2.B, w2.H, w2.N, w2.N, w2.D, True), 4 * q2.numel() * 2 + w2.B * w2.H * w2.N * 4,
                    f"{w2.name}: B={w2.B} H={w2.H} N={w2.N} D={w2.D} bf16 causal")

    def bwd_case(causal):  # backward over the headline shape: the forward's O and LSE, a seeded dO
        q, k, v = head()
        do = grad()
        o_f, lse_f = attn.fwd(q, k, v, causal=causal, sm_scale=w.sm_scale)
        ws_b = torch.empty(attn.bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
        return Case("bwd_causal" if causal else "bwd",
                    lambda: attn.bwd(q, k, v, o_f, do, lse_f, causal=causal, sm_scale=w.sm_scale, workspace=ws_b),
                    2.5 * dense_flops(w.B, w.H, w.N, w.N, w.D, causal), bwd_io,
                    f"{w.name} backward: B={w.B} H={w.H} N={w.N} D={w.D} bf16 causal={causal} (dQ, dK, dV)")

    def bwd_bias_case():  # backward of the per-head bias workload (the bias as a fixed operand)
        q, k, v = head()
        b, do = bias(), grad()
        o_b, lse_b = attn.fwd_bias(q, k, v, bias=b, sm_scale=w.sm_scale)
        ws_bb = torch.empty(attn.bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
        return Case("bwd_bias", lambda: attn.bwd_bias(q, k, v, o_b, do, lse_b, bias=b, sm_scale=w.sm_scale,
                                                      workspace=ws_bb),
                    2.5 * dense_flops(w.B, w.H, w.N, w.N, w.D, False), bwd_io + b.numel() * 2,
                    f"{w.name} backward: B={w.B} H={w.H} N={w.N} D={w.D} bf16 + bias [1,{w.H},{w.N},{w.N}] bf16 (dQ, dK, dV)")

    def jagged_ws():
        jq = jag()[0]
        return shared("jws", lambda: torch.empty(attn.jagged_workspace_bytes(w5.num_seqs, jq.shape[1]),
                                                 dtype=torch.uint8, device=dev))

    def jagged_case():
        jq, jk, jv, off = jag()
        ws = jagged_ws()
        return Case("jagged", lambda: attn.jagged_fwd(jq, jk, jv, off, w5.max_len, sm_scale=w5.sm_scale, workspace=ws),
                    jagged_flops(lengths.tolist(), w5.H, w5.D), 4 * jq.numel() * 2 + jq.shape[0] * jq.shape[1] * 4,
                    f"{w5.name}: 256 sequences U[1,1024], H=8 D=128 bf16, total_len={jq.shape[1]}")

    def jagged_bwd_case():  # jagged backward over the same sequences, from the forward's O and LSE
        jq, jk, jv, off = jag()
        jo, jl = attn.jagged_fwd(jq, jk, jv, off, w5.max_len, sm_scale=w5.sm_scale, workspace=jagged_ws())
        jdo = wl.grad_output(jq.shape, "bf16", 0).to(dev)
        jws = torch.empty(attn.jagged_bwd_workspace_bytes(w5.num_seqs, w5.H, jq.shape[1]), dtype=torch.uint8, device=dev)
        return Case("jagged_bwd", lambda: attn.jagged_bwd(jq, jk, jv, jo, jdo, jl, off, w5.max_len,
                                                          sm_scale=w5.sm_scale, workspace=jws),
                    2.5 * jagged_flops(lengths.tolist(), w5.H, w5.D), 8 * jq.numel() * 2 + jq.shape[0] * jq.shape[1] * 4,
                    f"{w5.name} backward: 256 sequences U[1,1024], H=8 D=128 bf16 (dQ, dK, dV)")

    builders = {
        "fwd": lambda: fwd_case(False), "fwd_causal": lambda: fwd_case(True), "fwd_fp16": fp16_case,
        "fwd_bias": bias_case, "fwd_mask": mask_case, "jvp": lambda: jvp_case(False),
        "jvp_causal": lambda: jvp_case(True), "causal_d64": causal_d64_case, "jagged": jagged_case,
        "tiny_fp32": tiny_case,
        "bwd": lambda: bwd_case(False), "bwd_causal": lambda: bwd_case(True), "bwd_bias": bwd_bias_case,
        "jagged_bwd": jagged_bwd_case,
    }
    names = [only] if only else list(builders)
    return {n: builders[n]() for n in names}


def time_case(torch, case, steps, warmup):
    """Average per-launch duration from HIP events on the launch stream, and
    the wall time of `steps` back-to-back launches."""
    durs, wall = time_launches(torch, case, steps, warmup)
    return sum(durs) / len(durs), min(durs), wall


def time_launches(torch, case, steps, warmup, flush=None):
    """Per-launch durations (ms) from HIP events on the launch stream around
    each launch, and the wall time of the whole loop.  With `flush` (a device
    buffer larger than L2 + MALL), the buffer is rewritten before every launch
    (outside the events), so each launch starts with cold caches."""
    for _ in range(warmup):
        case.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        if flush is not None:
            flush.fill_(i & 0xFF)
        a.record(stream)
        case.run()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in evs], wall


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def load_traffic(kernel_hash):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_hash:
        return None  # counters were taken on another version of the kernel
    return rec.get("fwd_bytes_per_launch")


def _host_info():
    from threadpoolctl import threadpool_info
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return int(threads), model


def _slices_until(budget_s, n_total, run_one):
    """Runs run_one(i) for i = 0, 1, ... until the budget is spent (at least
    once, at most n_total times); returns (count, seconds)."""
    n, t0 = 0, time.perf_counter()
    while n < n_total and (n == 0 or time.perf_counter() - t0 < budget_s):
        run_one(n)
        n += 1
    return n, time.perf_counter() - t0


def cpu_baseline(wl, budget_s=10.0):
    """The fp64 oracle on a bounded sample of the headline workload: whole
    (batch, head) slices of the same seeded B=4, H=32, N=4096, D=128 inputs,
    one after another until the time budget is spent (at most all 128)."""
    import oracle

    w = wl.WORKLOADS["long_d128"]
    q, k, v = wl.dense_inputs(w.B, w.H, w.N, w.N, w.D, "bf16", 0)
    scale = oracle.scale_as_passed(w.sm_scale)
    oracle.attention(q[:1, :1, :64], k[:1, :1, :64], v[:1, :1, :64], scale, False)  # warm the BLAS pool

    def one(i):
        b, h = divmod(i, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attention(q[sl], k[sl], v[sl], scale, False)
    heads, dt = _slices_until(budget_s, w.B * w.H, one)
    flops = dense_flops(1, heads, w.N, w.N, w.D, False)
    threads, model = _host_info()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_logical_cpus": os.cpu_count(), "seconds": round(dt, 3),
            "sample": f"{heads} of the 128 (batch, head) slices of the B=4 H=32 N=4096 D=128 non-causal "
                      f"forward in {dt:.1f} s (fp64 numpy oracle, BLAS threads = cores)"}


def cpu_baseline_jvp(wl, budget_s=8.0):
    """The oracle's closed-form JVP (O, tO, LSE) on whole (batch, head) slices
    of the B=4, H=16, N=2048, D=64 JVP workload, the metric's second half."""
    import oracle

    w = wl.WORKLOADS["jvp_d64"]
    ts = wl.dense_inputs(w.B, w.H, w.N, w.N, w.D, "bf16", 0, tangents=True)
    scale = oracle.scale_as_passed(w.sm_scale)

    def one(i):
        b, h = divmod(i, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attention_jvp(*(t[sl] for t in ts), scale, False)
    heads, dt = _slices_until(budget_s, w.B * w.H, one)
    flops = dense_flops(1, heads, w.N, w.N, w.D, False, jvp=True)
    threads, _ = _host_info()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{heads} of the 64 (batch, head) slices of the B=4 H=16 N=2048 D=64 non-causal JVP "
                      f"forward in {dt:.1f} s (fp64 numpy oracle, closed-form tangent)"}


def cpu_oracle_configs(wl, gpu_ms, budget_s=4.0):
    """Oracle seconds on the other workloads, with the GPU/CPU ratio against
    the GPU median of the same workload: the tiny fp32 forward whole (median
    of 5), the causal D=64 forward and the jagged forward on bounded samples
    (whole (batch, head) slices; whole sequences of all 8 heads), each scaled
    to the full workload by its flop share."""
    import oracle

    out = {}
    t = wl.WORKLOADS["tiny_fp32"]
    q, k, v = wl.dense_inputs(t.B, t.H, t.N, t.N, t.D, "fp32", 0)
    sc = oracle.scale_as_passed(t.sm_scale)
    ts = []
    for _ in range(5):
        t0 = time.perf_counter()
        oracle.attention(q, k, v, sc, False)
        ts.append(time.perf_counter() - t0)
    sec = median(ts)
    f = dense_flops(t.B, t.H, t.N, t.N, t.D, False)
    out["tiny_fp32"] = {"oracle_s": round(sec, 6), "oracle_gflops": round(f / sec / 1e9, 3),
                        "sample": "whole workload, median of 5"}

    c = wl.WORKLOADS["causal_d64"]
    q, k, v = wl.dense_inputs(c.B, c.H, c.N, c.N, c.D, "bf16", 0)
    sc = oracle.scale_as_passed(c.sm_scale)

    def one(i):
        b, h = divmod(i, c.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attention(q[sl], k[sl], v[sl], sc, True)
    n, dt = _slices_until(budget_s, c.B * c.H, one)
    sec = dt * (c.B * c.H) / n
    out["causal_d64"] = {"oracle_s": round(sec, 4), "oracle_gflops": round(dense_flops(c.B, c.H, c.N, c.N, c.D, True)
                                                                           / sec / 1e9, 3),
                         "sample": f"{n} of {c.B * c.H} (batch, head) slices in {dt:.1f} s, scaled"}

    j = wl.WORKLOADS["jagged_d128"]
    lengths = wl.jagged_lengths(j.num_seqs, j.max_len, 0)
    jq, jk, jv, off = wl.jagged_inputs(lengths, j.H, j.D, "bf16", 0)
    offs = off.numpy()
    sc = oracle.scale_as_passed(j.sm_scale)
    L = lengths.numpy()

    def one_seq(i):
        sl = slice(int(offs[i]), int(offs[i + 1]))
        oracle.jagged_attention(jq[:, sl], jk[:, sl], jv[:, sl], np.array([0, L[i]]), j.max_len, sc)
    n, dt = _slices_until(budget_s, j.num_seqs, one_seq)
    share = float(np.sum(L[:n].astype(np.float64) ** 2) / np.sum(L.astype(np.float64) ** 2))
    sec = dt / share
    out["jagged"] = {"oracle_s": round(sec, 4), "oracle_gflops": round(jagged_flops(L.tolist(), j.H, j.D)
                                                                            / sec / 1e9, 3),
                          "sample": f"{n} of {j.num_seqs} sequences (all 8 heads) in {dt:.1f} s, "
                                    f"{100 * share:.1f}% of the flops, scaled"}
    for name, ms in gpu_ms.items():
        if name in out and ms:
            out[name]["gpu_ms"] = round(ms, 5)
            out[name]["gpu_over_cpu"] = round(out[name]["oracle_s"] / (ms * 1e-3), 1)
    return out


def copy_calibration(torch, steps):
    """A plain device copy of 1 GiB (reads 1 GiB, writes 1 GiB) for scaling
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": 1 << 30, "launches": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (each (batch, head) is "
              "independent, so work would shard by head across GPUs). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_forward_online_attn_amd as attn
    from attention_forward_online_attn_amd import workloads as wl

    attn.load_library()
    if args.copy_calibration:
        copy_calibration(torch, args.steps)
        return
    cases = make_cases(torch, attn, wl, args.only)
    if args.only:
        c = cases[args.only]
        avg, mn, _ = time_case(torch, c, args.steps, args.warmup)
        print(json.dumps({"case": c.name, "desc": c.desc, "avg_ms": avg, "min_ms": mn,
                          "tflops": c.flops / (avg * 1e-3) / 1e12}), flush=True)
        return

    head = cases["fwd"]
    durs, wall = time_launches(torch, head, args.steps, args.warmup)
    avg, mn = sum(durs) / len(durs), min(durs)
    ms_per_step = wall * 1e3 / args.steps
    value = head.flops / (ms_per_step * 1e-3) / 1e12
    achieved = head.flops / (avg * 1e-3) / 1e12
    # cold caches: a 512 MiB buffer (more than 8 x 4 MB L2 + 256 MB MALL) is
    # rewritten before every launch, outside the timed events; medians over at
    # least 50 launches
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    n_cold = max(50, args.steps // 2)

    def summary(c, durs_w, durs_c):
        mw, mc = median(durs_w), median(durs_c)
        return {"workload": c.desc, "avg_ms": round(sum(durs_w) / len(durs_w), 4), "median_ms": round(mw, 4),
                "min_ms": round(min(durs_w), 4), "tflops": round(c.flops / (mw * 1e-3) / 1e12, 2),
                "frac_of_mfma_peak": round(c.flops / (mw * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "gbps_compulsory": round(c.bytes / (mw * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(c.bytes / (mw * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "cold_median_ms": round(mc, 4), "cold_min_ms": round(min(durs_c), 4),
                "cold_tflops": round(c.flops / (mc * 1e-3) / 1e12, 2)}

    extra = {"fwd": summary(head, durs, time_launches(torch, head, n_cold, 2, flush)[0])}
    warm = {}
    for name in ("fwd_causal", "fwd_fp16", "fwd_bias", "fwd_mask", "jvp", "jvp_causal", "causal_d64", "jagged",
                 "tiny_fp32", "bwd", "bwd_causal", "bwd_bias", "jagged_bwd"):
        c = cases[name]
        dw, _ = time_launches(torch, c, max(50, args.steps // 2), 10)
        dc, _ = time_launches(torch, c, n_cold, 2, flush)
        extra[name] = summary(c, dw, dc)
        warm[name] = dw
    del flush
    jvp_avg = sum(warm["jvp"]) / len(warm["jvp"])
    jvp_achieved = cases["jvp"].flops / (jvp_avg * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count}
    traffic = load_traffic(kernel_source_hash())
    out = {
        "metric": "attention fwd TFLOP/s (bf16, N=4096, D=128) + JVP fwd TFLOP/s, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs)",
        "config": {"workload": head.desc, "jvp_workload": cases["jvp"].desc,
                   "flops_per_step": head.flops,
                   "flop_convention": "4*B*H*Nq*Nkv*D (x0.5 causal, x3 JVP, x2.5 backward)",
                   "device": device},
        "jvp_value": extra["jvp"]["tflops"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd_bf16_kernel<128,64,false,4,false,0,0>",
                     "avg_launch_ms": round(avg, 4), "min_launch_ms": round(mn, 4),
                     "cold_median_ms": extra["fwd"]["cold_median_ms"]},
        "jvp_roofline": {"bound": "mfma", "achieved": round(jvp_achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(jvp_achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                         "kernel": "attn_fwd_bf16_kernel<64,32,true,4,false,0,0>",
                         "avg_launch_ms": round(jvp_avg, 4), "min_launch_ms": round(min(warm["jvp"]), 4),
                         "cold_median_ms": extra["jvp"]["cold_median_ms"],
                         "flops_per_launch": cases["jvp"].flops},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
        out["cpu_baseline_jvp"] = cpu_baseline_jvp(wl)
        out["cpu_baseline_jvp"]["gpu_over_cpu"] = round(jvp_achieved / out["cpu_baseline_jvp"]["value"], 1)
        out["cpu_baseline"]["gpu_over_cpu"] = round(achieved / out["cpu_baseline"]["value"], 1)
        out["cpu_oracle_configs"] = cpu_oracle_configs(
            wl, {n: extra[n]["median_ms"] for n in ("tiny_fp32", "causal_d64", "jagged")})
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
