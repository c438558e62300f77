"""KDA prefill + decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one pass of the whole hot path over one synthetic batch:
  * kda_prefill on the K3-shaped single-layer workload
    (B=1, H=96, T=65536, d_k=d_v=128, bf16 q/k/v, fp32 z/beta, fp32 state out), then
  * kda_decode on the batched decode workload
    (256 sequences x 96 heads, 128x128 fp32 state updated in place).
Inputs are seeded and already resident in HBM when timing starts.  W warmup
steps run untimed, then exactly K steps are timed between two device
synchronisations; HIP events on the launch stream time each entry point.
After the timed region, 1000 extra decode steps measure the decode state
bandwidth, and the fp64 oracle runs on a bounded sample on the host cores
(the CPU baseline).  Rank 0 prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s & MFMA % (H=96,d=128); decode state GB/s vs HBM peak"
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, AMD published
BF16_DENSE_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, AMD published
# Algorithmic work per (token, head) pair at d = 128, chunk 64:
#   bytes: q, k, v bf16 (3 x 256) + z fp32 (512) + beta (4) + o bf16 (256) = 1540
#   useful flops: 6 d^2 (W S, Q S, K^T V') + 5 C d (lower-triangular C x C products) + C^2/3 (solve)
PREFILL_BYTES_PER_PAIR = 1540
PREFILL_FLOPS_PER_PAIR = 6 * 128 * 128 + 5 * 64 * 128 + (64 * 64) // 3
# decode: state read + write (2 x 128 x 128 x 4) + q, k, v, o bf16 + z fp32 + beta = 132612
DECODE_BYTES_PER_PAIR = 2 * 128 * 128 * 4 + 4 * 128 * 2 + 128 * 4 + 4


# The sources of the kernels one kda_prefill launch runs (chunk table, intra, inter,
# combine) and the headers they include: a change to any of them makes the committed
# traffic figure stale.
PREFILL_SOURCES = ("kda_prefill.hip", "kda_intra.hip", "kda_intra_f32.hip", "kda_chunk.h", "kda_device.h",
                   "kda_internal.h")


def kernel_sources_digest() -> str:
    """sha256 (first 16 hex digits) over the prefill kernels' sources, with
    comments and whitespace removed: a figure taken on the kernels stays
    valid through comment edits and goes stale with any change to the code."""
    import hashlib
    import re
    files = [os.path.join(ROOT, "gated_delta_rule_21_amd", "csrc", f) for f in PREFILL_SOURCES]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, encoding="utf-8") as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", "", code, flags=re.S)     # block comments
        code = re.sub(r"//[^\n]*", "", code)                    # line comments
        h.update("".join(code.split()).encode())
    return h.hexdigest()[:16]


def profile_value(fname: str, key: str):
    """An integer `key: value` line of a committed rocprofv3 summary under
    profiles/, or None when the file is missing or the prefill kernels' sources
    have changed since it was taken (its `sources_sha256` line differs)."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            parts = line.strip().split(":")
            if len(parts) == 2 and parts[0] in (key, "sources_sha256"):
                vals[parts[0]] = parts[1].strip()
    if vals.get("sources_sha256") != kernel_sources_digest() or key not in vals:
        return None
    return int(vals[key])


def measured_traffic():
    """HBM bytes per kda_prefill launch (FETCH_SIZE / WRITE_SIZE summary)."""
    return profile_value("kda_k3_traffic.md", "prefill_traffic_bytes")


def counted_mfma_flops():
    """16-bit MFMA FLOPs per kda_prefill launch (SQ_INSTS_VALU_MFMA_MOPS_* x 512)."""
    return profile_value("kda_k3_prefill_counters.md", "prefill_mfma16_flops")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--decode-steps", type=int, default=1000)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-features", action="store_true",
                   help="skip the side measurements of the feature path, the output gate and the fused calls")
    p.add_argument("--no-backward", action="store_true",
                   help="skip the side measurement of the prefill backward")
    p.add_argument("--no-checkpoints", action="store_true",
                   help="skip the side measurement of the prefill with 512-token checkpoints")
    p.add_argument("--no-decode-window", action="store_true",
                   help="skip the side measurement of the speculative decode step")
    p.add_argument("--no-varlen", action="store_true",
                   help="skip the side measurement of the varlen packed prefill (32 sequences, 262144 tokens)")
    p.add_argument("--no-small-head", action="store_true",
                   help="skip the side measurement of the small-head prefill (B=2, H=8, T=8192)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the oracle sample")
    p.add_argument("--copy-probe-gib", type=float, default=0.0,
                   help="after timing, run one plain device copy of this many GiB (a known "
                        "byte count that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (or the platform string)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(pre: dict, target_s: float) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the prefill
    workload: the first `tok` tokens of every head, with `tok` grown until
    one run takes about target_s / 2 seconds or covers the whole sequence."""
    import numpy as np
    import oracle
    from gated_delta_rule_21_amd import workloads as W

    cores = os.cpu_count() or 1
    T, H = pre["q"].shape[0], pre["q"].shape[1]
    threads = min(cores, H)

    def run(tok):
        sl = lambda t: t[:tok]
        args = [W.as_numpy(sl(pre[n])) for n in ("q", "k", "v", "z")]
        beta = W.as_numpy(sl(pre["beta"]))
        A = W.as_numpy(pre["A"])
        cu = np.array([0, tok], np.int32)
        t0 = time.perf_counter()
        oracle.prefill(args[0], args[1], args[2], args[3], A, beta, None, cu, nthreads=threads)
        return time.perf_counter() - t0

    tok = 64
    dt = run(tok)
    while dt < target_s / 2 and tok < T:
        tok = min(T, int(tok * min(8.0, max(1.5, target_s / 2 / max(dt, 1e-3)))))
        dt = run(tok)
    return {"value": tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 token-loop oracle (C, OpenMP over heads) on the first %d of %d tokens "
                      "of all %d heads of the prefill workload, %.2f s wall; host CPU %s, %d logical "
                      "cores, %d threads used" % (tok, T, H, dt, cpu_model(), cores, threads)}


def small_head_prefill(kda, W, dev, reps: int = 12, sets: int = 3) -> dict:
    """Side measurement: the small-head prefill (B=2, H=8, T=8192 each,
    d=128, bf16), split into segments by the automatic choice and unsplit.
    One set of inputs and outputs is about 235 MB, under the 256 MB Infinity
    Cache, so the timed calls rotate over `sets` independently drawn sets
    (about 0.7 GB in all).  HIP events on the launch stream, inputs resident,
    workspace preallocated."""
    import torch
    ins = [W.make("small_head", device=dev, seed=W.BASE_SEED + 1 + 100 * i) for i in range(sets)]
    T, H, D = ins[0]["q"].shape
    N = ins[0]["cu_seqlens"].numel() - 1
    outs = [(torch.empty((T, H, D), dtype=torch.bfloat16, device=dev),
             torch.empty((N, H, D, D), dtype=torch.float32, device=dev)) for _ in range(sets)]
    out = {"workload": "small_head B=2 H=8 T=8192 per sequence d=128 bf16, h0 given; %d input sets "
                       "rotated" % sets}
    for P, key in ((0, "auto"), (1, "unsplit")):
        segs = P if P > 0 else kda.kda_prefill_segments(N, T, H, D, D, kda.KDA_BF16)
        ws = kda.prefill_workspace(N, T, H, D, kda.KDA_BF16, dev, segments=P)

        def run(i):
            d, (o, hT) = ins[i % sets], outs[i % sets]
            kda.prefill(d["q"], d["k"], d["v"], d["z"], d["A"], d["beta"], d["cu_seqlens"], h0=d["h0"],
                        o=o, hT=hT, workspace=ws, segments=P)
        for i in range(sets):
            run(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        del ws
        out[key] = {"segments": segs, "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1)}
    return out


def varlen_prefill(kda, W, dev, reps: int = 5) -> dict:
    """Side measurement: the varlen packed prefill (32 lognormal lengths
    summing to 262,144 tokens, H=96, d=128, bf16, h0 given), with the
    per-(token, head) algorithmic bytes of the K3 figure."""
    import torch
    d = W.make("k3_varlen", device=dev)
    T, H, D = d["q"].shape
    N = d["cu_seqlens"].numel() - 1
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    ws = kda.prefill_workspace(N, T, H, D, kda.KDA_BF16, dev)
    run = lambda: kda.prefill(d["q"], d["k"], d["v"], d["z"], d["A"], d["beta"], d["cu_seqlens"], h0=d["h0"],
                              o=o, hT=hT, workspace=ws)
    run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbps = PREFILL_BYTES_PER_PAIR * T * H / (ms * 1e-3) / 1e9
    lens = (d["cu_seqlens"][1:] - d["cu_seqlens"][:-1]).tolist()
    del ws, o, hT, d
    torch.cuda.empty_cache()
    return {"workload": "k3_varlen: 32 lognormal(ln 8192, 1) lengths summing to 262144 (shortest %d, longest %d), "
                        "H=96 d=128 bf16, h0 given" % (min(lens), max(lens)),
            "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "algorithmic_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def decode_window_step(kda, W, dev, reps: int = 200) -> dict:
    """Side measurement: one speculative-decode step, 256 sequences x 96
    heads x 128^2: replay of a 4-token window with n_accept ~ U{0..4}, then a
    new 4-token window.  Algorithmic bytes: the state read once, written once
    where something was accepted, the accepted replay tokens' k, v, z, beta,
    and the window's q, k, v, z, beta and o."""
    import torch
    Lr = L = 4
    d = W.random_decode_window(256, 96, 128, Lr=Lr, L=L, io="bf16", device=dev)
    N, H, D = d["N"], d["H"], d["dk"]
    S = d["S"].clone()
    o = torch.empty((N, L, H, D), dtype=torch.bfloat16, device=dev)
    run = lambda: kda.decode_window(d["A"], S, window=d["window"], replay=d["replay"],
                                    n_accept=d["n_accept"], o=o)
    for _ in range(5):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    acc = d["n_accept"].cpu()
    state = D * D * 4
    per_head = (state * N + state * int((acc > 0).sum()) + 1028 * int(acc.sum()) + 1540 * L * N)
    gbps = per_head * H / (ms * 1e-3) / 1e9
    return {"workload": "spec decode 256x96 d=128 bf16, replay 4 (n_accept ~ U{0..4}), window 4",
            "ms": round(ms, 4), "algorithmic_GBps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "accepted_tokens": int(acc.sum()), "window_tokens": N * L}


def prefill_checkpoint_cost(kda, pre, o, hT, ws, interval: int = 512, reps: int = 5) -> dict:
    """Side measurement: the same K3 prefill saving the state every
    `interval` tokens (prefix-reuse checkpoints)."""
    import torch
    T, H, D = pre["q"].shape
    ck = torch.empty((T // interval, H, D, D), dtype=torch.float32, device=pre["q"].device)
    run = lambda: kda.prefill_checkpoints(pre["q"], pre["k"], pre["v"], pre["z"], pre["A"], pre["beta"],
                                          pre["cu_seqlens"], interval, h0=None, o=o, hT=hT,
                                          checkpoints=ck, workspace=ws)
    run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del ck
    return {"interval": interval, "checkpoints": T // interval, "ms": round(ms, 4),
            "checkpoint_GB": round((T // interval) * H * D * D * 4 / 1e9, 3)}


def prefill_backward_cost(kda, W, pre, reps: int = 3) -> dict:
    """Side measurement: gradients of the K3 prefill (kda_prefill_backward:
    forward recompute with chunk-boundary states, then the fp32 backward
    kernels).  Algorithmic bytes per (token, head): q, k, v and dO read in
    bf16, z and beta in fp32, dq, dk, dv, dz and dbeta written in fp32."""
    import torch
    T, H, D = pre["q"].shape
    dev = pre["q"].device
    cot = W.random_cotangents(T, 1, H, D, "bf16", final_state=True, device=dev)
    ws = torch.empty(kda.kda_prefill_backward_workspace_size(1, T, H, D, D, kda.KDA_BF16), dtype=torch.uint8,
                     device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {n: torch.empty((T, H, D), **f32) for n in ("dq", "dk", "dv", "dz")}
    g.update(dbeta=torch.empty((T, H), **f32), dA=torch.empty((H,), **f32), dh0=torch.empty((1, H, D, D), **f32))
    run = lambda: kda.prefill_backward(pre["q"], pre["k"], pre["v"], pre["z"], pre["A"], pre["beta"],
                                       pre["cu_seqlens"], cot["dO"], h0=None, grad_hT=cot["dhT"], workspace=ws,
                                       grads=g)
    run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    per_pair = 4 * 2 * D + 4 * D + 4 + 4 * 4 * D + 4
    gbps = per_pair * T * H / (ms * 1e-3) / 1e9
    out = {"workload": "K3 shape T=65536 H=96 d=128 bf16, dO bf16, dhT fp32", "ms": round(ms, 3),
           "tokens_per_s": round(T / (ms * 1e-3), 1), "algorithmic_B_per_pair": per_pair,
           "algorithmic_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
           "workspace_GB": round(ws.numel() / 1e9, 2)}
    del ws, g, cot
    torch.cuda.empty_cache()
    return out


def feature_path_cost(kda, W, dev, pre, reps: int = 10) -> dict:
    """Side measurement at the K3 prefill shape (T=65536, H=96, d=128, bf16):
    the ShortConv -> Swish -> L2Norm feature path for q, k, v (with a carried
    window) and the Sigmoid(g) * RMSNorm(o) output gate, each alone; then the
    three separate calls (feature path, kda_prefill on its q, k, v, output
    gate) against kda_prefill_fused doing the same in one call.  Algorithmic
    bytes: three inputs read and three outputs written; o and g read and y
    written."""
    import torch
    f = W.random_features([65536], 96, 128, "bf16", window=True, device=dev)
    T, H, D = f["xq"].shape
    q, k, v = (torch.empty_like(f["xq"]) for _ in range(3))
    win_out = torch.empty_like(f["window"])
    y = torch.empty_like(f["o"])
    o = torch.empty_like(f["o"])
    hT = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = kda.prefill_workspace(1, T, H, D, kda.KDA_BF16, dev)
    wsf = torch.empty(kda.kda_prefill_fused_workspace_size(1, T, H, D, D, kda.KDA_BF16), dtype=torch.uint8,
                      device=dev)

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    qkv = lambda: kda.qkv_shortconv(f["xq"], f["xk"], f["xv"], f["wq"], f["wk"], f["wv"], f["cu_seqlens"],
                                    conv_state_in=f["window"], conv_state_out=win_out, q=q, k=k, v=v)
    gate = lambda: kda.output_gate(o, f["g"], f["w"], 1e-6, y=y)

    def separate():
        qkv()
        kda.prefill(q, k, v, pre["z"], pre["A"], pre["beta"], pre["cu_seqlens"], h0=None, o=o, hT=hT, workspace=ws)
        gate()

    def fused():
        kda.prefill_fused(f["xq"], f["xk"], f["xv"], f["wq"], f["wk"], f["wv"], pre["z"], pre["A"], pre["beta"],
                          pre["cu_seqlens"], f["g"], f["w"], 1e-6, conv_state_in=f["window"],
                          conv_state_out=win_out, y=y, hT=hT, workspace=wsf)

    ms_qkv = timed(qkv)
    ms_gate = timed(gate)
    ms_sep = timed(separate)
    ms_fused = timed(fused)
    row = T * H * D * 2
    del ws, wsf, f, q, k, v, o, y
    torch.cuda.empty_cache()
    return {"workload": "K3 shape T=65536 H=96 d=128 bf16",
            "qkv_shortconv": {"ms": round(ms_qkv, 4), "GBps": round(6 * row / (ms_qkv * 1e-3) / 1e9, 1)},
            "output_gate": {"ms": round(ms_gate, 4), "GBps": round(3 * row / (ms_gate * 1e-3) / 1e9, 1)},
            "separate_calls": {"ms": round(ms_sep, 4), "what": "kda_qkv_shortconv + kda_prefill + kda_output_gate"},
            "fused": {"ms": round(ms_fused, 4),
                      "what": "kda_prefill_fused (same inputs and outputs; pipelined here: a feature pass staging "
                              "q, k, v, then the intra kernel beside the gated output pass, o never stored)",
                      "tokens_per_s": round(T / (ms_fused * 1e-3), 1),
                      "saved_ms": round(ms_sep - ms_fused, 4)}}


def decode_fused_cost(kda, W, dev, reps: int = 100) -> dict:
    """Side measurement at the batched decode shape (256 sequences x 96 heads
    x 128, bf16, a carried window): one step as the three separate calls
    (feature path of the token, kda_decode, output gate) against
    kda_decode_fused, each repeated in place (state and window updated)."""
    import torch
    N, H, D = 256, 96, 128
    f = W.random_features([1] * N, H, D, "bf16", window=True, device=dev)
    dec = W.random_decode(N, H, D, "bf16", 0.05, device=dev)
    S = dec["S"]
    win = f["window"]
    cu = torch.arange(N + 1, dtype=torch.int32, device=dev)
    q, k, v = (torch.empty_like(f["xq"]) for _ in range(3))
    o = torch.empty_like(f["xq"])
    y = torch.empty_like(f["xq"])

    def separate():
        kda.qkv_shortconv(f["xq"], f["xk"], f["xv"], f["wq"], f["wk"], f["wv"], cu, conv_state_in=win,
                          conv_state_out=win, q=q, k=k, v=v)
        kda.decode(q, k, v, dec["z"], dec["A"], dec["beta"], S, o=o)
        kda.output_gate(o, f["g"], f["w"], 1e-6, y=y)

    def fused():
        kda.decode_fused(f["xq"], f["xk"], f["xv"], f["wq"], f["wk"], f["wv"], dec["z"], dec["A"], dec["beta"], S,
                         f["g"], f["w"], 1e-6, conv_state_in=win, conv_state_out=win, y=y)

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_sep = timed(separate)
    ms_fused = timed(fused)
    state_bytes = 2 * N * H * D * D * 4
    return {"workload": "k3_decode 256x96 d=128 bf16, window carried, state updated in place",
            "separate_calls": {"ms": round(ms_sep, 4), "what": "kda_qkv_shortconv + kda_decode + kda_output_gate"},
            "fused": {"ms": round(ms_fused, 4), "what": "kda_decode_fused",
                      "state_GBps": round(state_bytes / (ms_fused * 1e-3) / 1e9, 1),
                      "saved_ms": round(ms_sep - ms_fused, 4)}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU and shards nothing across GPUs; --gpus %d is not "
              "supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_21_amd as kda
    from gated_delta_rule_21_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pre = W.make("k3_prefill", device=dev)
    dec = W.make("k3_decode", device=dev)
    T, H, D = pre["q"].shape
    Nd = dec["q"].shape[0]
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = kda.prefill_workspace(1, T, H, D, kda.KDA_BF16, dev)
    S = dec["S"].clone()
    od = torch.empty((Nd, H, D), dtype=torch.bfloat16, device=dev)

    def prefill():
        kda.prefill(pre["q"], pre["k"], pre["v"], pre["z"], pre["A"], pre["beta"],
                    pre["cu_seqlens"], h0=None, o=o, hT=hT, workspace=ws)

    def decode():
        kda.decode(dec["q"], dec["k"], dec["v"], dec["z"], dec["A"], dec["beta"], S, o=od)

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        prefill()
        e[1].record()
        decode()
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    dec_ms_step = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    step_ms = wall * 1e3 / args.steps

    # decode state bandwidth over repeated in-place steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.decode_steps):
        decode()
    e1.record()
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / args.decode_steps

    if args.copy_probe_gib > 0:
        n = int(args.copy_probe_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    pairs = T * H
    traffic = measured_traffic()
    mfma_flops = counted_mfma_flops()
    pre_bytes = PREFILL_BYTES_PER_PAIR * pairs
    pre_gbps = pre_bytes / (pre_ms * 1e-3) / 1e9
    pre_tflops = PREFILL_FLOPS_PER_PAIR * pairs / (pre_ms * 1e-3) / 1e12
    dec_bytes = DECODE_BYTES_PER_PAIR * Nd * H
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9

    line = {
        "metric": METRIC,
        "value": round(T / (pre_ms * 1e-3), 1),
        "unit": "tokens/s",
        "value_is": "prefill tokens/s: %d tokens / the mean kda_prefill time (HIP events on the launch "
                    "stream) over the timed steps; decode is reported under 'decode'" % T,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit-norm bf16, v bf16, z and beta fp32)",
        "config": {"workload": "k3_prefill B=1 H=96 T=65536 d=128 bf16 + k3_decode 256x96 "
                               "fp32 128x128 state",
                   "global_batch": 1, "seq_len": T, "heads": H, "head_dim": D,
                   "decode_batch": Nd, "chunk": 64, "parallelism": "single GPU"},
        "prefill": {"ms": round(pre_ms, 4), "tokens_per_s": round(T / (pre_ms * 1e-3), 1),
                    "algorithmic_GBps": round(pre_gbps, 1),
                    "hbm_frac": round(pre_gbps / HBM_PEAK_GBPS, 4),
                    "useful_TFLOPs": round(pre_tflops, 2),
                    "mfma_useful_frac": round(pre_tflops / BF16_DENSE_PEAK_TFLOPS, 4),
                    "mfma_counted_frac": (None if mfma_flops is None else
                                          round(mfma_flops / (pre_ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 4)),
                    "mfma_counted_source": "profiles/kda_k3_prefill_counters.md: 16-bit MFMA MOPS x 512 per "
                                           "call (rocprofv3 --pmc) / this run's call time"},
        "decode": {"ms_per_step": round(dec_ms, 4), "steps": args.decode_steps,
                   "state_GBps": round(dec_gbps, 1), "hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "ms_in_step": round(dec_ms_step, 4)},
        "roofline": {"bound": "hbm", "achieved": round(pre_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(pre_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "kda_prefill (chunk table, then intra and inter kernels pipelined over three "
                               "chunk runs), 1540 algorithmic B per (token, head) x 6291456 pairs per call"},
    }
    if not args.no_features:
        line["feature_path"] = feature_path_cost(kda, W, dev, pre)
        line["decode_fused"] = decode_fused_cost(kda, W, dev)
    if not args.no_backward:
        line["prefill_backward"] = prefill_backward_cost(kda, W, pre)
    if not args.no_checkpoints:
        line["prefill_checkpoints"] = prefill_checkpoint_cost(kda, pre, o, hT, ws)
    if not args.no_varlen:
        line["varlen"] = varlen_prefill(kda, W, dev)
    if not args.no_small_head:
        line["small_head"] = small_head_prefill(kda, W, dev)
    if not args.no_decode_window:
        line["decode_window"] = decode_window_step(kda, W, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pre, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
