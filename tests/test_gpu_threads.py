"""Several host threads calling the library at once.

The entry points keep no state between calls (the workspace size is a pure
function of the arguments), so threads may size workspaces and launch
prefills and decode steps concurrently, each on its own stream with its own
buffers; a pipelined prefill uses the calling thread's own helper stream.
Five threads each run a different mix of calls (segmented, pipelined and
plain prefills, fp32 and bf16, decode steps on the prefill's state, a
pipelined fused prefill with its conv window carried in place) on streams of
the default priority, all at the same time; every result must equal the same
calls run one after the other on one stream, bit for bit."""
import threading

import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    # (lens, H, d, io, segments, blocks)
    ([700, 3, 129], 4, 128, "bf16", 3, 0),
    ([64, 0, 333], 3, 64, "f32", 1, 0),
    ([1500, 900], 2, 128, "bf16", 0, 3),
    ([17, 200, 65, 1], 5, 32, "bf16", 2, 0),
    ([1400, 0, 650], 3, 128, "fused", 0, 3),
]


def to(d, dev):
    return {n: (t.to(dev) if isinstance(t, torch.Tensor) else t) for n, t in d.items()}


def prepare(i):
    lens, H, d, io, P, B = CASES[i]
    dev = torch.device("cuda")
    p = to(W.random_prefill(lens, H, d, "bf16" if io == "fused" else io, h0_std=0.05, seed=8300 + i), dev)
    if io == "fused":
        p["f"] = to(W.random_features(lens, H, d, "bf16", window=True, seed=8350 + i), dev)
        return p, None, P, B
    dec = to(W.random_decode(len(lens), H, d, io, 0.05, seed=8400 + i), dev)
    return p, dec, P, B


def work_fused(p, P, B, reps=3):
    """The fused prefill with its window carried in place, repeated."""
    f = p["f"]
    win = f["window"].clone()
    outs = []
    for _ in range(reps):
        y, hT = kda.prefill_fused(f["xq"], f["xk"], f["xv"], f["wq"], f["wk"], f["wv"], p["z"], p["A"], p["beta"],
                                  p["cu_seqlens"], f["g"], f["w"], 1e-6, h0=p["h0"], conv_state_in=win,
                                  conv_state_out=win, segments=P, blocks=B)
        outs += [y, hT, win.clone()]
    return outs


def work(p, dec, P, B, reps=3):
    """Prefill into fresh buffers, then a decode step on its final state;
    repeated, returning every output."""
    if dec is None:
        return work_fused(p, P, B, reps)
    outs = []
    N = p["cu_seqlens"].numel() - 1
    T, H, d = p["q"].shape
    n = kda.kda_prefill_ex_workspace_size(N, T, H, d, d, kda._io_code(p["q"]), kda.options(P, blocks=B))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(reps):
        o, hT = kda.prefill(p["q"], p["k"], p["v"], p["z"], p["A"], p["beta"], p["cu_seqlens"], h0=p["h0"],
                            workspace=ws, segments=P, blocks=B)
        od = kda.decode(dec["q"], dec["k"], dec["v"], dec["z"], p["A"], dec["beta"], hT)
        outs += [o, hT, od]
    return outs


def test_concurrent_threads_match_serial():
    print("case five threads, one stream each", flush=True)
    inputs = [prepare(i) for i in range(len(CASES))]
    torch.cuda.synchronize()
    want = [work(*x) for x in inputs]
    torch.cuda.synchronize()

    got = [None] * len(CASES)
    errors = []
    start = threading.Barrier(len(CASES))

    def run(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            start.wait()
            with torch.cuda.stream(s):
                got[i] = work(*inputs[i])
            s.synchronize()
        except Exception as e:      # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(len(CASES)):
        for j, (x, y) in enumerate(zip(got[i], want[i])):
            assert torch.equal(x, y), "thread %d, output %d differs from the serial run" % (i, j)
