"""The entry points under HIP graph capture.

A serving-shaped sequence is captured once with torch.cuda.graph: a
segmented prefill of a ragged batch into caller-owned o, hT and workspace;
the same prefill through the chunk-block pipeline (a helper stream joined by
events); the fused prefill of the same batch, pipelined, its conv window
carried in place;
two decode steps on the prefill's final state, in place; one fused decode
step on that state with its conv window carried in place; and the prefill
without a workspace argument (its fixed device scratch).  The graph is
replayed several times, with other eager calls of the same entry points,
buffer scribbles and synchronisations between the replays.  Every replay
must equal the eager run of the same calls bit for bit: the kernels are
deterministic, and the library makes no allocation, host synchronisation or
memset on the capturing stream, and reads only what it is given."""
import threading

import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W

pytestmark = pytest.mark.gpu
EPS = 1e-6
LENS = [300, 1, 129, 0, 64]
H, D = 4, 128


def to(d, dev):
    return {n: (t.to(dev) if isinstance(t, torch.Tensor) else t) for n, t in d.items()}


def make_state(seed=8100, dev="cuda"):
    dev = torch.device(dev)
    p = to(W.random_prefill(LENS, H, D, "bf16", h0_std=0.05, seed=seed), dev)
    N = len(LENS)
    T = sum(LENS)
    dec = [to(W.random_decode(N, H, D, "bf16", 0.05, seed=seed + 10 + i), dev) for i in range(2)]
    f = to(W.random_features([1] * N, H, D, "bf16", window=True, seed=seed + 20), dev)
    fz = to(W.random_decode(N, H, D, "bf16", 0.05, seed=seed + 21), dev)
    ff = to(W.random_features(LENS, H, D, "bf16", window=True, seed=seed + 30), dev)
    bufs = dict(
        o=torch.empty((T, H, D), dtype=torch.bfloat16, device=dev),
        hT=torch.empty((N, H, D, D), dtype=torch.float32, device=dev),
        ws=torch.empty(kda.kda_prefill_ex_workspace_size(N, T, H, D, D, kda.KDA_BF16, kda.options(3)),
                       dtype=torch.uint8, device=dev),
        od=[torch.empty((N, H, D), dtype=torch.bfloat16, device=dev) for _ in range(2)],
        y=torch.empty((N, H, D), dtype=torch.bfloat16, device=dev),
        win=torch.empty_like(f["window"]),
        o2=torch.empty((T, H, D), dtype=torch.bfloat16, device=dev),
        hT2=torch.empty((N, H, D, D), dtype=torch.float32, device=dev),
        o3=torch.empty((T, H, D), dtype=torch.bfloat16, device=dev),
        hT3=torch.empty((N, H, D, D), dtype=torch.float32, device=dev),
        ws3=torch.empty(kda.kda_prefill_ex_workspace_size(N, T, H, D, D, kda.KDA_BF16, kda.options(blocks=3)),
                        dtype=torch.uint8, device=dev),
        ff=ff,
        fy=torch.empty((T, H, D), dtype=torch.bfloat16, device=dev),
        fhT=torch.empty((N, H, D, D), dtype=torch.float32, device=dev),
        fwin=torch.empty_like(ff["window"]),
        ws4=torch.empty(kda.kda_prefill_fused_workspace_size(N, T, H, D, D, kda.KDA_BF16, kda.options(blocks=3)),
                        dtype=torch.uint8, device=dev),
    )
    return p, dec, f, fz, bufs


def sequence(p, dec, f, fz, b):
    """The calls the graph holds, on the current stream."""
    b["win"].copy_(f["window"])
    kda.prefill(p["q"], p["k"], p["v"], p["z"], p["A"], p["beta"], p["cu_seqlens"], h0=p["h0"], o=b["o"],
                hT=b["hT"], workspace=b["ws"], segments=3)
    kda.prefill(p["q"], p["k"], p["v"], p["z"], p["A"], p["beta"], p["cu_seqlens"], h0=p["h0"], o=b["o3"],
                hT=b["hT3"], workspace=b["ws3"], blocks=3)
    ff = b["ff"]
    b["fwin"].copy_(ff["window"])
    kda.prefill_fused(ff["xq"], ff["xk"], ff["xv"], ff["wq"], ff["wk"], ff["wv"], p["z"], p["A"], p["beta"],
                      p["cu_seqlens"], ff["g"], ff["w"], EPS, h0=p["h0"], conv_state_in=b["fwin"],
                      conv_state_out=b["fwin"], y=b["fy"], hT=b["fhT"], workspace=b["ws4"], blocks=3)
    for i in range(2):
        kda.decode(dec[i]["q"], dec[i]["k"], dec[i]["v"], dec[i]["z"], p["A"], dec[i]["beta"], b["hT"],
                   o=b["od"][i])
    kda.decode_fused(f["xq"], f["xk"], f["xv"], f["wq"], f["wk"], f["wv"], fz["z"], p["A"], fz["beta"], b["hT"],
                     f["g"], f["w"], EPS, conv_state_in=b["win"], conv_state_out=b["win"], y=b["y"])
    N = len(LENS)
    st = kda.kda_prefill_noalloc(kda.KDA_BF16, p["q"].data_ptr(), p["k"].data_ptr(), p["v"].data_ptr(),
                                 p["z"].data_ptr(), p["A"].data_ptr(), p["beta"].data_ptr(), p["h0"].data_ptr(),
                                 p["cu_seqlens"].data_ptr(), N, sum(LENS), H, D, D, b["o2"].data_ptr(),
                                 b["hT2"].data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, kda.kda_status_string(st)


OUTS = ("o", "hT", "od0", "od1", "y", "win", "o2", "hT2", "o3", "hT3", "fy", "fhT", "fwin")


def outputs(b):
    return [b["od"][0] if n == "od0" else b["od"][1] if n == "od1" else b[n] for n in OUTS]


def snapshot(b):
    return [t.clone() for t in outputs(b)]


def scribble(b):
    for t in outputs(b):
        t.fill_(-7.0)


def test_capture_and_replay():
    print("case graph capture: prefill (3 segments), pipelined prefill, pipelined fused prefill, 2 decode steps, "
          "fused decode, noalloc prefill", flush=True)
    p, dec, f, fz, b = make_state()
    sequence(p, dec, f, fz, b)            # eager, also the warm-up before capture
    torch.cuda.synchronize()
    want = snapshot(b)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sequence(p, dec, f, fz, b)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # a second batch through the same entry points (the noalloc scratch
    # included), run eagerly between replays on other buffers
    p2, dec2, f2, fz2, b2 = make_state(seed=8200)
    for rep in range(4):
        scribble(b)
        torch.cuda.synchronize()
        g.replay()
        if rep % 2 == 0:
            sequence(p2, dec2, f2, fz2, b2)   # eager work between replays
        torch.cuda.synchronize()
        got = snapshot(b)
        for n, x, y in zip(OUTS, got, want):
            assert torch.equal(x, y), "replay %d: %s differs from the eager run" % (rep, n)
    g.reset()


def test_first_pipelined_call_under_capture():
    """A thread whose first pipelined call is made under graph capture: the
    thread's helper stream and events are created during the capture, and the
    replays equal the eager call bit for bit."""
    print("case first pipelined call of a thread under capture", flush=True)
    p = to(W.random_prefill(LENS, H, D, "bf16", h0_std=0.05, seed=8300), "cuda")
    N, T = len(LENS), sum(LENS)
    o_want, h_want = kda.prefill(p["q"], p["k"], p["v"], p["z"], p["A"], p["beta"], p["cu_seqlens"], h0=p["h0"],
                                 blocks=3)
    torch.cuda.synchronize()
    ws = torch.empty(kda.kda_prefill_ex_workspace_size(N, T, H, D, D, kda.KDA_BF16, kda.options(blocks=3)),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(o_want)
    hT = torch.empty_like(h_want)
    result = {}

    def body():
        try:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    kda.prefill(p["q"], p["k"], p["v"], p["z"], p["A"], p["beta"], p["cu_seqlens"], h0=p["h0"],
                                o=o, hT=hT, workspace=ws, blocks=3)
            torch.cuda.synchronize()
            for _ in range(3):
                o.fill_(-7.0)
                hT.fill_(-7.0)
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                result.setdefault("equal", []).append(torch.equal(o, o_want) and torch.equal(hT, h_want))
            g.reset()
        except Exception as e:           # reported by the main thread
            result["error"] = repr(e)

    t = threading.Thread(target=body)
    t.start()
    t.join(timeout=120)
    assert not t.is_alive()
    assert "error" not in result, result.get("error")
    assert result["equal"] == [True, True, True]
