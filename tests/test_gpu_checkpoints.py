"""Prefill with state checkpoints every `interval` tokens: HIP kernels vs the
fp64 oracle.  The expected checkpoint j of sequence n is the oracle's final
state over the sequence's first (j + 1) * interval tokens (from its h0)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
import oracle
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_prefill, compare_states, host, oracle_prefill, to_gpu

pytestmark = pytest.mark.gpu


def oracle_checkpoints(d, interval, heads=None, only=None):
    """Expected checkpoints [count, H', dv, dk] in the library's order
    (sequence-major, token order); `only` restricts to some indices."""
    cu = d["cu_seqlens"].cpu().tolist()
    pieces, h0s, idx = [], [], 0
    for n in range(len(cu) - 1):
        for j in range((cu[n + 1] - cu[n]) // interval):
            if only is None or idx in only:
                pieces.append((cu[n], cu[n] + (j + 1) * interval, n))
            idx += 1
    if not pieces:
        return np.zeros((0,)), idx
    sel = lambda t: t if heads is None else t[:, heads]
    cat = lambda name: torch.cat([sel(d[name][a:b].cpu()) for a, b, _ in pieces], 0)
    h0 = None
    if d.get("h0") is not None:
        h0 = torch.stack([sel(d["h0"].cpu())[n] for _, _, n in pieces])
    A = d["A"].cpu() if heads is None else d["A"].cpu()[heads]
    lens = [b - a for a, b, _ in pieces]
    _, hT = oracle.prefill(W.as_numpy(cat("q")), W.as_numpy(cat("k")), W.as_numpy(cat("v")), W.as_numpy(cat("z")),
                           W.as_numpy(A), W.as_numpy(cat("beta")), None if h0 is None else W.as_numpy(h0),
                           W.as_numpy(W.cu_from_lengths(lens)))
    return hT, idx


def run(g, interval, segments=0):
    T, H, d = g["q"].shape
    ck = torch.full((T // interval, H, d, d), 7.0, dtype=torch.float32, device="cuda")   # sentinel
    o, hT, ck, off = kda.prefill_checkpoints(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"],
                                             g["cu_seqlens"], interval, h0=g["h0"], checkpoints=ck,
                                             segments=segments)
    torch.cuda.synchronize()
    return o, hT, ck, off


@pytest.mark.parametrize("io,d,interval,segments", [("bf16", 128, 512, 0), ("bf16", 64, 128, 3),
                                                    ("f32", 32, 64, 0), ("f32", 128, 256, 5)])
def test_checkpoints_ragged(io, d, interval, segments):
    """Lengths that are multiples of the interval, one token short of it,
    empty, and below it; forced segments split sequences between checkpoints."""
    lens = [1600, 0, 512, 511, 1100, 64, 1024]
    inp = W.random_prefill(lens, 3, d, io, h0_std=0.05, seed=700 + d + interval)
    g = to_gpu(inp)
    o, hT, ck, off = run(g, interval, segments)
    exp, count = oracle_checkpoints(inp, interval)
    offsets = np.cumsum([0] + [n // interval for n in lens])
    assert off.cpu().tolist() == offsets.tolist()
    m = compare_states(host(ck[:count]), exp, io, what="checkpoints")
    print("checkpoints %s d=%d interval=%d segments=%d: %d, %s" % (io, d, interval, segments, count, m),
          flush=True)
    ro, rh = oracle_prefill(inp)
    compare_prefill(o, hT, ro, rh, inp["cu_seqlens"], io, label="checkpoint run outputs")
    assert bool((ck[count:] == 7.0).all()), "entries past the total must stay untouched"
    # outputs and final states: the same as without checkpoints, bit for bit
    o2, h2 = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"], h0=g["h0"],
                         segments=segments)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(hT, h2)


def test_checkpoint_at_sequence_end_equals_hT():
    inp = W.random_prefill([1024, 1536], 2, 128, "bf16", h0_std=0.05, seed=710)
    g = to_gpu(inp)
    o, hT, ck, off = run(g, 512)
    assert off.cpu().tolist() == [0, 2, 5]
    assert torch.equal(ck[1], hT[0]) and torch.equal(ck[4], hT[1])


def test_checkpoints_without_h0_and_offsets_only():
    inp = W.random_prefill([700, 300], 2, 64, "bf16", h0_std=None, seed=711)
    g = to_gpu(inp)
    off = torch.full((3,), -1, dtype=torch.int32, device="cuda")
    ws = kda.prefill_workspace(2, 1000, 2, 64, kda.KDA_BF16, "cuda")
    st = kda.kda_prefill_ex(kda.KDA_BF16, g["q"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(),
                            g["z"].data_ptr(), g["A"].data_ptr(), g["beta"].data_ptr(), None,
                            g["cu_seqlens"].data_ptr(), 2, 1000, 2, 64, 64,
                            torch.empty((1000, 2, 64), dtype=torch.bfloat16, device="cuda").data_ptr(),
                            None, kda.options(0, 256, None, off.data_ptr()), ws.data_ptr(), ws.numel(),
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0 and off.cpu().tolist() == [0, 2, 3]
    o, hT, ck, off2 = run(dict(g, h0=None), 256)
    exp, count = oracle_checkpoints(dict(inp, h0=None), 256)
    assert count == 3
    compare_states(host(ck[:3]), exp, "bf16", what="checkpoints")


def test_k3_prefill_checkpoints_sampled():
    """The K3 prefill (H=96, T=65536) with a checkpoint every 4096 tokens:
    checkpoints 0, 7 and 15 on two heads against the oracle."""
    d = W.make("k3_prefill", device="cuda")
    o, hT, ck, off = run(d, 4096)
    assert off.cpu().tolist() == [0, 16]
    heads = [5, 77]
    exp, count = oracle_checkpoints(d, 4096, heads=heads, only={0, 7, 15})
    got = host(ck[[0, 7, 15]][:, heads])
    m = compare_states(got, exp, "bf16", what="k3 checkpoints")
    print("k3 checkpoints %s" % m, flush=True)
    assert torch.equal(ck[15], hT[0])
