"""Prefill backward: HIP kernels vs the fp64 oracle's reverse sweep
(kda_oracle_backward), gradient by gradient, by relative L2.

The oracle gets the very values the GPU reads (bf16 inputs as their exact
values, dO in the io dtype).  Arithmetic after the forward recompute is fp32
on the GPU; for bf16 inputs the recomputed forward states carry the bf16
path's own error, so the bf16 bar is the forward's 2e-3."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
import oracle
from gated_delta_rule_21_amd import workloads as W
from gpu_util import BF16_TOL, host, rel_l2, to_gpu

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dz", "dbeta", "dA", "dh0")
F32_BWD_TOL = 1e-5


def oracle_grads(inp, cot, heads=None):
    sel = lambda t: t if heads is None else t[:, heads]
    q, k, v, z, beta = (W.as_numpy(sel(inp[n])) for n in ("q", "k", "v", "z", "beta"))
    A = W.as_numpy(inp["A"] if heads is None else inp["A"][heads])
    h0 = None if inp.get("h0") is None else W.as_numpy(sel(inp["h0"]))
    dO = host(sel(cot["dO"]))
    dhT = None if cot.get("dhT") is None else host(sel(cot["dhT"]))
    cu = W.as_numpy(inp["cu_seqlens"]).astype(np.int32)
    return oracle.backward(q, k, v, z, A, beta, h0, cu, dO, dhT)


def gpu_grads(g, gc, segments=0):
    out = kda.prefill_backward(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"], gc["dO"],
                               h0=g["h0"], grad_hT=gc["dhT"], segments=segments)
    torch.cuda.synchronize()
    return out


def check(got, exp, bar, heads=None):
    errs = {}
    for name in NAMES:
        x = host(got[name])
        if heads is not None:
            x = x[heads] if name == "dA" else x[:, heads]
        errs[name] = rel_l2(x, exp[name])
    print({k: "%.2e" % v for k, v in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= bar, (name, e, bar)


CASES = [
    # io, d, H, lengths, h0, dhT, segments
    ("f32", 32, 2, [256], False, True, 0),
    ("f32", 64, 3, [130, 0, 64, 1, 200], True, True, 0),
    ("f32", 128, 2, [100, 300], True, False, 0),
    ("bf16", 128, 3, [300, 64, 17, 0, 129], True, True, 0),
    ("bf16", 32, 2, [1000, 63], True, True, 3),
    ("bf16", 64, 2, [777], False, True, 0),
    # more (chunk, head) items than CUs, over several sequences: the persistent
    # local and grad kernels carry the next item's inputs across sequence ends
    ("bf16", 32, 2, [3000, 5000, 100, 0, 4100], True, True, 0),
    ("f32", 32, 2, [4100, 0, 3000, 5000, 100], True, True, 0),
]


@pytest.mark.parametrize("io,d,H,lens,h0,dhT,segments", CASES)
def test_backward_ragged(io, d, H, lens, h0, dhT, segments):
    print("backward", io, d, H, lens, h0, dhT, segments, flush=True)
    inp = W.random_prefill(lens, H, d, io, h0_std=0.1 if h0 else None, seed=900 + d + len(lens))
    cot = W.random_cotangents(sum(lens), len(lens), H, d, io, final_state=dhT, seed=950 + d)
    got = gpu_grads(to_gpu(inp), to_gpu(cot), segments)
    check(got, oracle_grads(inp, cot), F32_BWD_TOL if io == "f32" else BF16_TOL)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("z_shift,beta_zero", [(-30.0, True), (-30.0, False), (8.0, False)])
def test_backward_degenerate_gates(z_shift, beta_zero, io):
    """No decay and no write (constant state), no decay (the DeltaNet rule),
    and the strongest decay the gate allows (alpha -> e^-5), on both paths."""
    print("backward gates", z_shift, beta_zero, io, flush=True)
    inp = W.random_prefill([200, 70], 2, 64, io, h0_std=0.3, seed=990, z_shift=z_shift)
    if beta_zero:
        inp["beta"].zero_()
    cot = W.random_cotangents(270, 2, 2, 64, io, seed=991)
    got = gpu_grads(to_gpu(inp), to_gpu(cot))
    check(got, oracle_grads(inp, cot), F32_BWD_TOL if io == "f32" else BF16_TOL)


def test_backward_repeatable():
    """Two calls give the same bits (no atomics; fixed-order reductions)."""
    inp = W.random_prefill([500, 90], 2, 128, "bf16", h0_std=0.05, seed=995)
    cot = W.random_cotangents(590, 2, 2, 128, "bf16", seed=996)
    g, gc = to_gpu(inp), to_gpu(cot)
    a = gpu_grads(g, gc)
    b = gpu_grads(g, gc)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name


def test_backward_k3_sampled_heads():
    """The K3 prefill shape (H = 96, T = 65536, d = 128, bf16) on the GPU;
    the oracle on two of the heads (heads are independent)."""
    print("backward K3", flush=True)
    inp = W.make("k3_prefill")
    T, H = inp["q"].shape[0], inp["q"].shape[1]
    cot = W.random_cotangents(T, inp["N"], H, 128, "bf16", seed=997)
    got = gpu_grads(to_gpu(inp), to_gpu(cot))
    heads = [5, 77]
    check(got, oracle_grads(inp, cot, heads), BF16_TOL, heads)


@pytest.mark.parametrize("lens", [[0, 0], []])
def test_backward_empty(lens):
    """No tokens: dh0 = dhT, dA = 0 (and nothing else to write); no sequences at all."""
    print("backward empty", lens, flush=True)
    H, d = 2, 32
    inp = W.random_prefill(lens, H, d, "f32", h0_std=0.1, seed=998)
    cot = W.random_cotangents(0, len(lens), H, d, "f32", seed=999)
    got = gpu_grads(to_gpu(inp), to_gpu(cot))
    assert torch.equal(got["dh0"].cpu(), cot["dhT"])
    assert torch.equal(got["dA"].cpu(), torch.zeros(H))
