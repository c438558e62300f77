"""Decode step: HIP kernel vs the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
import oracle
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_outputs, host, rel_l2, to_gpu, tol

pytestmark = pytest.mark.gpu


def _run(d):
    g = to_gpu(d)
    S = g["S"].clone()
    o = kda.decode(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], S)
    torch.cuda.synchronize()
    ro, rS = oracle.decode(*(W.as_numpy(d[n]) for n in ("q", "k", "v", "z", "A", "beta")),
                           W.as_numpy(d["S"]))
    return host(o), host(S), ro, rS


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_small(io, d):
    print("decode", io, d, flush=True)
    inp = W.random_decode(5, 3, d, io, 0.05, seed=77 + d)
    o, S, ro, rS = _run(inp)
    compare_outputs(o, ro, io)
    assert rel_l2(S, rS) <= 1e-6, rel_l2(S, rS)


def test_decode_empty_batch():
    """N = 0: accepted, nothing launched."""
    inp = W.random_decode(0, 3, 64, "bf16", 0.05, seed=5)
    o, S, ro, rS = _run(inp)
    assert o.shape[0] == 0 and S.shape[0] == 0 and ro.shape[0] == 0


def test_decode_k3_full_shape():
    """256 sequences x 96 heads x 128 x 128, the batched decode workload."""
    inp = W.make("k3_decode")
    o, S, ro, rS = _run(inp)
    m = compare_outputs(o, ro, "bf16")
    e_s = rel_l2(S, rS)
    print("k3_decode o %s S=%.3e" % (m, e_s), flush=True)
    assert e_s <= 1e-6


@pytest.mark.parametrize("z_shift", [-4.0, 6.0])
def test_decode_stress_decay(z_shift):
    inp = W.random_decode(8, 4, 128, "bf16", 0.05, seed=91, z_shift=z_shift)
    o, S, ro, rS = _run(inp)
    compare_outputs(o, ro, "bf16")
    assert rel_l2(S, rS) <= 1e-6


def test_decode_alpha_one_beta_zero_keeps_state():
    inp = W.random_decode(4, 2, 64, "bf16", 0.5, seed=5)
    inp["z"][:] = -1e30
    inp["beta"][:] = 0
    g = to_gpu(inp)
    S = g["S"].clone()
    kda.decode(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], S)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), inp["S"])
