"""Segmented prefill (intra-device context parallelism): sequences cut into
segments whose affine state maps (M, S~) are composed from h0, then every
segment runs its outputs from its own incoming state.  Forced segment
counts through the C ABI, checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_outputs, compare_prefill, host, oracle_prefill, to_gpu

pytestmark = pytest.mark.gpu


def run(g, segments, h0="same", hT=None):
    o, hT_ = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"],
                         h0=g["h0"] if h0 == "same" else h0, hT=hT, segments=segments)
    torch.cuda.synchronize()
    return o, hT_


def test_segment_count_query():
    assert kda.kda_prefill_segments(1, 65536, 96, 128, 128, kda.KDA_BF16) == 1
    assert kda.kda_prefill_segments(2, 16384, 8, 128, 128, kda.KDA_BF16) > 1


@pytest.mark.parametrize("P", [2, 3, 5, 16])
@pytest.mark.parametrize("io,d", [("bf16", 128), ("bf16", 64), ("f32", 32), ("f32", 128)])
def test_forced_segments_ragged(io, d, P):
    """Long, short, one-chunk, one-token and empty sequences; with P = 16 the
    short ones get one segment per chunk."""
    lens = [1000, 0, 64, 1, 450, 77, 640]
    inp = W.random_prefill(lens, 3, d, io, h0_std=0.05, seed=500 + d + P)
    print("case segments P=%d %s d=%d" % (P, io, d), flush=True)
    g = to_gpu(inp)
    o, hT = run(g, P)
    ro, rh = oracle_prefill(inp)
    compare_prefill(o, hT, ro, rh, inp["cu_seqlens"], io, label="segments P=%d %s d=%d" % (P, io, d))


@pytest.mark.parametrize("z_shift", [-4.0, 6.0])
def test_forced_segments_decay_extremes(z_shift):
    """Weak decay (M close to a product of near-identity maps) and saturated decay."""
    inp = W.random_prefill([1500, 700], 4, 128, "bf16", h0_std=0.05, seed=61, z_shift=z_shift)
    g = to_gpu(inp)
    o, hT = run(g, 6)
    ro, rh = oracle_prefill(inp)
    compare_prefill(o, hT, ro, rh, inp["cu_seqlens"], "bf16", label="segments z_shift %g" % z_shift)


def test_segments_hT_may_alias_h0():
    inp = W.random_prefill([900, 300], 2, 128, "bf16", h0_std=0.1, seed=62)
    g = to_gpu(inp)
    o_ref, hT_ref = run(g, 4, hT=torch.empty_like(g["h0"]))
    S = g["h0"].clone()
    o, _ = run(g, 4, h0=S, hT=S)
    assert torch.equal(o, o_ref) and torch.equal(S, hT_ref)


def test_segments_without_h0():
    inp = W.random_prefill([800, 500], 2, 64, "bf16", h0_std=None, seed=63)
    g = to_gpu(inp)
    o, hT = run(g, 3, h0=None)
    ro, rh = oracle_prefill(inp)
    compare_prefill(o, hT, ro, rh, inp["cu_seqlens"], "bf16", label="segments without h0")


def test_segments_constant_state_exact():
    """alpha = 1 and beta = 0: every transition is exactly (I, 0), so the
    composed incoming states and hT equal h0 bit for bit."""
    inp = W.random_prefill([700, 260], 2, 128, "bf16", h0_std=0.3, seed=64)
    inp["z"][:] = -1e30
    inp["beta"][:] = 0.0
    g = to_gpu(inp)
    o, hT = run(g, 5)
    assert torch.equal(hT.cpu(), inp["h0"])
    ro, _ = oracle_prefill(inp)
    compare_outputs(host(o), ro, "bf16", inp["cu_seqlens"].tolist())


def test_segments_deterministic():
    inp = W.random_prefill([1200, 64], 3, 128, "bf16", h0_std=0.05, seed=65)
    g = to_gpu(inp)
    o1, h1 = run(g, 4)
    o2, h2 = run(g, 4)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_small_head_workload_split_and_unsplit():
    """B=2, H=8, T=8192 each, d=128: the automatic choice splits this
    workload; both it and the unsplit pass match the oracle on every output."""
    d = W.make("small_head")
    g = to_gpu(d)
    assert kda.kda_prefill_segments(2, 16384, 8, 128, 128, kda.KDA_BF16) > 1
    ro, rh = oracle_prefill(d, nthreads=0)
    for P in (0, 1):
        o, hT = run(g, P)
        compare_prefill(o, hT, ro, rh, d["cu_seqlens"], "bf16", label="small_head segments=%s" % (P or "auto"))
