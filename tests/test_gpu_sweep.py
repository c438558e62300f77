"""A seeded sweep of prefill shapes against the fp64 oracle: io dtype, head
dimension, head count, batch, length mix (empty, one token, exact and
off-by-one chunk multiples, longer), decay strength and segment count
drawn together, so
that combinations no hand-written case names are covered.  Every case is
compared by every measure of gpu_util."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_prefill, oracle_prefill, to_gpu

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 200, 333, 640]


def draw(seed):
    r = np.random.default_rng(seed)
    io = ["bf16", "f32"][r.integers(2)]
    d = [32, 64, 128][r.integers(3)]
    H = int(r.integers(1, 5))
    N = int(r.integers(1, 6))
    lens = [int(x) for x in r.choice(LENGTHS, size=N)]
    if sum(lens) == 0:
        lens[0] = 77
    h0 = None if r.integers(3) == 0 else 0.05
    P = [0, 1, 2, 3, 7][r.integers(5)]
    zs = [-4.0, 0.0, 0.0, 6.0][r.integers(4)]
    return io, d, H, lens, h0, P, zs


@pytest.mark.parametrize("seed", range(16))
def test_prefill_sweep(seed):
    io, d, H, lens, h0, P, zs = draw(7000 + seed)
    label = "sweep %d: %s d=%d H=%d lens=%s h0=%s segments=%d z_shift=%g" % (seed, io, d, H, lens, h0, P, zs)
    print(label, flush=True)
    inp = W.random_prefill(lens, H, d, io, h0_std=h0, seed=7100 + seed, z_shift=zs)
    g = to_gpu(inp)
    o, hT = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"], h0=g["h0"],
                        segments=P)
    torch.cuda.synchronize()
    ro, rh = oracle_prefill(inp)
    compare_prefill(o, hT, ro, rh, inp["cu_seqlens"], io, label=label)
