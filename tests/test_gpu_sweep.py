"""Seeded sweeps against the fp64 oracle, so that combinations no
hand-written case names are covered.  Prefill: io dtype, head dimension,
head count, batch, length mix (empty, one token, exact and off-by-one chunk
multiples, longer), decay strength and segment count drawn together, each
case compared by every measure of gpu_util.  Decode and speculative decode
windows: batch, heads, head size, dtype, decay strength, state scale, and
replay / window lengths with accepted counts drawn per sequence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
import oracle
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_outputs, compare_prefill, oracle_prefill, to_gpu

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


def draw_window(seed):
    r = np.random.default_rng(seed)
    io = ["bf16", "f32"][r.integers(2)]
    d = [32, 64, 128][r.integers(3)]
    H = int(r.integers(1, 5))
    N = int(r.integers(1, 9))
    Lr = int(r.choice([0, 1, 2, 4, 7, 16]))
    L = int(r.choice([0, 1, 3, 5, 16]))
    if Lr == 0 and L == 0:
        L = 2
    commit = bool(r.integers(2))
    state_std = float(r.choice([0.0, 0.05, 0.5]))
    return io, d, H, N, Lr, L, commit, state_std


@pytest.mark.parametrize("seed", range(12))
def test_decode_window_sweep(seed):
    """Speculative decoding: replay length, accepted counts (drawn per
    sequence, the ends included), window length, commit, state scale."""
    import test_gpu_decode_window as TW
    io, d, H, N, Lr, L, commit, std = draw_window(7300 + seed)
    label = "window sweep %d: %s d=%d H=%d N=%d Lr=%d L=%d commit=%s S std %g" % (seed, io, d, H, N, Lr, L,
                                                                                  commit, std)
    print(label, flush=True)
    inp = W.random_decode_window(N, H, d, Lr=Lr, L=L, io=io, state_std=std, seed=7400 + seed)
    if Lr > 0:
        r = np.random.default_rng(7500 + seed)
        acc = r.integers(0, Lr + 1, size=N)
        acc[0], acc[-1] = Lr, 0
        inp["n_accept"] = torch.tensor(acc, dtype=torch.int32)
    TW.check(inp, io, commit_window=commit, label=label)


@pytest.mark.parametrize("seed", range(8))
def test_decode_sweep(seed):
    """Single-token decode over random batch, heads, head size, dtype, decay
    strength and state scale."""
    r = np.random.default_rng(7600 + seed)
    io = ["bf16", "f32"][r.integers(2)]
    d = [32, 64, 128][r.integers(3)]
    H, N = int(r.integers(1, 7)), int(r.integers(1, 40))
    zs = float(r.choice([-4.0, 0.0, 6.0]))
    std = float(r.choice([0.0, 0.05, 0.5]))
    label = "decode sweep %d: %s d=%d H=%d N=%d z_shift=%g S std %g" % (seed, io, d, H, N, zs, std)
    print(label, flush=True)
    inp = W.random_decode(N, H, d, io, std, seed=7700 + seed, z_shift=zs)
    g = to_gpu(inp)
    S = g["S"].clone()
    o = kda.decode(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], S)
    torch.cuda.synchronize()
    ro, rS = oracle.decode(*(W.as_numpy(inp[n]) for n in ("q", "k", "v", "z", "A", "beta")), W.as_numpy(inp["S"]))
    compare_outputs(o.cpu().float().numpy().astype(np.float64), ro, io, label=label)
    from gpu_util import rel_l2
    e = rel_l2(S.cpu().numpy(), rS)
    assert e <= 1e-6, (label, e)
