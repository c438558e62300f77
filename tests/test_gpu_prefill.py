"""Chunkwise prefill: HIP kernels vs the fp64 oracle (through the C ABI).

Small cases run the oracle on every output; the K3-sized workloads run the
GPU on the full batch and the oracle on sampled heads (sliced inputs)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W
from gpu_util import (BF16_TOL, F32_TOL, compare_outputs, compare_prefill, host, oracle_prefill, rel_l2,
                      to_gpu)

pytestmark = pytest.mark.gpu


def gpu_prefill(g, h0="same", hT=True):
    h0t = g["h0"] if h0 == "same" else h0
    o, hT_ = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"],
                         h0=h0t, final_state=hT)
    torch.cuda.synchronize()
    return o, hT_


def check(d, io, heads=None, label=""):
    """GPU prefill against the oracle by every measure of gpu_util: whole
    tensor, per (sequence, head), compute-only and element-wise."""
    print("case", label, flush=True)
    g = to_gpu(d)
    o, hT = gpu_prefill(g)
    ro, rh = oracle_prefill(d, heads=heads)
    if heads is not None:
        o, hT = o[:, heads], hT[:, heads]
    return compare_prefill(o, hT, ro, rh, d["cu_seqlens"], io, label=label)


def test_tiny_f32_workload():
    """B=1, H=2, T=256, d=32, all fp32, h0 = 0."""
    check(W.make("tiny_f32"), "f32", label="tiny_f32")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_ragged_varlen(io, d):
    """Several chunks, partial last chunks, a one-token and an empty sequence."""
    lens = [200, 0, 64, 1, 130, 77]
    inp = W.random_prefill(lens, 3, d, io, h0_std=0.05, seed=300 + d)
    check(inp, io, label="ragged %s d=%d" % (io, d))


@pytest.mark.parametrize("z_shift", [-4.0, 6.0])
def test_stress_decay(z_shift):
    """Weak decay (mean g about -0.09) and saturated decay."""
    inp = W.random_prefill([300, 129], 4, 128, "bf16", h0_std=0.05, seed=41, z_shift=z_shift)
    check(inp, "bf16", label="z_shift %g" % z_shift)


@pytest.mark.parametrize("io,d", [("bf16", 128), ("bf16", 32), ("f32", 64), ("f32", 128)])
def test_deltanet_ragged(io, d):
    """alpha = 1 exactly (z = -1e30: the sigmoid underflows to 0, g = 0) with
    random beta: KDA reduces to the delta rule; ragged lengths."""
    inp = W.random_prefill([200, 0, 64, 1, 130, 77], 3, d, io, h0_std=0.05, seed=320 + d)
    inp["z"][:] = -1e30
    check(inp, io, label="deltanet %s d=%d" % (io, d))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decay_floor_attained(io):
    """z = +1e30: the sigmoid is exactly 1, so g = -5 on every token and
    channel and every 16-token window sums to exactly -80, the pages' bound
    attained (devpress K3 walk-through §3.2, Eq 5): the largest in-block
    decay factor, e^80, is reached on every diagonal block."""
    inp = W.random_prefill([300, 129, 64], 4, 128, io, h0_std=0.05, seed=330)
    inp["z"][:] = 1e30
    check(inp, io, label="decay floor %s" % io)


def test_no_h0_no_hT():
    inp = W.random_prefill([150, 90], 2, 64, "bf16", h0_std=None, seed=8)
    g = to_gpu(inp)
    o, hT = gpu_prefill(g, h0=None, hT=False)
    assert hT is None
    ro, _ = oracle_prefill(inp)
    compare_outputs(host(o), ro, "bf16", inp["cu_seqlens"].tolist())


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 128])
def test_empty_sequences_and_batch(io, d):
    """No tokens: every sequence empty leaves its state as it came in (hT
    equals h0 bit for bit, or zero without h0), and an empty batch (N = 0,
    T = 0) is accepted and does nothing."""
    print("empty", io, d, flush=True)
    for lens, h0_std in (([0, 0, 0], 0.05), ([0, 0], None), ([], None)):
        inp = W.random_prefill(lens, 2, d, io, h0_std=h0_std, seed=12)
        g = to_gpu(inp)
        o, hT = gpu_prefill(g)
        assert o.shape == (0, 2, d) and hT.shape == (len(lens), 2, d, d)
        want = g["h0"] if h0_std is not None else torch.zeros_like(hT)
        assert torch.equal(hT, want), lens
        _, rh = oracle_prefill(inp)
        assert np.array_equal(host(hT), rh), lens


def test_hT_may_alias_h0():
    inp = W.random_prefill([100, 70], 2, 128, "bf16", h0_std=0.1, seed=9)
    g = to_gpu(inp)
    o_ref, hT_ref = gpu_prefill(g)
    S = g["h0"].clone()
    o, _ = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"], h0=S, hT=S)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, hT_ref)


def test_deterministic():
    inp = W.random_prefill([333, 64], 3, 128, "bf16", h0_std=0.05, seed=10)
    g = to_gpu(inp)
    o1, h1 = gpu_prefill(g)
    o2, h2 = gpu_prefill(g)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_alpha_one_beta_zero_constant_state():
    """alpha = 1 (z = -1e30) and beta = 0: hT == h0 bit for bit, o = h0^T q."""
    inp = W.random_prefill([90, 40], 2, 64, "bf16", h0_std=0.3, seed=11)
    inp["z"][:] = -1e30
    inp["beta"][:] = 0.0
    g = to_gpu(inp)
    o, hT = gpu_prefill(g)
    assert torch.equal(hT.cpu(), inp["h0"])
    ro, _ = oracle_prefill(inp)
    compare_outputs(host(o), ro, "bf16", inp["cu_seqlens"].tolist())


@pytest.mark.parametrize("io,d", [("f32", 32), ("f32", 128), ("bf16", 128)])
def test_exact_write(io, d):
    """Unit keys with exact binary entries (four of +-0.5, exact in bf16 too),
    beta = 1, q = k: o_t = v_t whatever the decay, since
    S_t^T k_t = (Diag(a) S)^T (I - k k^T) k + v k^T k = v for |k| = 1.
    Several sequences and a partial chunk; the oracle agrees as well."""
    r = np.random.Generator(np.random.PCG64(12 + d))
    lens = [160, 37, 64]
    T, H = sum(lens), 2
    k = np.zeros((T, H, d), np.float32)
    for t in range(T):
        for h in range(H):
            idx = r.choice(d, 4, replace=False)
            k[t, h, idx] = r.choice([-0.5, 0.5], 4)
    inp = W.random_prefill(lens, H, d, io, h0_std=0.2, seed=12)
    inp["k"] = torch.from_numpy(k).to(inp["q"].dtype)
    inp["q"] = inp["k"].clone()
    inp["beta"][:] = 1.0
    g = to_gpu(inp)
    o, _ = gpu_prefill(g)
    cu = inp["cu_seqlens"].tolist()
    m = compare_outputs(host(o), inp["v"].double().numpy(), io, cu, what="o vs v")
    print("exact write %s d=%d %s" % (io, d, m), flush=True)
    ro, _ = oracle_prefill(inp)
    compare_outputs(host(o), ro, io, cu)


def test_split_and_carry():
    """prefill(T1) -> hT -> prefill(T2, h0=hT) matches one prefill of T1+T2."""
    inp = W.random_prefill([400], 2, 128, "bf16", h0_std=0.05, seed=13)
    g = to_gpu(inp)
    o, hT = gpu_prefill(g)
    t1 = 150
    part = lambda a, b: {n: (g[n][a:b] if n in ("q", "k", "v", "z", "beta") else g[n])
                         for n in ("q", "k", "v", "z", "beta", "A")}
    p1 = part(0, t1)
    o1, h1 = kda.prefill(p1["q"], p1["k"], p1["v"], p1["z"], p1["A"], p1["beta"],
                         torch.tensor([0, t1], dtype=torch.int32, device="cuda"), h0=g["h0"])
    p2 = part(t1, 400)
    o2, h2 = kda.prefill(p2["q"], p2["k"], p2["v"], p2["z"], p2["A"], p2["beta"],
                         torch.tensor([0, 400 - t1], dtype=torch.int32, device="cuda"), h0=h1)
    torch.cuda.synchronize()
    # against the oracle (the split point, 150, lies inside a chunk)
    ro, rh = oracle_prefill(inp)
    compare_prefill(torch.cat([o1, o2]), h2, ro, rh, [0, 400], "bf16", label="split and carry")
    assert rel_l2(host(torch.cat([o1, o2])), host(o)) <= BF16_TOL


def test_k3_prefill_sampled_heads():
    """B=1, H=96, T=65536: full GPU run, oracle on 6 sampled heads."""
    d = W.make("k3_prefill", device="cuda")
    check(d, "bf16", heads=[0, 17, 40, 63, 80, 95], label="k3_prefill")


def test_k3_varlen_sampled_heads():
    """32 lognormal sequences, 262144 tokens, H=96: oracle on 4 sampled heads."""
    d = W.make("k3_varlen", device="cuda")
    check(d, "bf16", heads=[3, 50, 77, 94], label="k3_varlen")
