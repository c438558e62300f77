"""Scale equivariance of the GPU path, exactly.

The recurrence is linear in (v, h0) together: scaling v and the initial
state by 2^s scales every output and every state by 2^s, with q, k, z, A
and beta unchanged.  The bf16 path keeps S, V' and U in fp16 only after a
power-of-two scaling chosen from their own magnitude, so its fp16 mantissas,
and with them every rounding it makes, do not depend on s: the outputs for
2^s v must equal 2^s times the outputs for v bit for bit, also where 2^s v
lies far outside the fp16 range.  The fp32 path and the decode kernels use
fp32 arithmetic throughout, where a power-of-two factor commutes with every
rounding.  Exponents are kept well inside the fp32 and bf16 ranges, so no
value over- or underflows.  One case of each is also checked against the
oracle, so that the property is not met by a path that is wrong at every
scale."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W
from gpu_util import compare_prefill, oracle_prefill, to_gpu

pytestmark = pytest.mark.gpu

SHIFTS = [-24, -7, 9, 24]


def scaled(d, s, keys):
    e = dict(d)
    for n in keys:
        if e.get(n) is not None:
            e[n] = (e[n].double() * 2.0 ** s).to(e[n].dtype)
    return e


def prefill(g, segments=0):
    o, hT = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"], h0=g["h0"],
                        segments=segments)
    torch.cuda.synchronize()
    return o.double(), hT.double()


@pytest.mark.parametrize("io,d,segments", [("bf16", 128, 0), ("bf16", 64, 3), ("bf16", 32, 1), ("f32", 64, 0)])
def test_prefill_scales_exactly(io, d, segments):
    lens = [300, 1, 129, 0, 64, 700]
    base = W.random_prefill(lens, 3, d, io, h0_std=0.05, seed=8500 + d)
    print("case prefill scaling %s d=%d segments=%d" % (io, d, segments), flush=True)
    g = to_gpu(base)
    o, hT = prefill(g, segments)
    if d == 128:
        ro, rh = oracle_prefill(base)
        compare_prefill(o.float(), hT.float(), ro, rh, base["cu_seqlens"], io, label="unscaled")
    for s in SHIFTS:
        o2, hT2 = prefill(to_gpu(scaled(base, s, ("v", "h0"))), segments)
        assert torch.equal(o2, o * 2.0 ** s), "o differs at 2^%d" % s
        assert torch.equal(hT2, hT * 2.0 ** s), "hT differs at 2^%d" % s


def test_decode_scales_exactly():
    print("case decode scaling", flush=True)
    base = W.random_decode(17, 4, 128, "bf16", 0.05, seed=8600)
    g = to_gpu(base)
    S = g["S"].clone()
    o = kda.decode(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], S).double()
    for s in SHIFTS:
        g2 = to_gpu(scaled(base, s, ("v", "S")))
        S2 = g2["S"].clone()
        o2 = kda.decode(g2["q"], g2["k"], g2["v"], g2["z"], g2["A"], g2["beta"], S2).double()
        torch.cuda.synchronize()
        assert torch.equal(o2, o * 2.0 ** s), "o differs at 2^%d" % s
        assert torch.equal(S2.double(), S.double() * 2.0 ** s), "S differs at 2^%d" % s


def test_decode_window_scales_exactly():
    print("case decode window scaling", flush=True)
    base = W.random_decode_window(6, 3, 128, Lr=4, L=3, io="bf16", seed=8700)
    base["n_accept"] = torch.tensor([0, 4, 2, 1, 4, 3], dtype=torch.int32)

    def run(d):
        S = d["S"].cuda()
        win = {n: t.cuda() for n, t in d["window"].items()}
        rep = {n: t.cuda() for n, t in d["replay"].items()}
        o = kda.decode_window(d["A"].cuda(), S, window=win, replay=rep, n_accept=d["n_accept"].cuda(),
                              commit_window=True)
        torch.cuda.synchronize()
        return o.double(), S.double()

    o, S = run(base)
    for s in SHIFTS:
        d2 = dict(base)
        d2["S"] = (base["S"].double() * 2.0 ** s).float()
        d2["window"] = dict(base["window"])
        d2["replay"] = dict(base["replay"])
        for part in ("window", "replay"):
            d2[part]["v"] = (base[part]["v"].double() * 2.0 ** s).to(base[part]["v"].dtype)
        o2, S2 = run(d2)
        assert torch.equal(o2, o * 2.0 ** s), "o differs at 2^%d" % s
        assert torch.equal(S2, S * 2.0 ** s), "S differs at 2^%d" % s
