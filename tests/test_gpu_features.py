"""Feature path (ShortConv -> Swish -> L2Norm) and output gate: HIP kernels
vs the fp64 oracle in oracle/features.py, through the C ABI."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
from gated_delta_rule_21_amd import workloads as W
from gpu_util import host, rel_l2, tol
from oracle import features as F

pytestmark = pytest.mark.gpu


def widen(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def oracle_qkv(d):
    return F.qkv_features(widen(d["xq"]), widen(d["xk"]), widen(d["xv"]), widen(d["wq"]), widen(d["wk"]),
                          widen(d["wv"]), d["cu_seqlens"].cpu().numpy(), widen(d["window"]))


def gpu_qkv(d, in_place=False):
    g = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
    win_in = g["window"]
    win_out = None
    if win_in is not None:
        win_out = win_in if in_place else torch.empty_like(win_in)
    elif d["N"] > 0:
        win_out = torch.empty((d["N"], 3, d["H"], 3 * d["d"]), dtype=g["xq"].dtype, device="cuda")
    q, k, v = kda.qkv_shortconv(g["xq"], g["xk"], g["xv"], g["wq"], g["wk"], g["wv"], g["cu_seqlens"],
                                conv_state_in=win_in, conv_state_out=win_out)
    torch.cuda.synchronize()
    return q, k, v, win_out


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_qkv_ragged(io, d):
    """Sequences shorter than the window, empty, and long; a carried window."""
    lens = [0, 1, 2, 3, 5, 70, 200, 0]
    inp = W.random_features(lens, 3, d, io, window=True, seed=800 + d)
    q, k, v, win = gpu_qkv(inp)
    rq, rk, rv, rwin = oracle_qkv(inp)
    errs = [rel_l2(host(a), b) for a, b in ((q, rq), (k, rk), (v, rv))]
    print("qkv %s d=%d rel-L2 q=%.3e k=%.3e v=%.3e" % (io, d, *errs), flush=True)
    assert max(errs) <= tol(io), errs
    # the window is a copy of input values: exact
    np.testing.assert_array_equal(widen(win), rwin)


def test_qkv_without_window_and_in_place():
    inp = W.random_features([9, 1, 40], 4, 128, "bf16", window=False, seed=810)
    q, k, v, win = gpu_qkv(inp)
    rq, rk, rv, rwin = oracle_qkv(inp)
    assert max(rel_l2(host(a), b) for a, b in ((q, rq), (k, rk), (v, rv))) <= tol("bf16")
    np.testing.assert_array_equal(widen(win), rwin)
    inp = W.random_features([9, 1, 0, 40], 4, 64, "bf16", window=True, seed=811)
    q, k, v, win = gpu_qkv(inp, in_place=True)
    rq, rk, rv, rwin = oracle_qkv(inp)
    assert max(rel_l2(host(a), b) for a, b in ((q, rq), (k, rk), (v, rv))) <= tol("bf16")
    np.testing.assert_array_equal(widen(win), rwin)


def test_decode_steps_carry_the_window():
    """Five one-token steps (T = N, cu = 0..N) with the window updated in
    place equal one call over the five tokens of every sequence."""
    N, H, d, steps = 6, 3, 128, 5
    full = W.random_features([steps] * N, H, d, "bf16", window=True, seed=812)
    rq, rk, rv, rwin = oracle_qkv(full)
    win = full["window"].cuda()
    cu = torch.arange(N + 1, dtype=torch.int32, device="cuda")
    for s in range(steps):
        pick = lambda t: t.view(N, steps, H, d)[:, s].contiguous().cuda()
        q, k, v = kda.qkv_shortconv(pick(full["xq"]), pick(full["xk"]), pick(full["xv"]), full["wq"].cuda(),
                                    full["wk"].cuda(), full["wv"].cuda(), cu, conv_state_in=win, conv_state_out=win)
        torch.cuda.synchronize()
        ref = lambda r: r.reshape(N, steps, H, d)[:, s]
        assert rel_l2(host(q), ref(rq)) <= tol("bf16")
        assert rel_l2(host(v), ref(rv)) <= tol("bf16")
    np.testing.assert_array_equal(widen(win), rwin)


def test_qkv_feeds_prefill():
    """The feature path's q, k are unit rows and drive kda_prefill like any
    unit-norm input: the prefill on them matches the KDA oracle."""
    from gpu_util import oracle_prefill
    inp = W.random_features([300, 77], 2, 128, "bf16", window=False, seed=813)
    q, k, v, _ = gpu_qkv(inp)
    norms = torch.linalg.vector_norm(q.float(), dim=-1)
    assert float((norms - 1).abs().max()) < 1e-2
    pre = W.random_prefill([300, 77], 2, 128, "bf16", h0_std=0.05, seed=814)
    pre.update(q=q.cpu(), k=k.cpu(), v=v.cpu())
    g = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in pre.items()}
    o, hT = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["A"], g["beta"], g["cu_seqlens"], h0=g["h0"])
    torch.cuda.synchronize()
    ro, rh = oracle_prefill(pre)
    from gpu_util import compare_prefill
    compare_prefill(o, hT, ro, rh, pre["cu_seqlens"], "bf16", label="feature path -> prefill")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_output_gate(io, d):
    inp = W.random_features([130, 7], 5, d, io, seed=820 + d)
    o, g, w = inp["o"].cuda(), inp["g"].cuda(), inp["w"].cuda()
    y = kda.output_gate(o, g, w, 1e-5)
    torch.cuda.synchronize()
    ry = F.output_gate(widen(inp["o"]), widen(inp["g"]), widen(inp["w"]), 1e-5)
    e = rel_l2(host(y), ry)
    print("gate %s d=%d rel-L2 %.3e" % (io, d, e), flush=True)
    assert e <= tol(io), e
    # in place over o gives the same bits
    o2 = o.clone()
    kda.output_gate(o2, g, w, 1e-5, y=o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, y)


def test_k3_shaped_feature_path_and_gate():
    """T = 65536, H = 96, d = 128 (the K3 prefill shape), one sequence with a
    carried window: tokens [0, 300) and [65000, 65536) against the oracle,
    each slice with its own window (the given one, or the three tokens
    before it)."""
    inp = W.random_features([65536], 96, 128, "bf16", window=True, seed=830, device="cuda")
    q, k, v, win = gpu_qkv(inp)
    y = kda.output_gate(inp["o"], inp["g"], inp["w"], 1e-6)
    torch.cuda.synchronize()
    names = ("xq", "xk", "xv")
    for a, b in ((0, 300), (65000, 65536)):
        if a == 0:
            w3 = inp["window"].cpu()
        else:
            w3 = torch.cat([inp[n][a - 3:a].cpu() for n in names], -1).unsqueeze(0)
        sub = {n: inp[n][a:b].cpu() for n in names}
        sub.update({n: inp[n].cpu() for n in ("wq", "wk", "wv")})
        sub.update(cu_seqlens=torch.tensor([0, b - a], dtype=torch.int32), window=w3)
        rq, rk, rv, _ = oracle_qkv(sub)
        for got, ref in ((q, rq), (k, rk), (v, rv)):
            e = rel_l2(host(got[a:b]), ref)
            assert e <= tol("bf16"), (a, e)
    ry = F.output_gate(widen(inp["o"][:2000]), widen(inp["g"][:2000]), widen(inp["w"]), 1e-6)
    assert rel_l2(host(y[:2000]), ry) <= tol("bf16")
