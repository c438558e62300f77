"""The fused decode step (feature path -> decode step -> output gate in one
pass over the state) against the composition of the three oracles, through
the C ABI, and against the three separate entry points.

The composition: q, k, v of the new token from the feature oracle in fp64
over the carried window (the fused step keeps them in fp32; the decode
oracle's C interface takes them as fp32, a 2^-24 perturbation); the decode
oracle; the gate oracle on the unrounded o.  y is compared by the output
measures of gpu_util and the gated element bound; the state by rel-L2 over
the batch and per (sequence, head) against S_TOL = 1e-6, decode_kernel's own
state bar: the step's fp32 work (the taps, Swish and the norm with the
hardware exp, reciprocal and reciprocal square root, each within a few ulp,
then the update) measured at most 2.1e-7 per (sequence, head).
The new window is compared bit for bit (a copy of inputs).  Against the
separate calls, which hand q, k, v and o over in bf16, the window is
bit-identical and the state and y differ by those roundings."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
import oracle
from gated_delta_rule_21_amd import workloads as W
from gpu_util import check_gated_elements, compare_outputs, compare_states, host, rel_l2
from oracle import features as F

pytestmark = pytest.mark.gpu
EPS = 1e-6
S_TOL = 1e-6


def widen(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def step_inputs(N, H, d, seed, window=True, z_shift=0.0):
    f = W.random_features([1] * N, H, d, "bf16", window=window, seed=seed)
    dec = W.random_decode(N, H, d, "bf16", 0.05, seed=seed + 1, z_shift=z_shift)
    return dict(xq=f["xq"], xk=f["xk"], xv=f["xv"], wq=f["wq"], wk=f["wk"], wv=f["wv"], window=f["window"],
                gate=f["g"], norm_w=f["w"], z=dec["z"], A=dec["A"], beta=dec["beta"], S=dec["S"])


def oracle_step(d, S, window):
    """(y, S_new, window_new, o, g) of the composition for one token per sequence."""
    N = d["xq"].shape[0]
    cu = np.arange(N + 1)
    q, k, v, wout = F.qkv_features(widen(d["xq"]), widen(d["xk"]), widen(d["xv"]), widen(d["wq"]), widen(d["wk"]),
                                   widen(d["wv"]), cu, window)
    f32 = lambda a: np.asarray(a, np.float32)
    ro, rS = oracle.decode(f32(q), f32(k), f32(v), W.as_numpy(d["z"]), W.as_numpy(d["A"]), W.as_numpy(d["beta"]), S)
    g = widen(d["gate"])
    return F.output_gate(ro, g, widen(d["norm_w"]), EPS), rS, wout, ro, g


def gpu_step(g, S, win_in, win_out):
    y = kda.decode_fused(g["xq"], g["xk"], g["xv"], g["wq"], g["wk"], g["wv"], g["z"], g["A"], g["beta"], S,
                         g["gate"], g["norm_w"], EPS, conv_state_in=win_in, conv_state_out=win_out)
    torch.cuda.synchronize()
    return y


def run_steps(N, H, d, steps, seed, window=True, in_place=False, z_shift=0.0, label=""):
    """`steps` fused steps in a row, the state and the window carried on both
    sides; every step checked against the oracle composition."""
    first = step_inputs(N, H, d, seed, window, z_shift)
    S_gpu = first["S"].cuda()
    S_ref = W.as_numpy(first["S"]).astype(np.float64)
    win_gpu = first["window"].cuda() if window else None
    win_ref = widen(first["window"]) if window else None
    for s in range(steps):
        inp = first if s == 0 else step_inputs(N, H, d, seed + 10 * s, window, z_shift)
        print("case %s step %d" % (label, s), flush=True)
        g = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
        out_win = None
        if window or s == 0:
            out_win = win_gpu if (in_place and win_gpu is not None) else torch.empty(
                (N, 3, H, 3 * d), dtype=torch.bfloat16, device="cuda")
        y = gpu_step(g, S_gpu, win_gpu, out_win)
        ry, S_ref, wref, ro, rg = oracle_step(inp, S_ref, win_ref)
        compare_outputs(host(y), ry, "bf16", None, what="y", label="%s step %d" % (label, s), elem=False)
        check_gated_elements(host(y), ry, ro, rg, widen(inp["norm_w"]), EPS, [0, N], "%s step %d" % (label, s))
        compare_states(host(S_gpu), S_ref, "bf16", what="S", whole_bar=S_TOL, unit_bar=S_TOL,
                       label="%s step %d" % (label, s))
        np.testing.assert_array_equal(widen(out_win), wref)
        win_gpu, win_ref = out_win, wref
        window = True        # later steps carry the window the first one produced


@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_fused_steps(d):
    run_steps(24, 3, d, 3, seed=1200 + d, label="d=%d" % d)


def test_decode_fused_without_window_and_in_place():
    run_steps(20, 2, 128, 2, seed=1300, window=False, label="no window")
    run_steps(20, 2, 64, 3, seed=1310, in_place=True, label="in place")


@pytest.mark.parametrize("z_shift", [-4.0, 6.0])
def test_decode_fused_decay_extremes(z_shift):
    run_steps(16, 4, 128, 2, seed=1320, z_shift=z_shift, label="z%+g" % z_shift)


def test_decode_fused_empty_batch():
    inp = step_inputs(0, 3, 64, seed=1330)
    g = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    y = gpu_step(g, g["S"], g["window"], None)
    assert y.shape == (0, 3, 64)


def test_decode_fused_matches_separate_calls():
    """qkv_shortconv + decode + output_gate: the same window bit for bit; the
    state and y within the bf16 roundings that the separate path makes, each
    at most 2^-9 relative: of k and v for the state (2 x 2^-9), of q, k, v and
    o for y (4 x 2^-9)."""
    N, H, d = 64, 8, 128
    inp = step_inputs(N, H, d, seed=1340)
    g = {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in inp.items()}
    S1, S2 = g["S"].clone(), g["S"].clone()
    w1, w2 = torch.empty_like(g["window"]), torch.empty_like(g["window"])
    y1 = gpu_step(g, S1, g["window"], w1)
    cu = torch.arange(N + 1, dtype=torch.int32, device="cuda")
    q, k, v = kda.qkv_shortconv(g["xq"], g["xk"], g["xv"], g["wq"], g["wk"], g["wv"], cu,
                                conv_state_in=g["window"], conv_state_out=w2)
    o = kda.decode(q, k, v, g["z"], g["A"], g["beta"], S2)
    y2 = kda.output_gate(o, g["gate"], g["norm_w"], EPS)
    torch.cuda.synchronize()
    assert torch.equal(w1, w2)
    e_s, e_y = rel_l2(host(S1), host(S2)), rel_l2(host(y1), host(y2))
    print("fused vs separate: S %.2e y %.2e" % (e_s, e_y), flush=True)
    assert 0 < e_s < 2 * 2.0 ** -9 and e_y < 4 * 2.0 ** -9


def test_decode_fused_k3_shape():
    """The batched decode workload's shape, 256 sequences x 96 heads x 128."""
    run_steps(256, 96, 128, 1, seed=1350, label="k3")
