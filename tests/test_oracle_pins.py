"""The fp64 oracle against the facts that pin it (see pins.py)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def _run(q, k, v, z, A, beta, h0, cu):
    return oracle.prefill(q, k, v, z, A, beta, h0, cu)


@pytest.mark.parametrize("check", pins.ALL_PREFILL_CHECKS, ids=lambda f: f.__name__)
def test_prefill_pin(check):
    check(_run)


def test_gate_closed_forms_c_and_numpy():
    lib = oracle.load()
    pins.check_gate_closed_forms(lambda a, z: lib.kda_oracle_gate(a, z))
    pins.check_gate_closed_forms(lambda a, z: float(oracle.gate(np.array([a]), np.array([[z]]))[0, 0]))


def _sig(x, n):
    return float("%.*g" % (n, x))


def test_pages_printed_constants():
    """The figures the pages print about the gate and the state follow from
    the definitions (rounded as printed)."""
    g = json.load(open(GOLDEN))
    gmin = g["g_min"]["printed"]
    assert gmin == oracle.G_MIN
    assert _sig(math.exp(gmin), 2) == g["alpha_lower_bound"]["printed"]
    assert _sig(100 * math.exp(gmin), 2) == g["min_retention_percent"]["printed"]
    assert g["window_tokens"]["printed"] * gmin == g["window_log_decay_lower"]["printed"]
    assert _sig(math.exp(-g["window_log_decay_lower"]["printed"]), 2) == g["rescale_bound"]["printed"]
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    assert _sig(bf16_max, 2) == g["bf16_max"]["printed"]
    assert math.exp(80) < bf16_max
    n = 96 * 128 * 128
    assert n == g["state_elements_per_layer_request"]["printed"]
    assert round(n * 2 / 2 ** 20) == g["state_mib_per_layer_bf16"]["printed"]
    assert round(69 * n * 2 / 2 ** 20) == g["state_mib_per_request_69_layers"]["printed"]
    assert 2 * g["state_mib_per_request_69_layers"]["printed"] == g["decode_state_traffic_mib_per_step"]["printed"]


def test_gate_bounds_random():
    """alpha in (e^-5, 1) on ordinary logits (devpress §3.2, Eq 5)."""
    r = pins.rng(5)
    A = r.uniform(-1, 1, 4)
    z = r.standard_normal((1000, 4, 16)) * 3
    a = np.exp(oracle.gate(A, z))
    assert np.all(a > math.exp(-5)) and np.all(a < 1)


def test_decode_is_one_prefill_token():
    """A decode step equals a prefill of one token per sequence, and T steps
    equal a prefill of T tokens ("Kimi K3：架构、训练与推理系统研究" §11.2: decode advances the state that
    prefill left, one token at a time)."""
    d = pins.rand_inputs(30, [1, 1, 1], H=2, dk=8, dv=6, h0_std=0.5)
    o, hT = pins.call(_run, d)
    od, Sd = oracle.decode(d["q"], d["k"], d["v"], d["z"], d["A"], d["beta"], d["h0"])
    assert np.array_equal(o, od) and np.array_equal(hT, Sd)
    T = 12
    e = pins.rand_inputs(31, [T], H=2, dk=8, dv=6, h0_std=0.5)
    o, hT = pins.call(_run, e)
    S = e["h0"].astype(np.float64)
    for t in range(T):
        sl = slice(t, t + 1)
        ot, S = oracle.decode(e["q"][sl], e["k"][sl], e["v"][sl], e["z"][sl], e["A"],
                              e["beta"][sl], S)
        assert np.allclose(ot[0], o[t], rtol=1e-14, atol=1e-15)
    assert np.allclose(S, hT, rtol=1e-14, atol=1e-15)


def test_bf16_bits_widen_exactly():
    """bf16 inputs are read as their exact values (the rounding happens once,
    when the inputs are made)."""
    x = np.array([1.0, -2.5, 3.140625, 1e-3], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    w = oracle.widen(bits)
    assert w[0] == 1.0 and w[1] == -2.5 and w[2] == 3.140625
    d = pins.rand_inputs(32, [10], H=1, dk=4, dv=4)
    tr = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    ob, hb = oracle.prefill(tr(d["q"]), tr(d["k"]), tr(d["v"]), d["z"], d["A"], d["beta"], None, d["cu"])
    f = lambda a: ((a.view(np.uint32) >> 16) << 16).view(np.float32)
    of, hf = oracle.prefill(f(d["q"]), f(d["k"]), f(d["v"]), d["z"], d["A"], d["beta"], None, d["cu"])
    assert np.array_equal(ob, of) and np.array_equal(hb, hf)
