"""Pins for the feature-path and output-gate oracle (oracle/features.py):
library routines and identities that do not depend on the oracle, plus
planted mistakes in copies of it that each pin must catch."""
import types

import numpy as np
import pytest
from scipy.special import expit

import oracle.features as F


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- the pins
def check_conv_is_numpy_convolve(mod):
    """Every sequence and channel: the causal 4-tap convolution equals
    numpy.convolve of [window, sequence] with the reversed taps."""
    r = rng(1)
    lens = [7, 0, 1, 5]
    cu = np.cumsum([0] + lens)
    H, d = 2, 3
    x = r.normal(size=(cu[-1], H, d))
    w = r.normal(size=(H, d, 4))
    win = r.normal(size=(len(lens), 3, H, d))
    y, out = mod.short_conv(x, w, cu, win)
    for n in range(len(lens)):
        for h in range(H):
            for c in range(d):
                s = np.concatenate([win[n, :, h, c], x[cu[n]:cu[n + 1], h, c]])
                full = np.convolve(s, w[h, c, ::-1])
                np.testing.assert_allclose(y[cu[n]:cu[n + 1], h, c], full[3:3 + lens[n]], rtol=1e-13, atol=1e-13)
                np.testing.assert_array_equal(out[n, :, h, c], s[-3:])


def check_conv_split_and_carry(mod):
    """One sequence in one call equals two calls that carry the window."""
    r = rng(2)
    x = r.normal(size=(11, 2, 4))
    w = r.normal(size=(2, 4, 4))
    win0 = r.normal(size=(1, 3, 2, 4))
    y, out = mod.short_conv(x, w, [0, 11], win0)
    y1, o1 = mod.short_conv(x[:2], w, [0, 2], win0)   # shorter than the window
    y2, o2 = mod.short_conv(x[2:], w, [0, 9], o1)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(o2, out)


def check_conv_impulse(mod):
    """A unit impulse at the first token with a zero window reads the taps
    back in order: y[t] = w[3 - t]."""
    w = np.arange(1.0, 5.0).reshape(1, 1, 4)
    x = np.zeros((6, 1, 1))
    x[0] = 1.0
    y, _ = mod.short_conv(x, w, [0, 6])
    assert y[:, 0, 0].tolist() == [4.0, 3.0, 2.0, 1.0, 0.0, 0.0]


def check_swish(mod):
    u = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(mod.swish(u), u * expit(u), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(mod.swish(u) - mod.swish(-u), u, rtol=1e-13, atol=1e-13)
    assert mod.swish(np.array(0.0)) == 0.0


def check_l2norm(mod):
    r = rng(3)
    u = r.normal(size=(5, 7))
    n = mod.l2norm(u)
    np.testing.assert_allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(n * np.linalg.norm(u, axis=-1, keepdims=True), u, rtol=1e-13)


def check_rmsnorm_and_gate(mod):
    r = rng(4)
    o = r.normal(size=(6, 3, 8)) * 3.0
    w = np.ones(8)
    y = mod.rmsnorm(o, w, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(mod.rmsnorm(5.0 * o, w, 0.0), y, rtol=1e-13)
    wv = r.normal(size=8)
    np.testing.assert_allclose(mod.rmsnorm(o, wv, 0.0), y * wv, rtol=1e-13)
    assert np.all(mod.rmsnorm(np.zeros((1, 8)), w, 1e-6) == 0.0)
    g = r.normal(size=o.shape)
    # Sigmoid(g) + Sigmoid(-g) = 1, Sigmoid(0) = 1/2
    np.testing.assert_allclose(mod.output_gate(o, g, wv, 1e-5) + mod.output_gate(o, -g, wv, 1e-5),
                               mod.rmsnorm(o, wv, 1e-5), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mod.output_gate(o, 0 * g, wv, 1e-5), 0.5 * mod.rmsnorm(o, wv, 1e-5), rtol=1e-14)
    np.testing.assert_allclose(mod.output_gate(o, g, wv, 1e-5), expit(g) * mod.rmsnorm(o, wv, 1e-5), rtol=1e-13)


def check_qkv_paths(mod):
    """q and k are unit vectors, v is not normalised, and the carried window
    is the q | k | v channels of the last three pre-convolution tokens."""
    r = rng(5)
    lens = [9, 2]
    cu = np.cumsum([0] + lens)
    H, dk, dv = 2, 4, 6
    xq, xk = r.normal(size=(11, H, dk)), r.normal(size=(11, H, dk))
    xv = r.normal(size=(11, H, dv))
    wq, wk, wv = r.normal(size=(H, dk, 4)), r.normal(size=(H, dk, 4)), r.normal(size=(H, dv, 4))
    win = r.normal(size=(2, 3, H, 2 * dk + dv))
    q, k, v, out = mod.qkv_features(xq, xk, xv, wq, wk, wv, cu, win)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-13)
    cv, _ = mod.short_conv(xv, wv, cu, win[..., 2 * dk:])
    np.testing.assert_allclose(v, cv * expit(cv), rtol=1e-13)
    ck, ok = mod.short_conv(xk, wk, cu, win[..., dk:2 * dk])
    np.testing.assert_allclose(k, mod.l2norm(ck * expit(ck)), rtol=1e-13)
    # sequence 1 (tokens 9, 10) keeps one carried token, then its own two
    np.testing.assert_array_equal(out[1, 0], win[1, 2])
    np.testing.assert_array_equal(out[1, 1:, :, :dk], xq[9:11])
    np.testing.assert_array_equal(out[1, 1:, :, dk:2 * dk], xk[9:11])
    np.testing.assert_array_equal(out[0, :, :, 2 * dk:], xv[6:9])


PINS = [check_conv_is_numpy_convolve, check_conv_split_and_carry, check_conv_impulse, check_swish,
        check_l2norm, check_rmsnorm_and_gate, check_qkv_paths]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_feature_pin(pin):
    pin(F)


# ---------------------------------------------------------------- mutants
SRC = open(F.__file__).read()
MUTANTS = {
    "taps_reversed": ('np.einsum("ihd,hdi->hd", seq[t:t + TAPS], w)', 'np.einsum("ihd,hdi->hd", seq[t:t + TAPS][::-1], w)'),
    "window_ignored": ("prev = np.zeros((TAPS - 1, H, d)) if window is None else np.asarray(window[n], np.float64)",
                       "prev = np.zeros((TAPS - 1, H, d))"),
    "window_out_oldest": ("out[n] = seq[-(TAPS - 1):]", "out[n] = seq[:TAPS - 1]"),
    "window_off_by_one": ("seq[t:t + TAPS]", "seq[t + 1:t + 1 + TAPS] if t + 1 + TAPS <= len(seq) else seq[t:t + TAPS]"),
    "swish_sign": ("return u / (1.0 + np.exp(-u))", "return u / (1.0 + np.exp(u))"),
    "l2norm_no_sqrt": ("return u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True))",
                       "return u / np.sum(u * u, axis=-1, keepdims=True)"),
    "rms_sum_not_mean": ("np.mean(o * o, axis=-1, keepdims=True) + eps", "np.sum(o * o, axis=-1, keepdims=True) + eps"),
    "rms_weight_dropped": ("+ eps) * np.asarray(w, np.float64)", "+ eps)"),
    "gate_sign": ("return sigmoid(np.asarray(g, np.float64)) * rmsnorm(o, w, eps)",
                  "return sigmoid(-np.asarray(g, np.float64)) * rmsnorm(o, w, eps)"),
    "v_normalised": ("v = swish(cv)", "v = l2norm(swish(cv))"),
    "k_from_q_window": ("ck, ok = short_conv(xk, wk, cu_seqlens, part(dk, 2 * dk))",
                        "ck, ok = short_conv(xk, wk, cu_seqlens, part(0, dk))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, name
    mod = types.ModuleType("features_" + name)
    exec(compile(SRC.replace(old, new), "features_" + name, "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
