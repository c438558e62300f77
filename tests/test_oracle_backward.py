"""Pins for the oracle's backward (kda_oracle_backward): reverse-mode
gradients of L = sum(dO * o) + sum(dhT * hT) through the token recurrence.

The pages give no backward formula, so the oracle's hand-derived reverse
sweep is pinned to:
  * torch.autograd (float64) through a plain torch forward of the recurrence,
  * central finite differences of the oracle's own (already pinned) forward,
  * a closed form (alpha = 1, beta = 0: the state is constant),
and planted mistakes in copies of the C source must each fail a pin."""
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle

G_MIN = -5.0


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def inputs(seed, lens, H, d, h0=True, unit=True):
    r = rng(seed)
    T = sum(lens)
    f = lambda *s: r.normal(size=s).astype(np.float32)
    q, k = f(T, H, d), f(T, H, d)
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=q, k=k, v=f(T, H, d), z=f(T, H, d), A=(r.uniform(-1, 1, size=H)).astype(np.float32),
                beta=(1 / (1 + np.exp(-f(T, H)))).astype(np.float32),
                h0=(r.normal(size=(len(lens), H, d, d)) * 0.3) if h0 else None,
                cu=np.cumsum([0] + list(lens)).astype(np.int32),
                dO=r.normal(size=(T, H, d)), dhT=r.normal(size=(len(lens), H, d, d)))


def torch_grads(d):
    """Autograd through a float64 torch forward of the recurrence."""
    t = lambda x: torch.tensor(np.asarray(x, np.float64), dtype=torch.float64, requires_grad=True)
    q, k, v, z, A, beta = (t(d[n]) for n in ("q", "k", "v", "z", "A", "beta"))
    N = len(d["cu"]) - 1
    H, dk = d["q"].shape[1], d["q"].shape[2]
    h0 = t(d["h0"]) if d["h0"] is not None else torch.zeros(N, H, dk, dk, dtype=torch.float64, requires_grad=True)
    outs, finals = [], []
    for n in range(N):
        heads = []
        for h in range(H):
            S = h0[n, h].T          # [dv][dk] in memory -> S_{i,j} = h0[j][i]
            for tt in range(int(d["cu"][n]), int(d["cu"][n + 1])):
                g = G_MIN * torch.sigmoid(torch.exp(A[h]) * z[tt, h])
                Sbar = torch.exp(g)[:, None] * S
                e = v[tt, h] - Sbar.T @ k[tt, h]
                S = Sbar + beta[tt, h] * torch.outer(k[tt, h], e)
                outs.append((tt, h, S.T @ q[tt, h]))
            heads.append(S.T)
        finals.append(torch.stack(heads))
    loss = torch.zeros((), dtype=torch.float64)
    dO = torch.tensor(d["dO"])
    for tt, h, o in outs:
        loss = loss + (o * dO[tt, h]).sum()
    if N:
        loss = loss + (torch.stack(finals) * torch.tensor(d["dhT"])).sum()
    loss.backward()
    g = lambda x: x.grad.numpy() if x.grad is not None else np.zeros(x.shape)
    return dict(dq=g(q), dk=g(k), dv=g(v), dz=g(z), dA=g(A), dbeta=g(beta), dh0=g(h0))


def run_oracle(d, lib_path=None):
    kw = {} if lib_path is None else {"lib_path": lib_path}
    return oracle.backward(d["q"], d["k"], d["v"], d["z"], d["A"], d["beta"], d["h0"], d["cu"], d["dO"],
                           d["dhT"], **kw)


def check_autograd(run):
    d = inputs(1, [7, 0, 13, 70], 2, 6)   # one sequence crosses a 64-token checkpoint
    got, ref = run(d), torch_grads(d)
    for name in ("dq", "dk", "dv", "dz", "dA", "dbeta", "dh0"):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-9, atol=1e-11, err_msg=name)


def check_finite_differences(run):
    """Directional derivative of L along a random direction in every input,
    by central differences of the forward oracle (float32 inputs widened;
    the step is applied in float64 where the oracle reads float64)."""
    d = inputs(2, [9, 5], 2, 5, unit=False)
    g = run(d)
    r = rng(3)
    dirs = {n: r.normal(size=np.shape(d[n])) for n in ("q", "k", "v", "z", "A", "beta", "h0")}

    def loss(eps):
        x = {n: (d[n].astype(np.float64) + eps * dirs[n]) for n in dirs}
        o, hT = oracle.prefill(x["q"].astype(np.float32), x["k"].astype(np.float32), x["v"].astype(np.float32),
                               x["z"].astype(np.float32), x["A"].astype(np.float32), x["beta"].astype(np.float32),
                               x["h0"], d["cu"])
        return float((o * d["dO"]).sum() + (hT * d["dhT"]).sum())

    # float32 rounding of the perturbed inputs limits the step: use 1e-2 and
    # compare against the gradient taken at the rounded base point
    eps = 1e-2
    fd = (loss(eps) - loss(-eps)) / (2 * eps)
    an = sum(float((g[{"q": "dq", "k": "dk", "v": "dv", "z": "dz", "A": "dA", "beta": "dbeta",
                       "h0": "dh0"}[n]] * dirs[n]).sum()) for n in dirs)
    assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (fd, an)


def check_constant_state(run):
    """alpha = 1, beta = 0: S_t = h0, o_t = h0^T q_t.  Then dq_t = h0 do_t,
    dh0 = dhT + sum_t q_t do_t^T, dk = dv = dz = dA = 0, and
    dbeta_t = k_t^T Lambda_t e_t with Lambda_t = dhT + sum_{tau >= t} q do^T,
    e_t = v_t - h0^T k_t."""
    d = inputs(4, [11], 2, 4)
    d["z"][:] = -1e30
    d["beta"][:] = 0.0
    g = run(d)
    T, H = 11, 2
    for h in range(H):
        S = d["h0"][0, h].T      # S_{i,j}
        lam = d["dhT"][0, h].T.copy()
        for t in range(T - 1, -1, -1):
            qq, kk, vv = (d[n][t, h].astype(np.float64) for n in ("q", "k", "v"))
            lam += np.outer(qq, d["dO"][t, h])
            np.testing.assert_allclose(g["dq"][t, h], S @ d["dO"][t, h], rtol=1e-12, atol=1e-12)
            e = vv - S.T @ kk
            np.testing.assert_allclose(g["dbeta"][t, h], kk @ lam @ e, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["dh0"][0, h], lam.T, rtol=1e-12, atol=1e-12)
    for name in ("dk", "dv", "dz", "dA"):
        assert np.all(g[name] == 0.0), name


PINS = [check_autograd, check_finite_differences, check_constant_state]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(run_oracle)


def test_chunkwise_backward_matches_token_sweep():
    """The chunk-form gradients (a second algorithm: matrix derivatives of
    the chunk formulas) equal the token sweep for several chunk sizes."""
    from oracle import chunkwise
    d = inputs(11, [5, 0, 70, 130], 2, 6)
    ref = run_oracle(d)
    for C in (1, 3, 16, 64):
        got = chunkwise.backward(d["q"], d["k"], d["v"], d["z"], d["A"], d["beta"], d["h0"], d["cu"], d["dO"],
                                 d["dhT"], chunk=C)
        for name in ref:
            np.testing.assert_allclose(got[name], ref[name], rtol=1e-10, atol=1e-12, err_msg="%s C=%d" % (name, C))


def test_backward_bf16_inputs_match_autograd():
    d = inputs(5, [20, 3], 2, 8)
    bits = {}
    for n in ("q", "k", "v"):
        b = (d[n].view(np.uint32) + 0x7FFF + ((d[n].view(np.uint32) >> 16) & 1)) >> 16
        bits[n] = b.astype(np.uint16)
        d[n] = (b.astype(np.uint32) << 16).view(np.float32)   # the values the bits stand for
    got = oracle.backward(bits["q"], bits["k"], bits["v"], d["z"], d["A"], d["beta"], d["h0"], d["cu"], d["dO"],
                          d["dhT"])
    ref = torch_grads(d)
    for name in ("dq", "dk", "dv", "dz", "dA", "dbeta", "dh0"):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-9, atol=1e-11, err_msg=name)


SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")
MUTANTS = {
    "no_q_do": ("L[(size_t)i * dv + j] += qq[i] * dOt[j];", "L[(size_t)i * dv + j] += 0.0 * qq[i] * dOt[j];"),
    "dq_from_prev_state": ("acc += Sn[(size_t)i * dv + j] * dOt[j];", "acc += Sp[(size_t)i * dv + j] * dOt[j];"),
    "dp_sign": ("w1[j] = -b * w1[j];", "w1[j] = b * w1[j];"),
    "dk_no_sbar": ("+ a[i] * Sp[(size_t)i * dv + j] * w1[j];", ";"),
    "no_decay_on_lambda": ("L[(size_t)i * dv + j] = a[i] * ds;", "L[(size_t)i * dv + j] = ds;"),
    "dalpha_with_new_state": ("da += ds * Sp[(size_t)i * dv + j];", "da += ds * Sn[(size_t)i * dv + j];"),
    "gate_derivative": ("const double dx = w2[i] * KDA_ORACLE_GMIN * s * (1.0 - s);",
                        "const double dx = w2[i] * KDA_ORACLE_GMIN * s;"),
    "dA_missing_z": ("gA += dx * x;", "gA += dx * eA;"),
    "beta_grad_sign": ("for (int j = 0; j < dv; ++j) db += w1[j] * e[j];", "for (int j = 0; j < dv; ++j) db -= w1[j] * e[j];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("mut_%s.so" % name))
    subprocess.run(["gcc", *oracle.CFLAGS, str(path), "-o", lib, "-lm"], check=True)
    failed = []
    for pin in PINS:
        try:
            pin(lambda d: run_oracle(d, lib))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
