"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each check takes `run(q, k, v, z, A, beta, h0, cu) -> (o, hT)` (a prefill
oracle) and raises AssertionError when the runner disagrees with a fact that
does not depend on the runner: a closed form, a special case that reduces to
an older rule the pages print, an exact identity, or a second algorithm.
The same checks are run against deliberately broken copies of the oracle
(test_oracle_mutants.py) to show that each plausible mistake fails one.

Page names used below:
  P1 = s1mplewind "kimi-k3" notes; P2 = "Hybrid KDA–MLA：Kimi K3 注意力机制解析";
  P3 = devpress K3 technical-report walk-through;
  P5 = "Kimi K3：架构、训练与推理系统研究".
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import hadamard
from scipy.special import expit

import oracle
from oracle import chunkwise

Z_ALPHA_ONE = -1.0e30   # sigmoid(-huge) = 0 exactly  => g = 0, alpha = 1
Z_ALPHA_MIN = 1.0e30    # sigmoid(+huge) = 1 exactly  => g = -5


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_inputs(seed, lens, H, dk, dv=None, h0_std=None, unit=True):
    """Small float32 inputs for oracle checks (q, k unit-norm rows)."""
    dv = dk if dv is None else dv
    r = rng(seed)
    T = int(sum(lens))
    q = r.standard_normal((T, H, dk)).astype(np.float32)
    k = r.standard_normal((T, H, dk)).astype(np.float32)
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, dv)).astype(np.float32)
    z = r.standard_normal((T, H, dk)).astype(np.float32)
    A = r.uniform(-1, 1, H).astype(np.float32)
    beta = expit(r.standard_normal((T, H))).astype(np.float32)
    N = len(lens)
    h0 = None
    if h0_std is not None:
        h0 = (r.standard_normal((N, H, dv, dk)) * h0_std).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(q=q, k=k, v=v, z=z, A=A, beta=beta, h0=h0, cu=cu)


def call(run, d):
    return run(d["q"], d["k"], d["v"], d["z"], d["A"], d["beta"], d["h0"], d["cu"])


def rel_l2(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm((x - y).ravel()) / max(np.linalg.norm(y.ravel()), 1e-300))


# --------------------------------------------------------------------------
# Gate (P3 §3.2 Eq 5; P5 §3.2; P2 decay design)
# --------------------------------------------------------------------------
def check_gate_closed_forms(gate_fn):
    """gate_fn(A_h, z) -> g.  sigmoid(0) = 1/2 gives g = -2.5 exactly; the
    saturated ends give g = 0 and g = g_min = -5 exactly."""
    assert gate_fn(0.0, 0.0) == -2.5
    assert gate_fn(0.7, 0.0) == -2.5
    assert gate_fn(0.0, Z_ALPHA_ONE) == 0.0
    assert gate_fn(0.3, Z_ALPHA_MIN) == -5.0
    # textbook logistic from scipy
    for a, z in [(0.0, 1.0), (-1.0, 2.5), (0.9, -3.0), (0.25, 0.125)]:
        want = -5.0 * expit(np.exp(a) * z)
        assert abs(gate_fn(a, z) - want) <= 4e-16 * 5, (a, z)


# --------------------------------------------------------------------------
# Special cases of the recurrence
# --------------------------------------------------------------------------
def check_constant_state(run):
    """alpha = 1 and beta = 0: the state never changes and o_t = h0^T q_t."""
    d = rand_inputs(11, [37, 0, 20], H=2, dk=8, dv=6, h0_std=1.0)
    d["z"][:] = Z_ALPHA_ONE
    d["beta"][:] = 0.0
    o, hT = call(run, d)
    assert np.array_equal(hT, d["h0"].astype(np.float64))
    cu = d["cu"]
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1]):
            for h in range(2):
                want = d["h0"][n, h].astype(np.float64) @ d["q"][t, h].astype(np.float64)
                assert np.allclose(o[t, h], want, rtol=1e-13, atol=1e-13)


def check_decay_only(run):
    """beta = 0: pure channel-wise decay, o_t = h0^T (Gamma_t * q_t) with
    Gamma_t = exp(sum_{j<=t} g_j) and hT = Diag(Gamma_T) h0."""
    d = rand_inputs(12, [29, 17], H=3, dk=8, dv=5, h0_std=1.0)
    d["beta"][:] = 0.0
    o, hT = call(run, d)
    g = oracle.gate(d["A"], d["z"])            # [T, H, dk]
    cu = d["cu"]
    for n in range(2):
        G = np.cumsum(g[cu[n]:cu[n + 1]], axis=0)   # inclusive
        for h in range(3):
            h0 = d["h0"][n, h].astype(np.float64)   # [dv, dk]
            for r, t in enumerate(range(cu[n], cu[n + 1])):
                want = h0 @ (np.exp(G[r, h]) * d["q"][t, h])
                assert np.allclose(o[t, h], want, rtol=1e-12, atol=1e-14)
            assert np.allclose(hT[n, h], h0 * np.exp(G[-1, h])[None, :], rtol=1e-12,
                               atol=1e-300)


def check_deltanet(run):
    """alpha = 1 reduces KDA to the delta rule (P1 "Delta Networks", with the
    write strength beta of P1's gated line), in P1's value-by-key state
    orientation: S <- S + beta (v - S k) k^T, o = S q."""
    d = rand_inputs(13, [41], H=2, dk=16, dv=12, h0_std=0.5)
    d["z"][:] = Z_ALPHA_ONE
    o, hT = call(run, d)
    for h in range(2):
        S = d["h0"][0, h].astype(np.float64)       # dv x dk, P1's orientation
        for t in range(41):
            kt = d["k"][t, h].astype(np.float64)
            vt = d["v"][t, h].astype(np.float64)
            qt = d["q"][t, h].astype(np.float64)
            S = S + float(d["beta"][t, h]) * np.outer(vt - S @ kt, kt)
            assert np.allclose(o[t, h], S @ qt, rtol=1e-12, atol=1e-12), t
        assert np.allclose(hT[0, h], S, rtol=1e-12, atol=1e-12)


def check_gdn(run):
    """A decay that is the same on every key channel reduces KDA to Gated
    DeltaNet in the form P1 sets beside KDA ("对比GDN的公式"):
    S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T."""
    d = rand_inputs(14, [33], H=2, dk=8, dv=8, h0_std=0.3)
    d["z"][:] = d["z"][:, :, :1]                    # constant across channels
    o, hT = call(run, d)
    g = oracle.gate(d["A"], d["z"])[:, :, 0]
    for h in range(2):
        S = d["h0"][0, h].astype(np.float64).T      # dk x dv
        for t in range(33):
            kt = d["k"][t, h].astype(np.float64)
            b = float(d["beta"][t, h])
            S = np.exp(g[t, h]) * (np.eye(8) - b * np.outer(kt, kt)) @ S \
                + b * np.outer(kt, d["v"][t, h].astype(np.float64))
            assert np.allclose(o[t, h], S.T @ d["q"][t, h], rtol=1e-12, atol=1e-12)
        assert np.allclose(hT[0, h], S.T, rtol=1e-12, atol=1e-12)


def check_product_form(run):
    """Eq 1 of P3 §3.1 (also P1 "Kimi Delta Attention", P5 §3.1) with explicit
    matrices: S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,
    o_t = S_t^T q_t -- including the single-token closed form."""
    d = rand_inputs(15, [1, 9], H=2, dk=6, dv=7, h0_std=0.8)
    o, hT = call(run, d)
    alpha = np.exp(oracle.gate(d["A"], d["z"]))
    cu = d["cu"]
    for n in range(2):
        for h in range(2):
            S = d["h0"][n, h].astype(np.float64).T
            for t in range(cu[n], cu[n + 1]):
                kt = d["k"][t, h].astype(np.float64)
                b = float(d["beta"][t, h])
                S = (np.eye(6) - b * np.outer(kt, kt)) @ np.diag(alpha[t, h]) @ S \
                    + b * np.outer(kt, d["v"][t, h])
                assert np.allclose(o[t, h], S.T @ d["q"][t, h], rtol=1e-12, atol=1e-13)
            assert np.allclose(hT[n, h], S.T, rtol=1e-12, atol=1e-13)


def _exact_unit_keys(r, T, dk):
    """Unit vectors that are exact in binary: four entries of +-1/2."""
    k = np.zeros((T, dk), dtype=np.float32)
    for t in range(T):
        idx = r.choice(dk, size=4, replace=False)
        k[t, idx] = r.choice([-0.5, 0.5], size=4)
    return k


def check_exact_write(run):
    """Unit-norm k and beta = 1 write v exactly: S_t^T k_t = v_t.  Reading
    with q = k therefore returns o_t = v_t (P2's prediction-error view: the
    error of the new state on its own key is zero)."""
    r = rng(16)
    d = rand_inputs(16, [24, 24], H=2, dk=16, dv=10, h0_std=1.0)
    for h in range(2):
        d["k"][:, h] = _exact_unit_keys(r, 48, 16)
    d["q"] = d["k"].copy()
    d["beta"][:] = 1.0
    o, _ = call(run, d)
    assert np.allclose(o, d["v"].astype(np.float64), rtol=0, atol=1e-13)


def check_linear_attention(run):
    """alpha = 1, beta = 1, h0 = 0 and orthonormal keys: every prediction
    error is the value itself, so KDA is plain linear attention (P1
    "Linear attn"): o_t = sum_{i<=t} (q_t . k_i) v_i."""
    dk, T = 16, 12
    Hd = hadamard(dk).astype(np.float32) / 4.0          # exactly orthonormal rows
    r = rng(17)
    d = rand_inputs(17, [T], H=1, dk=dk, dv=5)
    d["k"][:, 0] = Hd[r.permutation(dk)[:T]]
    d["z"][:] = Z_ALPHA_ONE
    d["beta"][:] = 1.0
    o, _ = call(run, d)
    q = d["q"][:, 0].astype(np.float64)
    k = d["k"][:, 0].astype(np.float64)
    v = d["v"][:, 0].astype(np.float64)
    want = np.tril(q @ k.T) @ v
    assert np.allclose(o[:, 0], want, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# A second algorithm and exact identities
# --------------------------------------------------------------------------
def check_chunkwise(run):
    """The chunkwise form of P1 ("Chunkwise 形式") equals the token loop for
    every chunk size, with partial chunks, an empty sequence and h0."""
    d = rand_inputs(18, [70, 0, 5, 64, 33], H=2, dk=8, dv=6, h0_std=0.5)
    o, hT = call(run, d)
    for C in (1, 3, 16, 64):
        oc, hc = chunkwise.prefill(d["q"], d["k"], d["v"], d["z"], d["A"], d["beta"],
                                   d["h0"], d["cu"], chunk=C)
        assert rel_l2(oc, o) < 1e-12 and rel_l2(hc, hT) < 1e-12, C


def check_split_and_carry(run):
    """Running T1 tokens, carrying hT as h0, then T2 tokens equals one run of
    T1 + T2 (the prefill -> decode state handoff of P5 §11.1-11.2)."""
    d = rand_inputs(19, [50], H=2, dk=8, dv=8, h0_std=0.2)
    o, hT = call(run, d)
    t1 = 23
    part = lambda a, s: a[s]
    d1 = dict(d, q=d["q"][:t1], k=d["k"][:t1], v=d["v"][:t1], z=d["z"][:t1],
              beta=d["beta"][:t1], cu=np.array([0, t1], np.int32))
    o1, h1 = call(run, d1)
    d2 = dict(d, q=d["q"][t1:], k=d["k"][t1:], v=d["v"][t1:], z=d["z"][t1:],
              beta=d["beta"][t1:], h0=h1, cu=np.array([0, 50 - t1], np.int32))
    o2, h2 = call(run, d2)
    assert np.allclose(np.concatenate([o1, o2]), o, rtol=1e-14, atol=1e-15)
    assert np.allclose(h2, hT, rtol=1e-14, atol=1e-15)
    del part


def check_varlen_packing(run):
    """Packed sequences equal separate runs; an empty sequence keeps h0."""
    lens = [9, 0, 31, 1]
    d = rand_inputs(20, lens, H=2, dk=8, dv=4, h0_std=0.4)
    o, hT = call(run, d)
    cu = d["cu"]
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        dn = dict(q=d["q"][sl], k=d["k"][sl], v=d["v"][sl], z=d["z"][sl], A=d["A"],
                  beta=d["beta"][sl], h0=d["h0"][n:n + 1],
                  cu=np.array([0, lens[n]], np.int32))
        on, hn = call(run, dn)
        assert np.allclose(on, o[sl], rtol=1e-15, atol=0)
        assert np.allclose(hn[0], hT[n], rtol=1e-15, atol=0)
    assert np.array_equal(hT[1], d["h0"][1].astype(np.float64))


def check_head_and_column_independence(run):
    """Heads are independent (permuting heads with their A_h permutes the
    outputs), and value channels are independent (the first dv/2 value
    channels of a run equal a run on those channels alone)."""
    d = rand_inputs(21, [19, 13], H=4, dk=8, dv=6, h0_std=0.3)
    o, hT = call(run, d)
    p = np.array([2, 0, 3, 1])
    dp = dict(d, q=d["q"][:, p], k=d["k"][:, p], v=d["v"][:, p], z=d["z"][:, p],
              A=d["A"][p], beta=d["beta"][:, p], h0=d["h0"][:, p])
    op, hp = call(run, dp)
    assert np.allclose(op, o[:, p], rtol=1e-15, atol=0)
    assert np.allclose(hp, hT[:, p], rtol=1e-15, atol=0)
    dh = dict(d, v=np.ascontiguousarray(d["v"][:, :, :3]),
              h0=np.ascontiguousarray(d["h0"][:, :, :3]))
    oh, hh = call(run, dh)
    assert np.allclose(oh, o[:, :, :3], rtol=1e-13, atol=1e-15)
    assert np.allclose(hh, hT[:, :, :3], rtol=1e-13, atol=1e-15)


def check_kcp_affine(run):
    """P3 §8.1, Eq 17 (KDA context parallelism): a segment maps its input
    state affinely, S_out = M S_in + S~, with M = prod_t (I - beta_t k_t
    k_t^T) Diag(alpha_t) and S~ the state reached from zero.  M is built here
    from explicit transition matrices; S~ and S_out come from the runner."""
    d = rand_inputs(22, [27], H=1, dk=6, dv=5, h0_std=1.0)
    alpha = np.exp(oracle.gate(d["A"], d["z"]))
    M = np.eye(6)
    for t in range(27):
        kt = d["k"][t, 0].astype(np.float64)
        Mt = (np.eye(6) - float(d["beta"][t, 0]) * np.outer(kt, kt)) @ np.diag(alpha[t, 0])
        M = Mt @ M
    _, h_zero = call(run, dict(d, h0=None))
    _, h_in = call(run, d)
    S_in = d["h0"][0, 0].astype(np.float64).T        # dk x dv
    want = M @ S_in + h_zero[0, 0].T
    assert np.allclose(h_in[0, 0].T, want, rtol=1e-12, atol=1e-13)


def check_decay_window_bound(run):
    """P3 §3.2 / P5 §3.2: any 16 consecutive tokens accumulate a log-decay
    in (-80, 0) on every channel, so relative rescale factors stay below e^80.
    Checked on the gate values the runner's decay implies: with beta = 0 and
    h0 = I-like probes, hT = Diag(exp(sum g)) h0 exposes the window sums."""
    r = rng(23)
    d = rand_inputs(23, [16] * 8, H=2, dk=8, dv=8, h0_std=None)
    d["z"] = (r.standard_normal(d["z"].shape) * 4.0).astype(np.float32)
    d["beta"][:] = 0.0
    eye = np.broadcast_to(np.eye(8, dtype=np.float32), (8, 2, 8, 8)).copy()
    d["h0"] = eye
    _, hT = call(run, d)
    diag = np.einsum("nhii->nhi", hT)              # exp(window sum) per channel
    logs = np.log(diag)
    assert np.all(logs < 0.0) and np.all(logs > -80.0)


ALL_PREFILL_CHECKS = [
    check_constant_state, check_decay_only, check_deltanet, check_gdn,
    check_product_form, check_exact_write, check_linear_attention, check_chunkwise,
    check_split_and_carry, check_varlen_packing, check_head_and_column_independence,
    check_kcp_affine, check_decay_window_bound,
]
