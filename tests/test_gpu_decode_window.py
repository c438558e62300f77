"""Multi-token decode with replay: HIP kernel vs the fp64 oracle.

The expected values come from the oracle's token recurrence: the committed
state is the recurrence over each sequence's accepted replay tokens, and the
window outputs continue from it."""
import numpy as np
import pytest
import torch

import gated_delta_rule_21_amd as kda
import oracle
from gated_delta_rule_21_amd import workloads as W
from gpu_util import host, rel_l2, tol

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-6   # rel-L2 of the fp32 state after a few fp32 token updates


def _pack(t, lens):
    """[N][len][H][...] -> the first lens[n] tokens of every sequence, packed."""
    return torch.cat([t[n, :lens[n]] for n in range(t.shape[0])], 0)


def oracle_window(d, commit_window=False):
    """(o [N, L, H, dv] or None, state written back) from the oracle."""
    N, H = d["N"], d["H"]
    A = W.as_numpy(d["A"])
    S = W.as_numpy(d["S"]).astype(np.float64)
    acc = d["n_accept"].tolist() if d["Lr"] > 0 else [0] * N
    if sum(acc) > 0:
        rp = d["replay"]
        kr = W.as_numpy(_pack(rp["k"], acc))
        _, S = oracle.prefill(kr, kr, W.as_numpy(_pack(rp["v"], acc)), W.as_numpy(_pack(rp["z"], acc)), A,
                              W.as_numpy(_pack(rp["beta"], acc)), S, W.as_numpy(W.cu_from_lengths(acc)))
    L = d["L"]
    if L == 0:
        return None, S
    wn = d["window"]
    flat = lambda t: W.as_numpy(t.reshape(N * L, *t.shape[2:]))
    o, Sw = oracle.prefill(flat(wn["q"]), flat(wn["k"]), flat(wn["v"]), flat(wn["z"]), A, flat(wn["beta"]), S,
                           W.as_numpy(W.cu_from_lengths([L] * N)))
    return o.reshape(N, L, H, -1), (Sw if commit_window else S)


def to_gpu(d):
    g = dict(d)
    for key in ("A", "S", "n_accept"):
        g[key] = d[key].cuda()
    for key in ("replay", "window"):
        g[key] = {n: t.cuda() for n, t in d[key].items()}
    return g


def gpu_window(g, commit_window=False):
    S = g["S"].clone()
    o = kda.decode_window(g["A"], S, window=g["window"] if g["L"] > 0 else None,
                          replay=g["replay"] if g["Lr"] > 0 else None, n_accept=g["n_accept"],
                          commit_window=commit_window)
    torch.cuda.synchronize()
    return o, S


def check(d, io, commit_window=False, label=""):
    o, S = gpu_window(to_gpu(d), commit_window)
    ro, rS = oracle_window(d, commit_window)
    eS = rel_l2(host(S), rS)
    eo = rel_l2(host(o), ro) if ro is not None else 0.0
    print("%s rel-L2 o=%.3e S=%.3e" % (label, eo, eS), flush=True)
    assert eS <= STATE_TOL, eS
    assert eo <= tol(io), eo


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_replay_and_window(io, d):
    inp = W.random_decode_window(6, 3, d, Lr=4, L=3, io=io, seed=900 + d)
    inp["n_accept"] = torch.tensor([0, 4, 2, 1, 4, 3], dtype=torch.int32)
    check(inp, io, label="window %s d=%d" % (io, d))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_commit_window(io):
    inp = W.random_decode_window(5, 4, 128, Lr=3, L=5, io=io, seed=910)
    check(inp, io, commit_window=True, label="commit %s" % io)


def test_longest_windows():
    inp = W.random_decode_window(4, 2, 64, Lr=16, L=16, io="bf16", seed=911)
    inp["n_accept"] = torch.tensor([16, 0, 9, 16], dtype=torch.int32)
    check(inp, "bf16", label="Lr=L=16")


def test_commit_only_and_window_only():
    inp = W.random_decode_window(5, 3, 128, Lr=5, L=0, io="bf16", seed=912)
    check(inp, "bf16", label="replay only")
    inp = W.random_decode_window(5, 3, 128, Lr=0, L=6, io="bf16", seed=913)
    check(inp, "bf16", label="window only")


def test_out_of_range_accept_is_clamped():
    inp = W.random_decode_window(4, 2, 32, Lr=3, L=2, io="f32", seed=914)
    g = to_gpu(inp)
    g["n_accept"] = torch.tensor([-5, 7, 3, 0], dtype=torch.int32, device="cuda")
    o, S = gpu_window(g)
    inp["n_accept"] = torch.tensor([0, 3, 3, 0], dtype=torch.int32)
    ro, rS = oracle_window(inp)
    assert rel_l2(host(S), rS) <= STATE_TOL
    assert rel_l2(host(o), ro) <= tol("f32")


def test_nothing_accepted_leaves_state_untouched():
    inp = W.random_decode_window(8, 3, 128, Lr=4, L=4, io="bf16", seed=915)
    inp["n_accept"][:] = 0
    o, S = gpu_window(to_gpu(inp))
    assert torch.equal(S.cpu(), inp["S"])


def test_single_token_window_is_a_decode_step():
    """Lr = 0, L = 1, commit: the same update as kda_decode."""
    inp = W.random_decode_window(7, 3, 128, Lr=0, L=1, io="bf16", seed=916)
    g = to_gpu(inp)
    o, S = gpu_window(g, commit_window=True)
    w = g["window"]
    S2 = g["S"].clone()
    o2 = kda.decode(w["q"][:, 0].contiguous(), w["k"][:, 0].contiguous(), w["v"][:, 0].contiguous(),
                    w["z"][:, 0].contiguous(), g["A"], w["beta"][:, 0].contiguous(), S2)
    torch.cuda.synchronize()
    assert rel_l2(host(S), host(S2)) <= STATE_TOL
    assert rel_l2(host(o[:, 0]), host(o2)) <= tol("bf16")
    check(inp, "bf16", commit_window=True, label="one token")


def test_serving_loop_matches_the_accepted_token_stream():
    """Three speculative steps: each call replays the accepted part of the
    previous window and runs the next one.  The committed state and every
    window output match the oracle over the accepted token stream."""
    N, H, d, L = 6, 3, 128, 4
    steps = [W.random_decode_window(N, H, d, Lr=0, L=L, io="bf16", seed=920 + i) for i in range(4)]
    A, S0 = steps[0]["A"], steps[0]["S"]
    gA, S = A.cuda(), S0.clone().cuda()
    accepted = [torch.randint(0, L + 1, (N,), generator=torch.Generator().manual_seed(930 + i),
                              dtype=torch.int32) for i in range(3)]
    prev = None
    S_ref = S0.numpy().astype(np.float64)
    for i in range(3):
        win = {n: t.cuda() for n, t in steps[i]["window"].items()}
        o = kda.decode_window(gA, S, window=win, replay=prev,
                              n_accept=accepted[i - 1].cuda() if prev is not None else None)
        torch.cuda.synchronize()
        # oracle: the state committed by this call's replay of the previous
        # window, then this window's outputs from it
        if prev is not None:
            acc = accepted[i - 1].tolist()
            rp = steps[i - 1]["window"]
            kr = W.as_numpy(_pack(rp["k"], acc))
            _, S_ref = oracle.prefill(kr, kr, W.as_numpy(_pack(rp["v"], acc)), W.as_numpy(_pack(rp["z"], acc)),
                                      W.as_numpy(A), W.as_numpy(_pack(rp["beta"], acc)), S_ref,
                                      W.as_numpy(W.cu_from_lengths(acc)))
            assert rel_l2(host(S), S_ref) <= STATE_TOL
        flat = lambda t: W.as_numpy(t.reshape(N * L, *t.shape[2:]))
        wn = steps[i]["window"]
        ro, _ = oracle.prefill(flat(wn["q"]), flat(wn["k"]), flat(wn["v"]), flat(wn["z"]), W.as_numpy(A),
                               flat(wn["beta"]), S_ref, W.as_numpy(W.cu_from_lengths([L] * N)))
        assert rel_l2(host(o), ro.reshape(N, L, H, d)) <= tol("bf16")
        prev = {n: win[n] for n in ("k", "v", "z", "beta")}


def test_k3_spec_decode_shape():
    """256 sequences x 96 heads x 128^2, replay 4 (random acceptance), window 4;
    the oracle on 12 sampled sequences."""
    inp = W.random_decode_window(256, 96, 128, Lr=4, L=4, io="bf16", seed=940)
    o, S = gpu_window(to_gpu(inp))
    sel = [0, 17, 40, 63, 99, 128, 150, 177, 200, 222, 240, 255]
    sub = dict(inp, N=len(sel), S=inp["S"][sel], n_accept=inp["n_accept"][sel],
               replay={n: t[sel] for n, t in inp["replay"].items()},
               window={n: t[sel] for n, t in inp["window"].items()})
    ro, rS = oracle_window(sub)
    eo, eS = rel_l2(host(o[sel]), ro), rel_l2(host(S[sel]), rS)
    print("k3 spec decode rel-L2 o=%.3e S=%.3e" % (eo, eS), flush=True)
    assert eS <= STATE_TOL and eo <= tol("bf16")
