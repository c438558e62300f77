"""The seeded workload generators (CPU): the shapes the bench and the parity
tests run, the lognormal length mix of the varlen batch, reproducibility
from the seed, and the input recipe the generators promise (unit-norm q and
k, beta in (0, 1), one A per head).  The K3 shapes are checked from their
registry entries and from a few generated rows, without drawing the full
tensors."""
import math

import numpy as np
import pytest
import torch

from gated_delta_rule_21_amd import workloads as W


def test_registry_shapes():
    k3 = W.WORKLOADS["k3_prefill"]
    assert (k3.kind, k3.N, k3.H, k3.d, k3.io, k3.lens) == ("prefill", 1, 96, 128, "bf16", (65536,))
    dec = W.WORKLOADS["k3_decode"]
    assert (dec.kind, dec.N, dec.H, dec.d) == ("decode", 256, 96, 128)
    var = W.WORKLOADS["k3_varlen"]
    assert (var.N, var.H, var.d, var.lognormal_total) == (32, 96, 128, 262144)
    sh = W.WORKLOADS["small_head"]
    assert (sh.N, sh.H, sh.d, sh.lens) == (2, 8, 128, (8192, 8192))
    assert len({w.index for w in W.WORKLOADS.values()}) == len(W.WORKLOADS)


def test_varlen_lengths():
    """32 lengths, every one at least 1, summing exactly to 262,144; the mix is
    lognormal (a wide spread: the longest several times the mean); the same
    seed gives the same lengths and another seed others."""
    var = W.WORKLOADS["k3_varlen"]
    lens = W.seq_lengths(var)
    assert len(lens) == 32 and sum(lens) == 262144 and min(lens) >= 1
    assert max(lens) > 4 * (262144 / 32)
    logs = np.log(np.array(lens, dtype=np.float64))
    assert 0.5 < logs.std() < 1.6              # sigma = 1 up to sampling and the rescale
    assert W.seq_lengths(var) == lens
    assert W.seq_lengths(var, seed=W.BASE_SEED + 99) != lens
    assert W.lognormal_lengths(5, 5, seed=3) == [1, 1, 1, 1, 1]


def test_cu_seqlens():
    cu = W.cu_from_lengths([3, 0, 5])
    assert cu.dtype == torch.int32 and cu.tolist() == [0, 3, 3, 8]


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_random_prefill_recipe(io):
    lens = [70, 0, 5]
    d = W.random_prefill(lens, 3, 32, io, h0_std=0.05, seed=123)
    T = sum(lens)
    dt = W.torch_dtype(io)
    assert d["q"].shape == (T, 3, 32) and d["q"].dtype == dt
    assert d["k"].dtype == dt and d["v"].dtype == dt
    assert d["z"].dtype == torch.float32 and d["z"].shape == (T, 3, 32)
    assert d["beta"].shape == (T, 3) and d["A"].shape == (3,)
    assert d["h0"].shape == (3, 3, 32, 32)
    assert d["cu_seqlens"].tolist() == [0, 70, 70, 75]
    # unit-norm q and k per (token, head), up to the io rounding
    for n in ("q", "k"):
        norms = d[n].double().norm(dim=-1)
        tol = 1e-2 if io == "bf16" else 1e-6
        assert torch.allclose(norms, torch.ones_like(norms), atol=tol)
    assert float(d["beta"].min()) > 0 and float(d["beta"].max()) < 1
    assert float(d["A"].abs().max()) <= 1
    # reproducible from the seed, different for another
    again = W.random_prefill(lens, 3, 32, io, h0_std=0.05, seed=123)
    other = W.random_prefill(lens, 3, 32, io, h0_std=0.05, seed=124)
    assert torch.equal(again["v"], d["v"]) and torch.equal(again["z"], d["z"])
    assert not torch.equal(other["v"], d["v"])


def test_random_prefill_without_h0():
    d = W.random_prefill([10], 2, 32, "bf16", h0_std=None, seed=5)
    assert d["h0"] is None
