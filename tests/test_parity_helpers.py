"""CPU checks of the comparison helpers the GPU parity tests use: the bf16
rounding of the oracle matches torch's round-to-nearest-even conversion, and
each measure catches the kind of mistake it is there for."""
import numpy as np
import pytest
import torch

from gpu_util import (BF16_COMPUTE_TOL, bf16_half_ulp, bf16_rne, check_gated_elements, compare_outputs,
                      compare_states)


def test_bf16_rne_matches_torch():
    r = np.random.Generator(np.random.PCG64(3))
    x = (r.standard_normal(200000) * np.exp(r.uniform(-20, 20, 200000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_rne(x.astype(np.float64)), want)


def test_bf16_rne_ties_and_carry():
    one = 1.0
    assert bf16_rne(one + 2.0 ** -8) == 1.0                      # tie, to the even neighbour
    assert bf16_rne(one + 3 * 2.0 ** -8) == one + 2.0 ** -6      # tie, to the even neighbour above
    assert bf16_rne(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    assert bf16_rne(2.0 - 2.0 ** -9) == 2.0                      # carry into the next binade
    assert bf16_rne(-1.5) == -1.5 and bf16_rne(0.0) == 0.0
    assert bf16_half_ulp(1.0) == 2.0 ** -8 and bf16_half_ulp(1.99) == 2.0 ** -8
    assert bf16_half_ulp(0.75) == 2.0 ** -9 and bf16_half_ulp(0.0) == 0.0


def _case(seed=0, T=300, H=3, d=32):
    r = np.random.Generator(np.random.PCG64(seed))
    y = r.standard_normal((T, H, d))
    return y, bf16_rne(y)


def test_exact_rounding_passes_every_measure():
    y, x = _case()
    m = compare_outputs(x, y, "bf16", cu=[0, 100, 100, 300])
    assert m["compute"] == 0.0 and m["elem_max"] == 0.0 and m["excess_rel"] == 0.0
    assert 1.4e-3 < m["rel"] < 1.8e-3       # the rounding alone


def test_one_wrong_element_fails_elementwise():
    y, x = _case()
    x[123, 1, 5] = bf16_rne(y[123, 1, 5] + 0.02 * max(abs(y[123, 1, 5]), np.sqrt(np.mean(y[:, 1] ** 2))))
    with pytest.raises(AssertionError, match=r"element \[123, 1, 5\]"):
        compare_outputs(x, y, "bf16")


def test_one_wrong_head_of_one_sequence_fails_per_unit():
    # a 2 % error on one (sequence, head) of a long tensor: the whole-tensor
    # rel-L2 stays under 2e-3, the per-(sequence, head) measure does not
    y, _ = _case(T=4000, H=8)
    x = y.copy()
    x[3000:3040, 6] *= 1.02
    x = bf16_rne(x)
    assert np.linalg.norm(x - y) / np.linalg.norm(y) < 2e-3
    with pytest.raises(AssertionError, match="sequence 1 head 6"):
        compare_outputs(x, y, "bf16", cu=[0, 3000, 3040, 4000])


def test_small_compute_error_fails_compute_only():
    # a uniform relative error of 1e-3 before the final rounding: the plain
    # rel-L2 (rounding included) stays under 2e-3, the compute-only one not
    y, _ = _case(T=2000)
    x = bf16_rne(y * (1 + 1e-3))
    assert np.linalg.norm(x - y) / np.linalg.norm(y) < 2e-3
    with pytest.raises(AssertionError, match="compute-only|rounding-excess"):
        compare_outputs(x, y, "bf16")
    assert np.linalg.norm(x - bf16_rne(y)) / np.linalg.norm(bf16_rne(y)) > BF16_COMPUTE_TOL


def test_errors_beyond_rounding_fail_the_excess_measure():
    # 2e-3 relative noise before the rounding: most of it exceeds what one
    # rounding explains
    y, _ = _case(T=2000)
    r = np.random.Generator(np.random.PCG64(9))
    x = bf16_rne(y * (1 + 2e-3 * r.standard_normal(y.shape)))
    with pytest.raises(AssertionError, match="rounding-excess|compute-only|rel-L2"):
        compare_outputs(x, y, "bf16")


def test_states_per_unit_and_exact_zero():
    r = np.random.Generator(np.random.PCG64(1))
    y = r.standard_normal((3, 4, 8, 8))
    y[1, 2] = 0.0
    x = y + 1e-7 * r.standard_normal(y.shape)
    x[1, 2] = 0.0
    compare_states(x, y, "bf16")
    x2 = x.copy()
    x2[2, 3] *= 1.004                      # one (sequence, head) off by 4e-3
    with pytest.raises(AssertionError, match="sequence 2 head 3"):
        compare_states(x2, y, "bf16", whole_bar=1.0)
    x3 = x.copy()
    x3[1, 2, 0, 0] = 1e-30
    with pytest.raises(AssertionError, match="exactly zero"):
        compare_states(x3, y, "bf16")


def test_gated_element_bound():
    """The rounding of an exact gated output passes; an error of 5 % of an
    element's scale (|Sigmoid(g) w| max(|o|, U) / r) fails."""
    r = np.random.Generator(np.random.PCG64(4))
    eps, cu = 1e-6, [0, 10, 40]
    o, g, w = r.standard_normal((40, 2, 32)), 2 * r.standard_normal((40, 2, 32)), 1 + 0.1 * r.standard_normal(32)
    rr = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    y = w / (1 + np.exp(-g)) * o / rr
    assert check_gated_elements(bf16_rne(y), y, o, g, w, eps, cu) < 0.5
    U = np.sqrt(np.mean(o[10:] ** 2, axis=(0, 2)))[1]
    x = bf16_rne(y)
    x[20, 1, 3] = y[20, 1, 3] + 0.05 * abs(w[3] / (1 + np.exp(-g[20, 1, 3]))) * max(abs(o[20, 1, 3]), U) / rr[20, 1, 0]
    with pytest.raises(AssertionError, match="gated element"):
        check_gated_elements(x, y, o, g, w, eps, cu)
