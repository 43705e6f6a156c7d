"""Pins for the element-importance weightings of the oracle.

Source: "ik_llama.cpp 量化权重之谜：weight[j] = qw[j] * sqrtf(sigma2 + xb[j]*xb[j])
的由来与原理", section 一 (the chosen form and the plain alternative weight =
qw) and section 二 (magnitude forms tried before it: x^2, |x|, sigma^2 + x^2,
sigma + |x|).

Checked against closed forms on exactly representable values, against the
block solver called directly with the weights a mode implies, and against
invariances that hold for every mode.
"""
import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

F32 = np.float32
MODES = list(oracle.WEIGHTINGS)


def test_closed_forms_on_exact_values():
    rng = np.random.default_rng(101)
    x = (rng.integers(-64, 65, 256) * 2.0 ** -6).astype(F32)
    q = (2.0 ** rng.integers(-3, 4, 256)).astype(F32)
    s2 = F32(0.25)                                  # sigma = 0.5 exactly
    xd, qd = x.astype(np.float64), q.astype(np.float64)
    want = {
        "x2": qd * xd * xd,
        "abs_x": qd * np.abs(xd),
        "sigma2_plus_x2": qd * (xd * xd + 0.25),
        "sigma_plus_abs_x": qd * (0.5 + np.abs(xd)),
        "imatrix_only": qd,
    }
    for mode, w in want.items():
        got = oracle.row_weights_mode(x, q, s2, mode).astype(np.float64)
        assert np.array_equal(got, w), mode
        got1 = oracle.row_weights_mode(x, None, s2, mode).astype(np.float64)
        assert np.array_equal(got1, w / qd), mode
    # the default form is the pages' formula
    got = oracle.row_weights_mode(x, q, s2, "sqrt_sigma2_x2")
    assert np.array_equal(got, oracle.row_weights(x, q, s2))


def test_imatrix_only_without_imatrix_is_the_unweighted_fit():
    # weight = qw with no imatrix is weight 1 for every element: each block
    # must be what the block solver gives with unit weights
    x, _ = synth.q4_0_matrix(4, 256, seed=102)
    out = oracle.quantize_rows_weighted("q4_0", x, None, "imatrix_only")
    ones = np.ones(32, F32)
    for r in range(4):
        for b in range(8):
            l, d, _ = oracle.solve_sym(x[r, 32 * b:32 * b + 32], ones, 8)
            blk = out[r, 20 * b:20 * b + 20]
            assert np.frombuffer(bytes(blk[:4]), F32)[0] == d
            u = l.astype(np.int64) + 8
            assert list(blk[4:]) == [int(u[i] | (u[i + 16] << 4)) for i in range(16)]


@pytest.mark.parametrize("mode", MODES)
def test_each_mode_passes_its_weights_to_the_solver(mode):
    # Q4_1 blocks of one row against solve_asym called with the mode's
    # weights computed by the weight function
    x, q = synth.q4_0_matrix(1, 128, seed=103)
    s2 = oracle.row_sigma2(x[0])
    w = oracle.row_weights_mode(x[0], q, s2, mode)
    out = oracle.quantize_rows_weighted("q4_1", x, q, mode)
    for b in range(4):
        l, d, m, _ = oracle.solve_asym(x[0, 32 * b:32 * b + 32], w[32 * b:32 * b + 32], 15)
        blk = out[0, 24 * b:24 * b + 24]
        assert np.frombuffer(bytes(blk[:8]), F32).tolist() == [d, m]


@pytest.mark.parametrize("mode", MODES)
def test_zero_importance_groups_fall_back_per_mode(mode):
    x, q = synth.q4_0_matrix(3, 256, seed=104)
    q0 = q.copy()
    q0[64:96] = 0.0                                  # no data on one group
    a = oracle.quantize_rows_weighted("q4_k", x, q0, mode)
    q1 = q.copy()
    q1[64:96] = 1.0                                  # unit importances there
    b = oracle.quantize_rows_weighted("q4_k", x, q1, mode)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", MODES)
def test_power_of_two_scaling_scales_the_scales(mode):
    x, q = synth.q4_0_matrix(2, 256, seed=105)
    a = oracle.quantize_rows_weighted("q4_0", x, q, mode)
    b = oracle.quantize_rows_weighted("q4_0", x * F32(4.0), q, mode)
    da = a.reshape(-1, 20)[:, :4].copy().view(F32)
    db = b.reshape(-1, 20)[:, :4].copy().view(F32)
    assert np.array_equal(db, da * F32(4.0))
    assert np.array_equal(a.reshape(-1, 20)[:, 4:], b.reshape(-1, 20)[:, 4:])


def test_default_mode_is_the_plain_quantizer():
    x, q = synth.q4_k_matrix(8, 512, seed=106)
    for t in ("q4_0", "q5_1", "q4_k"):
        assert np.array_equal(oracle.quantize_rows_weighted(t, x, q, 0), oracle.quantize_rows(t, x, q))


def test_invalid_mode_is_rejected():
    x = np.ones((1, 32), F32)
    with pytest.raises(ValueError):
        oracle.quantize_rows_weighted("q4_0", x, None, 6)
