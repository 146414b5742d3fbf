"""Pins of the oracle's fused epilogue  y = act(alpha*c + bias[n]) + beta*R[m, n].

The epilogue follows "gemm.rst" (alpha / beta: D = alpha*A@B + beta*C, with C
not read when beta is 0) and "Matmul2dFp4" (an optional per-element (row, col)
epilogue); the pages name no activation.  The pins below do not retype the
oracle's formulas: they compare with independent library routines (scipy's
logistic function and erf), with identities the definitions imply, and with
cases that tell the plausible misreadings apart (bias on the wrong axis,
activation after the residual, beta applied to the product).
"""
import math

import numpy as np
import pytest
from scipy import special

import oracle

ACTS = (oracle.ACT_NONE, oracle.ACT_RELU, oracle.ACT_SILU, oracle.ACT_GELU_TANH)
GRID = np.concatenate([np.linspace(-12.0, 12.0, 2401), [-60.0, -30.0, 30.0, 60.0, 0.0]])


def test_silu_is_x_times_logistic():
    for x in GRID:
        ref = x * special.expit(x)
        assert math.isclose(oracle.activation(oracle.ACT_SILU, x), ref, rel_tol=1e-14, abs_tol=1e-300)


def test_gelu_tanh_tracks_erf_gelu():
    # the tanh form approximates 0.5 x (1 + erf(x / sqrt 2)) to 4.7e-4; a wrong
    # constant (0.44715, no square root, pi/2 for 2/pi, no cubic term) misses
    # by more than 3e-2
    worst = max(abs(oracle.activation(oracle.ACT_GELU_TANH, x) - 0.5 * x * (1.0 + special.erf(x / math.sqrt(2.0))))
                for x in GRID)
    assert worst < 5e-4
    assert oracle.activation(oracle.ACT_GELU_TANH, 30.0) == 30.0
    assert abs(oracle.activation(oracle.ACT_GELU_TANH, -30.0)) < 1e-300 + 1e-30


@pytest.mark.parametrize("act", ACTS[1:])
def test_odd_part_identity(act):
    # relu, silu and the tanh-form gelu all satisfy act(x) - act(-x) = x
    for x in GRID:
        d = oracle.activation(act, x) - oracle.activation(act, -x)
        assert math.isclose(d, x, rel_tol=1e-13, abs_tol=1e-13)


def test_relu_and_identity():
    assert oracle.activation(oracle.ACT_RELU, -3.5) == 0.0
    assert oracle.activation(oracle.ACT_RELU, 2.25) == 2.25
    assert oracle.activation(oracle.ACT_NONE, -7.0) == -7.0
    assert math.isnan(oracle.activation(99, 1.0))


@pytest.mark.parametrize("act", ACTS)
def test_lipschitz_constants_bound_the_slope(act):
    x = np.linspace(-20.0, 20.0, 400001)
    y = np.array([oracle.activation(act, v) for v in x[::50]])
    slope = np.max(np.abs(np.diff(y) / np.diff(x[::50])))
    assert slope <= oracle.ACT_LIPSCHITZ[act]
    # and the constants are not loose by more than 3 %
    assert slope >= oracle.ACT_LIPSCHITZ[act] / 1.03


def _case(seed, M=5, N=7):
    rng = np.random.default_rng(seed)
    C = rng.standard_normal((M, N)) * 3.0
    bias_vals = rng.standard_normal(N)
    bias = np.array([oracle.round_bf16(v) for v in bias_vals], dtype=np.uint16)
    R = rng.standard_normal((M, N))
    return C, bias, R


def test_plain_settings_return_the_product():
    C, _, R = _case(0)
    assert np.array_equal(oracle.epilogue(C), C)
    assert np.array_equal(oracle.epilogue(C, 1.0, None, oracle.ACT_NONE, 0.0, R), C)


def test_alpha_scales_the_product():
    C, _, _ = _case(1)
    assert np.array_equal(oracle.epilogue(C, 4.0), 4.0 * C)
    assert np.array_equal(oracle.epilogue(C, -0.5), -0.5 * C)


def test_bias_runs_along_columns():
    C, bias, _ = _case(2)
    y = oracle.epilogue(C, 1.0, bias)
    for m in range(C.shape[0]):
        assert np.allclose(y[m] - C[m], oracle.bf16_values(bias), rtol=0, atol=1e-12)


def test_residual_is_added_after_the_activation():
    C = -np.ones((3, 4))
    R = np.full((3, 4), 5.0)
    # relu(-1) + 5 = 5; adding R before the activation would give relu(4) = 4
    assert np.array_equal(oracle.epilogue(C, 1.0, None, oracle.ACT_RELU, 1.0, R), np.full((3, 4), 5.0))
    # bias goes in before the activation: relu(-1 + 3) = 2
    bias = np.array([oracle.round_bf16(3.0)] * 4, dtype=np.uint16)
    assert np.array_equal(oracle.epilogue(C, 1.0, bias, oracle.ACT_RELU), np.full((3, 4), 2.0))


def test_beta_one_and_zero_as_in_the_gemm_primitive():
    C, _, R = _case(3)
    # beta = 1: D = A@B + C
    assert np.allclose(oracle.epilogue(C, 1.0, None, oracle.ACT_NONE, 1.0, R), C + R, rtol=0, atol=1e-15)
    # beta = 0: the input C is not read (NaNs in it do not propagate)
    Rnan = np.full_like(R, np.nan)
    assert np.array_equal(oracle.epilogue(C, 1.0, None, oracle.ACT_NONE, 0.0, Rnan), C)


def _fp32_epilogue(C, alpha, bias, act, beta, R):
    """An fp32 implementation of the same epilogue (what a kernel does)."""
    c = np.asarray(C, np.float32)
    v = np.float32(alpha) * c
    if bias is not None:
        v = v + oracle.bf16_values(bias).astype(np.float32)[None, :]
    if act == oracle.ACT_RELU:
        v = np.maximum(v, np.float32(0))
    elif act == oracle.ACT_SILU:
        v = v / (np.float32(1) + np.exp(-v))
    elif act == oracle.ACT_GELU_TANH:
        k = np.float32(math.sqrt(2.0 / math.pi))
        v = np.float32(0.5) * v * (np.float32(1) + np.tanh(k * (v + np.float32(0.044715) * v * v * v)))
    if R is not None and beta != 0.0:
        v = v + np.float32(beta) * np.asarray(R, np.float32)
    return v.astype(np.float64)


@pytest.mark.parametrize("act", ACTS)
def test_gate_accepts_fp32_epilogue_and_rejects_misreadings(act):
    C, bias, R = _case(10 + act, M=8, N=9)
    S = np.abs(C) * 4.0 + 1.0  # a plausible sum of |a w|
    alpha, beta = 0.75, 1.5
    Y = oracle.epilogue(C, alpha, bias, act, beta, R)
    ok = _fp32_epilogue(C, alpha, bias, act, beta, R)
    assert oracle.epilogue_gate_ratio(ok, C, S, alpha, bias, act, beta, R, Y, bf16_out=False) <= 1.0
    bf = np.array([oracle.bf16_value(oracle.round_bf16(v)) for v in ok.ravel()]).reshape(ok.shape)
    assert oracle.epilogue_gate_ratio(bf, C, S, alpha, bias, act, beta, R, Y, bf16_out=True) <= 1.0
    # plausible mistakes, each far outside the bound
    mistakes = {
        "alpha ignored": _fp32_epilogue(C, 1.0, bias, act, beta, R),
        "beta ignored": _fp32_epilogue(C, alpha, bias, act, 1.0, R),
        "bias dropped": _fp32_epilogue(C, alpha, None, act, beta, R),
        "residual dropped": _fp32_epilogue(C, alpha, bias, act, beta, None),
    }
    if act != oracle.ACT_NONE:
        mistakes["activation dropped"] = _fp32_epilogue(C, alpha, bias, oracle.ACT_NONE, beta, R)
        mistakes["residual inside the activation"] = _fp32_epilogue(
            C + (beta / alpha) * R, alpha, bias, act, 0.0, None)
    for name, y in mistakes.items():
        assert oracle.epilogue_gate_ratio(y, C, S, alpha, bias, act, beta, R, Y, bf16_out=False) > 1.0, name
