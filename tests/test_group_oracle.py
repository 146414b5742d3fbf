"""Pins of the oracle's int4 group size (formats INT4_G32 / INT4_G64).

The int4 page defines value = (code - zero[g]) * scale[g] with g the group of
`group` contiguous inputs (128 in its fixture).  These checks do not retype
that formula: they tie the group-32 / 64 oracle to the pinned group-128 one
through identities the definition implies, so that a wrong group index (k / G
vs k * G, the row stride of the scale array, an off-by-one group boundary)
fails one of them.
"""
import numpy as np
import pytest

import oracle
from weight_only_bit_w4a16_amd import inputs

SMALL = [oracle.INT4_G32, oracle.INT4_G64]


def _expand(arr, ratio):
    """Per-group array of the group-128 format repeated `ratio` times along K."""
    return np.repeat(arr, ratio, axis=1)


@pytest.mark.parametrize("fmt", SMALL)
def test_equal_group_parameters_reduce_to_group_128(fmt):
    # every small group of a 128-group carries that group's scale and zero:
    # the weights (exact and bf16) and the GEMM equal the group-128 ones
    N, K, M = 6, 384, 3
    case = inputs.make_case(oracle.INT4_G128, M, N, K, seed=11)
    ratio = 128 // oracle.GROUP[fmt]
    s_small, z_small = _expand(case.scales, ratio), _expand(case.zeros, ratio)
    w128, b128 = oracle.dequant(oracle.INT4_G128, case.packed, case.scales, case.zeros, N, K)
    w, b = oracle.dequant(fmt, case.packed, s_small, z_small, N, K)
    assert np.array_equal(w, w128) and np.array_equal(b, b128)
    C128, S128 = oracle.gemm(oracle.INT4_G128, case.A, case.packed, case.scales, case.zeros, M, N, K)
    C, S = oracle.gemm(fmt, case.A, case.packed, s_small, z_small, M, N, K)
    assert np.array_equal(C, C128) and np.array_equal(S, S128)


@pytest.mark.parametrize("fmt", SMALL)
def test_a_group_reaches_exactly_its_inputs(fmt):
    G = oracle.GROUP[fmt]
    N, K = 4, 256
    case = inputs.make_case(fmt, 0, N, K, seed=12)
    base, _ = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    for n, g in [(0, 0), (2, 1), (3, K // G - 1), (1, K // G // 2)]:
        s, z = case.scales.copy(), case.zeros.copy()
        s[n, g] = oracle.round_bf16(-3.0 * oracle.bf16_value(int(s[n, g])))
        z[n, g] = (int(z[n, g]) + 7) % 16
        w, _ = oracle.dequant(fmt, case.packed, s, z, N, K)
        changed = np.argwhere(w != base)
        assert changed.size, (n, g)
        assert np.all(changed[:, 0] == n)
        assert changed[:, 1].min() >= g * G and changed[:, 1].max() < (g + 1) * G


@pytest.mark.parametrize("fmt", SMALL)
def test_code_equal_to_zero_is_zero_and_steps_by_the_scale(fmt):
    G = oracle.GROUP[fmt]
    N, K = 3, 128
    case = inputs.make_case(fmt, 0, N, K, seed=13)
    # codes 0, 1, 2, ... cycling along k: neighbours inside a group differ by
    # one code, i.e. by exactly one scale
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w, _ = oracle.dequant(fmt, packed, case.scales, case.zeros, N, K)
    for n in range(N):
        for k in range(K - 1):
            g = k // G
            if (k + 1) // G != g or codes[n, k + 1] != codes[n, k] + 1:
                continue
            assert w[n, k + 1] - w[n, k] == oracle.bf16_value(int(case.scales[n, g]))
        for k in range(K):
            if codes[n, k] == case.zeros[n, k // G]:
                assert w[n, k] == 0.0


def test_ragged_last_group_is_the_shorter_rest():
    # K = 96 with groups of 64: group 0 covers k 0..63, group 1 the rest
    # (k 64..95) with its own scale and zero -- the same weights as groups of
    # 32 carrying (g0, g0, g1); likewise K = 160 with groups of 128
    for fmt, K, expand in ((oracle.INT4_G64, 96, [0, 0, 1]), (oracle.INT4_G128, 160, [0, 0, 0, 0, 1])):
        case = inputs.make_case(fmt, 2, 3, K, seed=14)
        assert case.scales.shape == (3, 2) and case.zeros.shape == (3, 2)
        w, b = oracle.dequant(fmt, case.packed, case.scales, case.zeros, 3, K)
        w32, b32 = oracle.dequant(oracle.INT4_G32, case.packed, case.scales[:, expand],
                                  case.zeros[:, expand], 3, K)
        assert np.array_equal(w, w32) and np.array_equal(b, b32)
        C, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, 2, 3, K)
        C32, S32 = oracle.gemm(oracle.INT4_G32, case.A, case.packed, case.scales[:, expand],
                               case.zeros[:, expand], 2, 3, K)
        assert np.array_equal(C, C32) and np.array_equal(S, S32)
    # arrays short of ceil(K / G) groups are refused before the C code runs
    case = inputs.make_case(oracle.INT4_G64, 0, 2, 96, seed=15)
    with pytest.raises(ValueError):
        oracle.dequant(oracle.INT4_G64, case.packed, case.scales[:, :1], case.zeros[:, :1], 2, 96)

@pytest.mark.parametrize("fmt", [oracle.INT4_G128, oracle.NVFP4, oracle.MXFP4, oracle.INT4_G32,
                                 oracle.INT4_G64, oracle.INT4_SYM])
def test_k_odd_multiple_of_16_is_a_prefix(fmt):
    """K = 16 * odd (the NVFP4 layout's (N, ceil(K/16)) scales): a row of K
    codes dequantises to the first K weights of the same row extended by 16
    codes, with the same scales (and zeros) -- the short last group takes its
    own group's scale, and nothing else moves."""
    N, K = 5, 208   # 13 * 16
    G = oracle.GROUP[fmt]
    big = inputs.make_case(fmt, 1, N, K + 16, seed=7)
    ng = (K + G - 1) // G
    packed = big.packed[:, :K // 2].copy()
    scales = big.scales[:, :ng].copy()
    zeros = None if big.zeros is None else big.zeros[:, :ng].copy()
    w, wb = oracle.dequant(fmt, packed, scales, zeros, N, K)
    wbig, wbbig = oracle.dequant(fmt, big.packed, big.scales, big.zeros, N, K + 16)
    assert np.array_equal(w, wbig[:, :K]) and np.array_equal(wb, wbbig[:, :K])
