"""Pins of the oracle's symmetric int4 format (INT4_SYM).

Reading (the int4 page gives only the asymmetric triple and, in its
tolerance table, what ignoring the zero point costs): symmetric int4 has no
zero array; every group of 128 takes the code midpoint 8 as its zero point.
These checks do not retype (code - 8) * scale: they tie the format to the
pinned asymmetric group-128 oracle with every zero byte 8, and check the
properties a symmetric quantiser must have (code 8 is exactly zero; codes
8 + d and 8 - d are negatives; the scale enters linearly), so that a wrong
zero point (0, 7, 15), a wrong group or a sign slip fails one of them.
"""
import numpy as np

import oracle
from weight_only_bit_w4a16_amd import inputs


def test_equals_asymmetric_with_zero_point_8():
    N, K, M = 5, 384, 3
    case = inputs.make_case(oracle.INT4_SYM, M, N, K, seed=31)
    assert case.zeros is None
    eights = np.full((N, K // 128), 8, np.uint8)
    w, b = oracle.dequant(oracle.INT4_SYM, case.packed, case.scales, None, N, K)
    wa, ba = oracle.dequant(oracle.INT4_G128, case.packed, case.scales, eights, N, K)
    assert np.array_equal(w, wa) and np.array_equal(b, ba)
    C, S = oracle.gemm(oracle.INT4_SYM, case.A, case.packed, case.scales, None, M, N, K)
    Ca, Sa = oracle.gemm(oracle.INT4_G128, case.A, case.packed, case.scales, eights, M, N, K)
    assert np.array_equal(C, Ca) and np.array_equal(S, Sa)


def test_code_8_is_zero_and_codes_mirror_about_it():
    N, K = 2, 256
    case = inputs.make_case(oracle.INT4_SYM, 0, N, K, seed=32)
    # row 0: codes 8 everywhere; row 1: codes 0..15 in order, repeated
    packed = np.empty((N, K // 2), np.uint8)
    packed[0] = 0x88
    lo = np.arange(0, K, 2) % 16
    packed[1] = (lo | ((lo + 1) % 16) << 4).astype(np.uint8)
    w, _ = oracle.dequant(oracle.INT4_SYM, packed, case.scales, None, N, K)
    assert np.all(w[0] == 0.0)
    codes = np.arange(K) % 16
    for d in range(1, 8):
        up, down = w[1][codes == 8 + d], w[1][codes == 8 - d]
        assert np.array_equal(up, -down)
        assert np.all(up != 0.0)
    # code 0 is the one without a mirror: one step below code 1
    g = np.arange(K) // 128
    step = w[1][codes == 9] - w[1][codes == 8]
    assert np.array_equal(w[1][codes == 0], -8.0 * step)
    assert np.all(np.sign(step) == np.sign(np.array([oracle.bf16_value(int(case.scales[1, j])) for j in g[codes == 9]])))


def test_scale_enters_linearly_per_group_of_128():
    N, K = 3, 384
    case = inputs.make_case(oracle.INT4_SYM, 0, N, K, seed=33)
    base, _ = oracle.dequant(oracle.INT4_SYM, case.packed, case.scales, None, N, K)
    s = case.scales.copy()
    s[1, 2] = oracle.round_bf16(2.0 * oracle.bf16_value(int(s[1, 2])))   # exact doubling
    w, _ = oracle.dequant(oracle.INT4_SYM, case.packed, s, None, N, K)
    changed = np.argwhere(w != base)
    assert np.all(changed[:, 0] == 1)
    assert changed[:, 1].min() >= 256 and changed[:, 1].max() < 384
    assert np.array_equal(w[1, 256:], 2.0 * base[1, 256:])
