"""Pins of the CPU oracle against things other than itself.

Each test ties a part of the oracle to a library routine (torch's float8 /
bf16 casts, numpy's matmul), a value the pages print, a closed-form invariant,
or exact rational brute force, chosen so that a plausible slip (a dropped
term, a wrong sign, bias or index, swapped nibbles, a transposed operand)
fails at least one of them.  All run on the CPU.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden
from weight_only_bit_w4a16_amd import inputs

FMTS = [oracle.INT4_G128, oracle.NVFP4, oracle.MXFP4]


def _bits_f32(x):
    return np.array([x], dtype=np.float32).view(np.uint32)[0]


# ---- element decoders ------------------------------------------------------

def test_e2m1_matches_page_bit_assembly_on_normal_codes():
    """fp4 codes with exponent 1..3 decode to the values of the bit-assembly
    helper on the TileLang fp4 page (golden file); the four codes with
    exponent 0 follow the subnormal reading instead."""
    rows = read_golden("fp4_bitassembly_bf16.txt")
    assert len(rows) == 16
    for code, bits, value, follows in rows:
        code, bits, value = int(code), int(bits, 16), float(value)
        # the printed bf16 pattern and its printed value agree (torch decode)
        t = torch.tensor([bits], dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
        assert float(t.float()) == value
        if follows == "same":
            assert oracle.e2m1_value(code) == value
        else:
            assert follows == "subnormal"
            assert oracle.e2m1_value(code) != value


def test_e2m1_subnormal_spacing_and_signs():
    v = [oracle.e2m1_value(c) for c in range(16)]
    # zero exponent field: m times the spacing of the lowest normal binade
    spacing = v[3] - v[2]
    assert v[0] == 0.0 and not np.signbit(v[0])
    assert v[1] == spacing == 0.5
    # code 8 is negative zero
    assert v[8] == 0.0 and np.signbit(v[8])
    for c in range(8):
        assert v[c | 8] == -v[c]
    # magnitudes increase with the code
    assert all(v[c] < v[c + 1] for c in range(7))
    # the mantissa bit adds half of the binade's base
    for c in (2, 4, 6):
        assert v[c + 1] == 1.5 * v[c]


def test_e2m1_against_torch_e4m3_decode():
    """Re-encode each e2m1 code as the e4m3 byte with the same sign, the same
    unbiased exponent and the same mantissa fraction (e4m3 has 3 mantissa bits
    and bias 7, so exponent +6, mantissa << 2; subnormal 0.5 = 2^-1 is the
    normal e4m3 0x30) and let torch's float8_e4m3fn cast decode it."""
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            byte = 0x00
        elif e == 0:
            byte = 6 << 3  # 2^(6-7) = 0.5
        else:
            byte = ((e + 6) << 3) | (m << 2)
        byte |= s << 7
        ref = float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).double())
        got = oracle.e2m1_value(c)
        assert got == ref
        assert np.signbit(got) == np.signbit(ref)


def test_e4m3_all_256_codes_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e8m0_all_256_codes_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_value(b) for b in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    # torch's float32 path cannot represent 2^-127 exactly as a normal, but
    # it is a float32 subnormal and the cast keeps it
    assert np.array_equal(got[:255], ref[:255])


def test_bf16_value_all_65536_patterns_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = oracle.bf16_values(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _torch_rne_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_round_bf16_against_torch_cast():
    rng = np.random.default_rng(123)
    # random fp32 bit patterns over the whole finite range, plus exact ties
    # (low 16 bits 0x8000) with even and odd kept LSB, near-ties, subnormals,
    # the overflow boundary and signed zeros
    raw = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    ties = (raw & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    near_lo = (raw & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    near_hi = (raw & np.uint32(0xFFFF0000)) | np.uint32(0x8001)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000,
                        0x007F8000, 0x007FFFFF, 0x00800000, 0x7F7F0000, 0x7F7F7FFF,
                        0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000, 0x3F808000, 0x3F818000,
                        0x3F800001, 0x7F800000, 0xFF800000], dtype=np.uint32)
    pats = np.concatenate([raw, ties, near_lo, near_hi, special])
    f = pats.view(np.float32)
    keep = np.isfinite(f) | np.isinf(f)
    f = f[keep & ~np.isnan(f)]
    ref = _torch_rne_bf16_bits(f)
    got = np.array([oracle.round_bf16(float(x)) for x in f], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(_bits_f32(f[i])), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_round_bf16_nan():
    assert (oracle.round_bf16(float("nan")) & 0x7FFF) > 0x7F80


# ---- weights ----------------------------------------------------------------

def _pack_codes(codes):
    """Pack an (N, K) array of 4-bit codes as the spec states: byte (n, i)
    holds input 2i in its low nibble and 2i+1 in its high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_nibble_order_low_nibble_is_even_k():
    N, K = 3, 256
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    packed = _pack_codes(codes)
    scales = np.full((N, K // 128), 0x3F80, np.uint16)  # bf16 1.0
    zeros = np.zeros((N, K // 128), np.uint8)
    w, wb = oracle.dequant(oracle.INT4_G128, packed, scales, zeros, N, K)
    assert np.array_equal(w, codes.astype(np.float64))
    # one byte by hand: 0xBA holds 0xA at the even position, 0xB at the odd one
    packed = np.full((1, 64), 0xBA, np.uint8)
    w, _ = oracle.dequant(oracle.INT4_G128, packed, scales[:1], zeros[:1], 1, 128)
    assert w[0, 0] == 10 and w[0, 1] == 11


def test_int4_zero_point_and_scale():
    N, K = 2, 256
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    packed = _pack_codes(codes)
    scale = 0.0146484375  # bf16-representable
    sbits = inputs.bf16_bits(np.full((N, K // 128), scale))
    zeros = np.array([[3, 15], [0, 8]], np.uint8)
    w, wb = oracle.dequant(oracle.INT4_G128, packed, sbits, zeros, N, K)
    for n in range(N):
        for k in range(K):
            z = zeros[n, k // 128]
            c = codes[n, k]
            assert w[n, k] == (int(c) - int(z)) * scale
            if c == z:
                assert w[n, k] == 0 and not np.signbit(w[n, k])
    # the bf16 copy is the single RNE rounding of the exact value (torch cast
    # of the exact value, which is representable in fp32)
    assert np.array_equal(wb, _torch_rne_bf16_bits(w.astype(np.float32)))


@pytest.mark.parametrize("fmt", FMTS)
def test_group_locality(fmt):
    """Changing the scale of group g of row n changes exactly the weights of
    that row in columns [g*G, (g+1)*G)."""
    G = oracle.GROUP[fmt]
    N, K = 4, 4 * max(G, 32)
    case = inputs.make_case(fmt, 1, N, K, seed=7)
    w0, _ = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    n, g = 2, 3
    s2 = case.scales.copy()
    if fmt == oracle.INT4_G128:
        s2[n, g] = 0x4000  # bf16 2.0
    elif fmt == oracle.NVFP4:
        s2[n, g] = 0x48  # e4m3 4.0 (not in the generated range's typical values)
    else:
        s2[n, g] = 130
    w1, _ = oracle.dequant(fmt, case.packed, s2, case.zeros, N, K)
    changed = w0 != w1
    expect = np.zeros_like(changed)
    expect[n, g * G:(g + 1) * G] = True
    # codes that decode to zero do not change; everything that changes is inside the group
    assert not np.any(changed & ~expect)
    assert changed.sum() >= G // 4
    if fmt == oracle.INT4_G128:
        z2 = case.zeros.copy()
        z2[n, g] = (int(z2[n, g]) + 1) % 16
        w2, _ = oracle.dequant(fmt, case.packed, case.scales, z2, N, K)
        ch = w0 != w2
        assert np.array_equal(ch, expect)  # every weight of the group shifts


@pytest.mark.parametrize("fmt", [oracle.NVFP4, oracle.MXFP4])
def test_fp4_weights_exact_in_bf16_at_workload_ranges(fmt):
    case = inputs.make_case(fmt, 1, 64, 1024, seed=3)
    w, wb = oracle.dequant(fmt, case.packed, case.scales, None, 64, 1024)
    back = torch.from_numpy(wb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(back, w)
    # negative zero from code 8 survives
    codes_lo = case.packed & 0xF
    neg0 = codes_lo == 8
    assert np.all(wb[:, 0::2][neg0] == 0x8000)


def test_mxfp4_unit_scale_is_plain_e2m1():
    N, K = 2, 64
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    scales = np.full((N, K // 32), 127, np.uint8)
    w, _ = oracle.dequant(oracle.MXFP4, _pack_codes(codes), scales, None, N, K)
    for c in range(16):
        assert w[0, c] == oracle.e2m1_value(c)
    scales[:, 1] = 128  # second block doubled
    w2, _ = oracle.dequant(oracle.MXFP4, _pack_codes(codes), scales, None, N, K)
    assert np.array_equal(w2[:, 32:], 2 * w[:, 32:])
    assert np.array_equal(w2[:, :32], w[:, :32])


def test_nvfp4_scale_enters_by_magnitude():
    N, K = 1, 32
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, 2))
    pos = np.full((N, 2), 0x38, np.uint8)  # e4m3 1.0
    neg = pos | 0x80                        # e4m3 -1.0
    w_pos, _ = oracle.dequant(oracle.NVFP4, _pack_codes(codes), pos, None, N, K)
    w_neg, _ = oracle.dequant(oracle.NVFP4, _pack_codes(codes), neg, None, N, K)
    assert np.array_equal(w_pos, w_neg)


# ---- GEMM -------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_identity_reduces_to_dequant(fmt):
    """A = I (M = K) gives C = W^T: pins operand order and indexing of the
    GEMM against the dequantised weights."""
    K = 128
    N = 5
    case = inputs.make_case(fmt, 1, N, K, seed=11)
    A = np.zeros((K, K), np.uint16)
    A[np.arange(K), np.arange(K)] = 0x3F80
    C, S = oracle.gemm(fmt, A, case.packed, case.scales, case.zeros, K, N, K)
    w, _ = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    assert np.array_equal(C, w.T)
    assert np.array_equal(S, np.abs(w.T))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_against_numpy_matmul(fmt):
    M, N, K = 16, 256, 512
    case = inputs.make_case(fmt, M, N, K, seed=5)
    C, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    w, _ = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    A64 = torch.from_numpy(case.A.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    ref = A64 @ w.T
    refS = np.abs(A64) @ np.abs(w.T)
    assert np.all(np.abs(C - ref) <= 1e-12 * refS + 1e-300)
    assert np.allclose(S, refS, rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_exact_rational_brute_force(fmt):
    """Tiny shapes: the fp64 sum is within one rounding per term of the exact
    rational sum of a * w (all values are dyadic)."""
    G = oracle.GROUP[fmt]
    M, N, K = 3, 3, 2 * max(G, 32)
    case = inputs.make_case(fmt, M, N, K, seed=13)
    C, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    w, _ = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    A64 = torch.from_numpy(case.A.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(A64[m, k])) * Fraction(float(w[n, k])) for k in range(K)),
                        Fraction(0))
            mag = sum((abs(Fraction(float(A64[m, k])) * Fraction(float(w[n, k]))) for k in range(K)),
                      Fraction(0))
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(K) * Fraction(2.0 ** -53) * mag
            assert abs(Fraction(S[m, n]) - mag) <= Fraction(K) * Fraction(2.0 ** -53) * mag


def test_gemm_linear_in_A_and_zero_codes():
    fmt = oracle.INT4_G128
    M, N, K = 4, 16, 256
    case = inputs.make_case(fmt, M, N, K, seed=17)
    C, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    # 2A: bf16 exponent + 1 (no overflow for N(0,1) draws)
    A2 = case.A + np.uint16(1 << 7)
    C2, _ = oracle.gemm(fmt, A2, case.packed, case.scales, case.zeros, M, N, K)
    assert np.array_equal(C2, 2 * C)
    # -A: sign flip
    Aneg = case.A ^ np.uint16(0x8000)
    Cn, _ = oracle.gemm(fmt, Aneg, case.packed, case.scales, case.zeros, M, N, K)
    assert np.array_equal(Cn, -C)
    # every code equal to its group's zero point -> C == 0
    zeros = np.full((N, K // 128), 9, np.uint8)
    packed = np.full((N, K // 2), 0x99, np.uint8)
    Cz, Sz = oracle.gemm(fmt, case.A, packed, case.scales, zeros, M, N, K)
    assert np.all(Cz == 0) and np.all(Sz == 0)


def test_gemm_at_matches_full():
    fmt = oracle.NVFP4
    M, N, K = 8, 48, 256
    case = inputs.make_case(fmt, M, N, K, seed=19)
    C, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    rng = np.random.default_rng(0)
    mi = rng.integers(0, M, 50)
    ni = rng.integers(0, N, 50)
    Ca, Sa = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    assert np.array_equal(Ca, C[mi, ni])
    assert np.array_equal(Sa, S[mi, ni])


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        oracle.dequant(oracle.INT4_G128, np.zeros((1, 50), np.uint8), np.zeros((1, 1), np.uint16),
                       np.zeros((1, 1), np.uint8), 1, 101)   # odd K
    with pytest.raises(ValueError):
        oracle.gemm(7, np.zeros((1, 32), np.uint16), np.zeros((1, 16), np.uint8),
                    np.zeros((1, 1), np.uint8), None, 1, 1, 32)


# ---- workload shapes ---------------------------------------------------------

def test_decode_chain_bytes_match_page():
    """The 197-matrix decode chain, plus the KV cache, moves exactly the bytes
    per step that the int4 decode spec prints."""
    g = {k: int(v) for k, v in read_golden("decode_step_bytes.txt")}
    shapes = inputs.decoder_chain_shapes()
    assert len(shapes) == 197
    packed = sum(n * k // 2 for _, n, k in shapes)
    meta = sum((n * k // 128) * (2 + 1) for _, n, k in shapes)  # bf16 scale + u8 zero
    c = inputs.DECODER_3B
    kv = g["kv_tokens"] * c["layers"] * 2 * c["n_kv"] * c["hd"] * 2
    assert packed + meta + kv == g["bytes_per_step"]
    head = [s for s in shapes if s[0] == "lm_head"][0]
    assert head[1] * head[2] // 2 == g["lm_head_packed_bytes"]


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_matmul_matches_gemm(fmt):
    """The matrix-product form (exact dequantisation + binary64 BLAS product,
    used for the large full-output comparisons) agrees with the
    element-by-element oracle to binary64 rounding, ragged last group included."""
    G = oracle.GROUP[fmt]
    M, N = 24, 96
    K = 3 * G + 32 if fmt in (oracle.INT4_G128, oracle.INT4_G64, oracle.INT4_SYM) else 8 * G
    case = inputs.make_case(fmt, M, N, K, seed=23)
    C, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    Cm, Sm = oracle.gemm_matmul(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    assert np.all(np.abs(Cm - C) <= K * 2.0 ** -52 * S)
    assert np.all(np.abs(Sm - S) <= K * 2.0 ** -52 * S)
    # a planted transposition of the weight is caught
    Ct, _ = oracle.gemm_matmul(fmt, case.A, case.packed[::-1].copy(), case.scales[::-1].copy(),
                               None if case.zeros is None else case.zeros[::-1].copy(), M, N, K)
    assert not np.allclose(Ct, C)
