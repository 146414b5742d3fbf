"""Parity of the int4 formats with groups of 32 and 64 (INT4_G32 / INT4_G64)
with the oracle, through the C ABI.

The dequantisation is bit-exact (every code, special scales, every zero
byte); the GEMM meets the gate on every kernel and its variants: the skinny
kernel with A staged in LDS, copied per wave and loaded per lane, grouped
launches, the mid kernel with scales in LDS and loaded per lane, the tiled
kernel with small and large tiles, partial k-blocks, and the fused
epilogue.  A weight equal to its zero point is exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
FMTS = [w4.INT4_G32, w4.INT4_G64]


def _dev(case):
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    p = torch.from_numpy(case.packed).to(DEV)
    s = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
    z = torch.from_numpy(case.zeros).to(DEV)
    return A, p, s, z


def _gate(fmt, M, N, K, path, odts=(torch.float32, torch.bfloat16), seed=None, case=None):
    case = case or inputs.make_case(fmt, M, N, K, M * 13 + N * 5 + K if seed is None else seed)
    A, p, s, z = _dev(case)
    print(f"[groups] fmt {fmt} {M}x{N}x{K} path {path}", flush=True)
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in odts:
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path)
        torch.cuda.synchronize()
        r = oracle.gate_ratio(C.double().cpu().numpy(), Cref, S, odt == torch.bfloat16)
        print(f"[gate] {odt}: max err/bound = {r:.3e}", flush=True)
        assert r <= 1.0, f"fmt {fmt} {M}x{N}x{K} {path} {odt}: gate ratio {r}"


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(8192, 3072), (33, 160), (7, 64)])
def test_dequant_bit_exact(fmt, N, K):
    # K = 160 with groups of 64: a last group of 32 (its own scale and zero)
    case = inputs.make_case(fmt, 0, N, K, seed=N + K)
    _, p, s, z = _dev(case)
    W = _bits(w4.dequant(fmt, p, s, z))
    _, ref = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    assert np.array_equal(W, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_special_scales_and_every_zero_byte(fmt):
    G = oracle.GROUP[fmt]
    N, K = 512, 2 * G
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    rng = np.random.default_rng(7)
    special = np.array([0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
                        0x7F80, 0xFF80, 0x7FC0, 0x3C23], np.uint16)
    scales = rng.integers(0, 65536, size=(N, 2)).astype(np.uint16)
    scales[:len(special), 1] = special
    zeros = rng.integers(0, 256, size=(N, 2)).astype(np.uint8)
    zeros[:256, 0] = np.arange(256)
    case = inputs.Case(fmt, 0, N, K, np.zeros((0, K), np.uint16), packed, scales, zeros)
    _, p, s, z = _dev(case)
    W = _bits(w4.dequant(fmt, p, s, z))
    _, ref = oracle.dequant(fmt, packed, scales, zeros, N, K)
    nan_ref = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_ref, (W & 0x7FFF) > 0x7F80)
    assert np.array_equal(W[~nan_ref], ref[~nan_ref])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [
    (1, 8192, 3072),   # decode GEMV: A in LDS
    (3, 200, 384),
    (16, 256, 512),
    (16, 96, 4096),    # A too large for the LDS copy: per-wave copies
    (5, 72, 8192),     # four k-blocks per wave
    (2, 50, 96),       # one partial k-block
    (1, 24, 32),       # a single chunk
])
def test_gemm_skinny(fmt, M, N, K):
    assert w4.gemm_path(fmt, M, N, K) == "skinny"
    _gate(fmt, M, N, K, "auto")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(40, 200, 384), (100, 130, 640), (24, 40, 16384), (70, 33, 96)])
def test_gemm_mid(fmt, M, N, K):
    _gate(fmt, M, N, K, "mid")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(300, 257, 640), (17, 40, 128), (130, 300, 192)])
def test_gemm_tiled_small_tiles(fmt, M, N, K):
    _gate(fmt, M, N, K, "tiled")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_tiled_large_tiles_sampled(fmt):
    M, N, K = 2050, 6150, 192
    assert w4.gemm_path(fmt, M, N, K) == "tiled"
    case = inputs.make_case(fmt, M, N, K, seed=fmt)
    A, p, s, z = _dev(case)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.bfloat16).double().cpu().numpy()
    rng = np.random.default_rng(fmt)
    mi = np.concatenate([rng.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    r = oracle.gate_ratio(C[mi, ni], Cref, S, True)
    print(f"[gate] large tiles fmt {fmt}: max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_grouped_matches_single_launches(fmt):
    M, K, Ns = 1, 3072, [3072, 1024, 1024]
    cases = [inputs.make_case(fmt, M, n, K, 300 + i) for i, n in enumerate(Ns)]
    A = torch.from_numpy(cases[0].A.view(np.int16)).to(DEV).view(torch.bfloat16)
    weights = [_dev(c)[1:] for c in cases]
    outs = w4.gemm_grouped(fmt, A, weights)
    singles = [w4.gemm(fmt, A, p, s, z) for p, s, z in weights]
    torch.cuda.synchronize()
    for i, (case, out, single) in enumerate(zip(cases, outs, singles)):
        assert torch.equal(out.view(torch.int16), single.view(torch.int16)), i
        Cref, S = oracle.gemm(fmt, cases[0].A, case.packed, case.scales, case.zeros, M, Ns[i], K)
        assert oracle.gate_ratio(out.double().cpu().numpy(), Cref, S, True) <= 1.0


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ["skinny", "mid", "tiled"])
def test_zero_point_weights_are_exactly_zero(fmt, path):
    M, N, K = 5, 48, 256
    case = inputs.make_case(fmt, M, N, K, seed=9)
    case.packed[:] = 0xBB
    case.zeros[:] = 11
    A, p, s, z = _dev(case)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    assert torch.all(C == 0)


@pytest.mark.parametrize("path", ["skinny", "mid", "tiled"])
def test_every_zero_byte(path):
    fmt, M, N, K = w4.INT4_G32, 4, 64, 512
    case = inputs.make_case(fmt, M, N, K, seed=21)
    case.zeros[:] = np.random.default_rng(22).integers(0, 256, size=case.zeros.shape, dtype=np.uint8)
    case.zeros.flat[:4] = [0, 127, 128, 255]
    _gate(fmt, M, N, K, path, case=case)


def test_epilogue_group_64():
    fmt, M, N, K = w4.INT4_G64, 3, 200, 384
    case = inputs.make_case(fmt, M, N, K, seed=31)
    A, p, s, z = _dev(case)
    rng = np.random.default_rng(32)
    bits = np.array([oracle.round_bf16(v) for v in rng.standard_normal(N)], dtype=np.uint16)
    bias = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    R = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(DEV)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, bias=bias, residual=R, alpha=0.5,
                beta=2.0, activation="silu")
    torch.cuda.synchronize()
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    R64 = R.double().cpu().numpy()
    Y = oracle.epilogue(Cref, 0.5, bits, w4.ACT_SILU, 2.0, R64)
    r = oracle.epilogue_gate_ratio(C.double().cpu().numpy(), Cref, S, 0.5, bits, w4.ACT_SILU, 2.0,
                                   R64, Y, False)
    assert r <= 1.0
