"""Parity of the skinny kernel's ring variant with the oracle, through the C ABI.

The variant serves few-row launches whose A slice is too large for the
one-time LDS copy (more than 64 KB, or more than the staging registers: e.g.
16 x 8192, 4 x 8192, 3 x 8192): every k-block's A rows and weight rows arrive
by asynchronous global -> LDS copies into per-wave ring slots, and the scale
(and zero) window by the same copies, once.  Covered: every format, row
slices of 3 .. 16 rows, ragged N, partial last k-blocks (K % 128 != 0), waves
with fewer k-blocks than ring slots, the two-slot ring (scale windows too
large for three slots), scale / zero arrays that start off a 4-byte
boundary and a grouped launch (the fused epilogue: the epilogue tests).
Every element within the gate |C - C_ref| <= 2e-3 S + 1e-6 (+ 2^-8 |C_ref|
for bf16 output).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _dev(case, s_off=0, z_off=0):
    """Device copies; scales / zeros placed s_off / z_off bytes into a larger
    buffer, so that the arrays start at that offset from an aligned address."""
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    p = torch.from_numpy(case.packed).to(DEV)
    sb = case.scales.view(np.uint8).reshape(-1)
    buf = torch.zeros(sb.size + s_off + 16, dtype=torch.uint8, device=DEV)
    buf[s_off:s_off + sb.size] = torch.from_numpy(sb.copy()).to(DEV)
    s = buf[s_off:s_off + sb.size]
    if case.fmt in w4.INT4_FORMATS:
        s = s.view(torch.bfloat16).view(case.scales.shape)
        zb = torch.zeros(case.zeros.size + z_off + 16, dtype=torch.uint8, device=DEV)
        zb[z_off:z_off + case.zeros.size] = torch.from_numpy(case.zeros.reshape(-1).copy()).to(DEV)
        z = zb[z_off:z_off + case.zeros.size].view(case.zeros.shape)
    else:
        s = s.view(case.scales.shape)
        z = None
    return A, p, s, z


def _check(fmt, M, N, K, seed=None, s_off=0, z_off=0, odts=(torch.float32, torch.bfloat16)):
    seed = M * 131 + N * 7 + K if seed is None else seed
    case = inputs.make_case(fmt, M, N, K, seed)
    A, p, s, z = _dev(case, s_off, z_off)
    print(f"[ring] fmt {fmt} {M}x{N}x{K} s_off {s_off} z_off {z_off}", flush=True)
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in odts:
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path="skinny")
        torch.cuda.synchronize()
        r = oracle.gate_ratio(C.double().cpu().numpy(), Cref, S, odt == torch.bfloat16)
        print(f"[gate] {odt}: max err/bound = {r:.3e}", flush=True)
        assert r <= 1.0, f"fmt {fmt} {M}x{N}x{K} {odt}: gate ratio {r}"


ALL_FMTS = [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64]


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("M", [3, 4, 13, 16])
def test_ring_rows_and_formats(fmt, M):
    # 64 k-blocks over 8 waves; ragged N (a partial column tile)
    _check(fmt, M, 50, 8192)


@pytest.mark.parametrize("fmt,M,N,K", [
    (w4.NVFP4, 16, 40, 4160),      # last k-block: two of four chunks
    (w4.MXFP4, 5, 33, 6176),       # last k-block: one chunk
    (w4.INT4_G32, 8, 24, 4128),    # int4, groups of 32, one-chunk tail
    (w4.INT4_G64, 16, 30, 4160),   # int4, groups of 64, two-chunk tail
    (w4.INT4_G128, 16, 72, 2176),  # 17 k-blocks: waves with 3 and 2 (fewer than the slots)
    (w4.NVFP4, 16, 17, 2080),      # 17 k-blocks, the last partial
])
def test_ring_partial_and_short(fmt, M, N, K):
    _check(fmt, M, N, K)


@pytest.mark.parametrize("fmt,M,N,K", [
    (w4.NVFP4, 16, 24, 32768),     # 32 KB scale window: two slots per wave
    (w4.INT4_G32, 4, 20, 32768),   # 48 KB of scale and zero windows: two slots
    (w4.MXFP4, 16, 20, 16384),     # 8 KB window: three slots
    (w4.NVFP4, 16, 20, 81920),     # 80 KB window: no ring fits, the per-pass copies instead
])
def test_ring_large_windows(fmt, M, N, K):
    _check(fmt, M, N, K, odts=(torch.float32,))


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32])
def test_ring_windows_off_dword_boundary(fmt):
    # the windows are copied from the 4-byte aligned address below their start
    offs = [1, 3] if fmt == w4.MXFP4 else [2]
    for off in offs:
        _check(fmt, 16, 36, 8192, s_off=off, z_off=off if fmt in w4.INT4_FORMATS else 0,
               odts=(torch.float32,))


def test_ring_zero_point_cancels_exactly():
    M, N, K = 16, 48, 8192
    case = inputs.make_case(w4.INT4_G128, M, N, K, seed=5)
    case.packed[:] = 0x77
    case.zeros[:] = 7
    A, p, s, z = _dev(case)
    C = w4.gemm(w4.INT4_G128, A, p, s, z, out_dtype=torch.float32, path="skinny")
    torch.cuda.synchronize()
    assert torch.all(C == 0)


def test_ring_workload_nvfp4_m16_sampled():
    """The 16 x 3072 x 8192 NVFP4 workload (the ring's main user) at full
    size: 4096 sampled outputs plus the corners, and run to run identical."""
    fmt, M, N, K = w4.NVFP4, 16, 3072, 8192
    case = inputs.make_case(fmt, M, N, K, seed=9)
    A, p, s, z = _dev(case)
    C1 = w4.gemm(fmt, A, p, s, z, out_dtype=torch.bfloat16)
    C2 = w4.gemm(fmt, A, p, s, z, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    C = C1.double().cpu().numpy()
    rng = np.random.default_rng(9)
    mi = np.concatenate([rng.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    r = oracle.gate_ratio(C[mi, ni], Cref, S, True)
    print(f"[gate] max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0


def test_ring_grouped_matches_single():
    fmt, M, K = w4.NVFP4, 16, 8192
    Ns = [40, 72, 16]
    cases = [inputs.make_case(fmt, M, N, K, 300 + i) for i, N in enumerate(Ns)]
    A = _dev(cases[0])[0]
    weights = [_dev(c)[1:] for c in cases]
    outs = w4.gemm_grouped(fmt, A, weights, out_dtype=torch.float32, path="skinny")
    singles = [w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path="skinny") for p, s, z in weights]
    torch.cuda.synchronize()
    for i, (case, out, single) in enumerate(zip(cases, outs, singles)):
        assert torch.equal(out.view(torch.int32), single.view(torch.int32)), f"member {i}"
        Cref, S = oracle.gemm(fmt, cases[0].A, case.packed, case.scales, case.zeros, M, Ns[i], K)
        assert oracle.gate_ratio(out.double().cpu().numpy(), Cref, S, False) <= 1.0


@pytest.mark.parametrize("fmt,M,N,K", [
    (w4.INT4_G128, 8, 6000, 4096),   # several rounds of workgroups: 4 waves x 2 slots
    (w4.MXFP4, 5, 4200, 6176),       # the same with a partial last k-block
    (w4.INT4_G64, 16, 2500, 4096),
])
def test_ring_several_rounds(fmt, M, N, K):
    _check(fmt, M, N, K, odts=(torch.bfloat16,))


def test_ring_several_rounds_sampled():
    """16 x 8192 x 8192 NVFP4 (512 workgroups) at full size, sampled."""
    fmt, M, N, K = w4.NVFP4, 16, 8192, 8192
    case = inputs.make_case(fmt, M, N, K, seed=13)
    A, p, s, z = _dev(case)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path="skinny")
    torch.cuda.synchronize()
    C = C.double().cpu().numpy()
    rng = np.random.default_rng(13)
    mi = np.concatenate([rng.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    assert oracle.gate_ratio(C[mi, ni], Cref, S, False) <= 1.0


def test_ring_grouped_several_rounds_matches_single():
    # the group's 320 workgroups run 4 waves each, every member alone (<= 256
    # workgroups) 8: the K split over 8 virtual waves keeps the bits equal
    fmt, M, K = w4.NVFP4, 16, 4096
    Ns = [3072, 1024, 1024]
    cases = [inputs.make_case(fmt, M, N, K, 400 + i) for i, N in enumerate(Ns)]
    A = _dev(cases[0])[0]
    weights = [_dev(c)[1:] for c in cases]
    outs = w4.gemm_grouped(fmt, A, weights, out_dtype=torch.bfloat16, path="skinny")
    singles = [w4.gemm(fmt, A, p, s, z, out_dtype=torch.bfloat16, path="skinny") for p, s, z in weights]
    torch.cuda.synchronize()
    for i, (case, out, single) in enumerate(zip(cases, outs, singles)):
        assert torch.equal(out.view(torch.int16), single.view(torch.int16)), f"member {i}"
        Cref, S = oracle.gemm(fmt, cases[0].A, case.packed, case.scales, case.zeros, M, Ns[i], K)
        assert oracle.gate_ratio(out.double().cpu().numpy(), Cref, S, True) <= 1.0
