"""Parity of the mid kernel (tiles of 32 columns x 32..64 rows, split-K over
the waves; chosen for 16 < M <= 384 on wide matrices) with the oracle,
through the C ABI.  Its ring variant (every operand through per-wave LDS copy
slots) runs whenever its LDS fits beside the scale windows -- 48- and 64-row
tiles that do not fit become 32-row tiles -- and the per-lane form beyond.

Every element within the gate |C - C_ref| <= 2e-3 S + 1e-6 (+ 2^-8 |C_ref|
for bf16 output).  Covered: the row-tile shapes (2, 3 and 4 slices of 16
rows, ragged last tiles), ragged N and partial k-blocks (K % 128 != 0), the
scale windows staged in LDS and loaded per lane (large K), several passes
over K, scale and zero arrays that start off a 4-byte boundary, tall A
forced onto the kernel, exact zero-point cancellation, and the decode-batch
shapes at full size (sampled).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
FMTS = [w4.INT4_G128, w4.NVFP4, w4.MXFP4]


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


def _check(fmt, M, N, K, path="auto", seed=None, s_off=0, z_off=0, odts=(torch.float32, torch.bfloat16)):
    seed = M * 31 + N * 7 + K if seed is None else seed
    case = inputs.make_case(fmt, M, N, K, seed)
    A, p, s, z = _dev(case, s_off, z_off)
    print(f"[mid] fmt {fmt} {M}x{N}x{K} path {path} s_off {s_off} z_off {z_off}", flush=True)
    if path == "auto":
        assert w4.gemm_path(fmt, M, N, K) == "mid"
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in odts:
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path)
        torch.cuda.synchronize()
        r = oracle.gate_ratio(C.double().cpu().numpy(), Cref, S, odt == torch.bfloat16)
        print(f"[gate] {odt}: max err/bound = {r:.3e}", flush=True)
        assert r <= 1.0, f"fmt {fmt} {M}x{N}x{K} {odt}: gate ratio {r}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [17, 32, 33, 48, 64, 65, 100, 128, 192, 384])
def test_mid_row_tiles(fmt, M):
    # 2, 3 and 4 row slices per tile, ragged last tiles, N not a multiple of 32
    _check(fmt, M, 200, 384, path="mid")


@pytest.mark.parametrize("fmt,M,N,K", [(w4.INT4_G128, 40, 5120, 256), (w4.MXFP4, 100, 8192, 128),
                                       (w4.NVFP4, 17, 65536, 64)])
def test_mid_chosen_automatically(fmt, M, N, K):
    _check(fmt, M, N, K, odts=(torch.bfloat16,))


@pytest.mark.parametrize("fmt,M,N,K", [
    (w4.NVFP4, 40, 72, 96),      # one partial k-block
    (w4.MXFP4, 20, 33, 160),     # a full and a partial k-block
    (w4.NVFP4, 70, 40, 32),      # a single 32-code chunk
    (w4.MXFP4, 24, 1, 224),      # one output column
    (w4.INT4_G128, 31, 5, 128),  # one k-block, a single wave
])
def test_mid_ragged_k_and_n(fmt, M, N, K):
    _check(fmt, M, N, K, path="mid")


@pytest.mark.parametrize("fmt,M,N,K", [
    (w4.INT4_G128, 40, 72, 8192),    # ring, 48-row tiles
    (w4.INT4_G128, 20, 40, 32768),   # ring, 24 KB of windows
    (w4.INT4_G32, 20, 40, 16384),    # ring, 48 KB of windows
    (w4.NVFP4, 40, 72, 8192),        # ring, 16 KB window
    (w4.NVFP4, 64, 72, 8192),        # 64-row tiles past the ring's LDS: 32-row tiles
    (w4.MXFP4, 36, 50, 8192),
    (w4.MXFP4, 24, 64, 6144),
    (w4.NVFP4, 24, 40, 3104),        # partial last k-block
    (w4.NVFP4, 20, 40, 65536),       # 128 KB window: the per-lane form
    (w4.INT4_G32, 24, 40, 32768),    # 96 KB of scale and zero windows: the per-lane form
])
def test_mid_large_k(fmt, M, N, K):
    _check(fmt, M, N, K, path="mid", odts=(torch.float32,))


@pytest.mark.parametrize("fmt", FMTS)
def test_mid_scale_windows_off_dword_boundary(fmt):
    # scales 2 bytes (MXFP4: 1 and 3) and zeros 1 byte past an aligned address
    offs = [1, 3] if fmt == w4.MXFP4 else [2]
    for off in offs:
        _check(fmt, 40, 100, 512, path="mid", s_off=off, z_off=1, odts=(torch.float32,))
    # and in the per-lane form (windows too large for the ring)
    _check(fmt, 20, 40, 65536 if fmt == w4.NVFP4 else 131072, path="mid", s_off=offs[0], z_off=3,
           odts=(torch.float32,))


def test_mid_forced_at_small_and_tall_m():
    _check(w4.NVFP4, 1, 96, 256, path="mid")
    _check(w4.INT4_G128, 16, 64, 256, path="mid")
    _check(w4.MXFP4, 1000, 40, 128, path="mid", odts=(torch.bfloat16,))


def test_mid_zero_point_cancels_exactly():
    M, N, K = 40, 48, 512
    case = inputs.make_case(w4.INT4_G128, M, N, K, seed=3)
    case.packed[:] = 0x99
    case.zeros[:] = 9
    A, p, s, z = _dev(case)
    C = w4.gemm(w4.INT4_G128, A, p, s, z, out_dtype=torch.float32, path="mid")
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    for fmt in (w4.NVFP4, w4.MXFP4):
        case = inputs.make_case(fmt, M, N, K, seed=4)
        case.A[:] = 0
        A, p, s, z = _dev(case)
        C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path="mid")
        torch.cuda.synchronize()
        assert torch.all(C == 0)


@pytest.mark.parametrize("fmt,N,K", [(w4.INT4_G128, 8192, 3072), (w4.NVFP4, 3072, 8192),
                                     (w4.MXFP4, 8192, 3072)])
@pytest.mark.parametrize("M", [32, 64, 128])
def test_mid_decode_batch_full_size_sampled(fmt, N, K, M):
    """The decode-batch shapes at full size: 2048 sampled outputs (every
    column tile band and row slice is hit) plus the corners."""
    case = inputs.make_case(fmt, M, N, K, seed=M)
    A, p, s, z = _dev(case)
    print(f"[mid] full size fmt {fmt} {M}x{N}x{K}", flush=True)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.bfloat16, path="mid")
    torch.cuda.synchronize()
    C = C.double().cpu().numpy()
    rng = np.random.default_rng(M)
    mi = np.concatenate([rng.integers(0, M, 2048), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 2048), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    r = oracle.gate_ratio(C[mi, ni], Cref, S, True)
    print(f"[gate] max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0
    assert np.all(np.isfinite(C))


def test_mid_matches_skinny_within_rounding():
    # two kernels, two summation orders: both within the gate of the oracle
    # and close to each other
    fmt, M, N, K = w4.INT4_G128, 64, 512, 3072
    case = inputs.make_case(fmt, M, N, K, seed=77)
    A, p, s, z = _dev(case)
    Cm = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path="mid")
    Cs = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path="skinny")
    torch.cuda.synchronize()
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for C in (Cm, Cs):
        assert oracle.gate_ratio(C.double().cpu().numpy(), Cref, S, False) <= 1.0
    assert torch.allclose(Cm, Cs, rtol=1e-4, atol=1e-4)
