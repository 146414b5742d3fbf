"""The largest K the library accepts (2^22, and 2^22 - 16 for the kernel of
K an odd multiple of 16) on every path, against the oracle: all outputs where
the oracle finishes in seconds, sampled outputs on the wider launches; the
dequantisation bit for bit; prepacked weights bit-equal to row-major ones.
At this K a scale window no longer fits LDS, A takes megabytes per row and
every 32-bit byte offset of a 256-row A tile is close to its limit.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
KMAX = 1 << 22


def to_dev(case):
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    packed = torch.from_numpy(case.packed).to(DEV)
    if case.fmt in w4.INT4_FORMATS:
        scales = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
        zeros = torch.from_numpy(case.zeros).to(DEV) if case.zeros is not None else None
    else:
        scales = torch.from_numpy(case.scales).to(DEV)
        zeros = None
    return A, packed, scales, zeros


def check(C, Cref, S, bf16_out, what):
    r = oracle.gate_ratio(C, Cref, S, bf16_out)
    print(f"[gate] {what}: max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0, f"{what}: gate ratio {r}"


def test_max_k_accepted_and_one_past_rejected():
    assert w4.gemm_path(w4.INT4_G128, 1, 16, KMAX) in ("skinny", "mid", "tiled")
    assert w4.gemm_path(w4.NVFP4, 1, 16, KMAX - 16) == "ragged"
    with pytest.raises(w4.W4A16Error):
        w4.gemm_path(w4.MXFP4, 1, 16, KMAX + 32)


@pytest.mark.parametrize("fmt,M,N,K,path", [
    (w4.INT4_G128, 1, 40, KMAX, "auto"),
    (w4.NVFP4, 1, 24, KMAX, "auto"),
    (w4.MXFP4, 3, 20, KMAX, "auto"),
    (w4.NVFP4, 16, 20, KMAX, "auto"),      # 16 rows of A: 128 MB
    (w4.INT4_SYM, 2, 18, KMAX, "skinny"),
    (w4.INT4_G128, 2, 24, KMAX - 16, "auto"),
    (w4.NVFP4, 5, 16, KMAX - 16, "auto"),
])
def test_gemm_max_k_full(fmt, M, N, K, path):
    print(f"[case] fmt {fmt} {M}x{N}x{K} {path}", flush=True)
    case = inputs.make_case(fmt, M, N, K, seed=31 + M + N)
    A, p, s, z = to_dev(case)
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in (torch.float32, torch.bfloat16):
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path)
        torch.cuda.synchronize()
        check(C.double().cpu().numpy(), Cref, S, odt == torch.bfloat16,
              f"K max fmt {fmt} {M}x{N}x{K} {path} {odt}")


@pytest.mark.parametrize("fmt,M,N,path", [
    (w4.INT4_G128, 40, 64, "mid"),
    (w4.MXFP4, 40, 64, "tiled"),
    (w4.INT4_G32, 24, 40, "tiled"),
    (w4.NVFP4, 17, 48, "skinny"),
])
def test_gemm_max_k_sampled(fmt, M, N, path):
    print(f"[case] fmt {fmt} {M}x{N}x{KMAX} {path}", flush=True)
    case = inputs.make_case(fmt, M, N, KMAX, seed=41 + M)
    A, p, s, z = to_dev(case)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    C = C.double().cpu().numpy()
    rng = np.random.default_rng(M + N)
    mi = np.concatenate([rng.integers(0, M, 60), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 60), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, KMAX, mi, ni)
    check(C[mi, ni], Cref, S, False, f"K max fmt {fmt} {M}x{N} {path} sampled")
    assert np.all(np.isfinite(C))


@pytest.mark.parametrize("fmt,N,K", [(w4.MXFP4, 8, KMAX), (w4.INT4_G128, 6, KMAX),
                                     (w4.NVFP4, 5, KMAX - 16)])
def test_dequant_max_k(fmt, N, K):
    case = inputs.make_case(fmt, 0, N, K, seed=51 + N)
    _, p, s, z = to_dev(case)
    W = w4.dequant(fmt, p, s, z)
    torch.cuda.synchronize()
    got = W.view(torch.int16).cpu().numpy().view(np.uint16)
    _, ref = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    nan_ref = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_ref, (got & 0x7FFF) > 0x7F80)
    assert np.array_equal(got[~nan_ref], ref[~nan_ref])


def test_prepacked_max_k():
    fmt, M, N = w4.INT4_G128, 1, 32
    case = inputs.make_case(fmt, M, N, KMAX, seed=61)
    A, p, s, z = to_dev(case)
    C = w4.gemm(fmt, A, p, s, z)
    Cp = w4.gemm(fmt, A, w4.prepack(p), s, z)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), Cp.view(torch.int16))


# ---- the widest weight matrices: the grid limit ------------------------------------

def _wide_operands(N, K, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    A = torch.randn((1, K), generator=g, device=DEV).to(torch.bfloat16)
    packed = torch.randint(0, 256, (N, K // 2), generator=g, device=DEV, dtype=torch.uint8)
    scales = (127 + torch.randint(-4, 5, (N, (K + 31) // 32), generator=g, device=DEV)).to(torch.uint8)
    return A, packed, scales


def test_widest_matrix_below_grid_limit():
    """K = 16 (the ragged-K kernel, one workgroup of 256 work-items per 64
    rows): 2^30 - 64 rows is the widest grid below 2^32 work-items; sampled
    rows, the first and the last against the oracle."""
    N, K = (1 << 30) - 64, 16
    A, packed, scales = _wide_operands(N, K, 71)
    C = w4.gemm(w4.MXFP4, A, packed, scales, None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(72)
    rows = np.unique(np.concatenate([rng.integers(0, N, 62), [0, N - 1]]))
    idx = torch.from_numpy(rows).to(DEV)
    a = A.view(torch.int16).cpu().numpy().view(np.uint16)
    p = packed[idx].cpu().numpy()
    s = scales[idx].cpu().numpy()
    Cref, S = oracle.gemm(w4.MXFP4, a, p, s, None, 1, len(rows), K)
    check(C[0, idx].double().cpu().numpy()[None, :], Cref, S, False, f"N = 2^30 - 64, K = {K}")


def test_grid_limit_refused_before_launch():
    """2^30 rows at K = 16 would need 2^32 work-items along the grid: the call
    returns W4A16_ERR_HIP without launching, and C is left untouched."""
    N, K = 1 << 30, 16
    A, packed, scales = _wide_operands(N, K, 73)
    C = torch.full((1, N), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w4.W4A16Error) as e:
        w4.gemm(w4.MXFP4, A, packed, scales, None, out=C)
    assert e.value.status == w4.ERR_HIP
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
