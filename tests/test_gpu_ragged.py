"""Parity of int4 weights whose last group is shorter than the others (K not
a multiple of the group: 128 for INT4_G128 / INT4_SYM, 64 for INT4_G64),
through the C ABI.

Groups start at k = 0 and run along K; the last group of each row is the
shorter rest, with its own scale (and zero): ceil(K/G) of them per row.  The
dequantisation is bit-exact; the GEMM meets the gate |C - C_ref| <= 2e-3 S +
1e-6 (+ 2^-8 |C_ref| for bf16 output) on the skinny kernel (A in LDS, the
ring variant), the mid kernel (ring variant), the tiled kernel (small and
large tiles), grouped launches; codes equal to the zero point give exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
FMTS = [w4.INT4_G128, w4.INT4_SYM, w4.INT4_G64]


def _dev(case):
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    p = torch.from_numpy(case.packed).to(DEV)
    s = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
    z = torch.from_numpy(case.zeros).to(DEV) if case.zeros is not None else None
    return A, p, s, z


def _ragged(fmt, K):
    G = oracle.GROUP[fmt]
    assert K % 32 == 0 and K % G != 0, (fmt, K)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(7, 160), (33, 224), (300, 3104)])
def test_ragged_dequant_bit_exact(fmt, N, K):
    _ragged(fmt, K)
    case = inputs.make_case(fmt, 0, N, K, seed=N + K)
    assert case.scales.shape == (N, -(-K // oracle.GROUP[fmt]))
    _, p, s, z = _dev(case)
    W = w4.dequant(fmt, p, s, z)
    torch.cuda.synchronize()
    got = W.view(torch.int16).cpu().numpy().view(np.uint16)
    _, ref = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K,path", [
    (1, 48, 160, "skinny"),        # A in LDS, one full and one partial k-block
    (3, 33, 3104, "skinny"),
    (16, 40, 8224, "skinny"),      # the ring variant (A of 16 x 8224)
    (40, 72, 3104, "mid"),         # the mid ring
    (100, 8192, 224, "auto"),      # mid, chosen
    (300, 257, 672, "tiled"),      # 128 x 128 tiles, partial last k-tile
])
def test_ragged_gemm(fmt, M, N, K, path):
    _ragged(fmt, K)
    case = inputs.make_case(fmt, M, N, K, seed=M * 7 + N + K)
    A, p, s, z = _dev(case)
    print(f"[ragged] fmt {fmt} {M}x{N}x{K} path {path} ({w4.gemm_path(fmt, M, N, K, path)})", flush=True)
    if M * N > 200_000:
        rng = np.random.default_rng(M)
        mi = np.concatenate([rng.integers(0, M, 2048), [0, 0, M - 1, M - 1]])
        ni = np.concatenate([rng.integers(0, N, 2048), [0, N - 1, 0, N - 1]])
        Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    else:
        mi = ni = None
        Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in (torch.float32, torch.bfloat16):
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path)
        torch.cuda.synchronize()
        C = C.double().cpu().numpy()
        r = oracle.gate_ratio(C[mi, ni] if mi is not None else C, Cref, S, odt == torch.bfloat16)
        print(f"[gate] {odt}: max err/bound = {r:.3e}", flush=True)
        assert r <= 1.0


def test_ragged_tiled_large_tiles_sampled():
    fmt, M, N, K = w4.INT4_G128, 4100, 3000, 288   # 204 large tiles; K = 2 groups + 32
    _ragged(fmt, K)
    assert w4.gemm_path(fmt, M, N, K) == "tiled"
    case = inputs.make_case(fmt, M, N, K, seed=5)
    A, p, s, z = _dev(case)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    C = C.double().cpu().numpy()
    rng = np.random.default_rng(5)
    mi = np.concatenate([rng.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    assert oracle.gate_ratio(C[mi, ni], Cref, S, True) <= 1.0


@pytest.mark.parametrize("path", ["skinny", "mid", "tiled"])
def test_ragged_zero_point_is_exactly_zero(path):
    M, N, K = 20, 48, 224
    case = inputs.make_case(w4.INT4_G128, M, N, K, seed=6)
    case.packed[:] = 0x55
    case.zeros[:] = 5
    A, p, s, z = _dev(case)
    C = w4.gemm(w4.INT4_G128, A, p, s, z, out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    assert torch.all(C == 0)


def test_ragged_grouped_matches_single():
    fmt, M, K = w4.INT4_G128, 4, 3104
    Ns = [300, 128, 64]
    cases = [inputs.make_case(fmt, M, N, K, 600 + i) for i, N in enumerate(Ns)]
    A = _dev(cases[0])[0]
    weights = [_dev(c)[1:] for c in cases]
    outs = w4.gemm_grouped(fmt, A, weights, out_dtype=torch.float32)
    singles = [w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32) for p, s, z in weights]
    torch.cuda.synchronize()
    for i, (case, out, single) in enumerate(zip(cases, outs, singles)):
        assert torch.equal(out.view(torch.int32), single.view(torch.int32)), f"member {i}"
        Cref, S = oracle.gemm(fmt, cases[0].A, case.packed, case.scales, case.zeros, M, Ns[i], K)
        assert oracle.gate_ratio(out.double().cpu().numpy(), Cref, S, False) <= 1.0
