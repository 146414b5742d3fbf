"""Seeded random shapes: every format, every kernel choice, single and grouped
launches, through the C ABI.

A hundred and twenty cases drawn once from a fixed seed: format (all six),
M in 1 .. 300, N in 1 .. 600, K a multiple of 32 up to 4096 (so int4 with
groups of 128 or 64 often has a shorter last group), output bf16 or fp32,
path auto / skinny / mid / tiled.  Each must meet the gate
|C - C_ref| <= 2e-3 S + 1e-6 (+ 2^-8 |C_ref| for bf16 output) against the
oracle in every element.  Forty grouped launches (1 .. 8 members of N up to
4000, M up to 64, path auto or skinny) must in addition equal their single
launches bit for bit.  Thirty dequantisations of random N and K must equal
the oracle's bf16 weights bit for bit.  Each case prints its shape before its
launch, so that a failure names it.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
FMTS = [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64, w4.INT4_SYM]
PATHS = ["auto", "skinny", "mid", "tiled"]


def _cases(n=120, seed=2024, budget=12_000_000):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        fmt = FMTS[rng.integers(len(FMTS))]
        M = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 24, 33, 48, 64, 100, 130, 200, 300]))
        N = int(rng.integers(1, 601))
        K = 32 * int(rng.integers(1, 129))
        if M * N * K > budget:
            continue
        out.append((fmt, M, N, K, PATHS[rng.integers(len(PATHS))], bool(rng.integers(2)), len(out)))
    return out


def _dev(case):
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    p = torch.from_numpy(case.packed).to(DEV)
    if case.fmt in w4.INT4_FORMATS:
        s = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        s = torch.from_numpy(case.scales).to(DEV)
    z = torch.from_numpy(case.zeros).to(DEV) if case.zeros is not None else None
    return A, p, s, z


@pytest.mark.parametrize("fmt,M,N,K,path,f32,i", _cases())
def test_random_shape(fmt, M, N, K, path, f32, i):
    odt = torch.float32 if f32 else torch.bfloat16
    print(f"[random {i}] fmt {fmt} {M}x{N}x{K} path {path} -> {w4.gemm_path(fmt, M, N, K, path)} "
          f"out {odt}", flush=True)
    case = inputs.make_case(fmt, M, N, K, seed=7000 + i)
    A, p, s, z = _dev(case)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path)
    torch.cuda.synchronize()
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    r = oracle.gate_ratio(C.double().cpu().numpy(), Cref, S, not f32)
    print(f"[gate] max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0


def _grouped_cases(n=40, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = FMTS[rng.integers(len(FMTS))]
        M = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 32, 64]))
        K = 32 * int(rng.integers(1, 161))
        Ns = tuple(int(rng.integers(1, 4001)) for _ in range(int(rng.integers(1, 9))))
        out.append((fmt, M, K, Ns, ["auto", "skinny"][rng.integers(2)], bool(rng.integers(2)), i))
    return out


@pytest.mark.parametrize("fmt,M,K,Ns,path,f32,i", _grouped_cases())
def test_random_grouped(fmt, M, K, Ns, path, f32, i):
    """Grouped launches of 1 .. 8 members sharing A: every member within the
    gate against the oracle and equal bit for bit to its single launch."""
    odt, view = (torch.float32, torch.int32) if f32 else (torch.bfloat16, torch.int16)
    print(f"[random grouped {i}] fmt {fmt} M {M} K {K} N {Ns} path {path} out {odt}", flush=True)
    cases = [inputs.make_case(fmt, M, N, K, seed=8000 + 10 * i + j) for j, N in enumerate(Ns)]
    A = _dev(cases[0])[0]
    weights = [_dev(c)[1:] for c in cases]
    outs = w4.gemm_grouped(fmt, A, weights, out_dtype=odt, path=path)
    singles = [w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path) for p, s, z in weights]
    torch.cuda.synchronize()
    for j, (case, out, single) in enumerate(zip(cases, outs, singles)):
        assert torch.equal(out.view(view), single.view(view)), f"member {j}"
        Cref, S = oracle.gemm(fmt, cases[0].A, case.packed, case.scales, case.zeros, M, Ns[j], K)
        assert oracle.gate_ratio(out.double().cpu().numpy(), Cref, S, not f32) <= 1.0, f"member {j}"


def _dequant_cases(n=30, seed=2027):
    rng = np.random.default_rng(seed)
    return [(FMTS[rng.integers(len(FMTS))], int(rng.integers(1, 3000)), 32 * int(rng.integers(1, 257)), i)
            for i in range(n)]


@pytest.mark.parametrize("fmt,N,K,i", _dequant_cases())
def test_random_dequant_bit_exact(fmt, N, K, i):
    """Random N (1 .. 2999) and K (multiples of 32 up to 8192): the bf16
    weights equal the oracle's bit for bit."""
    print(f"[random dequant {i}] fmt {fmt} {N}x{K}", flush=True)
    case = inputs.make_case(fmt, 0, N, K, seed=9000 + i)
    _, p, s, z = _dev(case)
    W = w4.dequant(fmt, p, s, z)
    torch.cuda.synchronize()
    got = W.view(torch.int16).cpu().numpy().view(np.uint16)
    _, ref = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
    assert np.array_equal(got, ref)
