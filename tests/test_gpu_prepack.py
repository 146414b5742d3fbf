"""Prepacked weights (w4a16_prepack, W4A16_PREPACKED) through the C ABI.

* The prepacked bytes equal the documented permutation of the row-major
  packed array (reference below: plain numpy index arithmetic, no method
  arithmetic), ragged N padded with zero bytes.
* Every entry point gives on prepacked weights the same bits as on the
  row-major ones -- each kernel variant (skinny with A in LDS, the streaming
  variant, the ring variant, grouped / batched launches, mid and mid ring,
  both tiled configurations, the fused epilogue) and the dequantisation --
  and the GEMM stays within the gate against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
FORMATS = [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64, w4.INT4_SYM]


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


def reference_prepack(packed):
    """The header's formula: out[((t*KB + b)*64 + l)*16 + i] =
    packed[(16t + l%16)*K/2 + 64b + 16(l/16) + i], zero past N."""
    N, K2 = packed.shape
    KB, T = K2 // 64, (N + 15) // 16
    padded = np.zeros((T * 16, K2), np.uint8)
    padded[:N] = packed
    # (t, r, b, g, i) -> (t, b, g, r, i): slot l = r + 16 g
    x = padded.reshape(T, 16, KB, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(x).reshape(T * 16, K2)


def same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("N,K", [(1, 128), (15, 384), (16, 256), (17, 3072), (300, 1024), (4097, 640)])
def test_prepack_bytes(N, K):
    rng = np.random.default_rng(N + K)
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    pre = w4.prepack(torch.from_numpy(packed).to(DEV))
    torch.cuda.synchronize()
    assert pre.data.shape == ((N + 15) // 16 * 16, K // 2)
    np.testing.assert_array_equal(pre.data.cpu().numpy(), reference_prepack(packed))


# (what, M, N, K, path): one case per kernel variant
CASES = [
    ("skinny A in LDS", 1, 1000, 3072, "auto"),
    ("skinny 16 rows", 16, 520, 2048, "auto"),
    ("skinny 5 rows", 5, 9000, 1024, "auto"),
    ("skinny stream", 1, 16400, 384, "auto"),
    ("skinny ring", 16, 300, 8192, "auto"),
    ("skinny forced, M = 40", 40, 200, 512, "skinny"),
    ("mid", 64, 2050, 512, "mid"),
    ("mid ring", 64, 2048, 8192, "mid"),
    ("tiled small tiles", 300, 520, 256, "tiled"),
    ("tiled large tiles", 1536, 8200, 384, "auto"),
]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("what,M,N,K,path", CASES, ids=[c[0] for c in CASES])
def test_gemm_prepacked_equals_row_major(fmt, what, M, N, K, path):
    case = inputs.make_case(fmt, M, N, K, seed=fmt * 7 + M)
    A, p, s, z = to_dev(case)
    pre = w4.prepack(p)
    print(f"[prepack] fmt {fmt} {what}: {M}x{N}x{K} path {w4.gemm_path(fmt | w4.PREPACKED, M, N, K, path)}",
          flush=True)
    for odt in (torch.bfloat16, torch.float32):
        ref = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path)
        got = w4.gemm(fmt, A, pre, s, z, out_dtype=odt, path=path)
        torch.cuda.synchronize()
        assert same_bits(got, ref), f"{what} {odt}"
    if M * N * K <= 3_000_000_000:
        C = got.double().cpu().numpy()
        rng = np.random.default_rng(K)
        mi, ni = rng.integers(0, M, 1024), rng.integers(0, N, 1024)
        Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
        assert oracle.gate_ratio(C[mi, ni], Cref, S, False) <= 1.0


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.MXFP4])
def test_epilogue_prepacked(fmt):
    for M, N, K, path in [(4, 3000, 1024, "auto"), (1536, 8200, 256, "auto"), (64, 2048, 512, "mid")]:
        case = inputs.make_case(fmt, M, N, K, seed=M + N)
        A, p, s, z = to_dev(case)
        pre = w4.prepack(p)
        bias = torch.randn(N, device=DEV).to(torch.bfloat16)
        R = torch.randn(M, N, device=DEV).to(torch.bfloat16)
        kw = dict(bias=bias, residual=R, alpha=0.5, beta=1.0, activation="silu", path=path)
        ref = w4.gemm(fmt, A, p, s, z, **kw)
        got = w4.gemm(fmt, A, pre, s, z, **kw)
        torch.cuda.synchronize()
        assert same_bits(got, ref), (M, N, K)


@pytest.mark.parametrize("fmt", FORMATS)
def test_dequant_prepacked(fmt):
    for N, K in [(33, 384), (4096, 1024)]:
        case = inputs.make_case(fmt, 1, N, K, seed=N)
        _, p, s, z = to_dev(case)
        ref = w4.dequant(fmt, p, s, z)
        got = w4.dequant(fmt, w4.prepack(p), s, z)
        torch.cuda.synchronize()
        assert same_bits(got, ref)


def test_grouped_and_batched_prepacked():
    fmt, M, K = w4.INT4_G128, 1, 3072
    shapes = [3072, 1024, 1024, 8192]
    cases = [inputs.make_case(fmt, M, n, K, seed=40 + i) for i, n in enumerate(shapes)]
    devs = [to_dev(c) for c in cases]
    A = devs[0][0]
    weights = [(p, s, z) for _, p, s, z in devs]
    pweights = [(w4.prepack(p), s, z) for p, s, z in weights]
    ref = w4.gemm_grouped(fmt, A, weights)
    got = w4.gemm_grouped(fmt, A, pweights)
    items = [(a, p, s, z) for a, p, s, z in devs] * 3
    pitems = [(a, w4.prepack(p), s, z) for a, p, s, z in devs] * 3
    bref = w4.gemm_batched(fmt, items)
    bgot = w4.gemm_batched(fmt, pitems)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert same_bits(g, r)
    for r, g in zip(bref, bgot):
        assert same_bits(g, r)
    with pytest.raises(ValueError):
        w4.gemm_grouped(fmt, A, [weights[0], pweights[1]])


def _random_cases(n=60, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        fmt = FORMATS[rng.integers(len(FORMATS))]
        M = int(rng.choice([1, 2, 5, 8, 16, 17, 33, 64, 130, 300]))
        N = int(rng.integers(1, 601))
        K = 128 * int(rng.integers(1, 33))
        if M * N * K > 12_000_000:
            continue
        out.append((fmt, M, N, K, ["auto", "skinny", "mid", "tiled"][rng.integers(4)], bool(rng.integers(2)),
                    len(out)))
    return out


@pytest.mark.parametrize("fmt,M,N,K,path,f32,i", _random_cases())
def test_random_shapes_prepacked_equal_row_major(fmt, M, N, K, path, f32, i):
    odt = torch.float32 if f32 else torch.bfloat16
    print(f"[prepack random {i}] fmt {fmt} {M}x{N}x{K} path {path} -> "
          f"{w4.gemm_path(fmt | w4.PREPACKED, M, N, K, path)} out {odt}", flush=True)
    case = inputs.make_case(fmt, M, N, K, seed=9000 + i)
    A, p, s, z = to_dev(case)
    ref = w4.gemm(fmt, A, p, s, z, out_dtype=odt, path=path)
    got = w4.gemm(fmt, A, w4.prepack(p), s, z, out_dtype=odt, path=path)
    torch.cuda.synchronize()
    assert same_bits(got, ref)


def test_prepacked_batched_graph_replay():
    fmt, K = w4.INT4_G128, 3072
    cases = [inputs.make_case(fmt, 1, n, K, 60 + i) for i, n in enumerate([1024, 1024, 3072, 8192])]
    items = [(A, w4.prepack(p), s, z) for A, p, s, z in (to_dev(c) for c in cases)]
    eager = w4.gemm_batched(fmt, items)
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    call = w4.PreparedBatchedGemm(fmt, items, outs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert same_bits(o, e), rep
