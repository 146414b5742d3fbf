"""Private staging of the skinny kernel (int4 with groups of 128 and the fp4
formats, at most 8 A rows x k-blocks per wave): each wave copies its own A pieces, scales and
zeros to LDS and starts without a workgroup barrier.  The streaming variant
(>= 1024 tiles of 16 columns) stages A and the scale windows once per
workgroup instead; both feed the same operands in the same order, so the
columns of a wide launch and those of a narrow launch of its first rows agree
bit for bit.  Also against the oracle, with ragged K and a partial last tile.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def to_dev(case):
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    packed = torch.from_numpy(case.packed).to(DEV)
    if case.fmt in w4.INT4_FORMATS:
        scales = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        scales = torch.from_numpy(case.scales).to(DEV)
    zeros = torch.from_numpy(case.zeros).to(DEV) if case.zeros is not None else None
    return A, packed, scales, zeros


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.INT4_SYM, w4.NVFP4, w4.MXFP4])
@pytest.mark.parametrize("M,K", [(1, 3072), (2, 1024), (1, 8192), (4, 512), (3, 1280)])
def test_private_staging_equals_streaming_variant(fmt, M, K):
    N, n = 16384, 4096
    case = inputs.make_case(fmt, M, N, K, seed=81 + M + K)
    A, p, s, z = to_dev(case)
    wide = w4.gemm(fmt, A, p, s, z)  # 1024 tiles: the streaming variant
    narrow = w4.gemm(fmt, A, p[:n], s[:n], None if z is None else z[:n])  # one-tile, private staging
    torch.cuda.synchronize()
    assert torch.equal(wide[:, :n].view(torch.int16), narrow.view(torch.int16))


@pytest.mark.parametrize("fmt,M,N,K", [(w4.INT4_G128, 1, 1000, 3104), (w4.INT4_G128, 2, 77, 4064),
                                       (w4.INT4_SYM, 1, 333, 2080), (w4.INT4_G128, 4, 129, 544),
                                       (w4.NVFP4, 1, 500, 8224), (w4.MXFP4, 2, 300, 3104),
                                       (w4.NVFP4, 4, 77, 544), (w4.MXFP4, 1, 1000, 8192)])
def test_private_staging_against_oracle(fmt, M, N, K):
    case = inputs.make_case(fmt, M, N, K, seed=91 + N)
    A, p, s, z = to_dev(case)
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in (torch.float32, torch.bfloat16):
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt).double().cpu().numpy()
        r = oracle.gate_ratio(C, Cref, S, odt == torch.bfloat16)
        print(f"[gate] private staging fmt {fmt} {M}x{N}x{K} {odt}: {r:.3e}", flush=True)
        assert r <= 1.0


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.INT4_SYM])
def test_private_staging_fp16_and_bf16_routes_in_one_launch(fmt):
    """A values outside fp16's exact range (huge, tiny, NaN-free) in some
    waves' k-ranges: those waves take the bf16 route, the others the fp16 one;
    the result still equals the streaming variant bit for bit and the oracle."""
    M, N, n, K = 1, 16384, 4096, 3072
    case = inputs.make_case(fmt, M, N, K, seed=97)
    bits = case.A.copy()
    to_bf16 = lambda x: np.array([x], np.float32).view(np.uint32)[0] >> 16
    bits[0, 5] = to_bf16(1.5e30)      # k-block 0: wave 0's range
    bits[0, 700] = to_bf16(3.0e-30)   # k-block 5: wave 2's range (2 k-blocks per wave)
    bits[0, 2900] = to_bf16(-70000.0)  # k-block 22: past fp16's largest value
    case.A[:] = bits
    A, p, s, z = to_dev(case)
    wide = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32)
    narrow = w4.gemm(fmt, A, p[:n], s[:n], None if z is None else z[:n], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(wide[:, :n].view(torch.int32), narrow.view(torch.int32))
    zn = None if case.zeros is None else case.zeros[:n]
    Cref, S = oracle.gemm(fmt, case.A, case.packed[:n], case.scales[:n], zn, M, n, K)
    r = oracle.gate_ratio(narrow.double().cpu().numpy(), Cref, S, False)
    print(f"[gate] mixed fp16 / bf16 routes fmt {fmt}: {r:.3e}", flush=True)
    assert r <= 1.0


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.INT4_SYM])
@pytest.mark.parametrize("N,K", [(4096, 3072), (3072, 8192)])
def test_private_staging_two_virtual_waves_equal_one(fmt, N, K):
    """A batched launch of 8 GEMVs has more than four rounds of workgroups, so
    each wave runs two virtual waves of the K split; a single GEMV of the same
    shape keeps one per wave.  Both sum the same k-blocks in the same order,
    so every member equals its single launch bit for bit -- also when some
    members' A holds values outside fp16's exact range (those waves take the
    bf16 route, the others may take the fp16 one)."""
    items, cases = [], []
    for i in range(8):
        case = inputs.make_case(fmt, 1, N, K, seed=300 + i)
        if i % 2:
            to_bf16 = lambda x: np.array([x], np.float32).view(np.uint32)[0] >> 16
            case.A[0, (997 * i) % K] = to_bf16(2.5e-31 if i % 4 == 1 else -1.0e9)
        cases.append(case)
        items.append(to_dev(case))
    outs = w4.gemm_batched(fmt, items, out_dtype=torch.float32)
    singles = [w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32) for A, p, s, z in items]
    torch.cuda.synchronize()
    for i, (o, s1) in enumerate(zip(outs, singles)):
        assert torch.equal(o.view(torch.int32), s1.view(torch.int32)), f"member {i}"
    c = cases[1]
    Cref, S = oracle.gemm(fmt, c.A, c.packed, c.scales, c.zeros, 1, N, K)
    r = oracle.gate_ratio(outs[1].double().cpu().numpy(), Cref, S, False)
    print(f"[gate] two virtual waves fmt {fmt} {N}x{K}: {r:.3e}", flush=True)
    assert r <= 1.0
