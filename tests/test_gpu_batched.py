"""w4a16_gemm_batched (through the C ABI): independent GEMMs, each with its own
activations, weights and output, several per launch.

Every item's output must equal w4a16_gemm's for that item alone, bit for bit
(the skinny kernel's split of K depends only on format, M and K), and lie
within the gate against the oracle.  Covered: items of one shape beyond one
launch's 32 members, shapes mixed in one call, a lone item that takes the
streaming variant, the ring variant (A too large for the one-time LDS copy),
M > 16 (one launch per item), empty items, the whole 197-matrix decode chain,
and HIP graph capture.
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
        zeros = torch.from_numpy(case.zeros).to(DEV) if case.zeros is not None else None
    else:
        scales = torch.from_numpy(case.scales).to(DEV)
        zeros = None
    return A, packed, scales, zeros


def same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def check_items(fmt, M, shapes, out_dtype, oracle_check=True, seed=0):
    cases = [inputs.make_case(fmt, M, N, K, seed + 17 * i) for i, (N, K) in enumerate(shapes)]
    items = [to_dev(c) for c in cases]
    print(f"[batched] fmt {fmt} M {M} {len(items)} items, shapes {sorted(set(shapes))} {out_dtype}",
          flush=True)
    outs = w4.gemm_batched(fmt, items, out_dtype=out_dtype)
    singles = [w4.gemm(fmt, *it, out_dtype=out_dtype) for it in items]
    torch.cuda.synchronize()
    for i, (o, s) in enumerate(zip(outs, singles)):
        assert same_bits(o, s), f"item {i} ({shapes[i]}) differs from its single launch"
    if oracle_check:
        for i, c in enumerate(cases):
            if c.N * c.K > 40_000_000:
                continue
            Cref, S = oracle.gemm(fmt, c.A, c.packed, c.scales, c.zeros, M, c.N, c.K)
            r = oracle.gate_ratio(outs[i].double().cpu().numpy(), Cref, S, out_dtype == torch.bfloat16)
            assert r <= 1.0, f"item {i}: gate ratio {r}"


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64, w4.INT4_SYM])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_batched_mixed_shapes(fmt, M):
    shapes = [(256, 512), (96, 512), (256, 512), (40, 1024), (256, 512), (96, 512), (8, 256),
              (1000, 512)]
    check_items(fmt, M, shapes, torch.bfloat16)


def test_batched_more_than_one_launch_of_one_shape():
    # 70 items of one (K, N): launches of 32, 32 and 6 members
    check_items(w4.INT4_G128, 1, [(128, 256)] * 70, torch.float32, oracle_check=False)
    check_items(w4.MXFP4, 3, [(64, 512)] * 33, torch.bfloat16)


def test_batched_lone_item_takes_the_streaming_variant():
    # one 16384 x 256 item (>= 1024 tiles of 16 columns) among smaller ones
    check_items(w4.INT4_G128, 1, [(16384, 256), (512, 256), (512, 256)], torch.bfloat16)


def test_batched_ring_variant():
    # 16 rows x K = 8192 of A: past the one-time LDS copy (the ring variant)
    check_items(w4.NVFP4, 16, [(48, 8192), (48, 8192), (80, 8192)], torch.bfloat16)
    check_items(w4.INT4_G128, 12, [(64, 8192)] * 3, torch.float32)


def test_batched_larger_m_one_launch_per_item():
    check_items(w4.MXFP4, 64, [(512, 256), (512, 256), (300, 512)], torch.bfloat16)
    check_items(w4.INT4_G128, 300, [(256, 256), (520, 512)], torch.float32)


def test_batched_skips_empty_items():
    cases = [inputs.make_case(w4.MXFP4, 2, N, 256, 5 + N) for N in (64, 0, 32)]
    items = [to_dev(c) for c in cases]
    outs = w4.gemm_batched(w4.MXFP4, items)
    torch.cuda.synchronize()
    assert outs[1].shape == (2, 0)
    assert same_bits(outs[0], w4.gemm(w4.MXFP4, *items[0]))
    assert same_bits(outs[2], w4.gemm(w4.MXFP4, *items[2]))


@pytest.mark.timeout(300)
def test_batched_decode_chain_equals_single_launches():
    """All 197 int4 GEMVs of the 3B decode chain in one batched call (a
    handful of launches), each equal bit for bit to its single launch."""
    shapes = inputs.decoder_chain_shapes()
    items = []
    for i, (_, n, k) in enumerate(shapes):
        items.append(to_dev(inputs.make_case(w4.INT4_G128, 1, n, k, inputs.chain_seed(0, i))))
    outs = w4.gemm_batched(w4.INT4_G128, items)
    torch.cuda.synchronize()
    for i, it in enumerate(items):
        s = w4.gemm(w4.INT4_G128, *it)
        torch.cuda.synchronize()
        assert same_bits(outs[i], s), f"chain matrix {i} ({shapes[i][0]}) differs"


def test_batched_graph_capture_replay():
    cases = [inputs.make_case(w4.INT4_G128, 1, N, K, 30 + i)
             for i, (N, K) in enumerate([(1024, 3072), (1024, 3072), (3072, 3072), (3072, 8192)])]
    items = [to_dev(c) for c in cases]
    eager = w4.gemm_batched(w4.INT4_G128, items)
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    call = w4.PreparedBatchedGemm(w4.INT4_G128, items, outs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        _ = (items[0][0].float() * (rep + 1)).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert same_bits(o, e), rep


@pytest.mark.parametrize("fmt,M,K", [(w4.INT4_G128, 1, 3072), (w4.NVFP4, 4, 2048), (w4.MXFP4, 16, 1024),
                                     (w4.INT4_SYM, 2, 4096), (w4.INT4_G32, 1, 1024)])
def test_wave_count_does_not_change_bits(fmt, M, K):
    """A launch of many workgroups computes two of the K split's partial sums
    per wave (half the waves); a launch that fits the CUs at once computes one.
    A column's bits must not depend on which: every 1024-column slice of a
    wide matrix equals the same columns computed by a narrow launch."""
    N = 12288
    case = inputs.make_case(fmt, M, N, K, seed=fmt + M)
    A, p, s, z = to_dev(case)
    wide = w4.gemm(fmt, A, p, s, z)
    for c0 in range(0, N, 4096):
        sl = slice(c0, c0 + 1024)
        narrow = w4.gemm(fmt, A, p[sl].contiguous(), s[sl].contiguous(), None if z is None else z[sl].contiguous())
        torch.cuda.synchronize()
        assert same_bits(wide[:, sl].contiguous(), narrow), c0
