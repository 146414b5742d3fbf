"""K an odd multiple of 16 (through the C ABI): rows of K/2 bytes are only
8-byte aligned, and the ragged-K kernel serves every format, M, output type
and entry point; the dequantisation takes 16-code chunks.  Checked against
the oracle: bit-exact weights, GEMM within the gate, the fused epilogue, and
grouped / batched calls equal to single ones."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
FMTS = [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64, w4.INT4_SYM]


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
    v = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(v), b.view(v))


SHAPES = [(1, 1, 16), (1, 200, 48), (5, 17, 80), (16, 64, 1040), (40, 130, 272), (300, 70, 3088),
          (1, 3072, 8208)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt", FMTS)
def test_ragged_k_gemm(fmt, M, N, K):
    assert K % 32 == 16 and w4.gemm_path(fmt, M, N, K) == "ragged"
    case = inputs.make_case(fmt, M, N, K, seed=M + N + K + fmt)
    A, p, s, z = to_dev(case)
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in (torch.float32, torch.bfloat16):
        print(f"[ragged k] fmt {fmt} {M}x{N}x{K} {odt}", flush=True)
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt).double().cpu().numpy()
        r = oracle.gate_ratio(C, Cref, S, odt == torch.bfloat16)
        print(f"[gate] ragged k fmt {fmt} {M}x{N}x{K} {odt}: {r:.3e}", flush=True)
        assert r <= 1.0


@pytest.mark.parametrize("fmt", FMTS)
def test_ragged_k_dequant_bit_exact(fmt):
    for N, K in ((3, 16), (64, 48), (130, 1040), (7, 8208)):
        case = inputs.make_case(fmt, 0, N, K, seed=N + K)
        _, p, s, z = to_dev(case)
        W = w4.dequant(fmt, p, s, z)
        torch.cuda.synchronize()
        got = W.view(torch.int16).cpu().numpy().view(np.uint16)
        _, ref = oracle.dequant(fmt, case.packed, case.scales, case.zeros, N, K)
        assert np.array_equal(got, ref), (fmt, N, K)


def test_ragged_k_mxfp4_nan_scale():
    M, N, K = 4, 32, 80
    case = inputs.make_case(w4.MXFP4, M, N, K, seed=3)
    case.scales[5, 2] = 0xFF          # the short last block of row 5
    case.scales[9, 0] = 0xFF
    A, p, s, z = to_dev(case)
    C = w4.gemm(w4.MXFP4, A, p, s, z, out_dtype=torch.float32).double().cpu().numpy()
    assert np.all(np.isnan(C[:, [5, 9]]))
    keep = [n for n in range(N) if n not in (5, 9)]
    Cref, S = oracle.gemm(w4.MXFP4, case.A, case.packed, case.scales, None, M, N, K)
    assert oracle.gate_ratio(C[:, keep], Cref[:, keep], S[:, keep], False) <= 1.0


@pytest.mark.parametrize("act", ["none", "relu", "silu", "gelu_tanh"])
def test_ragged_k_epilogue(act):
    fmt, M, N, K = w4.NVFP4, 20, 100, 272
    case = inputs.make_case(fmt, M, N, K, seed=len(act))
    A, p, s, z = to_dev(case)
    rng = np.random.default_rng(len(act))
    bits = np.array([oracle.round_bf16(v) for v in rng.standard_normal(N)], np.uint16)
    bias = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    for odt in (torch.float32, torch.bfloat16):
        R = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(DEV).to(odt)
        Rv = R.double().cpu().numpy()
        C = w4.gemm(fmt, A, p, s, z, out=R, bias=bias, residual=R, alpha=0.5, beta=1.0, activation=act)
        torch.cuda.synchronize()
        Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, None, M, N, K)
        a_id = w4.ACTIVATIONS[act]
        Y = oracle.epilogue(Cref, 0.5, bits, a_id, 1.0, Rv)
        r = oracle.epilogue_gate_ratio(C.double().cpu().numpy(), Cref, S, 0.5, bits, a_id, 1.0, Rv, Y,
                                       odt == torch.bfloat16)
        assert r <= 1.0, (act, odt, r)


def test_ragged_k_grouped_and_batched_equal_single():
    fmt, M, K = w4.INT4_G128, 1, 1040
    cases = [inputs.make_case(fmt, M, N, K, seed=N) for N in (64, 96, 64)]
    items = [to_dev(c) for c in cases]
    singles = [w4.gemm(fmt, *it) for it in items]
    batched = w4.gemm_batched(fmt, items)
    A0 = items[0][0]   # a group shares one A
    singles0 = [w4.gemm(fmt, A0, *it[1:]) for it in items]
    grouped = w4.gemm_grouped(fmt, A0, [it[1:] for it in items])
    torch.cuda.synchronize()
    for s, b in zip(singles, batched):
        assert same_bits(s, b)
    for s, g in zip(singles0, grouped):
        assert same_bits(s, g)
