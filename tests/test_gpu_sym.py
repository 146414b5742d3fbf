"""Parity of symmetric int4 (W4A16_INT4_SYM: bf16 scale per 128, zero point 8,
no zero array) with the oracle, through the C ABI, on every kernel.

* dequant: bit-exact bf16 weights;
* GEMM: every element within the gate |C - C_ref| <= 2e-3 S + 1e-6
  (+ 2^-8 |C_ref| for bf16 output) on the skinny kernel (A in LDS, the ring
  variant for a long A slice, the streaming variant for >= 1024 column
  tiles), the mid kernel and the tiled kernel (both tile sizes), ragged
  shapes included; a grouped launch equal bit for bit to its single ones;
  codes all 8 give exactly 0 on every kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
FMT = w4.INT4_SYM


def _dev(case):
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    p = torch.from_numpy(case.packed).to(DEV)
    s = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
    return A, p, s


@pytest.mark.parametrize("N,K", [(7, 128), (256, 512), (3072, 8192)])
def test_sym_dequant_bit_exact(N, K):
    case = inputs.make_case(FMT, 0, N, K, seed=N + K)
    _, p, s = _dev(case)
    W = w4.dequant(FMT, p, s, None)
    torch.cuda.synchronize()
    got = W.view(torch.int16).cpu().numpy().view(np.uint16)
    _, ref = oracle.dequant(FMT, case.packed, case.scales, None, N, K)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K,path", [
    (1, 16, 128, "skinny"),        # one k-block, A in LDS (even / odd order)
    (3, 33, 384, "skinny"),        # ragged N
    (16, 256, 512, "skinny"),
    (1, 16384, 256, "auto"),       # the streaming variant (1024 column tiles)
    (16, 72, 8192, "skinny"),      # the ring variant (16 x 8192 A rows)
    (5, 600, 8192, "skinny"),      # the ring variant, several rounds of workgroups
    (40, 200, 384, "mid"),
    (100, 8192, 128, "auto"),      # mid, chosen
    (300, 257, 640, "tiled"),      # 128 x 128 tiles, ragged
    (4100, 3000, 256, "auto"),     # tiled, 256 x 256 tiles (204 of them), ragged (sampled)
])
def test_sym_gemm(M, N, K, path):
    case = inputs.make_case(FMT, M, N, K, seed=M * 7 + N + K)
    A, p, s = _dev(case)
    print(f"[sym] {M}x{N}x{K} path {path} ({w4.gemm_path(FMT, M, N, K, path)})", flush=True)
    for odt in (torch.float32, torch.bfloat16):
        C = w4.gemm(FMT, A, p, s, None, out_dtype=odt, path=path)
        torch.cuda.synchronize()
        C = C.double().cpu().numpy()
        if M * N > 1_000_000:
            rng = np.random.default_rng(M)
            mi = np.concatenate([rng.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
            ni = np.concatenate([rng.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
            Cref, S = oracle.gemm_at(FMT, case.A, case.packed, case.scales, None, M, N, K, mi, ni)
            r = oracle.gate_ratio(C[mi, ni], Cref, S, odt == torch.bfloat16)
        else:
            Cref, S = oracle.gemm(FMT, case.A, case.packed, case.scales, None, M, N, K)
            r = oracle.gate_ratio(C, Cref, S, odt == torch.bfloat16)
        print(f"[gate] {odt}: max err/bound = {r:.3e}", flush=True)
        assert r <= 1.0


@pytest.mark.parametrize("M,N,K,path", [(1, 64, 256, "skinny"), (1, 16384, 128, "auto"),
                                        (16, 40, 8192, "skinny"), (40, 96, 256, "mid"),
                                        (200, 128, 256, "tiled")])
def test_sym_code_8_gives_exact_zero(M, N, K, path):
    case = inputs.make_case(FMT, M, N, K, seed=3)
    case.packed[:] = 0x88
    A, p, s = _dev(case)
    C = w4.gemm(FMT, A, p, s, None, out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    assert torch.all(C == 0)


def test_sym_grouped_matches_single():
    M, K = 4, 3072
    Ns = [3072, 1024, 1024]
    cases = [inputs.make_case(FMT, M, N, K, 500 + i) for i, N in enumerate(Ns)]
    A = _dev(cases[0])[0]
    weights = [(*_dev(c)[1:], None) for c in cases]
    outs = w4.gemm_grouped(FMT, A, weights, out_dtype=torch.bfloat16)
    singles = [w4.gemm(FMT, A, p, s, z, out_dtype=torch.bfloat16) for p, s, z in weights]
    torch.cuda.synchronize()
    for i, (case, out, single) in enumerate(zip(cases, outs, singles)):
        assert torch.equal(out.view(torch.int16), single.view(torch.int16)), f"member {i}"
        Cref, S = oracle.gemm(FMT, cases[0].A, case.packed, case.scales, None, M, Ns[i], K)
        assert oracle.gate_ratio(out.double().cpu().numpy(), Cref, S, True) <= 1.0


def test_sym_binding_rejects_zeros():
    case = inputs.make_case(FMT, 1, 16, 128, seed=1)
    A, p, s = _dev(case)
    with pytest.raises(ValueError):
        w4.gemm(FMT, A, p, s, torch.zeros((16, 1), dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("M,N,K,path", [(1, 48, 384, "skinny"), (1, 16384, 256, "auto"),
                                        (16, 40, 8192, "skinny"), (40, 200, 384, "mid"),
                                        (300, 257, 640, "tiled")])
def test_sym_equals_asymmetric_with_zero_bytes_8(M, N, K, path):
    # the same kernel arithmetic with the zero point as a constant: bit for bit
    # the asymmetric group-128 result with every zero byte 8
    case = inputs.make_case(FMT, M, N, K, seed=M + 2 * N + K)
    A, p, s = _dev(case)
    z = torch.full((N, K // 128), 8, dtype=torch.uint8, device=DEV)
    for odt, view in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        Cs = w4.gemm(FMT, A, p, s, None, out_dtype=odt, path=path)
        Ca = w4.gemm(w4.INT4_G128, A, p, s, z, out_dtype=odt, path=path)
        torch.cuda.synchronize()
        assert torch.equal(Cs.view(view), Ca.view(view)), f"{M}x{N}x{K} {path} {odt}"
    Ws = w4.dequant(FMT, p, s, None)
    Wa = w4.dequant(w4.INT4_G128, p, s, z)
    torch.cuda.synchronize()
    assert torch.equal(Ws.view(torch.int16), Wa.view(torch.int16))
