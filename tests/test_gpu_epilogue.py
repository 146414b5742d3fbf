"""Parity of the fused epilogue (w4a16_gemm_ex, through the C ABI) with the oracle.

C = act(alpha * (A . W^T) + bias[n]) + beta * R[m, n] must match the oracle's
binary64 GEMM followed by its binary64 epilogue within the epilogue bound
(the GEMM gate carried through alpha and the activation's Lipschitz constant,
fp32 rounding of the epilogue, one bf16 rounding of bf16 output).  Covered:
every activation on the skinny, mid and tiled kernels and the streaming
skinny variant (single matrices of >= 1024 column tiles), both output dtypes,
bias and residual on and off, the residual being the output itself (in
place), beta = 0 with a residual that must not be read, and alpha = 0.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
ACTS = ["none", "relu", "silu", "gelu_tanh"]

# (fmt, M, N, K, path): skinny, mid, tiled, a launch the streaming variant
# takes and one the ring variant takes
SHAPES = {
    "skinny": (w4.INT4_G128, 3, 200, 384, "skinny"),
    "mid": (w4.MXFP4, 40, 136, 320, "mid"),
    "tiled": (w4.NVFP4, 40, 136, 256, "tiled"),
    "stream": (w4.INT4_G128, 1, 16384, 256, "auto"),
    # 12 x 8192 A rows: the skinny kernel's ring variant (A through LDS copies)
    "ring": (w4.MXFP4, 12, 80, 8192, "skinny"),
}


def _dev(case):
    A = torch.from_numpy(case.A.view(np.int16)).to(DEV).view(torch.bfloat16)
    p = torch.from_numpy(case.packed).to(DEV)
    if case.fmt in w4.INT4_FORMATS:
        s = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
        z = torch.from_numpy(case.zeros).to(DEV) if case.zeros is not None else None
    else:
        s = torch.from_numpy(case.scales).to(DEV)
        z = None
    return A, p, s, z


def _bias(N, seed):
    rng = np.random.default_rng(seed)
    bits = np.array([oracle.round_bf16(v) for v in rng.standard_normal(N) * 2.0], dtype=np.uint16)
    return bits, torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def _residual(M, N, dtype, seed):
    rng = np.random.default_rng(seed)
    R = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(DEV).to(dtype)
    return R


def _check(name, fmt, M, N, K, path, act, out_dtype, with_bias, with_res, alpha, beta,
           in_place=False, seed=0):
    case = inputs.make_case(fmt, M, N, K, seed)
    A, p, s, z = _dev(case)
    bits, bias = _bias(N, seed + 1) if with_bias else (None, None)
    R = _residual(M, N, out_dtype, seed + 2) if with_res else None
    R_vals = None if R is None else R.double().cpu().numpy()
    print(f"[epilogue] {name}: fmt {fmt} {M}x{N}x{K} {path} act {act} {out_dtype} "
          f"bias {with_bias} res {with_res} alpha {alpha} beta {beta} in_place {in_place}", flush=True)
    if in_place:
        out = R
        C = w4.gemm(fmt, A, p, s, z, out=out, path=path, bias=bias, residual=out,
                    alpha=alpha, beta=beta, activation=act)
    else:
        C = w4.gemm(fmt, A, p, s, z, out_dtype=out_dtype, path=path, bias=bias, residual=R,
                    alpha=alpha, beta=beta, activation=act)
    torch.cuda.synchronize()
    Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    act_id = w4.ACTIVATIONS[act]
    Y = oracle.epilogue(Cref, alpha, bits, act_id, beta, R_vals)
    r = oracle.epilogue_gate_ratio(C.double().cpu().numpy(), Cref, S, alpha, bits, act_id, beta,
                                   R_vals, Y, out_dtype == torch.bfloat16)
    print(f"[gate] max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0, f"{name}: epilogue gate ratio {r}"


@pytest.mark.parametrize("kernel", list(SHAPES))
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_epilogue_bias_residual(kernel, act, out_dtype):
    fmt, M, N, K, path = SHAPES[kernel]
    if kernel == "stream":
        assert w4.gemm_path(fmt, M, N, K, path) == "skinny"
    _check(kernel, fmt, M, N, K, path, act, out_dtype, True, True, 0.75, 1.5)


@pytest.mark.parametrize("kernel", list(SHAPES))
def test_epilogue_in_place_residual(kernel):
    # the residual is the output buffer: each element is read, then overwritten
    fmt, M, N, K, path = SHAPES[kernel]
    _check(kernel, fmt, M, N, K, path, "silu", torch.bfloat16, True, True, 1.0, 1.0, in_place=True)


@pytest.mark.parametrize("kernel", ["skinny", "mid", "tiled"])
def test_epilogue_partial_features(kernel):
    fmt, M, N, K, path = SHAPES[kernel]
    _check(kernel, fmt, M, N, K, path, "none", torch.float32, True, False, 1.0, 0.0)     # bias only
    _check(kernel, fmt, M, N, K, path, "none", torch.float32, False, True, 1.0, -2.0)    # residual only
    _check(kernel, fmt, M, N, K, path, "relu", torch.float32, False, False, 1.0, 0.0)    # activation only
    _check(kernel, fmt, M, N, K, path, "gelu_tanh", torch.float32, True, False, 0.0, 0.0)  # alpha 0


@pytest.mark.parametrize("kernel", ["skinny", "mid", "tiled"])
def test_epilogue_beta_zero_does_not_read_residual(kernel):
    fmt, M, N, K, path = SHAPES[kernel]
    case = inputs.make_case(fmt, M, N, K, 5)
    A, p, s, z = _dev(case)
    R = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path=path, residual=R, beta=0.0,
                activation="relu")
    torch.cuda.synchronize()
    assert torch.isfinite(C).all()
    plain = w4.gemm(fmt, A, p, s, z, out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    assert torch.equal(C, torch.relu(plain))


def test_epilogue_identity_settings_match_plain_gemm():
    # alpha 1, no bias, no activation, beta 0: bit for bit the plain GEMM
    for kernel in SHAPES:
        fmt, M, N, K, path = SHAPES[kernel]
        case = inputs.make_case(fmt, M, N, K, 7)
        A, p, s, z = _dev(case)
        R = _residual(M, N, torch.bfloat16, 8)
        plain = w4.gemm(fmt, A, p, s, z, path=path)
        ex = w4.gemm(fmt, A, p, s, z, path=path, residual=R, beta=0.0, activation="none")
        torch.cuda.synchronize()
        assert torch.equal(plain.view(torch.int16), ex.view(torch.int16)), kernel


def _random_cases(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    fmts = [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64, w4.INT4_SYM]
    out = []
    while len(out) < n:
        fmt = fmts[rng.integers(len(fmts))]
        M = int(rng.choice([1, 2, 5, 16, 17, 40, 64, 130, 260]))
        N = int(rng.integers(1, 700))
        K = 32 * int(rng.integers(1, 200))
        if M * N * K > 15_000_000:
            continue
        path = ["auto", "skinny", "mid", "tiled"][rng.integers(4)]
        act = ACTS[rng.integers(len(ACTS))]
        odt = [torch.bfloat16, torch.float32][rng.integers(2)]
        wb, wr, inp = bool(rng.integers(2)), bool(rng.integers(2)), bool(rng.integers(4) == 0)
        alpha = float(rng.choice([1.0, 0.5, -1.25, 2.0]))
        beta = float(rng.choice([1.0, 0.0, 0.75, -2.0])) if (wr or inp) else 0.0
        out.append((fmt, M, N, K, path, act, odt, wb, wr or inp, alpha, beta, inp, len(out)))
    return out


@pytest.mark.parametrize("fmt,M,N,K,path,act,odt,wb,wr,alpha,beta,inp,i", _random_cases())
def test_epilogue_random(fmt, M, N, K, path, act, odt, wb, wr, alpha, beta, inp, i):
    """Seeded random shapes, formats, paths and epilogue settings (bias or not,
    residual or not, in place or not, alpha / beta, every activation)."""
    _check(f"random {i}", fmt, M, N, K, path, act, odt, wb, wr, alpha, beta, in_place=inp, seed=600 + i)
