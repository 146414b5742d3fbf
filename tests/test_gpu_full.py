"""Every output of the large launches against the oracle (through the C ABI).

The tiled kernel's 256 x 256 tile configuration -- the one the M = 4096 MXFP4
workload runs, chosen from 192 such tiles on -- compared element by element:
* every weight format, bf16 and fp32 output, ragged M and N, K spanning
  several scale tiles (and a short last group where the format allows one);
* the fused epilogue on it: bias, residual, every activation, alpha, in place;
* the M = 4096 MXFP4 workload itself (4096 x 8192 x 3072), all 33.5 M outputs,
  seeds 0 and 1;
and the 3B decode chain's distinct shapes with the second seed, the LM head
(128256 x 3072) in full.

The reference for the large shapes is oracle.gemm_matmul (the oracle's exact
dequantisation and a binary64 matrix product), pinned against the
element-by-element oracle in tests/test_oracle_pins.py.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)

# 1528 x 8200: 6 x 33 = 198 tiles of 256 x 256, both dimensions ragged.
# K per format: at least two scale tiles of the tiled kernel (int4 groups of
# 128: 16 k-tiles per scale tile; NVFP4 4; the rest 8), K % 64 == 32 for a
# ragged last k-tile, and for int4 with groups of 128 / 64 a short last group.
LM, LN = 1528, 8200
LARGE_K = {w4.INT4_G128: 2080, w4.INT4_SYM: 2080, w4.INT4_G64: 1056, w4.INT4_G32: 1056,
           w4.NVFP4: 800, w4.MXFP4: 1056}


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


_REF = {}


def large_case(fmt):
    """The large-tile case of a format and its (C, S) reference (cached)."""
    if fmt not in _REF:
        K = LARGE_K[fmt]
        case = inputs.make_case(fmt, LM, LN, K, seed=fmt + 60)
        _REF[fmt] = (case, oracle.gemm_matmul(fmt, case.A, case.packed, case.scales, case.zeros, LM, LN, K))
    return _REF[fmt]


def check(C, Cref, S, bf16_out, what):
    r = oracle.gate_ratio(C, Cref, S, bf16_out)
    print(f"[gate] {what}: max err/bound = {r:.3e} over {C.size} outputs", flush=True)
    assert r <= 1.0, f"{what}: gate ratio {r}"


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64, w4.INT4_SYM])
def test_large_tiles_every_output(fmt, out):
    K = LARGE_K[fmt]
    assert w4.gemm_path(fmt, LM, LN, K) == "tiled"
    assert ((LM + 255) // 256) * ((LN + 255) // 256) >= 192  # the 256 x 256 configuration
    case, (Cref, S) = large_case(fmt)
    A, p, s, z = to_dev(case)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    print(f"[full] fmt {fmt} {LM}x{LN}x{K} out {out}", flush=True)
    C = w4.gemm(fmt, A, p, s, z, out_dtype=odt).double().cpu().numpy()
    check(C, Cref, S, out == "bf16", f"large tiles fmt {fmt} {LM}x{LN}x{K} {out}")


EPI = [  # (fmt, out, activation, bias, residual, alpha, beta, in place)
    (w4.MXFP4, "bf16", "none", True, True, 1.0, 1.0, False),
    (w4.MXFP4, "bf16", "relu", True, True, 0.5, 1.0, False),
    (w4.MXFP4, "bf16", "silu", True, False, 1.0, 0.0, False),
    (w4.MXFP4, "f32", "gelu_tanh", True, True, 1.0, 0.5, True),
    (w4.MXFP4, "f32", "silu", False, True, 2.0, -1.0, False),
    (w4.INT4_G128, "bf16", "gelu_tanh", True, True, 1.0, 1.0, True),
    (w4.INT4_G128, "f32", "relu", True, True, 1.0, 1.0, False),
    (w4.INT4_G32, "bf16", "silu", True, True, 1.0, 1.0, False),
    (w4.NVFP4, "f32", "none", True, True, 0.25, 1.0, True),
    (w4.INT4_SYM, "bf16", "relu", False, True, 1.0, 1.0, False),
]


@pytest.mark.parametrize("fmt,out,act,with_bias,with_res,alpha,beta,in_place", EPI)
def test_large_tiles_epilogue_every_output(fmt, out, act, with_bias, with_res, alpha, beta, in_place):
    case, (Cref, S) = large_case(fmt)
    K = LARGE_K[fmt]
    A, p, s, z = to_dev(case)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    rng = np.random.default_rng(fmt * 10 + len(act))
    bits = bias = None
    if with_bias:
        bits = np.array([oracle.round_bf16(v) for v in rng.standard_normal(LN) * 2.0], np.uint16)
        bias = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    R = R_vals = None
    if with_res:
        R = torch.from_numpy(rng.standard_normal((LM, LN)).astype(np.float32)).to(DEV).to(odt)
        R_vals = R.double().cpu().numpy()
    print(f"[full epilogue] fmt {fmt} out {out} act {act} bias {with_bias} res {with_res} "
          f"alpha {alpha} beta {beta} in place {in_place}", flush=True)
    if in_place:
        C = w4.gemm(fmt, A, p, s, z, out=R, bias=bias, residual=R, alpha=alpha, beta=beta, activation=act)
    else:
        C = w4.gemm(fmt, A, p, s, z, out_dtype=odt, bias=bias, residual=R, alpha=alpha, beta=beta,
                    activation=act)
    torch.cuda.synchronize()
    act_id = w4.ACTIVATIONS[act]
    Y = oracle.epilogue(Cref, alpha, bits, act_id, beta, R_vals)
    r = oracle.epilogue_gate_ratio(C.double().cpu().numpy(), Cref, S, alpha, bits, act_id, beta,
                                   R_vals, Y, out == "bf16")
    print(f"[gate] large tiles epilogue: max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp4_m4096_every_output(seed):
    """The compute-bound workload at full size, all 33.5 M outputs."""
    fmt, M, N, K = w4.MXFP4, 4096, 8192, 3072
    case = inputs.make_case(fmt, M, N, K, seed)
    A, p, s, z = to_dev(case)
    print(f"[full] mxfp4 {M}x{N}x{K} seed {seed}", flush=True)
    C = w4.gemm(fmt, A, p, s, z).double().cpu().numpy()
    Cref, S = oracle.gemm_matmul(fmt, case.A, case.packed, case.scales, None, M, N, K)
    check(C, Cref, S, True, f"mxfp4 m4096 seed {seed}")


@pytest.mark.timeout(300)
def test_decode_chain_second_seed():
    """Every distinct shape of the 3B decode chain with the second seed
    (q / o 3072 x 3072, k / v 1024 x 3072, gate / up 8192 x 3072, down
    3072 x 8192, LM head 128256 x 3072), every output."""
    shapes = inputs.decoder_chain_shapes()
    seen = {}
    for i, (name, n, k) in enumerate(shapes):
        seen.setdefault((n, k), (i, name))
    for (n, k), (i, name) in seen.items():
        case = inputs.make_case(w4.INT4_G128, 1, n, k, inputs.chain_seed(1, i))
        A, p, s, z = to_dev(case)
        print(f"[chain seed 1] {name} {n}x{k}", flush=True)
        C = w4.gemm(w4.INT4_G128, A, p, s, z).double().cpu().numpy()
        Cref, S = oracle.gemm(w4.INT4_G128, case.A, case.packed, case.scales, case.zeros, 1, n, k)
        check(C, Cref, S, True, f"chain seed 1 {name} ({n}x{k})")
