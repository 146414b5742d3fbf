"""Parity of w4a16_gemm_grouped (through the C ABI) with the CPU oracle.

Several weight matrices share one A: every member's C must pass the element
gate against the oracle and equal, bit for bit, what w4a16_gemm computes for
that member alone (the grouped launch runs the same kernel on each member's
column tiles).  Covers ragged N, a skipped empty member, the maximum group
size, both kernels and the decoder layer's q/k/v and gate/up groups.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _dev_weights(case):
    p = torch.from_numpy(case.packed).to(DEV)
    if case.fmt in w4.INT4_FORMATS:
        s = torch.from_numpy(case.scales.view(np.int16)).to(DEV).view(torch.bfloat16)
        z = torch.from_numpy(case.zeros).to(DEV)
    else:
        s = torch.from_numpy(case.scales).to(DEV)
        z = None
    return p, s, z


def _group(fmt, M, Ns, K, seed):
    """Member i's weights from seed 100*seed + i; A is member 0's."""
    cases = [inputs.make_case(fmt, M, N, K, 100 * seed + i) for i, N in enumerate(Ns)]
    A = torch.from_numpy(cases[0].A.view(np.int16)).to(DEV).view(torch.bfloat16)
    return cases, A, [_dev_weights(c) for c in cases]


def _check_group(fmt, M, Ns, K, seed, out_dtype, path):
    cases, A, weights = _group(fmt, M, Ns, K, seed)
    print(f"[grouped] fmt {fmt} M {M} N {Ns} K {K} seed {seed} {out_dtype} path {path}", flush=True)
    outs = w4.gemm_grouped(fmt, A, weights, out_dtype=out_dtype, path=path)
    singles = [w4.gemm(fmt, A, p, s, z, out_dtype=out_dtype, path=path) for p, s, z in weights]
    torch.cuda.synchronize()
    bf16 = out_dtype == torch.bfloat16
    for i, (case, out, single) in enumerate(zip(cases, outs, singles)):
        if Ns[i] == 0:
            assert out.numel() == 0
            continue
        assert torch.equal(out.view(torch.int16) if bf16 else out.view(torch.int32),
                           single.view(torch.int16) if bf16 else single.view(torch.int32)), \
            f"member {i} differs from its single launch"
        Cref, S = oracle.gemm(fmt, cases[0].A, case.packed, case.scales, case.zeros, M, Ns[i], K)
        r = oracle.gate_ratio(out.double().cpu().numpy(), Cref, S, bf16)
        print(f"[gate] member {i} ({Ns[i]} cols): max err/bound = {r:.3e}", flush=True)
        assert r <= 1.0, f"member {i}: gate ratio {r}"


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.NVFP4, w4.MXFP4])
@pytest.mark.parametrize("M", [1, 7, 16])
def test_grouped_ragged(fmt, M):
    _check_group(fmt, M, [96, 40, 200, 16], 640, 0, torch.bfloat16, "auto")


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.MXFP4])
def test_grouped_f32_and_max_members(fmt):
    _check_group(fmt, 3, [16 * (i + 1) + (i % 3) for i in range(w4.MAX_GROUP)], 256,
                 1, torch.float32, "skinny")


def test_grouped_skips_empty_member():
    _check_group(w4.NVFP4, 2, [64, 0, 48], 512, 2, torch.bfloat16, "auto")


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.NVFP4])
def test_grouped_tiled_path(fmt):
    # the tiled kernel: one launch per member
    _check_group(fmt, 40, [96, 200], 384, 3, torch.bfloat16, "tiled")


@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.MXFP4])
def test_grouped_mid_m(fmt):
    # the mid kernel: one launch per member
    _check_group(fmt, 40, [96, 200], 384, 6, torch.bfloat16, "mid")


def test_grouped_mid_m_auto():
    # 16 < M <= 384 and a wide member: the mid kernel, chosen for the widest
    assert w4.gemm_path(w4.NVFP4, 40, 5120, 256) == "mid"
    _check_group(w4.NVFP4, 40, [5120, 1024], 256, 7, torch.bfloat16, "auto")


@pytest.mark.parametrize("fmt", [w4.NVFP4, w4.MXFP4])
def test_grouped_mid_m_forced_skinny(fmt):
    # the skinny kernel over 16-row slices, all members in one launch
    _check_group(fmt, 40, [96, 0, 200], 384, 8, torch.float32, "skinny")


@pytest.mark.parametrize("members", [("q", "k", "v"), ("gate", "up")])
def test_grouped_decoder_layer(members):
    shapes = {name.split(".")[1]: (n, k) for name, n, k in inputs.decoder_chain_shapes(1) if "." in name}
    Ns = [shapes[m][0] for m in members]
    K = shapes[members[0]][1]
    _check_group(w4.INT4_G128, 1, Ns, K, 4, torch.bfloat16, "auto")


def test_grouped_graph_replay():
    cases, A, weights = _group(w4.INT4_G128, 1, [3072, 1024, 1024], 3072, 5)
    outs = [torch.empty((1, c.N), dtype=torch.bfloat16, device=DEV) for c in cases]
    call = w4.PreparedGroupedGemm(w4.INT4_G128, A, weights, outs)
    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}"
