"""Parity of the HIP path (through the C ABI) with the CPU oracle.

* dequant: bit-exact bf16 weights, every format, at the workloads' (N, K),
  ragged shapes and special scale / zero values;
* GEMM: every element within the gate |C - C_ref| <= 2e-3 S + 1e-6
  (+ 2^-8 |C_ref| for bf16 output), S = sum_k |a w|, on the workloads
  (seeds 0 and 1, both kernels), ragged shapes and degenerate inputs.  At
  the full large shapes the oracle is sampled element by element.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_w4a16_amd as w4
from weight_only_bit_w4a16_amd import inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


# ---- helpers ------------------------------------------------------------------

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


def bits_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_dequant_exact(fmt, packed, scales, zeros, N, K):
    """GPU dequant of the given host arrays equals the oracle bit for bit
    (NaN matches any NaN)."""
    case = inputs.Case(fmt, 0, N, K, np.zeros((0, K), np.uint16), packed, scales, zeros)
    _, p, s, z = to_dev(case)
    W = w4.dequant(fmt, p, s, z)
    torch.cuda.synchronize()
    got = bits_u16(W)
    _, ref = oracle.dequant(fmt, packed, scales, zeros, N, K)
    nan_ref = (ref & 0x7FFF) > 0x7F80
    nan_got = (got & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_ref, nan_got)
    diff = (got != ref) & ~nan_ref
    if diff.any():
        i = np.argwhere(diff)[:5]
        raise AssertionError(f"{diff.sum()} weights differ, e.g. at {i.tolist()}: "
                             f"gpu {[hex(got[tuple(x)]) for x in i]} "
                             f"oracle {[hex(ref[tuple(x)]) for x in i]}")


def run_gemm(case, out_dtype, path):
    A, p, s, z = to_dev(case)
    C = w4.gemm(case.fmt, A, p, s, z, out_dtype=out_dtype, path=path)
    torch.cuda.synchronize()
    return C.double().cpu().numpy()


def check_gate(C, Cref, S, bf16_out, what):
    r = oracle.gate_ratio(C, Cref, S, bf16_out)
    print(f"[gate] {what}: max err/bound = {r:.3e}", flush=True)
    assert r <= 1.0, f"{what}: gate ratio {r}"
    return r


# ---- dequant ---------------------------------------------------------------------

DEQ_SHAPES = [
    (w4.INT4_G128, 256, 512), (w4.INT4_G128, 8192, 3072), (w4.INT4_G128, 3072, 8192),
    (w4.NVFP4, 3072, 8192), (w4.NVFP4, 7, 96), (w4.NVFP4, 5, 32),
    (w4.MXFP4, 8192, 3072), (w4.MXFP4, 33, 160),
]


@pytest.mark.parametrize("fmt,N,K", DEQ_SHAPES)
def test_dequant_bit_exact(fmt, N, K):
    case = inputs.make_case(fmt, 0, N, K, seed=N + K)
    assert_dequant_exact(fmt, case.packed, case.scales, case.zeros, N, K)


def test_dequant_lm_head_rows():
    """Rows sampled from the 128256 x 3072 int4 LM head."""
    case = inputs.make_case(w4.INT4_G128, 0, 128256, 3072, seed=0)
    _, p, s, z = to_dev(case)
    W = bits_u16(w4.dequant(w4.INT4_G128, p, s, z))
    rows = np.random.default_rng(0).choice(128256, 96, replace=False)
    rows = np.concatenate([rows, [0, 128255]])
    _, ref = oracle.dequant(w4.INT4_G128, case.packed[rows], case.scales[rows], case.zeros[rows],
                            len(rows), 3072)
    assert np.array_equal(W[rows], ref)


def _all_codes(N, K):
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_dequant_every_e4m3_scale():
    """NVFP4: all 256 e4m3 scale bytes (NaN, subnormal, negative) x all 16 codes."""
    N, K = 256, 32
    packed = _all_codes(N, K)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    assert_dequant_exact(w4.NVFP4, packed, scales, None, N, K)


def test_dequant_every_e8m0_scale():
    """MXFP4: all 256 e8m0 bytes (2^-127 .. 2^127 and NaN) x all 16 codes."""
    N, K = 256, 32
    packed = _all_codes(N, K)
    scales = np.arange(256, dtype=np.uint8)[:, None].copy()
    assert_dequant_exact(w4.MXFP4, packed, scales, None, N, K)


def test_dequant_int4_special_scales_and_zeros():
    """int4: scale bit patterns across the bf16 range (subnormal, huge ->
    overflow, negative, zero, inf, NaN) with every zero byte and code."""
    rng = np.random.default_rng(5)
    N, K = 1024, 128
    packed = _all_codes(N, K)
    special = np.array([0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
                        0x7E00, 0x7F80, 0xFF80, 0x7FC0, 0x3C23, 0x3BA4], np.uint16)
    scales = rng.integers(0, 65536, size=(N, 1)).astype(np.uint16)
    scales[:len(special), 0] = special
    zeros = rng.integers(0, 256, size=(N, 1)).astype(np.uint8)
    zeros[:16, 0] = np.arange(16)
    assert_dequant_exact(w4.INT4_G128, packed, scales, zeros, N, K)


# ---- GEMM on the workloads -------------------------------------------------------

WORKLOADS = {
    "tiny_int4_m16": (w4.INT4_G128, 16, 256, 512, torch.float32),
    "decode_gemv_int4_m1": (w4.INT4_G128, 1, 8192, 3072, torch.bfloat16),
    "nvfp4_m16": (w4.NVFP4, 16, 3072, 8192, torch.bfloat16),
}


_REF_CACHE = {}


def _workload_ref(name, seed):
    if (name, seed) not in _REF_CACHE:
        fmt, M, N, K, _ = WORKLOADS[name]
        case = inputs.make_case(fmt, M, N, K, seed)
        ref = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
        _REF_CACHE[(name, seed)] = (case, ref)
    return _REF_CACHE[(name, seed)]


@pytest.mark.parametrize("path", ["auto", "skinny", "mid", "tiled"])
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_gemm_workloads_full(name, seed, path):
    fmt, M, N, K, odt = WORKLOADS[name]
    case, (Cref, S) = _workload_ref(name, seed)
    C = run_gemm(case, odt, path)
    check_gate(C, Cref, S, odt == torch.bfloat16, f"{name} seed {seed} path {path}")


@pytest.mark.parametrize("path", ["auto", "skinny"])
@pytest.mark.parametrize("seed", [0, 1])
def test_gemm_mxfp4_m4096_sampled(seed, path):
    """The compute-bound MXFP4 workload at full size; 4096 sampled outputs
    (every tile row and column band is hit) plus corners."""
    fmt, M, N, K = w4.MXFP4, 4096, 8192, 3072
    case = inputs.make_case(fmt, M, N, K, seed)
    C = run_gemm(case, torch.bfloat16, path)
    rng = np.random.default_rng(100 + seed)
    mi = np.concatenate([rng.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, None, M, N, K, mi, ni)
    check_gate(C[mi, ni], Cref, S, True, f"mxfp4 m4096 seed {seed} path {path}")
    assert np.all(np.isfinite(C))


def test_decode_chain_shapes():
    """One matrix of each distinct shape of the 3B decode chain at M = 1:
    k/v (1024 x 3072), q/o (3072 x 3072), gate/up (8192 x 3072),
    down (3072 x 8192) in full, and the LM head sampled."""
    shapes = inputs.decoder_chain_shapes()
    seen = {}
    for i, (name, n, k) in enumerate(shapes):
        seen.setdefault((n, k), (i, name))
    for (n, k), (i, name) in seen.items():
        case = inputs.make_case(w4.INT4_G128, 1, n, k, inputs.chain_seed(0, i))
        C = run_gemm(case, torch.bfloat16, "auto")
        if n > 10000:
            ni = np.random.default_rng(i).integers(0, n, 4096)
            mi = np.zeros_like(ni)
            Cref, S = oracle.gemm_at(w4.INT4_G128, case.A, case.packed, case.scales, case.zeros,
                                     1, n, k, mi, ni)
            check_gate(C[0, ni], Cref, S, True, f"chain {name} ({n}x{k}) sampled")
        else:
            Cref, S = oracle.gemm(w4.INT4_G128, case.A, case.packed, case.scales, case.zeros,
                                  1, n, k)
            check_gate(C, Cref, S, True, f"chain {name} ({n}x{k})")


# ---- ragged shapes, forced paths, degenerate inputs ------------------------------

RAGGED = [
    (w4.INT4_G128, 1, 16, 128), (w4.INT4_G128, 3, 33, 256), (w4.INT4_G128, 17, 200, 384),
    (w4.INT4_G128, 300, 257, 640),
    (w4.NVFP4, 1, 40, 32), (w4.NVFP4, 5, 19, 96), (w4.NVFP4, 16, 512, 160),
    (w4.NVFP4, 130, 300, 224),
    (w4.MXFP4, 2, 17, 32), (w4.MXFP4, 9, 64, 96), (w4.MXFP4, 260, 520, 192),
    (w4.MXFP4, 513, 129, 64),
    # short N / few rows: the skinny kernel splits K inside the MFMA (k-parts),
    # here with part counts that do not divide the k-blocks evenly
    (w4.MXFP4, 1, 200, 288), (w4.NVFP4, 2, 100, 480), (w4.INT4_G128, 3, 50, 1280),
    (w4.INT4_G128, 1, 1024, 3072), (w4.NVFP4, 1, 72, 8192),
    # long fp4 scale windows: per-lane scale loads at one row, the LDS-staged
    # window from two rows on
    (w4.NVFP4, 4, 72, 8192), (w4.MXFP4, 1, 40, 8192), (w4.MXFP4, 3, 40, 8192),
]


@pytest.mark.parametrize("path", ["skinny", "mid", "tiled"])
@pytest.mark.parametrize("fmt,M,N,K", RAGGED)
def test_gemm_ragged(fmt, M, N, K, path):
    case = inputs.make_case(fmt, M, N, K, seed=M * 7 + N * 3 + K)
    for odt in (torch.float32, torch.bfloat16):
        C = run_gemm(case, odt, path)
        Cref, S = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
        check_gate(C, Cref, S, odt == torch.bfloat16, f"ragged {fmt} {M}x{N}x{K} {path} {odt}")


@pytest.mark.parametrize("fmt,M,N,K", [(w4.NVFP4, 2050, 6150, 96), (w4.INT4_G128, 1999, 6200, 256),
                                       (w4.MXFP4, 4100, 3000, 160)])
def test_gemm_large_tiles_ragged_sampled(fmt, M, N, K):
    """The tiled kernel's 256 x 256 tiles (chosen from 192 of them up) with
    every dimension ragged; 4096 sampled outputs plus the four corners."""
    assert w4.gemm_path(fmt, M, N, K) == "tiled"
    case = inputs.make_case(fmt, M, N, K, seed=M + N + K)
    C = run_gemm(case, torch.bfloat16, "auto")
    rng = np.random.default_rng(M)
    mi = np.concatenate([rng.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([rng.integers(0, N, 4096), [0, N - 1, 0, N - 1]])
    Cref, S = oracle.gemm_at(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K, mi, ni)
    check_gate(C[mi, ni], Cref, S, True, f"large tiles {fmt} {M}x{N}x{K}")
    assert np.all(np.isfinite(C))


@pytest.mark.parametrize("path", ["skinny", "mid", "tiled"])
def test_gemm_degenerate(path):
    # every int4 code equal to its zero point -> exactly 0
    M, N, K = 4, 48, 256
    case = inputs.make_case(w4.INT4_G128, M, N, K, seed=3)
    case.packed[:] = 0x77
    case.zeros[:] = 7
    C = run_gemm(case, torch.float32, path)
    assert np.all(C == 0)
    # A = 0 -> exactly 0 for every format
    for fmt in (w4.NVFP4, w4.MXFP4):
        case = inputs.make_case(fmt, M, N, K, seed=4)
        case.A[:] = 0
        assert np.all(run_gemm(case, torch.float32, path) == 0)


@pytest.mark.parametrize("path,M,K", [
    ("skinny", 1, 512),     # A staged in LDS (even / odd k order)
    ("skinny", 16, 4096),   # A too large for the LDS copy: natural k order
    ("mid", 40, 512), ("tiled", 40, 512)])
def test_gemm_int4_any_zero_byte(path, M, K):
    # zero points across the whole byte range (the format itself stores 0..15)
    N = 96
    case = inputs.make_case(w4.INT4_G128, M, N, K, seed=11 + M)
    rng = np.random.default_rng(12 + M)
    case.zeros[:] = rng.integers(0, 256, size=case.zeros.shape, dtype=np.uint8)
    case.zeros.flat[:4] = [0, 127, 128, 255]
    Cref, S = oracle.gemm(w4.INT4_G128, case.A, case.packed, case.scales, case.zeros, M, N, K)
    for odt in (torch.float32, torch.bfloat16):
        C = run_gemm(case, odt, path)
        check_gate(C, Cref, S, odt == torch.bfloat16, f"int4 zeros 0..255 {M}x{N}x{K} {path} {odt}")


@pytest.mark.parametrize("path,M,N,K", [
    ("skinny", 1, 96, 512), ("skinny", 16, 72, 8192), ("mid", 40, 96, 512),
    ("tiled", 40, 96, 512), ("tiled", 300, 257, 224), ("auto", 5, 40, 48)])
def test_gemm_nvfp4_negative_scale_bytes(path, M, N, K):
    """NVFP4 scale bytes with the sign bit set on a random half: the scale
    enters by magnitude (the NVFP4 dequantisation writes |scale|), so the
    result matches the oracle and equals, bit for bit, the run with every
    sign bit clear."""
    case = inputs.make_case(w4.NVFP4, M, N, K, seed=21 + M + K)
    rng = np.random.default_rng(22 + M)
    pos = case.scales.copy()
    case.scales |= (rng.integers(0, 2, size=pos.shape, dtype=np.uint8) << 7).astype(np.uint8)
    assert (case.scales >= 0x80).any() and (case.scales < 0x80).any()
    Cref, S = oracle.gemm(w4.NVFP4, case.A, case.packed, case.scales, None, M, N, K)
    for odt in (torch.float32, torch.bfloat16):
        C = run_gemm(case, odt, path)
        check_gate(C, Cref, S, odt == torch.bfloat16, f"nvfp4 signed scales {M}x{N}x{K} {path}")
        neg_bits = C.copy()
        case_pos = inputs.Case(case.fmt, M, N, K, case.A, case.packed, pos, None)
        assert np.array_equal(run_gemm(case_pos, odt, path), neg_bits)


def test_gemm_zero_extent():
    case = inputs.make_case(w4.MXFP4, 0, 64, 64, seed=0)
    A, p, s, _ = to_dev(case)
    C = w4.gemm(w4.MXFP4, A, p, s, None)
    assert C.shape == (0, 64)
    A1 = torch.zeros((3, 64), dtype=torch.bfloat16, device=DEV)
    C = w4.gemm(w4.MXFP4, A1, p[:0], s[:0], None)
    assert C.shape == (3, 0)


# ---- determinism and streams --------------------------------------------------------

@pytest.mark.parametrize("fmt,M,N,K", [(w4.INT4_G128, 1, 8192, 3072), (w4.NVFP4, 16, 3072, 8192),
                                       (w4.INT4_G128, 64, 8192, 3072), (w4.MXFP4, 512, 1024, 3072)])
def test_deterministic_and_stream(fmt, M, N, K):
    case = inputs.make_case(fmt, M, N, K, seed=9)
    A, p, s, z = to_dev(case)
    C1 = w4.gemm(fmt, A, p, s, z)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        C2 = w4.gemm(fmt, A, p, s, z, stream=st)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("fmt,M,N,K,path", [(w4.INT4_G128, 1, 4096, 3072, "auto"),
                                            (w4.NVFP4, 16, 1024, 512, "auto"),
                                            (w4.NVFP4, 64, 1024, 512, "mid"),
                                            (w4.NVFP4, 16, 1024, 8192, "auto"),   # skinny ring
                                            (w4.MXFP4, 300, 512, 256, "tiled"),
                                            (w4.INT4_G64, 40, 300, 512, "skinny")])
def test_hip_graph_capture_replay(fmt, M, N, K, path):
    """The C ABI call is capturable: replays of a captured graph, with eager
    work and synchronisations between them, match the eager result."""
    case = inputs.make_case(fmt, M, N, K, seed=21)
    A, p, s, z = to_dev(case)
    eager = w4.gemm(fmt, A, p, s, z, path=path)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    call = w4.PreparedGemm(fmt, A, p, s, z, out, path=path)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        out.fill_(float("nan"))
        _ = (A.float() * (i + 1)).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"


# ---- exact single-atom and chain-graph checks ----------------------------------------

@pytest.mark.parametrize("fmt", [w4.INT4_G128, w4.NVFP4, w4.MXFP4, w4.INT4_G32, w4.INT4_G64, w4.INT4_SYM])
@pytest.mark.parametrize("path", ["skinny", "mid", "tiled"])
def test_integer_data_is_exact(fmt, path):
    """One MFMA atom's worth of rows and columns (16 x 16) over one or a few
    k-blocks, with small-integer activations and unit scales: every product
    and partial sum is an integer below 2^24, so any correct kernel returns the
    oracle's value bit for bit -- a transposed operand, a wrong k-slot order
    or a misplaced nibble cannot hide inside the tolerance."""
    M, N, K = 16, 16, 256
    case = inputs.make_case(fmt, M, N, K, seed=40 + fmt)
    rng = np.random.default_rng(41 + fmt)
    a = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    case.A[:] = np.array([oracle.round_bf16(v) for v in a.ravel()], np.uint16).reshape(M, K)
    if fmt in w4.INT4_FORMATS:
        case.scales[:] = oracle.round_bf16(1.0)
    elif fmt == w4.NVFP4:
        case.scales[:] = 0x38   # e4m3 1.0
    else:
        case.scales[:] = 127    # e8m0 1.0
    C = run_gemm(case, torch.float32, path)
    Cref, _ = oracle.gemm(fmt, case.A, case.packed, case.scales, case.zeros, M, N, K)
    assert np.all(np.abs(Cref) < 2 ** 20) and np.all(Cref == np.round(Cref * 2) / 2)
    assert np.array_equal(C, Cref), np.argwhere(C != Cref)[:5]


def test_decode_chain_graph_replay():
    """Two decoder layers of the chain (8 launches: grouped q/k/v, o, grouped
    gate/up, down) captured in one graph; every replay equals eager calls."""
    shapes = inputs.decoder_chain_shapes(2)
    groups = inputs.decoder_chain_groups(2)[:-1]  # without the LM head
    dev_w, dev_a = [], []
    for i, (name, n, k) in enumerate(shapes[:-1]):
        case = inputs.make_case(w4.INT4_G128, 1, n, k, inputs.chain_seed(0, i))
        A, p, s, z = to_dev(case)
        dev_w.append((p, s, z))
        dev_a.append(A)
    outs = [[torch.empty((1, shapes[i][1]), dtype=torch.bfloat16, device=DEV) for i in g] for g in groups]
    calls = [w4.PreparedGroupedGemm(w4.INT4_G128, dev_a[g[0]], [dev_w[i] for i in g], o)
             for g, o in zip(groups, outs)]
    eager = [[w4.gemm(w4.INT4_G128, dev_a[g[0]], *dev_w[i]) for i in g] for g in groups]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    for rep in range(3):
        for o in outs:
            for t in o:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            for t, ref in zip(o, e):
                assert torch.equal(t.view(torch.int16), ref.view(torch.int16)), rep
