import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def read_golden(name):
    """Rows of a golden fixture, '#' comments stripped, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def int4_rounding_adversary(fmt, M, N, K, seed):
    """An int4 case on which weights rounded to bf16 BEFORE the sum fail the
    GEMM gate by a wide margin (with fp32 output), while exact weights pass.

    Every group holds one repeated code c with zero point z and a bf16 scale s
    chosen so that the exact weight (c - z) * s lies just above a bf16
    rounding boundary: rounding it moves it down by more than 3e-3 of its
    value (the gate allows 2e-3 of S).  Every activation is positive, so the
    rounding errors of a row add up coherently: |sum a w~ - sum a w| > 3e-3 S.
    Returns an inputs.Case (the oracle's round_bf16 / bf16_value choose the
    pairs; nothing comes from the GPU path)."""
    import numpy as np
    import oracle
    from weight_only_bit_w4a16_amd import inputs

    # (d, scale bits) with d = c - z in 1..7 and scale m * 2^-14, m = 128..255:
    # relative change of d * s when rounded to bf16
    pairs = []
    for d in range(1, 8):
        for m in range(128, 256):
            bits = (120 << 7) | (m - 128)
            s = oracle.bf16_value(bits)
            w = d * s
            r = (oracle.bf16_value(oracle.round_bf16(w)) - w) / w
            if r < -3e-3:
                pairs.append((d, bits))
    assert pairs, "no adversarial (code - zero, scale) pair"
    case = inputs.make_case(fmt, M, N, K, seed)
    rng = np.random.default_rng(seed + 7)
    G = oracle.GROUP[fmt]
    ng = (K + G - 1) // G
    pick = rng.integers(0, len(pairs), size=(N, ng))
    d = np.array([p[0] for p in pairs])[pick]
    sbits = np.array([p[1] for p in pairs], dtype=np.uint16)[pick]
    if fmt == oracle.INT4_SYM:
        z = np.full((N, ng), 8)
    else:
        z = (rng.integers(0, 16, size=(N, ng)) % (16 - d)).astype(np.int64)
        case.zeros[:] = z.astype(np.uint8)
    c = (z + d).astype(np.uint8)                       # the code of every weight of the group
    codes = np.repeat(c, G, axis=1)[:, :K]
    case.packed[:] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    case.scales[:] = sbits
    case.A[:] = case.A & np.uint16(0x7FFF)             # |a|: every product has the weight's sign
    return case


def int4_cancellation_adversary(fmt, M, N, K, seed):
    """An int4 case whose exact result is tiny beside the terms a kernel could
    form on the way: every code of a group equals its zero point except one,
    which is one step away, and that code meets the one small activation of
    the group (2^-12) while the other activations are large (about 2^8).  The
    exact sum is then a handful of small products, and a kernel that adds
    sum(a * code) and sum(a * (-zero)) separately leaves fp32 rounding errors
    of the large sums (about 2^-24 * 2^12) that exceed the gate by orders of
    magnitude; a kernel that forms code - zero before multiplying is exact.
    Scales are 1.0.  Returns an inputs.Case."""
    import numpy as np
    import oracle
    from weight_only_bit_w4a16_amd import inputs

    case = inputs.make_case(fmt, M, N, K, seed)
    rng = np.random.default_rng(seed + 11)
    G = oracle.GROUP[fmt]
    ng = (K + G - 1) // G
    z = np.full((N, ng), 8) if fmt == oracle.INT4_SYM else rng.integers(1, 15, size=(N, ng))
    if case.zeros is not None:
        case.zeros[:] = z.astype(np.uint8)
    codes = np.repeat(z, G, axis=1)[:, :K].astype(np.int64)
    # one position per group and row: code = zero +- 1, at the group's small activation
    pos = np.minimum(np.arange(ng) * G + rng.integers(0, G, size=ng), K - 1)  # same for every row
    step = rng.choice([-1, 1], size=(N, ng))
    codes[:, pos] += step
    codes = codes.astype(np.uint8)
    case.packed[:] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    case.scales[:] = oracle.round_bf16(1.0)
    a = (rng.standard_normal((M, K)) * 256.0).astype(np.float32)
    a[:, pos] = np.float32(2.0 ** -12) * rng.choice([-1, 1], size=(M, ng))
    case.A[:] = inputs.bf16_bits(a)
    return case
