"""Seeded synthetic inputs for the W4A16 dequantise-GEMM workloads.

This module only draws random numbers and stores them in the operand
dtypes; it holds none of the method's arithmetic.  Both the HIP path and the
CPU oracle consume the same arrays it returns.  Type conversions of the drawn
reals (to bf16 and to float8 e4m3) use torch's CPU dtype casts.

Recipe (numpy PCG64 ``default_rng(seed)``; draw order A, packed, zeros, scales):

* A      : bf16(N(0, 1)), shape (M, K)
* packed : uniform bytes 0..255, shape (N, K/2) -- i.e. independent uniform
           4-bit codes, low nibble = even k
* int4   : zeros uniform 0..15 and scales bf16(U[0.005, 0.02]), (N, K/128)
* NVFP4  : scales e4m3(U[2^-4, 4]), (N, K/16), stored as raw bytes
* MXFP4  : e8m0 bytes 127 + uniform integer in [-4, 4], (N, K/32)

The shapes are those of the workloads on the pages: the 3B decoder's layer
matrices from the "megakernel_int4_weight_decode.py" spec (d 3072, ffn 8192,
24 query and 8 KV heads of 128, vocab 128256, tied LM head), and the NVFP4
layout of the "Matmul2dFp4" reference.  No dataset or trained weight is used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

INT4_G128, NVFP4, MXFP4, INT4_G32, INT4_G64, INT4_SYM = 0, 1, 2, 3, 4, 5
FORMAT_NAMES = {INT4_G128: "int4_g128", NVFP4: "nvfp4", MXFP4: "mxfp4",
                INT4_G32: "int4_g32", INT4_G64: "int4_g64", INT4_SYM: "int4_sym"}
GROUP = {INT4_G128: 128, NVFP4: 16, MXFP4: 32, INT4_G32: 32, INT4_G64: 64, INT4_SYM: 128}
INT4_FORMATS = (INT4_G128, INT4_G32, INT4_G64, INT4_SYM)  # bf16 scales
ZERO_FORMATS = (INT4_G128, INT4_G32, INT4_G64)  # with a zero array


@dataclass
class Case:
    fmt: int
    M: int
    N: int
    K: int
    A: np.ndarray        # uint16 bf16 bits (M, K)
    packed: np.ndarray   # uint8 (N, K/2)
    scales: np.ndarray   # uint16 bf16 bits (int4) or uint8 bytes (fp4), (N, K/G)
    zeros: np.ndarray | None  # uint8 (N, K/G) for asymmetric int4, else None


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store reals as bf16 (torch's round-to-nearest-even cast), as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """Store reals as float8 e4m3fn (torch's cast), as raw bytes."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def make_activations(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    return bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def make_weights(rng: np.random.Generator, fmt: int, N: int, K: int):
    G = GROUP[fmt]
    if K % 2:
        raise ValueError(f"K={K} must be even")
    ng = (K + G - 1) // G  # groups per row; the last one may be shorter
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    zeros = None
    if fmt in ZERO_FORMATS:
        zeros = rng.integers(0, 16, size=(N, ng), dtype=np.uint8)
        scales = bf16_bits(rng.uniform(0.005, 0.02, size=(N, ng)))
    elif fmt == INT4_SYM:
        scales = bf16_bits(rng.uniform(0.005, 0.02, size=(N, ng)))
    elif fmt == NVFP4:
        scales = e4m3_bytes(rng.uniform(2.0 ** -4, 4.0, size=(N, ng)))
    elif fmt == MXFP4:
        scales = (127 + rng.integers(-4, 5, size=(N, ng))).astype(np.uint8)
    else:
        raise ValueError(f"unknown format {fmt}")
    return packed, scales, zeros


def make_case(fmt: int, M: int, N: int, K: int, seed: int) -> Case:
    rng = np.random.default_rng(seed)
    A = make_activations(rng, M, K)
    packed, scales, zeros = make_weights(rng, fmt, N, K)
    return Case(fmt, M, N, K, A, packed, scales, zeros)


# ---- the workloads ------------------------------------------------------------

# name -> (format, M, N, K, output dtype)
CONFIGS = {
    "tiny_int4_m16": (INT4_G128, 16, 256, 512, "f32"),
    "decode_gemv_int4_m1": (INT4_G128, 1, 8192, 3072, "bf16"),
    "nvfp4_m16": (NVFP4, 16, 3072, 8192, "bf16"),
    "mxfp4_m4096": (MXFP4, 4096, 8192, 3072, "bf16"),
}

# 3B decoder: per layer q, k, v, o, gate, up, down as (out, in); then the tied
# LM head.  Applied as h @ W^T, so out = N and in = K.
DECODER_3B = dict(layers=28, d=3072, ffn=8192, n_q=24, n_kv=8, hd=128, vocab=128256)


def decoder_chain_shapes(layers: int = 28):
    c = DECODER_3B
    d, ffn, hd = c["d"], c["ffn"], c["hd"]
    per_layer = [
        ("q", c["n_q"] * hd, d),
        ("k", c["n_kv"] * hd, d),
        ("v", c["n_kv"] * hd, d),
        ("o", d, c["n_q"] * hd),
        ("gate", ffn, d),
        ("up", ffn, d),
        ("down", d, ffn),
    ]
    shapes = []
    for layer in range(layers):
        for name, n, k in per_layer:
            shapes.append((f"layer{layer}.{name}", n, k))
    shapes.append(("lm_head", c["vocab"], d))
    return shapes


def decoder_chain_groups(layers: int = 28):
    """The decode chain's matrices grouped by shared input: per layer [q, k, v]
    (the normalised layer input), [o], [gate, up] (the normalised attention
    output), [down]; then [lm_head].  Lists of indices into
    decoder_chain_shapes(layers)."""
    groups = []
    for layer in range(layers):
        b = 7 * layer
        groups += [[b, b + 1, b + 2], [b + 3], [b + 4, b + 5], [b + 6]]
    groups.append([7 * layers])
    return groups


def chain_seed(seed: int, index: int) -> int:
    """Seed of the index-th matrix of the decode chain for chain seed `seed`."""
    return 1000 * seed + index
