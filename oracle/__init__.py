"""Plain CPU oracle for the W4A16 dequantise-GEMM ``C = A . dequant(B)^T``.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path
(``weight_only_bit_w4a16_amd``) never does, and the two share no code.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, IEEE binary64, one
element at a time); this module only compiles it with gcc and marshals numpy
arrays to it.  Sources, per function, are cited in the C file:

* "megakernel_int4_weight_decode.py" task spec -- "The weight format", the
  nibble-order paragraph and "Precision": int4 asymmetric, group 128,
  value = (code - zero) * scale, low nibble = even input index.
* "Matmul2dFp4" (Mojo) -- NVFP4 operand layout and decode_e2m1 * |scale|.
* "example_dequant_gemm_bf16_fp4_hopper.py" -- fp4 sign/exponent/mantissa
  split and ``C = A @ B^T`` with B packed (N, K/2).

Formats: ``INT4_G128 = 0``, ``NVFP4 = 1``, ``MXFP4 = 2``, and the same int4 with
groups of 32 / 64 inputs, ``INT4_G32 = 3``, ``INT4_G64 = 4`` (the group is a
configuration value of the int4 page, 128 in its fixture), and symmetric int4
``INT4_SYM = 5`` (groups of 128, no zero array, zero point 8).  Scales are
passed as their raw storage: uint16 bf16 bits (int4) or uint8 bytes (e4m3 /
e8m0).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

INT4_G128, NVFP4, MXFP4, INT4_G32, INT4_G64, INT4_SYM = 0, 1, 2, 3, 4, 5
GROUP = {INT4_G128: 128, NVFP4: 16, MXFP4: 32, INT4_G32: 32, INT4_G64: 64, INT4_SYM: 128}
INT4_FORMATS = (INT4_G128, INT4_G32, INT4_G64, INT4_SYM)  # bf16 scales
ZERO_FORMATS = (INT4_G128, INT4_G32, INT4_G64)  # with a zero array

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libw4a16_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint]
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0_value.restype = ctypes.c_double
    lib.orc_round_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_bf16.restype = ctypes.c_uint16
    lib.orc_dequant.argtypes = [I, P, P, P, I64, I64, P, P]
    lib.orc_dequant.restype = I
    lib.orc_gemm.argtypes = [I, P, P, P, P, I64, I64, I64, I, P, P]
    lib.orc_gemm.restype = I
    lib.orc_gemm_at.argtypes = [I, P, P, P, P, I64, I64, I64, I64, P, P, P, P]
    lib.orc_gemm_at.restype = I
    lib.orc_activation.argtypes = [I, ctypes.c_double]
    lib.orc_activation.restype = ctypes.c_double
    lib.orc_epilogue.argtypes = [I64, I64, P, ctypes.c_double, P, I, ctypes.c_double, P]
    lib.orc_epilogue.restype = I
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = I
    lib.orc_set_num_threads.argtypes = [I]
    lib.orc_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _scales(fmt, scales):
    return _c(scales, np.uint16 if fmt in INT4_FORMATS else np.uint8)


# ---- element decoders ------------------------------------------------------

def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(int(bits))


def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().orc_e4m3_value(int(byte))


def e8m0_value(byte: int) -> float:
    return _load().orc_e8m0_value(int(byte))


def round_bf16(x: float) -> int:
    return int(_load().orc_round_bf16(float(x)))


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """Vector form of bf16_value (element by element through the C code)."""
    f = _load().orc_bf16_value
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


_BF16_TABLE = None


def _bf16_table() -> np.ndarray:
    """bf16_value of all 65536 bit patterns (the C decoder, called once per
    pattern), for decoding large arrays by lookup."""
    global _BF16_TABLE
    if _BF16_TABLE is None:
        _BF16_TABLE = bf16_values(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    return _BF16_TABLE


# ---- dequant / GEMM ---------------------------------------------------------

def _check_sizes(fmt, N, K, packed, scales, zeros, A=None, M=0):
    """The C code trusts its arguments: refuse arrays too small for (M, N, K)
    before any of it runs (groups per row = ceil(K / G), the last one may be
    shorter)."""
    if fmt not in GROUP or K <= 0 or K % 2 or N < 0 or M < 0:
        raise ValueError("oracle: bad format or shape")
    ng = (K + GROUP[fmt] - 1) // GROUP[fmt]
    if packed is None or packed.size < N * (K // 2):
        raise ValueError("oracle: packed smaller than (N, K/2)")
    if scales is None or scales.size < N * ng:
        raise ValueError("oracle: scales smaller than (N, ceil(K/G))")
    if fmt in ZERO_FORMATS and (zeros is None or zeros.size < N * ng):
        raise ValueError("oracle: zeros smaller than (N, ceil(K/G))")
    if A is not None and A.size < M * K:
        raise ValueError("oracle: A smaller than (M, K)")


def dequant(fmt: int, packed, scales, zeros, N: int, K: int):
    """Return (w_exact float64 (N, K), w_bf16 uint16 (N, K))."""
    packed = _c(packed, np.uint8)
    scales = _scales(fmt, scales)
    zeros = _c(zeros, np.uint8)
    _check_sizes(fmt, N, K, packed, scales, zeros)
    w = np.empty((N, K), np.float64)
    wb = np.empty((N, K), np.uint16)
    rc = _load().orc_dequant(fmt, _ptr(packed), _ptr(scales), _ptr(zeros), N, K,
                             _ptr(w), _ptr(wb))
    if rc != 0:
        raise ValueError("oracle dequant: bad format or shape")
    return w, wb


def gemm(fmt: int, A_bits, packed, scales, zeros, M: int, N: int, K: int,
         weights_bf16: bool = False):
    """Return (C float64 (M, N), S float64 (M, N)); A_bits is bf16 as uint16."""
    A_bits = _c(A_bits, np.uint16)
    packed = _c(packed, np.uint8)
    scales = _scales(fmt, scales)
    zeros = _c(zeros, np.uint8)
    _check_sizes(fmt, N, K, packed, scales, zeros, A_bits, M)
    C = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    rc = _load().orc_gemm(fmt, _ptr(A_bits), _ptr(packed), _ptr(scales), _ptr(zeros),
                          M, N, K, int(bool(weights_bf16)), _ptr(C), _ptr(S))
    if rc != 0:
        raise ValueError("oracle gemm: bad format or shape")
    return C, S


def gemm_matmul(fmt: int, A_bits, packed, scales, zeros, M: int, N: int, K: int):
    """The (C, S) of :func:`gemm` for shapes too large for its element-by-element
    loop: the oracle's exact dequantisation, then binary64 matrix products
    (numpy's, a library primitive) C = A . W^T and S = |A| . |W|^T.  The sums
    run in another order than gemm()'s k-ascending loop, so the two differ by
    binary64 rounding only (at most about K * 2^-53 * S).  Finite weights only:
    a BLAS product is not required to propagate NaN."""
    A_bits = _c(A_bits, np.uint16)
    _check_sizes(fmt, N, K, _c(packed, np.uint8), _scales(fmt, scales), _c(zeros, np.uint8), A_bits, M)
    w, _ = dequant(fmt, packed, scales, zeros, N, K)
    if not np.all(np.isfinite(w)):
        raise ValueError("oracle gemm_matmul: weights must be finite")
    a = _bf16_table()[A_bits].reshape(M, K)
    C = a @ w.T
    S = np.abs(a) @ np.abs(w).T
    return C, S


def gemm_at(fmt: int, A_bits, packed, scales, zeros, M: int, N: int, K: int,
            m_idx, n_idx):
    """Sampled reference: (C[i], S[i]) for each (m_idx[i], n_idx[i])."""
    A_bits = _c(A_bits, np.uint16)
    packed = _c(packed, np.uint8)
    scales = _scales(fmt, scales)
    zeros = _c(zeros, np.uint8)
    _check_sizes(fmt, N, K, packed, scales, zeros, A_bits, M)
    mi = _c(m_idx, np.int64)
    ni = _c(n_idx, np.int64)
    C = np.empty(len(mi), np.float64)
    S = np.empty(len(mi), np.float64)
    rc = _load().orc_gemm_at(fmt, _ptr(A_bits), _ptr(packed), _ptr(scales), _ptr(zeros),
                             M, N, K, len(mi), _ptr(mi), _ptr(ni), _ptr(C), _ptr(S))
    if rc != 0:
        raise ValueError("oracle gemm_at: bad format, shape or index")
    return C, S


# ---- fused epilogue ----------------------------------------------------------

ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH = 0, 1, 2, 3
# Lipschitz constants of the activations (max |act'|): SiLU's derivative peaks
# at 1.0998 near x = 2.40, the tanh-form GELU's at 1.1289 near x = 1.50
ACT_LIPSCHITZ = {ACT_NONE: 1.0, ACT_RELU: 1.0, ACT_SILU: 1.1, ACT_GELU_TANH: 1.13}


def activation(act: int, x: float) -> float:
    return float(_load().orc_activation(act, float(x)))


def epilogue(C, alpha: float = 1.0, bias=None, act: int = ACT_NONE, beta: float = 0.0, R=None):
    """y = act(alpha*C + bias[n]) + beta*R, in fp64 (C, R: float arrays (M, N);
    bias: bf16 bits (N)).  Returns a new array."""
    y = np.array(C, dtype=np.float64, order="C", copy=True)
    M, N = y.shape
    b = None if bias is None else _c(bias, np.uint16)
    r = None if R is None else _c(np.asarray(R, dtype=np.float64), np.float64)
    if b is not None and b.shape != (N,):
        raise ValueError("oracle epilogue: bias must have N elements")
    if r is not None and r.shape != (M, N):
        raise ValueError("oracle epilogue: R must be (M, N)")
    rc = _load().orc_epilogue(M, N, _ptr(y), float(alpha), _ptr(b), int(act), float(beta), _ptr(r))
    if rc != 0:
        raise ValueError("oracle epilogue: bad activation")
    return y


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (timing only: results do not depend on it)."""
    _load().orc_set_num_threads(int(n))


# ---- the correctness gate ---------------------------------------------------

GATE_REL = 2e-3
GATE_ABS = 1e-6
BF16_OUT_REL = 2.0 ** -8


def gate_bound(C_ref, S, bf16_out: bool):
    """Per-element allowed |C_gpu - C_ref|: 2e-3*S + 1e-6, plus 2^-8*|C_ref|
    when the output is stored as bf16 (one bf16 unit roundoff)."""
    b = GATE_REL * np.asarray(S) + GATE_ABS
    if bf16_out:
        b = b + BF16_OUT_REL * np.abs(np.asarray(C_ref))
    return b


def epilogue_gate_bound(C_ref, S, alpha: float, bias, act: int, beta: float, R, Y_ref,
                        bf16_out: bool):
    """Per-element allowed |Y_gpu - Y_ref| for y = act(alpha*c + bias) + beta*R:
    the GEMM bound carried through alpha and the activation's Lipschitz
    constant, fp32 rounding of the epilogue's operations (2^-20 of the
    magnitudes involved), and one bf16 rounding of y when stored as bf16."""
    C_ref = np.asarray(C_ref, dtype=np.float64)
    pre = abs(alpha) * np.abs(C_ref)
    if bias is not None:
        pre = pre + np.abs(bf16_values(np.asarray(bias, dtype=np.uint16)))[None, :]
    post = np.abs(np.asarray(Y_ref, dtype=np.float64))
    if R is not None and beta != 0.0:
        post = post + abs(beta) * np.abs(np.asarray(R, dtype=np.float64))
    b = (ACT_LIPSCHITZ[act] * abs(alpha) * (GATE_REL * np.asarray(S) + GATE_ABS)
         + 2.0 ** -20 * (pre + post) + GATE_ABS)
    if bf16_out:
        b = b + BF16_OUT_REL * np.abs(np.asarray(Y_ref))
    return b


def epilogue_gate_ratio(Y_test, C_ref, S, alpha, bias, act, beta, R, Y_ref, bf16_out: bool):
    """max |Y_test - Y_ref| / epilogue bound (<= 1 passes); NaN fails."""
    err = np.abs(np.asarray(Y_test, dtype=np.float64) - np.asarray(Y_ref))
    r = err / epilogue_gate_bound(C_ref, S, alpha, bias, act, beta, R, Y_ref, bf16_out)
    if not np.all(np.isfinite(r)):
        return float("inf")
    return float(r.max()) if r.size else 0.0


def gate_ratio(C_test, C_ref, S, bf16_out: bool):
    """max |C_test - C_ref| / bound (<= 1 passes); NaN anywhere fails (inf)."""
    C_test = np.asarray(C_test, dtype=np.float64)
    err = np.abs(C_test - np.asarray(C_ref))
    r = err / gate_bound(C_ref, S, bf16_out)
    if not np.all(np.isfinite(r)):
        return float("inf")
    return float(r.max()) if r.size else 0.0
