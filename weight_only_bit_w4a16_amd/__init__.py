"""W4A16 dequantise-GEMM for MI355X (gfx950): Python binding of libw4a16.so.

``C = A . dequant(packed, scales, zeros)^T`` with bf16 activations A (M, K),
4-bit weights packed (N, K/2) uint8 (low nibble = even k) and fp32
accumulation.  Formats: ``INT4_G128`` (bf16 scale + uint8 zero per 128 k;
``INT4_G32`` / ``INT4_G64``: the same per 32 / 64 k; ``INT4_SYM``: bf16 scale
per 128 k, zero point 8, no zero array), ``NVFP4`` (e2m1 codes, e4m3 scale per
16 k), ``MXFP4`` (e2m1 codes, e8m0 scale per 32 k).  K is a multiple of 16;
the last group of a row may be shorter than the group size.

This module only marshals arguments to the C ABI declared in
``include/w4a16.h``: it checks that tensor shapes, dtypes and devices agree
with M, N, K (so no kernel can read past a tensor), then passes raw device
pointers and the current HIP stream.  Every step of the computation runs in
the library's HIP kernels; there is no fallback.  PyTorch is used for device
memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

INT4_G128, NVFP4, MXFP4, INT4_G32, INT4_G64, INT4_SYM = 0, 1, 2, 3, 4, 5
GROUP = {INT4_G128: 128, NVFP4: 16, MXFP4: 32, INT4_G32: 32, INT4_G64: 64, INT4_SYM: 128}
FORMAT_NAMES = {INT4_G128: "int4_g128", NVFP4: "nvfp4", MXFP4: "mxfp4",
                INT4_G32: "int4_g32", INT4_G64: "int4_g64", INT4_SYM: "int4_sym"}
INT4_FORMATS = (INT4_G128, INT4_G32, INT4_G64, INT4_SYM)  # bf16 scales
ZERO_FORMATS = (INT4_G128, INT4_G32, INT4_G64)  # with a zero array (symmetric int4: zero point 8)
OUT_BF16, OUT_F32 = 0x000, 0x100
PREPACKED = 0x400  # packed weights in the prepacked layout (w4a16_prepack)
PATH_AUTO, PATH_SKINNY, PATH_TILED, PATH_MID = 0x0000, 0x1000, 0x2000, 0x3000
PATH_RAGGED = 0x4000  # reported by gemm_path for K % 32 == 16 (never a flag)
PATHS = {"auto": PATH_AUTO, "skinny": PATH_SKINNY, "mid": PATH_MID, "tiled": PATH_TILED}

OK, ERR_FORMAT, ERR_SHAPE, ERR_NULL, ERR_ALIGN, ERR_HIP, ERR_EPILOGUE, ERR_OVERLAP = 0, -1, -2, -3, -4, -5, -6, -7
MAX_GROUP = 8  # members of one w4a16_gemm_grouped call

# fused epilogue: C = act(alpha * (A . W^T) + bias[n]) + beta * residual[m, n]
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_TANH = 0, 1, 2, 3
ACTIVATIONS = {"none": ACT_NONE, "relu": ACT_RELU, "silu": ACT_SILU, "gelu_tanh": ACT_GELU_TANH}


class Epilogue(ctypes.Structure):
    """struct w4a16_epilogue of include/w4a16.h."""
    _fields_ = [("bias", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("activation", ctypes.c_int), ("reserved", ctypes.c_int)]

class BatchItem(ctypes.Structure):
    """struct w4a16_batch_item of include/w4a16.h."""
    _fields_ = [("A", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a16.so")
_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def load_library():
    """Load the built HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(or python weight_only_bit_w4a16_amd/_build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.w4a16_gemm.argtypes = [I, P, P, P, P, P, I64, I64, I64, P]
    lib.w4a16_gemm.restype = I
    lib.w4a16_gemm_ex.argtypes = [I, P, P, P, P, P, I64, I64, I64, ctypes.POINTER(Epilogue), P]
    lib.w4a16_gemm_ex.restype = I
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.w4a16_gemm_grouped.argtypes = [I, P, I, PP, PP, PP, PP, ctypes.POINTER(I64), I64, I64, P]
    lib.w4a16_gemm_grouped.restype = I
    lib.w4a16_gemm_batched.argtypes = [I, I64, I, ctypes.POINTER(BatchItem), P]
    lib.w4a16_gemm_batched.restype = I
    lib.w4a16_dequant.argtypes = [I, P, P, P, P, I64, I64, P]
    lib.w4a16_dequant.restype = I
    lib.w4a16_gemm_path.argtypes = [I, I64, I64, I64]
    lib.w4a16_prepacked_bytes.restype = I64
    lib.w4a16_prepacked_bytes.argtypes = [I64, I64]
    lib.w4a16_prepack.restype = I
    lib.w4a16_prepack.argtypes = [P, P, I64, I64, P]
    lib.w4a16_gemm_path.restype = I
    lib.w4a16_strerror.argtypes = [I]
    lib.w4a16_strerror.restype = ctypes.c_char_p
    lib.w4a16_version.argtypes = []
    lib.w4a16_version.restype = I
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().w4a16_strerror(int(status)).decode()


def version() -> int:
    return int(load_library().w4a16_version())


def gemm_path(fmt: int, M: int, N: int, K: int, path: str = "auto") -> str:
    """Name of the kernel w4a16_gemm would launch: 'skinny', 'mid', 'tiled' or
    'ragged' (K % 32 == 16, whatever the path)."""
    rc = load_library().w4a16_gemm_path(int(fmt) | PATHS[path], M, N, K)
    if rc < 0:
        raise W4A16Error(rc, "w4a16_gemm_path")
    return {PATH_SKINNY: "skinny", PATH_MID: "mid", PATH_TILED: "tiled", PATH_RAGGED: "ragged"}[rc]


# ---- argument checks (host side, before any pointer reaches the library) ----

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, shape, itemsize, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.element_size() != itemsize:
        raise ValueError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class PrepackedWeights:
    """Packed weights (N, K/2) in the library's prepacked layout (made by
    :func:`prepack`): ``data`` is the uint8 buffer of ceil(N/16)*16 rows.
    Pass it wherever ``packed`` is taken (scales and zeros are unchanged)."""

    def __init__(self, data: torch.Tensor, N: int, K: int):
        self.data, self.N, self.K = data, int(N), int(K)
        self.shape = (self.N, self.K // 2)  # the logical packed shape
        self.device = data.device
        self.is_cuda = data.is_cuda


def _weights_view(packed):
    """(tensor passed to the library, logical rows N, PREPACKED flag or 0)."""
    if isinstance(packed, PrepackedWeights):
        return packed.data, packed.N, PREPACKED
    return packed, packed.shape[0], 0


def prepack(packed: torch.Tensor, stream=None) -> PrepackedWeights:
    """The prepacked layout of row-major packed weights (N, K/2), K % 128 == 0
    (asynchronous, on ``stream``)."""
    if not isinstance(packed, torch.Tensor) or not packed.is_cuda:
        raise ValueError("packed must be a GPU tensor")
    N, K2 = packed.shape
    K = 2 * K2
    _check(packed, "packed", (N, K2), 1, packed.device)
    nbytes = load_library().w4a16_prepacked_bytes(N, K)
    if nbytes < 0:
        raise W4A16Error(int(nbytes), "w4a16_prepacked_bytes")
    rows = (N + 15) // 16 * 16
    out = torch.empty((rows, K2), dtype=torch.uint8, device=packed.device)
    rc = load_library().w4a16_prepack(_ptr(packed), _ptr(out), N, K, _stream_handle(stream))
    if rc != OK:
        raise W4A16Error(rc, "w4a16_prepack")
    return PrepackedWeights(out, N, K)


def _check_weights(fmt, packed, scales, zeros, N, K, device):
    if fmt not in GROUP:
        raise ValueError(f"unknown format {fmt}")
    G = GROUP[fmt]
    if K % 16:
        raise ValueError(f"K={K} must be a multiple of 16")
    groups = (K + G - 1) // G  # the last group may be shorter
    if isinstance(packed, PrepackedWeights):
        if packed.K != K or packed.N != N:
            raise ValueError(f"prepacked weights are {packed.N} x {packed.K}, expected {N} x {K}")
        _check(packed.data, "packed", ((N + 15) // 16 * 16, K // 2), 1, device)
    else:
        _check(packed, "packed", (N, K // 2), 1, device)
    _check(scales, "scales", (N, groups), 2 if fmt in INT4_FORMATS else 1, device)
    if fmt in ZERO_FORMATS:
        if zeros is None:
            raise ValueError("asymmetric int4 weights need zeros")
        _check(zeros, "zeros", (N, groups), 1, device)
    elif zeros is not None:
        raise ValueError(f"{FORMAT_NAMES[fmt]} weights take no zeros")


def _epilogue(bias, residual, alpha, beta, activation, out, M, N, device):
    """The epilogue struct for these arguments, or None for a plain GEMM."""
    if bias is None and residual is None and alpha == 1.0 and activation in ("none", ACT_NONE):
        return None
    act = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
    if bias is not None:
        if bias.dtype != torch.bfloat16:
            raise ValueError("bias must be bf16")
        _check(bias, "bias", (N,), 2, device)
    if residual is not None:
        if residual.dtype != out.dtype:
            raise ValueError("residual must have the output's dtype")
        _check(residual, "residual", (M, N), out.element_size(), device)
    return Epilogue(None if bias is None else bias.data_ptr(),
                    None if residual is None else residual.data_ptr(),
                    float(alpha), float(beta), act, 0)


def gemm(fmt: int, A: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
         zeros: torch.Tensor | None = None, out: torch.Tensor | None = None,
         out_dtype: torch.dtype = torch.bfloat16, path: str = "auto", stream=None,
         bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
         alpha: float = 1.0, beta: float = 1.0, activation="none") -> torch.Tensor:
    """C = A . dequant(packed, scales, zeros)^T on the GPU (asynchronous).

    With any of bias / residual / alpha / activation set, the fused epilogue
    C = act(alpha * (A . W^T) + bias[n]) + beta * residual[m, n] is applied
    in the kernel (residual may be ``out`` itself)."""
    if not A.is_cuda:
        raise ValueError("A must be a GPU tensor")
    device = A.device
    M, K = A.shape
    wt, N, pre = _weights_view(packed)
    _check(A, "A", (M, K), 2, device)
    _check_weights(fmt, packed, scales, zeros, N, K, device)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be bf16 or fp32")
    _check(out, "out", (M, N), out.element_size(), device)
    flags = (OUT_F32 if out.dtype == torch.float32 else OUT_BF16) | PATHS[path] | pre
    ep = _epilogue(bias, residual, alpha, beta, activation, out, M, N, device)
    lib = load_library()
    if ep is None:
        rc = lib.w4a16_gemm(int(fmt) | flags, _ptr(A), _ptr(wt), _ptr(scales),
                            _ptr(zeros), _ptr(out), M, N, K, _stream_handle(stream))
    else:
        rc = lib.w4a16_gemm_ex(int(fmt) | flags, _ptr(A), _ptr(wt), _ptr(scales),
                               _ptr(zeros), _ptr(out), M, N, K, ctypes.byref(ep),
                               _stream_handle(stream))
    if rc != OK:
        raise W4A16Error(rc, "w4a16_gemm")
    return out


def _grouped_args(fmt, A, weights, outs, out_dtype):
    """Check a grouped call's tensors; return (flags, outs, ctypes arrays)."""
    if not A.is_cuda:
        raise ValueError("A must be a GPU tensor")
    if not 1 <= len(weights) <= MAX_GROUP:
        raise ValueError(f"a group has 1 .. {MAX_GROUP} weight matrices, got {len(weights)}")
    device = A.device
    M, K = A.shape
    _check(A, "A", (M, K), 2, device)
    if outs is None:
        outs = [torch.empty((M, _weights_view(w[0])[1]), dtype=out_dtype, device=device) for w in weights]
    if len(outs) != len(weights):
        raise ValueError("one output per weight matrix")
    dt = outs[0].dtype
    if dt not in (torch.bfloat16, torch.float32) or any(o.dtype != dt for o in outs):
        raise ValueError("outputs must all be bf16 or all fp32")
    n = len(weights)
    arr = lambda: (ctypes.c_void_p * n)()
    P, S, Z, Cs, Ns = arr(), arr(), arr(), arr(), (ctypes.c_int64 * n)()
    pres = set()
    for i, ((packed, scales, zeros), out) in enumerate(zip(weights, outs)):
        wt, N, pre = _weights_view(packed)
        pres.add(pre)
        _check_weights(fmt, packed, scales, zeros, N, K, device)
        _check(out, f"out[{i}]", (M, N), out.element_size(), device)
        P[i], S[i], Cs[i], Ns[i] = wt.data_ptr(), scales.data_ptr(), out.data_ptr(), N
        Z[i] = zeros.data_ptr() if zeros is not None else None
    if len(pres) > 1:
        raise ValueError("a group's weights must all be prepacked or all row-major")
    flags = (OUT_F32 if dt == torch.float32 else OUT_BF16) | pres.pop()
    zarr = Z if fmt in ZERO_FORMATS else None
    return flags, outs, (P, S, zarr, Cs, Ns), (M, K)


def gemm_grouped(fmt: int, A: torch.Tensor, weights, outs=None,
                 out_dtype: torch.dtype = torch.bfloat16, path: str = "auto", stream=None):
    """C_i = A . dequant(packed_i, scales_i, zeros_i)^T for every
    (packed_i, scales_i, zeros_i) in `weights` (all with A's K), in one launch
    on the skinny path.  Returns the list of outputs (asynchronous)."""
    flags, outs, (P, S, Z, Cs, Ns), (M, K) = _grouped_args(fmt, A, weights, outs, out_dtype)
    rc = load_library().w4a16_gemm_grouped(int(fmt) | flags | PATHS[path], _ptr(A), len(weights),
                                           P, S, Z, Cs, Ns, M, K, _stream_handle(stream))
    if rc != OK:
        raise W4A16Error(rc, "w4a16_gemm_grouped")
    return outs


class PreparedGroupedGemm:
    """One w4a16_gemm_grouped call marshalled once (see :class:`PreparedGemm`)."""

    def __init__(self, fmt: int, A, weights, outs, path: str = "auto"):
        flags, outs, arrays, (M, K) = _grouped_args(fmt, A, weights, outs, torch.bfloat16)
        self.tensors = (A, list(weights), outs)
        self.kernel = gemm_path(fmt | (flags & PREPACKED), M, int(arrays[4][0]), K, path)
        self._fn = load_library().w4a16_gemm_grouped
        self._args = (int(fmt) | flags | PATHS[path], _ptr(A), len(weights), *arrays, M, K)

    def __call__(self, stream=None):
        rc = self._fn(*self._args, _stream_handle(stream))
        if rc != OK:
            raise W4A16Error(rc, "w4a16_gemm_grouped")


def _batched_args(fmt, items, outs, out_dtype):
    """Check a batched call's tensors; return (flags, outs, item array, M)."""
    items = list(items)
    if not items:
        return (OUT_F32 if out_dtype == torch.float32 else OUT_BF16), [], (BatchItem * 1)(), 0
    if outs is None:
        outs = [torch.empty((A.shape[0], _weights_view(packed)[1]), dtype=out_dtype, device=A.device)
                for A, packed, _, _ in items]
    if len(outs) != len(items):
        raise ValueError("one output per item")
    dt = outs[0].dtype
    if dt not in (torch.bfloat16, torch.float32) or any(o.dtype != dt for o in outs):
        raise ValueError("outputs must all be bf16 or all fp32")
    M = items[0][0].shape[0]
    arr = (BatchItem * len(items))()
    pres = set()
    for i, ((A, packed, scales, zeros), out) in enumerate(zip(items, outs)):
        if not A.is_cuda:
            raise ValueError(f"A[{i}] must be a GPU tensor")
        device = A.device
        if A.dim() != 2 or A.shape[0] != M:
            raise ValueError(f"A[{i}] must have the batch's M = {M} rows")
        K = A.shape[1]
        wt, N, pre = _weights_view(packed)
        pres.add(pre)
        _check(A, f"A[{i}]", (M, K), 2, device)
        _check_weights(fmt, packed, scales, zeros, N, K, device)
        _check(out, f"out[{i}]", (M, N), out.element_size(), device)
        arr[i] = BatchItem(A.data_ptr(), wt.data_ptr(), scales.data_ptr(),
                           None if zeros is None else zeros.data_ptr(), out.data_ptr(), N, K)
    if len(pres) > 1:
        raise ValueError("a batch's weights must all be prepacked or all row-major")
    flags = (OUT_F32 if dt == torch.float32 else OUT_BF16) | pres.pop()
    return flags, outs, arr, M


def gemm_batched(fmt: int, items, outs=None, out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """C_i = A_i . dequant(packed_i, scales_i, zeros_i)^T for every item
    (A_i, packed_i, scales_i, zeros_i) -- independent GEMMs with their own
    activations (all with M rows) and outputs; for M <= 16 the items of one
    (K, N) share a launch.  Returns the list of outputs (asynchronous)."""
    flags, outs, arr, M = _batched_args(fmt, items, outs, out_dtype)
    rc = load_library().w4a16_gemm_batched(int(fmt) | flags, M, len(outs), arr, _stream_handle(stream))
    if rc != OK:
        raise W4A16Error(rc, "w4a16_gemm_batched")
    return outs


class PreparedBatchedGemm:
    """One w4a16_gemm_batched call marshalled once (see :class:`PreparedGemm`)."""

    def __init__(self, fmt: int, items, outs):
        items = list(items)
        flags, outs, arr, M = _batched_args(fmt, items, outs, torch.bfloat16)
        self.tensors = (items, outs)
        self.kernel = gemm_path(fmt | (flags & PREPACKED), M, int(arr[0].N), int(arr[0].K)) if items else None
        self._fn = load_library().w4a16_gemm_batched
        self._args = (int(fmt) | flags, M, len(outs), arr)

    def __call__(self, stream=None):
        rc = self._fn(*self._args, _stream_handle(stream))
        if rc != OK:
            raise W4A16Error(rc, "w4a16_gemm_batched")


def dequant(fmt: int, packed: torch.Tensor, scales: torch.Tensor,
            zeros: torch.Tensor | None = None, out: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """W = dequant(packed, scales, zeros) as bf16 (N, K), bit-exact."""
    if not packed.is_cuda:
        raise ValueError("packed must be a GPU tensor")
    device = packed.device
    wt, N, pre = _weights_view(packed)
    K = 2 * packed.shape[1]
    _check_weights(fmt, packed, scales, zeros, N, K, device)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=device)
    _check(out, "out", (N, K), 2, device)
    rc = load_library().w4a16_dequant(int(fmt) | pre, _ptr(wt), _ptr(scales), _ptr(zeros),
                                      _ptr(out), N, K, _stream_handle(stream))
    if rc != OK:
        raise W4A16Error(rc, "w4a16_dequant")
    return out


class PreparedGemm:
    """One w4a16_gemm call whose tensors were checked and marshalled once.

    Calling it re-issues the C call with the same device pointers on the
    given (default: current) stream -- for timing loops and graph capture,
    where the per-call Python checks of :func:`gemm` would dominate.
    The tensors are kept referenced for the object's lifetime.
    """

    def __init__(self, fmt: int, A, packed, scales, zeros, out, path: str = "auto",
                 bias=None, residual=None, alpha: float = 1.0, beta: float = 1.0,
                 activation="none"):
        device = A.device
        M, K = A.shape
        wt, N, pre = _weights_view(packed)
        _check(A, "A", (M, K), 2, device)
        _check_weights(fmt, packed, scales, zeros, N, K, device)
        _check(out, "out", (M, N), out.element_size(), device)
        if out.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("out must be bf16 or fp32")
        self.tensors = (A, packed, scales, zeros, out, bias, residual)
        flags = (OUT_F32 if out.dtype == torch.float32 else OUT_BF16) | PATHS[path] | pre
        self.kernel = gemm_path(fmt | pre, M, N, K, path)
        self._ep = _epilogue(bias, residual, alpha, beta, activation, out, M, N, device)
        lib = load_library()
        self._args = (int(fmt) | flags, _ptr(A), _ptr(wt), _ptr(scales), _ptr(zeros),
                      _ptr(out), M, N, K)
        if self._ep is None:
            self._fn = lib.w4a16_gemm
        else:
            self._fn = lib.w4a16_gemm_ex
            self._args = self._args + (ctypes.byref(self._ep),)

    def __call__(self, stream=None):
        rc = self._fn(*self._args, _stream_handle(stream))
        if rc != OK:
            raise W4A16Error(rc, "w4a16_gemm")
