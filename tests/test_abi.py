"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before touching the HIP
runtime.  No call here reaches a kernel launch (no GPU is needed)."""
import ctypes
import os
import re

import pytest

import weight_only_bit_w4a16_amd as w4
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "w4a16.h")


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(w4a16_\w+)\s*\(", text, re.M)))


def _header_defines():
    text = open(HEADER).read()
    out = {}
    for name, val in re.findall(r"#define\s+(W4A16_\w+)\s+\(?(-?0x[0-9A-Fa-f]+|-?\d+)\)?", text):
        out[name] = int(val, 0)
    return out


def test_library_exports_every_declared_function():
    lib = w4.load_library()
    names = _header_functions()
    assert set(names) == {"w4a16_gemm", "w4a16_gemm_ex", "w4a16_gemm_grouped", "w4a16_gemm_batched",
                          "w4a16_dequant", "w4a16_gemm_path", "w4a16_strerror", "w4a16_version",
                          "w4a16_prepack", "w4a16_prepacked_bytes"}
    for name in names:
        assert hasattr(lib, name), name


def test_python_constants_match_header():
    d = _header_defines()
    assert d["W4A16_INT4_G128"] == w4.INT4_G128
    assert d["W4A16_NVFP4"] == w4.NVFP4
    assert d["W4A16_MXFP4"] == w4.MXFP4
    assert d["W4A16_INT4_G32"] == w4.INT4_G32 and d["W4A16_INT4_G64"] == w4.INT4_G64
    assert d["W4A16_INT4_SYM"] == w4.INT4_SYM
    assert d["W4A16_OUT_F32"] == w4.OUT_F32
    assert d["W4A16_PREPACKED"] == w4.PREPACKED
    assert d["W4A16_PATH_SKINNY"] == w4.PATH_SKINNY
    assert d["W4A16_PATH_TILED"] == w4.PATH_TILED
    assert d["W4A16_PATH_MID"] == w4.PATH_MID
    for code in ("OK", "ERR_FORMAT", "ERR_SHAPE", "ERR_NULL", "ERR_ALIGN", "ERR_HIP", "ERR_EPILOGUE",
                 "ERR_OVERLAP"):
        assert d["W4A16_" + code] == getattr(w4, code)
    assert d["W4A16_MAX_GROUP"] == w4.MAX_GROUP
    for name in ("NONE", "RELU", "SILU", "GELU_TANH"):
        assert d["W4A16_ACT_" + name] == getattr(w4, "ACT_" + name)


def test_epilogue_struct_layout():
    # struct w4a16_epilogue: two pointers, two floats, two ints
    assert ctypes.sizeof(w4.Epilogue) == 32
    assert w4.Epilogue.alpha.offset == 16 and w4.Epilogue.activation.offset == 24


def test_version_and_strerror():
    assert w4.version() == 106
    for code in (w4.OK, w4.ERR_FORMAT, w4.ERR_SHAPE, w4.ERR_NULL, w4.ERR_ALIGN, w4.ERR_HIP,
                 w4.ERR_EPILOGUE, w4.ERR_OVERLAP):
        assert w4.strerror(code) != "unknown status"
    assert w4.strerror(12345) == "unknown status"


def test_path_choice():
    assert w4.gemm_path(w4.INT4_G128, 1, 8192, 3072) == "skinny"
    assert w4.gemm_path(w4.NVFP4, 16, 3072, 8192) == "skinny"
    # a small tiled grid: the mid kernel (workgroups of 32 columns x 64 rows)
    # while it has 160 .. 896 workgroups (3.5 rounds of 256),
    # the skinny kernel below 160 workgroups, else the tiled kernel
    assert w4.gemm_path(w4.MXFP4, 17, 64, 64) == "skinny"
    assert w4.gemm_path(w4.INT4_G128, 64, 1024, 3072) == "skinny"
    assert w4.gemm_path(w4.NVFP4, 64, 3072, 8192) == "skinny"        # 96 workgroups
    assert w4.gemm_path(w4.NVFP4, 65, 3072, 8192) == "mid"           # 192
    assert w4.gemm_path(w4.INT4_G128, 17, 5120, 3072) == "mid"       # 160
    assert w4.gemm_path(w4.MXFP4, 192, 8192, 3072) == "mid"          # 768 workgroups
    assert w4.gemm_path(w4.MXFP4, 193, 8192, 3072) == "tiled"        # 1024
    assert w4.gemm_path(w4.MXFP4, 96, 14336, 4096) == "mid"          # 896
    assert w4.gemm_path(w4.INT4_G128, 64, 28672, 4096) == "mid"      # 896 (112 large tiles)
    assert w4.gemm_path(w4.INT4_G128, 65, 28672, 4096) == "tiled"    # 1792
    assert w4.gemm_path(w4.INT4_G128, 192, 8192, 3072) == "mid"
    assert w4.gemm_path(w4.INT4_G128, 193, 8192, 3072) == "tiled"
    assert w4.gemm_path(w4.INT4_SYM, 192, 8192, 3072) == "mid"
    assert w4.gemm_path(w4.INT4_SYM, 193, 8192, 3072) == "tiled"
    assert w4.gemm_path(w4.INT4_G128, 384, 1024, 3072) == "mid"      # 192 workgroups
    assert w4.gemm_path(w4.INT4_G128, 400, 512, 3072) == "tiled"
    # a large tiled grid (>= 256 tiles): the mid kernel up to 48 rows
    assert w4.gemm_path(w4.INT4_G128, 64, 65536, 3072) == "mid"
    assert w4.gemm_path(w4.INT4_G128, 65, 65536, 3072) == "tiled"
    assert w4.gemm_path(w4.MXFP4, 4096, 8192, 3072) == "tiled"
    assert w4.gemm_path(w4.MXFP4, 4096, 8192, 3072, "skinny") == "skinny"
    assert w4.gemm_path(w4.INT4_G128, 1, 64, 128, "tiled") == "tiled"
    assert w4.gemm_path(w4.NVFP4, 1, 64, 128, "mid") == "mid"
    assert w4.gemm_path(w4.NVFP4, 4096, 64, 128, "mid") == "mid"
    # K an odd multiple of 16: the ragged-K kernel, whatever the path flag
    assert w4.gemm_path(w4.NVFP4, 1, 64, 48) == "ragged"
    assert w4.gemm_path(w4.INT4_G128, 4096, 8192, 3088, "tiled") == "ragged"
    assert w4.gemm_path(w4.MXFP4, 16, 64, 80, "skinny") == "ragged"


# fake, aligned device addresses: every call below fails validation (or is a
# zero-extent no-op) before any pointer could be used
PA, PB, PS, PZ, PC = (ctypes.c_void_p(0x100000 * i) for i in range(1, 6))


def _gemm(fmt, A=PA, B=PB, S=PS, Z=PZ, C=PC, M=16, N=64, K=128):
    return w4.load_library().w4a16_gemm(fmt, A, B, S, Z, C, M, N, K, None)


@pytest.mark.parametrize("fmt,M,N,K,expect", [
    (6, 16, 64, 128, w4.ERR_FORMAT),                          # unknown format
    (w4.INT4_SYM, 16, 64, 100, w4.ERR_SHAPE),                 # K % 16
    (w4.INT4_G64, 16, 64, 88, w4.ERR_SHAPE),                  # K % 16
    (w4.INT4_G32, 16, 64, 40, w4.ERR_SHAPE),                  # K % 16
    (w4.INT4_G128 | 0x4000, 16, 64, 128, w4.ERR_FORMAT),      # unknown flag
    (w4.INT4_G128 | 0x8000, 16, 64, 128, w4.ERR_FORMAT),      # unknown flag
    (w4.INT4_G128, -1, 64, 128, w4.ERR_SHAPE),
    (w4.INT4_G128, 16, -5, 128, w4.ERR_SHAPE),
    (w4.INT4_G128, 16, 64, 0, w4.ERR_SHAPE),
    (w4.INT4_G128, 16, 64, 104, w4.ERR_SHAPE),                # K % 16
    (w4.NVFP4, 16, 64, 24, w4.ERR_SHAPE),                     # K % 16 (a whole NVFP4 block)
    (w4.MXFP4, 16, 64, 2 ** 22 + 32, w4.ERR_SHAPE),
    (w4.MXFP4, 2 ** 31, 64, 64, w4.ERR_SHAPE),
])
def test_gemm_rejects_format_and_shape(fmt, M, N, K, expect):
    Z = PZ if (fmt & 0xFF) in w4.ZERO_FORMATS else None
    assert _gemm(fmt, Z=Z, M=M, N=N, K=K) == expect


def test_gemm_rejects_null_and_alignment():
    assert _gemm(w4.INT4_G128, A=None) == w4.ERR_NULL
    assert _gemm(w4.INT4_G128, B=None) == w4.ERR_NULL
    assert _gemm(w4.INT4_G128, S=None) == w4.ERR_NULL
    assert _gemm(w4.INT4_G128, C=None) == w4.ERR_NULL
    assert _gemm(w4.INT4_G128, Z=None) == w4.ERR_NULL           # int4 needs zeros
    assert _gemm(w4.INT4_G32, Z=None) == w4.ERR_NULL
    assert _gemm(w4.INT4_G64, Z=None) == w4.ERR_NULL
    assert _gemm(w4.INT4_G64, S=ctypes.c_void_p(0x100001)) == w4.ERR_ALIGN
    assert _gemm(w4.NVFP4, Z=PZ) == w4.ERR_NULL                  # fp4 takes none
    assert _gemm(w4.INT4_SYM, Z=PZ) == w4.ERR_NULL               # symmetric int4 takes none
    assert _gemm(w4.INT4_SYM, Z=None, S=ctypes.c_void_p(0x100001)) == w4.ERR_ALIGN
    odd = ctypes.c_void_p(0x100008)
    assert _gemm(w4.INT4_G128, A=odd) == w4.ERR_ALIGN
    assert _gemm(w4.INT4_G128, B=odd) == w4.ERR_ALIGN
    assert _gemm(w4.INT4_G128, S=ctypes.c_void_p(0x100001)) == w4.ERR_ALIGN
    assert _gemm(w4.NVFP4, Z=None, S=ctypes.c_void_p(0x100001)) == w4.ERR_ALIGN
    assert _gemm(w4.INT4_G128 | w4.OUT_F32, C=ctypes.c_void_p(0x100002)) == w4.ERR_ALIGN
    # zero extents are no-ops that look at no pointer
    assert _gemm(w4.MXFP4, Z=None, S=ctypes.c_void_p(0x100001), M=0) == w4.OK
    assert _gemm(w4.INT4_G128, A=None, C=None, N=0) == w4.OK


def test_zero_extent_is_a_noop():
    assert _gemm(w4.INT4_G128, M=0) == w4.OK
    assert _gemm(w4.INT4_G128, N=0) == w4.OK
    lib = w4.load_library()
    assert lib.w4a16_dequant(w4.MXFP4, PB, PS, None, PC, 0, 64, None) == w4.OK


def _gemm_ex(ep, fmt=w4.INT4_G128, C=PC, M=16, N=64, K=128):
    return w4.load_library().w4a16_gemm_ex(fmt, PA, PB, PS, PZ, C, M, N, K,
                                           None if ep is None else ctypes.byref(ep), None)


@pytest.mark.parametrize("fields,fmt,expect", [
    (dict(activation=4), w4.INT4_G128, w4.ERR_EPILOGUE),           # unknown activation
    (dict(activation=-1), w4.INT4_G128, w4.ERR_EPILOGUE),
    (dict(reserved=1), w4.INT4_G128, w4.ERR_EPILOGUE),             # reserved must be 0
    (dict(bias=0x100001), w4.INT4_G128, w4.ERR_ALIGN),             # bf16 bias, odd address
    (dict(residual=0x200001, beta=1.0), w4.INT4_G128, w4.ERR_ALIGN),
    (dict(residual=0x200002, beta=1.0), w4.INT4_G128 | w4.OUT_F32, w4.ERR_ALIGN),  # fp32: 4 B
    # residual overlapping C (C at 0x500000, 16 x 64 bf16 = 2 KB) without being C
    (dict(residual=0x500000 + 64, beta=1.0), w4.INT4_G128, w4.ERR_EPILOGUE),
    (dict(residual=0x500000 - 64, beta=1.0), w4.INT4_G128, w4.ERR_EPILOGUE),
])
def test_gemm_ex_rejects_bad_epilogue(fields, fmt, expect):
    ep = w4.Epilogue(None, None, 1.0, 0.0, 0, 0)
    for k, v in fields.items():
        setattr(ep, k, v)
    assert _gemm_ex(ep, fmt) == expect


def test_gemm_ex_validation_order_and_noops():
    # shape errors come first; a bad activation is caught even at zero extent;
    # with beta = 0 the residual is not read, so its address is not checked
    bad = w4.Epilogue(None, None, 1.0, 0.0, 9, 0)
    assert _gemm_ex(bad, fmt=7) == w4.ERR_FORMAT
    assert _gemm_ex(bad, M=0) == w4.ERR_EPILOGUE
    ok = w4.Epilogue(None, 0x500000 + 64, 1.0, 0.0, w4.ACT_SILU, 0)
    assert _gemm_ex(ok, M=0) == w4.OK
    assert _gemm_ex(None, M=0, N=0) == w4.OK
    # a residual that is C itself (in place) and disjoint ones pass validation
    # (the zero-extent calls never launch)
    assert _gemm_ex(w4.Epilogue(None, 0x500000, 1.0, 1.0, 0, 0), M=0) == w4.OK


def test_dequant_rejects_bad_arguments():
    lib = w4.load_library()
    assert lib.w4a16_dequant(w4.INT4_G128 | w4.OUT_F32, PB, PS, PZ, PC, 4, 128, None) == w4.ERR_FORMAT
    assert lib.w4a16_dequant(w4.INT4_G128, PB, PS, PZ, PC, 4, 40, None) == w4.ERR_SHAPE
    assert lib.w4a16_dequant(w4.INT4_G128, PB, PS, None, PC, 4, 128, None) == w4.ERR_NULL
    assert lib.w4a16_dequant(w4.MXFP4, PB, PS, PZ, PC, 4, 64, None) == w4.ERR_NULL
    assert lib.w4a16_dequant(w4.INT4_SYM, PB, PS, PZ, PC, 4, 128, None) == w4.ERR_NULL
    assert lib.w4a16_dequant(w4.INT4_SYM, PB, PS, None, PC, 4, 88, None) == w4.ERR_SHAPE
    assert lib.w4a16_dequant(6, PB, PS, None, PC, 4, 128, None) == w4.ERR_FORMAT
    assert lib.w4a16_dequant(w4.MXFP4, PB, PS, None, ctypes.c_void_p(0x100008), 4, 64,
                             None) == w4.ERR_ALIGN


def test_binding_shape_checks_before_library(monkeypatch):
    """The binding refuses inconsistent tensors (CPU tensors here: it must
    never reach the library)."""
    import torch
    A = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w4.gemm(w4.INT4_G128, A, torch.zeros(8, 64, dtype=torch.uint8),
                torch.zeros(8, 1, dtype=torch.bfloat16), torch.zeros(8, 1, dtype=torch.uint8))


# ---- w4a16_gemm_grouped validation (no call below reaches a launch) ---------

def _grouped(fmt, count=3, N=(64, 32, 48), M=1, K=128, A=PA, packed=True, scales=True,
             zeros="auto", C=True, Nnull=False, bad=None):
    n = max(count, 1)
    mk = lambda base: (ctypes.c_void_p * n)(*[0x100000 * (base + 8 * i) for i in range(n)])
    P, S, Cs = mk(2), mk(3), mk(5)
    Z = mk(4) if (zeros == "auto" and (fmt & 0xFF) in w4.ZERO_FORMATS) or zeros is True else None
    if bad:
        arr, i, val = bad
        {"P": P, "S": S, "C": Cs, "Z": Z}[arr][i] = val
    Ns = None if Nnull else (ctypes.c_int64 * n)(*(list(N) + [64] * n)[:n])
    return w4.load_library().w4a16_gemm_grouped(
        fmt, A, count, P if packed else None, S if scales else None, Z, Cs if C else None,
        Ns, M, 0 if K is None else K, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(fmt=6), w4.ERR_FORMAT),
    (dict(fmt=w4.INT4_SYM, zeros=True), w4.ERR_NULL),          # symmetric int4 takes no zeros
    (dict(fmt=w4.INT4_SYM, K=200), w4.ERR_SHAPE),              # K % 16
    (dict(fmt=w4.INT4_G128, count=0), w4.ERR_SHAPE),
    (dict(fmt=w4.INT4_G64, K=88), w4.ERR_SHAPE),               # K % 16
    (dict(fmt=w4.INT4_G32, zeros=False), w4.ERR_NULL),
    (dict(fmt=w4.INT4_G128, count=9), w4.ERR_SHAPE),
    (dict(fmt=w4.INT4_G128, K=104), w4.ERR_SHAPE),             # K % 16
    (dict(fmt=w4.NVFP4, K=40), w4.ERR_SHAPE),                  # K % 16
    (dict(fmt=w4.NVFP4, N=(64, -1, 32)), w4.ERR_SHAPE),
    (dict(fmt=w4.NVFP4, Nnull=True), w4.ERR_NULL),
    (dict(fmt=w4.NVFP4, A=None), w4.ERR_NULL),
    (dict(fmt=w4.NVFP4, packed=False), w4.ERR_NULL),
    (dict(fmt=w4.NVFP4, C=False), w4.ERR_NULL),
    (dict(fmt=w4.NVFP4, zeros=True), w4.ERR_NULL),             # fp4 takes no zeros
    (dict(fmt=w4.INT4_G128, zeros=False), w4.ERR_NULL),        # int4 needs zeros
    (dict(fmt=w4.INT4_G128, bad=("Z", 1, None)), w4.ERR_NULL),
    (dict(fmt=w4.MXFP4, bad=("S", 2, None)), w4.ERR_NULL),
    (dict(fmt=w4.MXFP4, bad=("P", 1, 0x100008)), w4.ERR_ALIGN),
    (dict(fmt=w4.NVFP4, bad=("S", 0, 0x100001)), w4.ERR_ALIGN),
    (dict(fmt=w4.NVFP4 | w4.OUT_F32, bad=("C", 2, 0x100002)), w4.ERR_ALIGN),
    (dict(fmt=w4.NVFP4, A=ctypes.c_void_p(0x100008)), w4.ERR_ALIGN),
])
def test_grouped_validation(kw, expect):
    assert _grouped(**kw) == expect


def test_grouped_zero_extents_check_no_pointer():
    # M = 0, or every member with N = 0: a valid no-op, NULL pointers allowed
    assert _grouped(w4.INT4_G128, M=0, A=None, packed=False, scales=False, C=False, zeros=False) == w4.OK
    assert _grouped(w4.MXFP4, N=(0, 0, 0), A=None, packed=False, scales=False, C=False) == w4.OK
    # a skipped member's pointers are not checked, the others still are
    assert _grouped(w4.NVFP4, N=(64, 0, 32), bad=("P", 1, None), C=False) == w4.ERR_NULL


# ---- w4a16_gemm_batched validation (no call below reaches a launch) ---------

def test_batch_item_struct_layout():
    # struct w4a16_batch_item: five pointers, two int64
    assert ctypes.sizeof(w4.BatchItem) == 56
    assert w4.BatchItem.N.offset == 40 and w4.BatchItem.K.offset == 48


def _batched(fmt, n=3, M=1, items=None, bad=None, count=None):
    arr = (w4.BatchItem * max(n, 1))()
    for i in range(n):
        z = 0x100000 * (40 + i) if (fmt & 0xFF) in w4.ZERO_FORMATS else None
        arr[i] = w4.BatchItem(0x100000 * (8 + i), 0x100000 * (16 + i), 0x100000 * (24 + i), z,
                              0x100000 * (32 + i), 64 + 32 * i, 128)
    if bad:
        i, field, val = bad
        setattr(arr[i], field, val)
    return w4.load_library().w4a16_gemm_batched(fmt, M, n if count is None else count,
                                                None if items == "null" else arr, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(fmt=6), w4.ERR_FORMAT),
    (dict(fmt=w4.MXFP4 | w4.PATH_SKINNY), w4.ERR_FORMAT),      # no path flags
    (dict(fmt=w4.MXFP4, count=-1), w4.ERR_SHAPE),
    (dict(fmt=w4.MXFP4, M=-1), w4.ERR_SHAPE),
    (dict(fmt=w4.MXFP4, items="null"), w4.ERR_NULL),
    (dict(fmt=w4.NVFP4, bad=(1, "K", 40)), w4.ERR_SHAPE),      # K % 16
    (dict(fmt=w4.NVFP4, bad=(2, "K", 0)), w4.ERR_SHAPE),
    (dict(fmt=w4.NVFP4, bad=(0, "N", -1)), w4.ERR_SHAPE),
    (dict(fmt=w4.NVFP4, bad=(1, "A", None)), w4.ERR_NULL),
    (dict(fmt=w4.NVFP4, bad=(2, "C", None)), w4.ERR_NULL),
    (dict(fmt=w4.NVFP4, bad=(0, "zeros", 0x100000)), w4.ERR_NULL),   # fp4 takes no zeros
    (dict(fmt=w4.INT4_G128, bad=(1, "zeros", None)), w4.ERR_NULL),   # int4 needs zeros
    (dict(fmt=w4.MXFP4, bad=(1, "A", 0x100008)), w4.ERR_ALIGN),
    (dict(fmt=w4.MXFP4, bad=(2, "packed", 0x100008)), w4.ERR_ALIGN),
    (dict(fmt=w4.NVFP4, bad=(0, "scales", 0x100001)), w4.ERR_ALIGN),
    (dict(fmt=w4.NVFP4 | w4.OUT_F32, bad=(2, "C", 0x100002)), w4.ERR_ALIGN),
])
def test_batched_validation(kw, expect):
    assert _batched(**kw) == expect


def test_batched_empty_calls_check_no_pointer():
    assert _batched(w4.MXFP4, count=0, items="null") == w4.OK
    assert _batched(w4.MXFP4, M=0, bad=(1, "A", None)) == w4.OK          # M = 0: nothing read
    # an item with N = 0 is skipped unchecked; the others still are
    arr_ok = _batched(w4.NVFP4, n=1, bad=(0, "N", 0))
    assert arr_ok == w4.OK


# ---- prepacked weights ------------------------------------------------------------

def test_prepacked_bytes():
    lib = w4.load_library()
    assert lib.w4a16_prepacked_bytes(1, 128) == 16 * 64          # one 16-row tile, one 1-KB block
    assert lib.w4a16_prepacked_bytes(16, 384) == 16 * 192
    assert lib.w4a16_prepacked_bytes(17, 256) == 32 * 128        # two tiles, the second padded
    assert lib.w4a16_prepacked_bytes(8192, 3072) == 8192 * 1536
    assert lib.w4a16_prepacked_bytes(0, 128) == 0
    assert lib.w4a16_prepacked_bytes(16, 64) == w4.ERR_SHAPE      # K % 128
    assert lib.w4a16_prepacked_bytes(16, 160) == w4.ERR_SHAPE
    assert lib.w4a16_prepacked_bytes(-1, 128) == w4.ERR_SHAPE
    assert lib.w4a16_prepacked_bytes(16, 2 ** 22 + 128) == w4.ERR_SHAPE


def test_prepack_host_checks():
    lib = w4.load_library()
    P, O = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x900000)
    assert lib.w4a16_prepack(P, O, 16, 64, None) == w4.ERR_SHAPE
    assert lib.w4a16_prepack(P, O, -1, 128, None) == w4.ERR_SHAPE
    assert lib.w4a16_prepack(None, O, 16, 128, None) == w4.ERR_NULL
    assert lib.w4a16_prepack(P, None, 16, 128, None) == w4.ERR_NULL
    assert lib.w4a16_prepack(ctypes.c_void_p(0x100008), O, 16, 128, None) == w4.ERR_ALIGN
    assert lib.w4a16_prepack(P, ctypes.c_void_p(0x900004), 16, 128, None) == w4.ERR_ALIGN
    # 16 x 64 bytes from 0x100000: an output starting inside (or ending inside) overlaps
    assert lib.w4a16_prepack(P, ctypes.c_void_p(0x100200), 16, 128, None) == w4.ERR_OVERLAP
    assert lib.w4a16_prepack(P, ctypes.c_void_p(0x100000 - 512), 16, 128, None) == w4.ERR_OVERLAP
    assert lib.w4a16_prepack(None, None, 0, 128, None) == w4.OK  # nothing to move


def test_prepacked_flag_checks():
    lib = w4.load_library()
    pre = w4.PREPACKED
    # K % 128 for every entry point that takes the flag
    assert _gemm(w4.INT4_G128 | pre, K=192) == w4.ERR_SHAPE
    assert _gemm(w4.INT4_G128 | pre, K=256, M=0) == w4.OK
    assert lib.w4a16_gemm_path(w4.MXFP4 | pre, 1, 64, 96) == w4.ERR_SHAPE
    for M, N, K in [(1, 8192, 3072), (64, 2048, 3072), (4096, 8192, 3072), (300, 256, 512)]:
        assert lib.w4a16_gemm_path(w4.MXFP4 | pre, M, N, K) == lib.w4a16_gemm_path(w4.MXFP4, M, N, K)
    assert lib.w4a16_dequant(w4.NVFP4 | pre, PB, PS, None, PA, 64, 96, None) == w4.ERR_SHAPE
    assert lib.w4a16_dequant(w4.NVFP4 | pre | w4.OUT_F32, PB, PS, None, PA, 64, 128, None) == w4.ERR_FORMAT
    item = w4.BatchItem(PA.value, PB.value, PS.value, None, PC.value, 64, 160)
    assert lib.w4a16_gemm_batched(w4.MXFP4 | pre, 1, 1, ctypes.byref(item), None) == w4.ERR_SHAPE


# ---- the measurement kernels (libw4a16_probe.so, bench.py --bounds) ----------------

def _probe_lib():
    from weight_only_bit_w4a16_amd import _build
    lib = ctypes.CDLL(_build.PROBE_LIB)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.w4a16_probe_read.argtypes = [P, I64, I, I, P, P]
    lib.w4a16_probe_mfma.argtypes = [I, I, I, P, P]
    lib.w4a16_probe_handoff.argtypes = [P, P, P, I, I, I, P]
    return lib


def test_probe_library_exports_its_header():
    text = open(os.path.join(ROOT, "include", "w4a16_probe.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(w4a16_probe_\w+)\s*\(", text, re.M)))
    assert names == ["w4a16_probe_empty", "w4a16_probe_handoff", "w4a16_probe_mfma", "w4a16_probe_read"]
    lib = _probe_lib()
    for name in names:
        assert hasattr(lib, name), name


def test_probe_host_checks():
    lib = _probe_lib()
    p, s = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    bad = -2
    assert lib.w4a16_probe_read(None, 1024, 256, 1, s, None) == bad
    assert lib.w4a16_probe_read(p, 1000, 256, 1, s, None) == bad          # bytes % 16
    assert lib.w4a16_probe_read(p, 1024, 100, 1, s, None) == bad          # threads % 64
    assert lib.w4a16_probe_read(p, 1024, 256, 3, s, None) == bad          # loads per thread
    assert lib.w4a16_probe_read(ctypes.c_void_p(0x100008), 1024, 256, 1, s, None) == bad
    assert lib.w4a16_probe_mfma(0, 256, 10, s, None) == bad
    assert lib.w4a16_probe_mfma(1, 2048, 10, s, None) == bad
    assert lib.w4a16_probe_handoff(p, p, p, 4, 2, 4, None) == bad          # mode
    assert lib.w4a16_probe_handoff(p, None, p, 4, 2, 1, None) == bad
