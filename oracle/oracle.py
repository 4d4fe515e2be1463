"""ctypes wrapper around the C oracle (``nvfp4_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The product package never imports this module.
Arrays are numpy; every function works on the *logical* layout (one 4-bit
code per byte, rows of 128 elements), not on the paged device layout.
"""
from __future__ import annotations

import ctypes
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

D = 128
BLOCK = 16
NBLK = D // BLOCK
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)

_lib = None
_lock = threading.Lock()

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int)


def lib():
    """Load (building first if needed) the oracle shared library.  The
    environment variable NVFP4_ORACLE_LIB names another build of the same
    source to load instead (the sanitized one, see build.py)."""
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("NVFP4_ORACLE_LIB")
            if not path:
                path = _build.LIB
                if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                    _build.build()
            L = ctypes.CDLL(path)
            L.orc_e2m1_value.restype = ctypes.c_double
            L.orc_e2m1_value.argtypes = [ctypes.c_uint]
            L.orc_e4m3_value.restype = ctypes.c_double
            L.orc_e4m3_value.argtypes = [ctypes.c_uint]
            L.orc_tensor_scale.restype = ctypes.c_float
            L.orc_tensor_scale.argtypes = [_f32p, ctypes.c_size_t]
            L.orc_tensor_scale_from_amax.restype = ctypes.c_float
            L.orc_tensor_scale_from_amax.argtypes = [ctypes.c_float]
            L.orc_abs_max.restype = ctypes.c_float
            L.orc_abs_max.argtypes = [_f32p, ctypes.c_size_t]
            L.orc_block_scale_code.restype = ctypes.c_uint
            L.orc_block_scale_code.argtypes = [ctypes.c_float, ctypes.c_float]
            L.orc_element_code.restype = ctypes.c_uint
            L.orc_element_code.argtypes = [ctypes.c_float, ctypes.c_uint, ctypes.c_float]
            L.orc_element_codes.restype = None
            L.orc_element_codes.argtypes = [_f32p, ctypes.c_size_t, ctypes.c_uint,
                                            ctypes.c_float, _u8p]
            L.orc_block_scale_codes.restype = None
            L.orc_block_scale_codes.argtypes = [_f32p, ctypes.c_size_t, ctypes.c_float, _u8p]
            L.orc_quantize_rows.restype = None
            L.orc_quantize_rows.argtypes = [_f32p, ctypes.c_size_t, ctypes.c_float, _u8p, _u8p]
            L.orc_dequant_value.restype = ctypes.c_float
            L.orc_dequant_value.argtypes = [ctypes.c_uint, ctypes.c_uint, ctypes.c_float]
            L.orc_dequant_rows.restype = None
            L.orc_dequant_rows.argtypes = [_u8p, _u8p, ctypes.c_size_t, ctypes.c_float, _f32p]
            L.orc_f32_to_bf16_array.restype = None
            L.orc_f32_to_bf16_array.argtypes = [_f32p, ctypes.c_size_t, _u16p]
            L.orc_attend.restype = ctypes.c_int
            L.orc_attend.argtypes = [_f32p, ctypes.c_int, ctypes.c_int,
                                     _u8p, _u8p, ctypes.c_float,
                                     _u8p, _u8p, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_double, _f64p, _f32p]
            L.orc_prefill_rows.restype = ctypes.c_int
            L.orc_prefill_rows.argtypes = [_f32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           _u8p, _u8p, ctypes.c_float,
                                           _u8p, _u8p, ctypes.c_float,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, _f64p, _f32p]
            L.orc_block_sq_error.restype = ctypes.c_double
            L.orc_block_sq_error.argtypes = [_f32p, ctypes.c_uint, ctypes.c_float]
            L.orc_block_scale_code_mse.restype = ctypes.c_uint
            L.orc_block_scale_code_mse.argtypes = [_f32p, ctypes.c_float]
            L.orc_quantize_rows_mse.restype = None
            L.orc_quantize_rows_mse.argtypes = [_f32p, ctypes.c_size_t, ctypes.c_float, _u8p, _u8p]
            L.orc_mx_block_exp.restype = ctypes.c_int
            L.orc_mx_block_exp.argtypes = [ctypes.c_float]
            L.orc_e8m0_value.restype = ctypes.c_double
            L.orc_e8m0_value.argtypes = [ctypes.c_uint]
            L.orc_mx_element_code.restype = ctypes.c_uint
            L.orc_mx_element_code.argtypes = [ctypes.c_float, ctypes.c_int]
            L.orc_mx_quantize_rows.restype = None
            L.orc_mx_quantize_rows.argtypes = [_f32p, ctypes.c_size_t, _u8p, _u8p]
            L.orc_mx_dequant_rows.restype = None
            L.orc_mx_dequant_rows.argtypes = [_u8p, _u8p, ctypes.c_size_t, _f32p]
            L.orc_nvfp4_to_fp8_code.restype = ctypes.c_uint
            L.orc_nvfp4_to_fp8_code.argtypes = [ctypes.c_uint, ctypes.c_uint, ctypes.c_float, ctypes.c_float]
            L.orc_nvfp4_to_fp8.restype = None
            L.orc_nvfp4_to_fp8.argtypes = [_u8p, _u8p, ctypes.c_size_t, ctypes.c_float, ctypes.c_float, _u8p]
            L.orc_fp8_tensor_scale_from_amax.restype = ctypes.c_float
            L.orc_fp8_tensor_scale_from_amax.argtypes = [ctypes.c_float]
            L.orc_fp8_code.restype = ctypes.c_uint
            L.orc_fp8_code.argtypes = [ctypes.c_float, ctypes.c_float]
            L.orc_fp8_codes.restype = None
            L.orc_fp8_codes.argtypes = [_f32p, ctypes.c_size_t, ctypes.c_float, _u8p]
            L.orc_fp8_value.restype = ctypes.c_float
            L.orc_fp8_value.argtypes = [ctypes.c_uint, ctypes.c_float]
            L.orc_fp8_dequant.restype = None
            L.orc_fp8_dequant.argtypes = [_u8p, ctypes.c_size_t, ctypes.c_float, _f32p]
            L.orc_attend_dense.restype = ctypes.c_int
            L.orc_attend_dense.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, _f32p, _f32p,
                                           ctypes.c_int, ctypes.c_double, _f64p, _f32p]
            _lib = L
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ scalars

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(int(byte))


def block_scale_code(amax_block: float, s_t: float) -> int:
    return lib().orc_block_scale_code(float(amax_block), float(s_t))


def element_code(x: float, sb_code: int, s_t: float) -> int:
    return lib().orc_element_code(float(x), int(sb_code), float(s_t))


def dequant_value(code: int, sb_code: int, s_t: float) -> float:
    return lib().orc_dequant_value(int(code), int(sb_code), float(s_t))


# ------------------------------------------------------------------- arrays

def abs_max(x) -> float:
    x = _c(x, np.float32).reshape(-1)
    return float(lib().orc_abs_max(_p(x, _f32p), x.size))


def tensor_scale(x) -> float:
    """s_t = amax(|x|) / (6 * 448), FP32."""
    x = _c(x, np.float32).reshape(-1)
    return float(np.float32(lib().orc_tensor_scale(_p(x, _f32p), x.size)))


def tensor_scale_from_amax(amax: float) -> float:
    return float(np.float32(lib().orc_tensor_scale_from_amax(float(amax))))


def element_codes(x, sb_code: int, s_t: float) -> np.ndarray:
    x = _c(x, np.float32).reshape(-1)
    out = np.empty(x.size, np.uint8)
    lib().orc_element_codes(_p(x, _f32p), x.size, int(sb_code), float(s_t), _p(out, _u8p))
    return out


def block_scale_codes(amax, s_t: float) -> np.ndarray:
    a = _c(amax, np.float32).reshape(-1)
    out = np.empty(a.size, np.uint8)
    lib().orc_block_scale_codes(_p(a, _f32p), a.size, float(s_t), _p(out, _u8p))
    return out


def quantize_rows(x, s_t: float):
    """x: [..., 128] FP32 -> (codes [..., 128] u8 one code per byte, scales [..., 8] u8)."""
    x = _c(x, np.float32)
    shape = x.shape
    assert shape[-1] == D
    flat = x.reshape(-1, D)
    n = flat.shape[0]
    codes = np.empty((n, D), np.uint8)
    scales = np.empty((n, NBLK), np.uint8)
    if n:
        lib().orc_quantize_rows(_p(flat, _f32p), n, float(s_t), _p(codes, _u8p), _p(scales, _u8p))
    return codes.reshape(shape), scales.reshape(shape[:-1] + (NBLK,))


def block_sq_error(x16, sb_code: int, s_t: float) -> float:
    """Squared error of one 16-element block under block-scale code sb_code
    (the MSE search's criterion, summed in element order)."""
    x16 = _c(x16, np.float32)
    assert x16.size == BLOCK
    return float(lib().orc_block_sq_error(_p(x16, _f32p), int(sb_code), float(s_t)))


def block_scale_code_mse(x16, s_t: float) -> int:
    x16 = _c(x16, np.float32)
    assert x16.size == BLOCK
    return int(lib().orc_block_scale_code_mse(_p(x16, _f32p), float(s_t)))


def quantize_rows_mse(x, s_t: float):
    """quantize_rows with the MSE-searched block scale."""
    x = _c(x, np.float32)
    shape = x.shape
    assert shape[-1] == D
    flat = x.reshape(-1, D)
    n = flat.shape[0]
    codes = np.empty((n, D), np.uint8)
    scales = np.empty((n, NBLK), np.uint8)
    if n:
        lib().orc_quantize_rows_mse(_p(flat, _f32p), n, float(s_t), _p(codes, _u8p), _p(scales, _u8p))
    return codes.reshape(shape), scales.reshape(shape[:-1] + (NBLK,))


def dequant_rows(codes, scales, s_t: float) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    shape = codes.shape
    n = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    out = np.empty((n, D), np.float32)
    if n:
        lib().orc_dequant_rows(_p(codes, _u8p), _p(scales, _u8p), n, float(s_t), _p(out, _f32p))
    return out.reshape(shape)


def f32_to_bf16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_p(x, _f32p), x.size, _p(out, _u16p))
    return out


# ---------------------------------------------------------------- attention

def attend(q, Hkv, kcodes, kscales, s_tk, vcodes, vscales, s_tv, scale=None):
    """Attention of q [Hq][128] over L cached tokens of one sequence.

    kcodes/vcodes: [L][Hkv][128] (one code per byte); kscales/vscales:
    [L][Hkv][8].  Returns [Hq][128] FP32; L == 0 gives zeros."""
    q = _c(q, np.float32)
    Hq = q.shape[0]
    L = kcodes.shape[0]
    if L == 0:
        kcodes = np.zeros((1, Hkv, D), np.uint8)
        vcodes = kcodes
        kscales = np.zeros((1, Hkv, NBLK), np.uint8)
        vscales = kscales
    kcodes = _c(kcodes, np.uint8)
    vcodes = _c(vcodes, np.uint8)
    kscales = _c(kscales, np.uint8)
    vscales = _c(vscales, np.uint8)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((Hq, D), np.float32)
    work = np.empty(max(L, 1), np.float64)
    rc = lib().orc_attend(_p(q, _f32p), Hq, Hkv, _p(kcodes, _u8p), _p(kscales, _u8p), float(s_tk),
                          _p(vcodes, _u8p), _p(vscales, _u8p), float(s_tv), L, float(scale),
                          _p(work, _f64p), _p(out, _f32p))
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return out


def decode_batch(q, seqs, Hkv, s_tk, s_tv, scale=None, threads=None):
    """Decode attention for a batch.

    q: [B][Hq][128] FP32; seqs: list of B tuples (kcodes [L][Hkv][128],
    kscales [L][Hkv][8], vcodes, vscales), one per sequence.  The (sequence,
    KV head) pairs run on a thread pool (the C call releases the GIL); each
    pair is an independent call on that KV head's slice.  Returns
    [B][Hq][128]."""
    q = _c(q, np.float32)
    B, Hq = q.shape[0], q.shape[1]
    G = Hq // Hkv
    out = np.empty(q.shape, np.float32)
    threads = threads or os.cpu_count() or 1

    def one(unit):
        b, h = divmod(unit, Hkv)
        kc, ks, vc, vs = seqs[b]
        out[b, h * G:(h + 1) * G] = attend(q[b, h * G:(h + 1) * G], 1, kc[:, h:h + 1], ks[:, h:h + 1],
                                           s_tk, vc[:, h:h + 1], vs[:, h:h + 1], s_tv, scale)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(B * Hkv)))
    return out


def prefill_rows(q_rows, rows, Hkv, kcodes, kscales, s_tk, vcodes, vscales, s_tv,
                 prefix, causal=True, scale=None, threads=None):
    """Causal chunk attention for selected query rows.

    q_rows: [n][Hq][128] FP32 (the selected rows of the chunk's queries);
    rows: their indices i within the chunk (query i sits at absolute
    position prefix + i); kcodes...: the whole cache [Ltot][Hkv][...].
    Rows are split over a thread pool.  Returns [n][Hq][128]."""
    q_rows = _c(q_rows, np.float32)
    rows = np.asarray(rows, np.int32)
    n, Hq = q_rows.shape[0], q_rows.shape[1]
    kcodes = _c(kcodes, np.uint8)
    vcodes = _c(vcodes, np.uint8)
    kscales = _c(kscales, np.uint8)
    vscales = _c(vscales, np.uint8)
    total = kcodes.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((n, Hq, D), np.float32)
    threads = max(1, min(threads or os.cpu_count() or 1, n))
    bounds = np.linspace(0, n, threads + 1).astype(int)

    def one(c):
        a, e = bounds[c], bounds[c + 1]
        if a == e:
            return
        r = np.ascontiguousarray(rows[a:e])
        qi = np.ascontiguousarray(q_rows[a:e])
        o = np.empty((e - a, Hq, D), np.float32)
        work = np.empty(max(total, 1), np.float64)
        rc = lib().orc_prefill_rows(_p(qi, _f32p), _p(r, _i32p), e - a, Hq, Hkv,
                                    _p(kcodes, _u8p), _p(kscales, _u8p), float(s_tk),
                                    _p(vcodes, _u8p), _p(vscales, _u8p), float(s_tv),
                                    int(prefix), int(bool(causal)), total, float(scale),
                                    _p(work, _f64p), _p(o, _f32p))
        if rc != 0:
            raise MemoryError("oracle scratch allocation failed")
        out[a:e] = o

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(threads)))
    return out


# ------------------------------------------------ comparison formats (FP8, BF16)

def fp8_tensor_scale(x) -> float:
    """FP8 cache tensor scale: amax(|X|) / 448 in FP32."""
    return float(lib().orc_fp8_tensor_scale_from_amax(ctypes.c_float(abs_max(x))))


def fp8_code(x: float, s_t: float) -> int:
    return int(lib().orc_fp8_code(float(x), float(s_t)))


def fp8_codes(x, s_t: float) -> np.ndarray:
    """E4M3 codes of x / s_t (nearest, ties to even, clamped to 448), any shape."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_fp8_codes(_p(x, _f32p), x.size, float(s_t), _p(out, _u8p))
    return out


def fp8_value(code: int, s_t: float) -> float:
    return float(lib().orc_fp8_value(int(code), float(s_t)))


def fp8_dequant(codes, s_t: float) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float32)
    lib().orc_fp8_dequant(_p(codes, _u8p), codes.size, float(s_t), _p(out, _f32p))
    return out


# ------------------------------------------------------------------ MXFP4

MX_BLOCK = 32


def mx_block_exp(amax: float) -> int:
    return int(lib().orc_mx_block_exp(float(amax)))


def e8m0_value(byte: int) -> float:
    return float(lib().orc_e8m0_value(int(byte)))


def mx_element_code(x: float, e: int) -> int:
    return int(lib().orc_mx_element_code(float(x), int(e)))


def mx_quantize_rows(x):
    """MXFP4 of rows [...][128]: (codes [...][128], E8M0 scales [...][4])."""
    x = _c(x, np.float32)
    shape = x.shape
    assert shape[-1] == D
    n = x.size // D
    codes = np.empty((n, D), np.uint8)
    scales = np.empty((n, D // MX_BLOCK), np.uint8)
    if n:
        lib().orc_mx_quantize_rows(_p(x.reshape(-1, D), _f32p), n, _p(codes, _u8p), _p(scales, _u8p))
    return codes.reshape(shape), scales.reshape(shape[:-1] + (D // MX_BLOCK,))


def mx_dequant_rows(codes, scales) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    shape = codes.shape
    n = codes.size // D
    out = np.empty((n, D), np.float32)
    if n:
        lib().orc_mx_dequant_rows(_p(codes.reshape(-1, D), _u8p), _p(scales.reshape(-1, D // MX_BLOCK), _u8p),
                                  n, _p(out, _f32p))
    return out.reshape(shape)


def nvfp4_to_fp8_code(code: int, sb_code: int, g: float, s8: float) -> int:
    return int(lib().orc_nvfp4_to_fp8_code(int(code), int(sb_code), float(g), float(s8)))


def nvfp4_to_fp8(codes, scales, g: float, s8: float) -> np.ndarray:
    """FP8 codes [rows][cols] of a row-major NVFP4 tensor: codes as one
    nibble per element [rows][cols] (low nibble of the packed byte first),
    block scales [rows][cols/16]; dequantize dividing by the global scale g,
    then encode over the output scale s8."""
    codes = _c(codes, np.uint8)
    packed = (codes[:, 0::2] & 15) | ((codes[:, 1::2] & 15) << 4)
    return nvfp4_to_fp8_packed(packed.astype(np.uint8), scales, g, s8)


def nvfp4_to_fp8_packed(packed, scales, g: float, s8: float) -> np.ndarray:
    """nvfp4_to_fp8 from packed bytes [rows][cols/2] (element 2j in the low
    nibble of byte j)."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint8)
    rows, cols = packed.shape[0], packed.shape[1] * 2
    assert cols % 16 == 0 and scales.shape == (rows, cols // 16)
    out = np.empty((rows, cols), np.uint8)
    if out.size:
        lib().orc_nvfp4_to_fp8(_p(packed, _u8p), _p(scales, _u8p), out.size, float(g), float(s8), _p(out, _u8p))
    return out


def attend_dense(q, Hkv, kh, vh, scale=None):
    """Attention of q [Hq][128] over an already dequantized cache kh, vh
    [L][Hkv][128] FP32 (the comparison formats).  Returns [Hq][128]."""
    q = _c(q, np.float32)
    Hq = q.shape[0]
    L = kh.shape[0]
    if L == 0:
        kh = np.zeros((1, Hkv, D), np.float32)
        vh = kh
    kh = _c(kh, np.float32)
    vh = _c(vh, np.float32)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((Hq, D), np.float32)
    work = np.empty(max(L, 1), np.float64)
    lib().orc_attend_dense(_p(q, _f32p), Hq, Hkv, _p(kh, _f32p), _p(vh, _f32p), L, float(scale),
                           _p(work, _f64p), _p(out, _f32p))
    return out


def decode_batch_dense(q, seqs, Hkv, scale=None, threads=None):
    """Decode attention for a batch over dequantized caches: seqs is a list of
    B pairs (kh [L][Hkv][128], vh [L][Hkv][128]) FP32.  Returns [B][Hq][128]."""
    q = _c(q, np.float32)
    B, Hq = q.shape[0], q.shape[1]
    G = Hq // Hkv
    out = np.empty(q.shape, np.float32)
    threads = threads or os.cpu_count() or 1

    def one(unit):
        b, h = divmod(unit, Hkv)
        kh, vh = seqs[b]
        out[b, h * G:(h + 1) * G] = attend_dense(q[b, h * G:(h + 1) * G], 1, kh[:, h:h + 1],
                                                 vh[:, h:h + 1], scale)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(B * Hkv)))
    return out
