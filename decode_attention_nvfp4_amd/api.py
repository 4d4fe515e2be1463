"""Thin ctypes binding over libnvfp4kv.so (include/nvfp4kv.h).

Argument marshalling only: PyTorch provides device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

from . import build as _build

F32, BF16 = 0, 1
PREFILL_FP8, PREFILL_F16 = 0, 1
CMP_FP8, CMP_BF16 = 1, 2          # comparison KV formats (nvfp4_cmp_format)
HEAD_DIM, PAGE_SIZE, BLOCK = 128, 16, 16

_lib = None
_lock = threading.Lock()


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str, detail: str):
        super().__init__(f"{fn}: {text} ({status}): {detail}")
        self.status = status


class CacheStruct(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("k_tensor_scale", ctypes.c_float), ("v_tensor_scale", ctypes.c_float),
        ("num_pages", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
    ]


class CmpCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("format", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
    ]


class MxCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("k_exp_offset", ctypes.c_int32), ("v_exp_offset", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
    ]


_VP, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_CP = ctypes.POINTER(CacheStruct)
_XP = ctypes.POINTER(CmpCacheStruct)
_MP = ctypes.POINTER(MxCacheStruct)

_SIGS = {
    "nvfp4_status_string": (ctypes.c_char_p, [_I32]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_kv_plane_bytes": (_SZ, [_I32, _I32, _I32]),
    "nvfp4_kv_cache_bytes": (_SZ, [_I32, _I32]),
    "nvfp4_tensor_scale_from_amax": (_F, [_F]),
    "nvfp4_abs_max": (_I32, [_VP, _I32, _I64, _VP, _VP]),
    "nvfp4_kv_append": (_I32, [_CP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _I32, _VP]),
    "nvfp4_kv_append_mse": (_I32, [_CP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _I32, _VP]),
    "nvfp4_to_fp8": (_I32, [_VP, _VP, _I64, _F, _F, _VP, _VP]),
    "nvfp4_kv_dequant": (_I32, [_CP, _VP, _I32, _I32, _VP, _VP, _I32, _VP]),
    "nvfp4_decode_num_splits": (_I32, [_I32, _I32, _I32, _I32]),
    "nvfp4_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "nvfp4_decode_attn": (_I32, [_CP, _VP, _I32, _I32, _I32, _VP, _I32, _VP, _I32, _F, _I32,
                                 _VP, _SZ, _VP, _VP]),
    "nvfp4_decode_gather_probe": (_I32, [_CP, _I32, _VP, _I32, _VP, _I32, _I32, _VP, _SZ, _VP]),
    "nvfp4_decode_attn_noalloc": (_I32, [_CP, _VP, _I32, _I32, _I32, _VP, _I32, _VP, _I32, _F, _I32,
                                         _VP, _VP]),
    "nvfp4_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "nvfp4_prefill_attn": (_I32, [_CP, _VP, _I32, _I32, _I32, _VP, _I32, _I32, _I32, _F, _VP, _SZ,
                                  _VP, _VP]),
    "nvfp4_cmp_plane_bytes": (_SZ, [_I32, _I32, _I32]),
    "nvfp4_cmp_fp8_scale_from_amax": (_F, [_F]),
    "nvfp4_cmp_append": (_I32, [_XP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _I32, _VP]),
    "nvfp4_cmp_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "nvfp4_cmp_decode_attn": (_I32, [_XP, _VP, _I32, _I32, _I32, _VP, _I32, _VP, _I32, _F, _I32,
                                     _VP, _SZ, _VP, _VP]),
    "nvfp4_mx_plane_bytes": (_SZ, [_I32, _I32, _I32]),
    "nvfp4_mx_exp_offset_from_amax": (_I32, [_F]),
    "nvfp4_mx_append": (_I32, [_MP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _I32, _VP]),
    "nvfp4_mx_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "nvfp4_mx_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "nvfp4_mx_prefill_attn": (_I32, [_MP, _VP, _I32, _I32, _I32, _VP, _I32, _I32, _F, _VP, _SZ, _VP, _VP]),
    "nvfp4_mx_decode_attn": (_I32, [_MP, _VP, _I32, _I32, _I32, _VP, _I32, _VP, _I32, _F, _I32,
                                    _VP, _SZ, _VP, _VP]),
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded library.  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_build.LIB):
                raise RuntimeError(
                    f"{_build.LIB} is missing: build it with `python -m decode_attention_nvfp4_amd.build` "
                    "(there is no fallback implementation)")
            L = ctypes.CDLL(_build.LIB)
            for name, (res, args) in _SIGS.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        L = lib()
        raise Nvfp4Error(fn, status, L.nvfp4_status_string(status).decode(),
                         L.nvfp4_last_error().decode())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


# ------------------------------------------------------------------- sizes

def plane_bytes(num_pages: int, num_kv_heads: int, plane: int) -> int:
    return lib().nvfp4_kv_plane_bytes(num_pages, num_kv_heads, plane)


def kv_cache_bytes(num_pages: int, num_kv_heads: int) -> int:
    return lib().nvfp4_kv_cache_bytes(num_pages, num_kv_heads)


def tensor_scale_from_amax(amax: float) -> float:
    return float(lib().nvfp4_tensor_scale_from_amax(float(amax)))


def decode_num_splits(batch, num_kv_heads, max_seq_len, num_splits=0) -> int:
    return lib().nvfp4_decode_num_splits(batch, num_kv_heads, max_seq_len, num_splits)


def decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, num_splits=0) -> int:
    return lib().nvfp4_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, num_splits)


def prefill_workspace_bytes(num_tokens, num_q_heads, num_kv_heads, prefix_len, mode=PREFILL_FP8) -> int:
    return lib().nvfp4_prefill_workspace_bytes(num_tokens, num_q_heads, num_kv_heads, prefix_len, mode)


# ------------------------------------------------------------------- cache

class KVCache:
    """The four device planes of a paged NVFP4 cache plus its tensor scales.

    fill: initial byte value of every plane (None leaves memory uninitialised)."""

    def __init__(self, num_pages: int, num_kv_heads: int, k_tensor_scale: float,
                 v_tensor_scale: float, device="cuda", fill: int | None = 0):
        self.num_pages = int(num_pages)
        self.num_kv_heads = int(num_kv_heads)
        self.k_tensor_scale = float(k_tensor_scale)
        self.v_tensor_scale = float(v_tensor_scale)
        planes = []
        for p in range(4):
            n = plane_bytes(self.num_pages, self.num_kv_heads, p)
            t = torch.empty(n, dtype=torch.uint8, device=device)
            if fill is not None:
                t.fill_(fill)
            planes.append(t)
        self.k_codes, self.k_scales, self.v_codes, self.v_scales = planes

    def struct(self) -> CacheStruct:
        return CacheStruct(self.k_codes.data_ptr(), self.k_scales.data_ptr(),
                           self.v_codes.data_ptr(), self.v_scales.data_ptr(),
                           self.k_tensor_scale, self.v_tensor_scale,
                           self.num_pages, self.num_kv_heads, PAGE_SIZE, HEAD_DIM)

    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales))


# ---------------------------------------------------------------- compute

def abs_max(x: torch.Tensor, stream=None) -> torch.Tensor:
    """max |x| as a one-element device float tensor (exact)."""
    _dev(x, "x")
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check("nvfp4_abs_max", lib().nvfp4_abs_max(_ptr(x), _dtype_code(x), x.numel(), _ptr(out),
                                                _stream(stream)))
    return out


def append(cache: KVCache, k_new, v_new, tok_seq, tok_pos, page_table, stream=None):
    """Quantize rows k_new/v_new [n][Hkv][128] into the cache at (tok_seq, tok_pos)."""
    _append("nvfp4_kv_append", cache, k_new, v_new, tok_seq, tok_pos, page_table, stream)


def append_mse(cache: KVCache, k_new, v_new, tok_seq, tok_pos, page_table, stream=None):
    """append() with the MSE-searched block scale."""
    _append("nvfp4_kv_append_mse", cache, k_new, v_new, tok_seq, tok_pos, page_table, stream)


def _append(name, cache, k_new, v_new, tok_seq, tok_pos, page_table, stream):
    n = k_new.shape[0] if k_new.dim() else 0
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, nm)
        if tuple(t.shape[1:]) != (cache.num_kv_heads, HEAD_DIM):
            raise ValueError(f"{nm} must be [n][{cache.num_kv_heads}][128], got {tuple(t.shape)}")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must match in shape and dtype")
    _dev(tok_seq, "tok_seq", torch.int32)
    _dev(tok_pos, "tok_pos", torch.int32)
    _dev(page_table, "page_table", torch.int32)
    if tok_seq.numel() < n or tok_pos.numel() < n:
        raise ValueError("tok_seq / tok_pos shorter than the number of rows")
    cs = cache.struct()
    _check(name, getattr(lib(), name)(
        ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), n, _ptr(tok_seq),
        _ptr(tok_pos), _ptr(page_table), page_table.shape[-1], _stream(stream)))


def to_fp8(codes, scales, global_scale: float, out_scale: float, out=None, stream=None):
    """FP8 codes (uint8, one per element) of a row-major NVFP4 tensor: packed
    codes (uint8, n/2 bytes) and block scales (uint8, n/16 bytes); the
    values divide by the global encode scale and encode over out_scale."""
    _dev(codes, "codes", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    n = codes.numel() * 2
    if scales.numel() * 16 != n:
        raise ValueError("scales must hold one byte per 16 elements")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    elif out.numel() != n or out.dtype != torch.uint8:
        raise ValueError("out must be uint8 with one byte per element")
    _check("nvfp4_to_fp8", lib().nvfp4_to_fp8(_ptr(codes), _ptr(scales), n, float(global_scale),
                                              float(out_scale), _ptr(out), _stream(stream)))
    return out


def dequant(cache: KVCache, page_table_row, pos0: int, n: int, out_dtype=torch.float32,
            want_k=True, want_v=True, stream=None):
    """(K, V) of positions pos0..pos0+n-1 of one sequence, [n][Hkv][128]."""
    _dev(page_table_row, "page_table_row", torch.int32)
    dev = cache.k_codes.device
    k = torch.empty((n, cache.num_kv_heads, HEAD_DIM), dtype=out_dtype, device=dev) if want_k else None
    v = torch.empty((n, cache.num_kv_heads, HEAD_DIM), dtype=out_dtype, device=dev) if want_v else None
    code = F32 if out_dtype == torch.float32 else BF16 if out_dtype == torch.bfloat16 else -1
    cs = cache.struct()
    _check("nvfp4_kv_dequant", lib().nvfp4_kv_dequant(
        ctypes.byref(cs), _ptr(page_table_row), pos0, n, _ptr(k), _ptr(v), code, _stream(stream)))
    return k, v


def decode(cache: KVCache, q, page_table, seq_lens, max_seq_len: int, softmax_scale=None,
           num_splits: int = 0, workspace=None, out=None, stream=None):
    """Decode attention: q [B][Hq][128] -> out [B][Hq][128] FP32."""
    _dev(q, "q")
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    B, Hq = q.shape[0], q.shape[1]
    if q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, cache.num_kv_heads, max_seq_len, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    _check("nvfp4_decode_attn", lib().nvfp4_decode_attn(
        ctypes.byref(cs), _ptr(q), _dtype_code(q), B, Hq, _ptr(page_table), page_table.shape[-1],
        _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(num_splits), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _ptr(out), _stream(stream)))
    return out


def decode_gather_probe(cache: KVCache, page_table, seq_lens, max_seq_len: int, num_splits: int = 0,
                        sink=None, stream=None):
    """The decode's page walk and loads without the math (a timing aid)."""
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    B = seq_lens.numel()
    if sink is None:
        w = decode_num_splits(B, cache.num_kv_heads, max_seq_len, num_splits)
        sink = torch.empty(max(1, w) * 64, dtype=torch.int32, device=page_table.device)
    cs = cache.struct()
    _check("nvfp4_decode_gather_probe", lib().nvfp4_decode_gather_probe(
        ctypes.byref(cs), B, _ptr(page_table), page_table.shape[-1], _ptr(seq_lens), int(max_seq_len),
        int(num_splits), _ptr(sink), sink.numel() * sink.element_size(), _stream(stream)))
    return sink


NOALLOC_SCRATCH_BYTES = 40 << 20   # NVFP4_DECODE_NOALLOC_SCRATCH_BYTES


def decode_noalloc(cache: KVCache, q, page_table, seq_lens, max_seq_len: int, softmax_scale=None,
                   num_splits: int = 0, out=None, stream=None):
    """decode() through nvfp4_decode_attn_noalloc: no workspace, the
    library's fixed per-device scratch holds the partial results."""
    _dev(q, "q")
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    B, Hq = q.shape[0], q.shape[1]
    if q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    cs = cache.struct()
    _check("nvfp4_decode_attn_noalloc", lib().nvfp4_decode_attn_noalloc(
        ctypes.byref(cs), _ptr(q), _dtype_code(q), B, Hq, _ptr(page_table), page_table.shape[-1],
        _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(num_splits), _ptr(out), _stream(stream)))
    return out


def prefill(cache: KVCache, q, page_table_row, prefix_len: int, causal: bool = True,
            softmax_scale=None, workspace=None, out=None, stream=None, mode=PREFILL_FP8):
    """Chunked prefill: q [T][Hq][128] -> out [T][Hq][128] FP32.  mode:
    PREFILL_FP8 (FP8 operands) or PREFILL_F16 (exact 16-bit operands)."""
    _dev(q, "q")
    _dev(page_table_row, "page_table_row", torch.int32)
    T, Hq = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((T, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = prefill_workspace_bytes(T, Hq, cache.num_kv_heads, prefix_len, mode)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    _check("nvfp4_prefill_attn", lib().nvfp4_prefill_attn(
        ctypes.byref(cs), _ptr(q), _dtype_code(q), T, Hq, _ptr(page_table_row), int(prefix_len),
        int(bool(causal)), int(mode), float(softmax_scale), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------ comparison KV formats

def cmp_plane_bytes(num_pages: int, num_kv_heads: int, fmt: int) -> int:
    return lib().nvfp4_cmp_plane_bytes(num_pages, num_kv_heads, fmt)


def cmp_fp8_scale_from_amax(amax: float) -> float:
    return float(lib().nvfp4_cmp_fp8_scale_from_amax(float(amax)))


def cmp_decode_workspace_bytes(fmt, batch, num_q_heads, num_kv_heads, max_seq_len, num_splits=0) -> int:
    return lib().nvfp4_cmp_decode_workspace_bytes(fmt, batch, num_q_heads, num_kv_heads, max_seq_len,
                                                  num_splits)


class CmpCache:
    """The two device planes (k, v) of a paged FP8 or BF16 cache.  The scales
    are the FP8 tensor scales (ignored for BF16)."""

    def __init__(self, fmt: int, num_pages: int, num_kv_heads: int, k_scale: float = 1.0,
                 v_scale: float = 1.0, device="cuda", fill: int | None = 0):
        self.fmt = int(fmt)
        self.num_pages = int(num_pages)
        self.num_kv_heads = int(num_kv_heads)
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)
        n = cmp_plane_bytes(self.num_pages, self.num_kv_heads, self.fmt)
        if n == 0:
            raise ValueError(f"bad comparison cache ({fmt}, {num_pages}, {num_kv_heads})")
        self.k = torch.empty(n, dtype=torch.uint8, device=device)
        self.v = torch.empty(n, dtype=torch.uint8, device=device)
        if fill is not None:
            self.k.fill_(fill)
            self.v.fill_(fill)

    def struct(self) -> CmpCacheStruct:
        return CmpCacheStruct(self.k.data_ptr(), self.v.data_ptr(), self.k_scale, self.v_scale, self.fmt,
                              self.num_pages, self.num_kv_heads, PAGE_SIZE, HEAD_DIM)

    def nbytes(self) -> int:
        return self.k.numel() + self.v.numel()


def cmp_append(cache: CmpCache, k_new, v_new, tok_seq, tok_pos, page_table, stream=None):
    """Store rows k_new/v_new [n][Hkv][128] into the comparison cache."""
    n = k_new.shape[0] if k_new.dim() else 0
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, nm)
        if tuple(t.shape[1:]) != (cache.num_kv_heads, HEAD_DIM):
            raise ValueError(f"{nm} must be [n][{cache.num_kv_heads}][128], got {tuple(t.shape)}")
    if k_new.shape != v_new.shape or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must match in shape and dtype")
    _dev(tok_seq, "tok_seq", torch.int32)
    _dev(tok_pos, "tok_pos", torch.int32)
    _dev(page_table, "page_table", torch.int32)
    if tok_seq.numel() < n or tok_pos.numel() < n:
        raise ValueError("tok_seq / tok_pos shorter than the number of rows")
    cs = cache.struct()
    _check("nvfp4_cmp_append", lib().nvfp4_cmp_append(
        ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), n, _ptr(tok_seq),
        _ptr(tok_pos), _ptr(page_table), page_table.shape[-1], _stream(stream)))


def cmp_decode(cache: CmpCache, q, page_table, seq_lens, max_seq_len: int, softmax_scale=None,
               num_splits: int = 0, workspace=None, out=None, stream=None):
    """Decode attention over a comparison cache: q [B][Hq][128] -> [B][Hq][128] FP32."""
    _dev(q, "q")
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    B, Hq = q.shape[0], q.shape[1]
    if q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = cmp_decode_workspace_bytes(cache.fmt, B, Hq, cache.num_kv_heads, max_seq_len, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    _check("nvfp4_cmp_decode_attn", lib().nvfp4_cmp_decode_attn(
        ctypes.byref(cs), _ptr(q), _dtype_code(q), B, Hq, _ptr(page_table), page_table.shape[-1],
        _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(num_splits), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------------------- MXFP4

def mx_plane_bytes(num_pages: int, num_kv_heads: int, plane: int) -> int:
    return lib().nvfp4_mx_plane_bytes(num_pages, num_kv_heads, plane)


def mx_exp_offset_from_amax(amax: float) -> int:
    return lib().nvfp4_mx_exp_offset_from_amax(float(amax))


class MxCache:
    """The four device planes of a paged MXFP4 cache plus the power-of-two
    offsets its decode takes the K and V values relative to."""

    def __init__(self, num_pages: int, num_kv_heads: int, k_exp_offset: int = 0, v_exp_offset: int = 0,
                 device="cuda", fill: int | None = 0):
        self.num_pages = int(num_pages)
        self.num_kv_heads = int(num_kv_heads)
        self.k_exp_offset = int(k_exp_offset)
        self.v_exp_offset = int(v_exp_offset)
        planes = []
        for p in range(4):
            n = mx_plane_bytes(self.num_pages, self.num_kv_heads, p)
            if n == 0:
                raise ValueError(f"bad MXFP4 cache ({num_pages}, {num_kv_heads})")
            t = torch.empty(n, dtype=torch.uint8, device=device)
            if fill is not None:
                t.fill_(fill)
            planes.append(t)
        self.k_codes, self.k_scales, self.v_codes, self.v_scales = planes

    def struct(self) -> MxCacheStruct:
        return MxCacheStruct(self.k_codes.data_ptr(), self.k_scales.data_ptr(),
                             self.v_codes.data_ptr(), self.v_scales.data_ptr(),
                             self.k_exp_offset, self.v_exp_offset,
                             self.num_pages, self.num_kv_heads, PAGE_SIZE, HEAD_DIM)

    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales))


def mx_append(cache: MxCache, k_new, v_new, tok_seq, tok_pos, page_table, stream=None):
    """Quantize rows k_new/v_new [n][Hkv][128] to MXFP4 at (tok_seq, tok_pos)."""
    _append("nvfp4_mx_append", cache, k_new, v_new, tok_seq, tok_pos, page_table, stream)


def mx_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, num_splits=0) -> int:
    return lib().nvfp4_mx_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, num_splits)


def mx_decode(cache: MxCache, q, page_table, seq_lens, max_seq_len: int, softmax_scale=None,
              num_splits: int = 0, workspace=None, out=None, stream=None):
    """Decode attention over an MXFP4 cache: q [B][Hq][128] -> [B][Hq][128] FP32."""
    _dev(q, "q")
    _dev(page_table, "page_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    B, Hq = q.shape[0], q.shape[1]
    if q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = mx_decode_workspace_bytes(B, Hq, cache.num_kv_heads, max_seq_len, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    _check("nvfp4_mx_decode_attn", lib().nvfp4_mx_decode_attn(
        ctypes.byref(cs), _ptr(q), _dtype_code(q), B, Hq, _ptr(page_table), page_table.shape[-1],
        _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(num_splits), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _ptr(out), _stream(stream)))
    return out


def mx_prefill_workspace_bytes(num_tokens, num_q_heads, num_kv_heads, prefix_len) -> int:
    return lib().nvfp4_mx_prefill_workspace_bytes(num_tokens, num_q_heads, num_kv_heads, prefix_len)


def mx_prefill(cache: MxCache, q, page_table_row, prefix_len: int, causal: bool = True,
               softmax_scale=None, workspace=None, out=None, stream=None):
    """Chunked prefill over an MXFP4 cache: q [T][Hq][128] -> out [T][Hq][128]
    FP32 (FP4 K operand with its block scales, FP8 Q, P and V)."""
    _dev(q, "q")
    _dev(page_table_row, "page_table_row", torch.int32)
    T, Hq = q.shape[0], q.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(HEAD_DIM)
    if out is None:
        out = torch.empty((T, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = mx_prefill_workspace_bytes(T, Hq, cache.num_kv_heads, prefix_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cs = cache.struct()
    _check("nvfp4_mx_prefill_attn", lib().nvfp4_mx_prefill_attn(
        ctypes.byref(cs), _ptr(q), _dtype_code(q), T, Hq, _ptr(page_table_row), int(prefix_len),
        int(bool(causal)), float(softmax_scale), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _ptr(out), _stream(stream)))
    return out
