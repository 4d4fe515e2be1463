"""Helpers for the GPU parity tests: build caches through the C-ABI library,
compute the oracle's answer on the same seeded inputs, compare."""
from __future__ import annotations

import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from decode_attention_nvfp4_amd import api
from decode_attention_nvfp4_amd import workloads as W
from layout import Planes, sequence_tokens

TOL = 2e-2   # pass iff |o - r| <= TOL * max(1, |r|) for every output element

# Host threads for input generation and the oracle (its C calls release the
# GIL); a GPU machine's share is 16 cores.
THREADS = max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    """list(map(fn, items)) on THREADS threads."""
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        return list(ex.map(fn, items))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
    return t.to(dev())


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev())


def planes(cache) -> Planes:
    """The layout reader over a copy of an NVFP4 or MXFP4 cache's planes."""
    torch.cuda.synchronize()
    nblk = 4 if isinstance(cache, api.MxCache) else 8
    return Planes(cache.k_codes.cpu().numpy(), cache.k_scales.cpu().numpy(),
                  cache.v_codes.cpu().numpy(), cache.v_scales.cpu().numpy(),
                  cache.num_pages, cache.num_kv_heads, nblk=nblk)


def check_planes(P: Planes, page_table, lens, codes, seqs):
    """The device planes (layout reader P) hold, for every listed sequence,
    exactly the oracle's codes and scales (codes[b] = (k codes, k scales,
    v codes, v scales))."""
    def one(b):
        pages, slots = sequence_tokens(page_table[b], int(lens[b]))
        got = P.gather(pages, slots)
        for g, e, nm in zip(got, codes[b], ("k codes", "k scales", "v codes", "v scales")):
            if not np.array_equal(g, e):
                bad = np.argwhere(g != e)[:5]
                return f"seq {b}: {nm} differ at {bad.tolist()}"
        return None
    errs = [e for e in pmap(one, list(seqs)) if e]
    assert not errs, errs[:4]


def compare(got: np.ndarray, ref: np.ndarray, tol: float = TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    ratio = float((err / np.maximum(1.0, np.abs(ref))).max()) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)) if err.size else 0.0
    stats = {"max_abs": float(err.max()) if err.size else 0.0, "mixed": ratio, "rel_l2": rel_l2}
    return ratio <= tol and np.all(np.isfinite(got)), stats


# The decode path multiplies exact 16-bit operands; its rounding of note is
# that of the weights, P to FP16 (relative u = 2^-11 per weight).  The 4-bit
# formats use the rounded weights in the numerator and (on the matrix core) in
# the row sum alike, so a normalized weight becomes w_t (1 + e_t - e_bar) with
# |e| <= u, and an output moves by at most
# sum_t w_t (|e_t| + |e_bar|) |v_t| <= 2 u A with A = sum_t w_t |v_t|.  The
# check allows 3 u A, plus FP32 accumulation noise.
DECODE_P_BOUND = 3.0 * 2.0 ** -11


def check_decode(out, ref, mag, factor=1.0):
    """The 2e-2 gate plus the decode path's derived bound; returns stats."""
    ok, st = compare(out, ref)
    err = np.abs(np.asarray(out, np.float64) - ref)
    bound = 1e-5 * np.maximum(1.0, np.abs(ref)) + factor * DECODE_P_BOUND * mag
    st["worst_err_over_bound"] = float((err / bound).max()) if err.size else 0.0
    assert ok, st
    assert np.all(err <= bound), st
    return st


def calibrate(w: W.DecodeWorkload, oracle, data=None):
    """(s_tK, s_tV) over the whole K and V tensors of a workload, including
    the tokens its decode steps append, with the oracle's definition."""
    ka = va = 0.0
    for b in range(w.B):
        k, v = data[b] if data is not None else w.kv(b)
        ka = max(ka, oracle.abs_max(k))
        va = max(va, oracle.abs_max(v))
    for s in range(w.steps):
        k, v = w.append_kv(s)
        ka = max(ka, oracle.abs_max(k))
        va = max(va, oracle.abs_max(v))
    return oracle.tensor_scale_from_amax(ka), oracle.tensor_scale_from_amax(va)


class BuiltDecode:
    """A decode workload appended into a device cache, plus the oracle's
    logical codes for the sequences it may check."""

    def __init__(self, w: W.DecodeWorkload, oracle, keep=None, fill=0xA5, chunk=16, mse=False):
        self.w = w
        # mse: the cache is written with the MSE-searched block scale
        self._append = api.append_mse if mse else api.append
        self._quant = oracle.quantize_rows_mse if mse else oracle.quantize_rows
        self.keep = set(range(w.B)) if keep is None else set(keep)
        data = pmap(w.kv, range(w.B))
        # tensor scales: static calibration over the whole tensor (all
        # sequences plus the appended steps), with the oracle's definition
        self.s_tk, self.s_tv = calibrate(w, oracle, data)
        self.cache = api.KVCache(w.num_pages, w.Hkv, self.s_tk, self.s_tv, fill=fill)
        self.pt = i32(w.page_table)
        kept = sorted(self.keep)
        self.codes = dict(zip(kept, pmap(lambda b: (*self._quant(data[b][0], self.s_tk),
                                                    *self._quant(data[b][1], self.s_tv)), kept)))
        for b0 in range(0, w.B, chunk):
            ks, vs, seqs, poss = [], [], [], []
            for b in range(b0, min(w.B, b0 + chunk)):
                k, v = data[b]
                ks.append(k)
                vs.append(v)
                seqs.append(np.full(len(k), b, np.int32))
                poss.append(np.arange(len(k), dtype=np.int32))
            k = np.concatenate(ks)
            if len(k) == 0:
                continue
            self._append(self.cache, to_dev(k, w.dtype), to_dev(np.concatenate(vs), w.dtype),
                       i32(np.concatenate(seqs)), i32(np.concatenate(poss)), self.pt)
        del data
        self.lens = w.lens.copy()
        torch.cuda.synchronize()

    def append_step(self, step, oracle=None):
        w = self.w
        k, v = w.append_kv(step)
        pos = self.lens.copy()
        self._append(self.cache, to_dev(k, w.dtype), to_dev(v, w.dtype), i32(np.arange(w.B)), i32(pos), self.pt)
        if oracle is not None:
            for b in self.keep:
                kc, ksc = self._quant(k[b:b + 1], self.s_tk)
                vc, vsc = self._quant(v[b:b + 1], self.s_tv)
                c = self.codes[b]
                self.codes[b] = (np.concatenate([c[0], kc]), np.concatenate([c[1], ksc]),
                                 np.concatenate([c[2], vc]), np.concatenate([c[3], vsc]))
        self.lens += 1

    def decode(self, q: np.ndarray, num_splits=0, dtype=None):
        qd = to_dev(q, dtype or self.w.dtype)
        return api.decode(self.cache, qd, self.pt, i32(self.lens), int(self.lens.max()),
                          num_splits=num_splits)

    def oracle_decode(self, oracle, q: np.ndarray, seqs, scale=None):
        """(reference, magnitude): the oracle's output, and the same attention
        over |v| (codes with the sign bit cleared), i.e. A = sum_t w_t |v_t|."""
        seqs = list(seqs)
        codes = [self.codes[b] for b in seqs]
        ref = oracle.decode_batch(q[seqs], codes, self.w.Hkv, self.s_tk, self.s_tv, scale=scale)
        mag = oracle.decode_batch(q[seqs], [(c[0], c[1], c[2] & 7, c[3]) for c in codes], self.w.Hkv,
                                  self.s_tk, self.s_tv, scale=scale)
        return ref, mag

    def check_codes(self, seqs):
        """Bit-exact comparison of the device planes with the oracle's codes."""
        check_planes(planes(self.cache), self.w.page_table, self.lens, self.codes, seqs)


# ------------------------------------------------ comparison formats

class BuiltCmp:
    """A decode workload appended into an FP8 or BF16 comparison cache, plus
    the oracle's stored values for every sequence.  FP8 tensor scales come
    from the oracle's calibration over the whole tensor (steps included)."""

    def __init__(self, w: W.DecodeWorkload, oracle, fmt: int, fill=0xA5, chunk=16):
        from layout import CmpPlanes  # noqa: F401  (used by check_codes)
        self.w, self.fmt = w, fmt
        data = pmap(w.kv, range(w.B))
        if fmt == api.CMP_FP8:
            ka = max([oracle.abs_max(k) for k, _ in data] + [oracle.abs_max(w.append_kv(s)[0]) for s in range(w.steps)])
            va = max([oracle.abs_max(v) for _, v in data] + [oracle.abs_max(w.append_kv(s)[1]) for s in range(w.steps)])
            self.s_k = oracle.fp8_tensor_scale(np.array([ka], np.float32))
            self.s_v = oracle.fp8_tensor_scale(np.array([va], np.float32))
        else:
            self.s_k = self.s_v = 1.0
        self.cache = api.CmpCache(fmt, w.num_pages, w.Hkv, self.s_k, self.s_v, fill=fill)
        self.pt = i32(w.page_table)
        self.vals = {}
        for b0 in range(0, w.B, chunk):
            ks, vs, seqs, poss = [], [], [], []
            for b in range(b0, min(w.B, b0 + chunk)):
                k, v = data[b]
                ks.append(k)
                vs.append(v)
                seqs.append(np.full(len(k), b, np.int32))
                poss.append(np.arange(len(k), dtype=np.int32))
                self.vals[b] = (self.encode(oracle, k, self.s_k), self.encode(oracle, v, self.s_v))
            k = np.concatenate(ks)
            if len(k) == 0:
                continue
            api.cmp_append(self.cache, to_dev(k, w.dtype), to_dev(np.concatenate(vs), w.dtype),
                           i32(np.concatenate(seqs)), i32(np.concatenate(poss)), self.pt)
        self.lens = w.lens.copy()
        torch.cuda.synchronize()

    def encode(self, oracle, x, s):
        """The stored elements: FP8 codes, or bf16 bit patterns."""
        return oracle.fp8_codes(x, s) if self.fmt == api.CMP_FP8 else oracle.f32_to_bf16_bits(x)

    def values(self, oracle, enc, s):
        if self.fmt == api.CMP_FP8:
            return oracle.fp8_dequant(enc, s)
        return (enc.astype(np.uint32) << 16).view(np.float32)

    def append_step(self, step, oracle):
        w = self.w
        k, v = w.append_kv(step)
        api.cmp_append(self.cache, to_dev(k, w.dtype), to_dev(v, w.dtype), i32(np.arange(w.B)),
                       i32(self.lens.copy()), self.pt)
        for b in range(w.B):
            ek, ev = self.vals[b]
            self.vals[b] = (np.concatenate([ek, self.encode(oracle, k[b:b + 1], self.s_k)]),
                            np.concatenate([ev, self.encode(oracle, v[b:b + 1], self.s_v)]))
        self.lens += 1

    def check_codes(self, seqs):
        from layout import CmpPlanes
        torch.cuda.synchronize()
        R = CmpPlanes(self.cache.k.cpu().numpy(), self.cache.v.cpu().numpy(), self.w.num_pages, self.w.Hkv,
                      self.fmt)
        for b in seqs:
            pages, slots = sequence_tokens(self.w.page_table[b], int(self.lens[b]))
            gk, gv = R.gather(pages, slots)
            for g, e, nm in ((gk, self.vals[b][0], "k"), (gv, self.vals[b][1], "v")):
                if not np.array_equal(g, e):
                    bad = np.argwhere(g != e)[:5]
                    raise AssertionError(f"seq {b}: {nm} differ at {bad.tolist()}")

    def decode(self, q: np.ndarray, num_splits=0, dtype=None):
        qd = to_dev(q, dtype or self.w.dtype)
        return api.cmp_decode(self.cache, qd, self.pt, i32(self.lens), int(self.lens.max()),
                              num_splits=num_splits)

    def oracle_decode(self, oracle, q: np.ndarray, seqs, scale=None):
        """(reference, magnitude) as in BuiltDecode, over the stored values."""
        seqs = list(seqs)
        kv = [(self.values(oracle, self.vals[b][0], self.s_k), self.values(oracle, self.vals[b][1], self.s_v))
              for b in seqs]
        ref = oracle.decode_batch_dense(q[seqs], kv, self.w.Hkv, scale=scale)
        mag = oracle.decode_batch_dense(q[seqs], [(k, np.abs(v)) for k, v in kv], self.w.Hkv, scale=scale)
        return ref, mag


# ------------------------------------------------------------------ MXFP4

def mx_exp_offset(amax: float) -> int:
    """floor(log2(amax)) - 10 (the offset the header states)."""
    return math.frexp(amax)[1] - 1 - 10 if amax > 0 else 0


class BuiltMx:
    """A decode workload appended into an MXFP4 cache, plus the oracle's
    codes and scales for every sequence.  The exp offsets come from the
    whole tensor's amax (steps included)."""

    def __init__(self, w: W.DecodeWorkload, oracle, fill=0xA5, chunk=16, keep=None):
        self.w = w
        self.keep = set(range(w.B)) if keep is None else set(keep)
        data = pmap(w.kv, range(w.B))
        ka = max([oracle.abs_max(k) for k, _ in data] + [oracle.abs_max(w.append_kv(s)[0]) for s in range(w.steps)])
        va = max([oracle.abs_max(v) for _, v in data] + [oracle.abs_max(w.append_kv(s)[1]) for s in range(w.steps)])
        self.k_exp, self.v_exp = mx_exp_offset(ka), mx_exp_offset(va)
        self.cache = api.MxCache(w.num_pages, w.Hkv, self.k_exp, self.v_exp, fill=fill)
        self.pt = i32(w.page_table)
        kept = sorted(self.keep)
        self.codes = dict(zip(kept, pmap(lambda b: (*oracle.mx_quantize_rows(data[b][0]),
                                                    *oracle.mx_quantize_rows(data[b][1])), kept)))
        for b0 in range(0, w.B, chunk):
            ks, vs, seqs, poss = [], [], [], []
            for b in range(b0, min(w.B, b0 + chunk)):
                k, v = data[b]
                ks.append(k)
                vs.append(v)
                seqs.append(np.full(len(k), b, np.int32))
                poss.append(np.arange(len(k), dtype=np.int32))
            k = np.concatenate(ks)
            if len(k) == 0:
                continue
            api.mx_append(self.cache, to_dev(k, w.dtype), to_dev(np.concatenate(vs), w.dtype),
                          i32(np.concatenate(seqs)), i32(np.concatenate(poss)), self.pt)
        self.lens = w.lens.copy()
        torch.cuda.synchronize()

    def append_step(self, step, oracle):
        w = self.w
        k, v = w.append_kv(step)
        api.mx_append(self.cache, to_dev(k, w.dtype), to_dev(v, w.dtype), i32(np.arange(w.B)),
                      i32(self.lens.copy()), self.pt)
        for b in self.keep:
            c = self.codes[b]
            kc, ksc = oracle.mx_quantize_rows(k[b:b + 1])
            vc, vsc = oracle.mx_quantize_rows(v[b:b + 1])
            self.codes[b] = (np.concatenate([c[0], kc]), np.concatenate([c[1], ksc]),
                             np.concatenate([c[2], vc]), np.concatenate([c[3], vsc]))
        self.lens += 1

    def check_codes(self, seqs):
        check_planes(planes(self.cache), self.w.page_table, self.lens, self.codes, seqs)

    def decode(self, q: np.ndarray, num_splits=0, dtype=None):
        qd = to_dev(q, dtype or self.w.dtype)
        return api.mx_decode(self.cache, qd, self.pt, i32(self.lens), int(self.lens.max()), num_splits=num_splits)

    def oracle_decode(self, oracle, q: np.ndarray, seqs, scale=None):
        """(reference, magnitude) as in BuiltDecode, over the MXFP4 values."""
        seqs = list(seqs)
        kv = [(oracle.mx_dequant_rows(self.codes[b][0], self.codes[b][1]),
               oracle.mx_dequant_rows(self.codes[b][2], self.codes[b][3])) for b in seqs]
        ref = oracle.decode_batch_dense(q[seqs], kv, self.w.Hkv, scale=scale)
        mag = oracle.decode_batch_dense(q[seqs], [(k, np.abs(v)) for k, v in kv], self.w.Hkv, scale=scale)
        return ref, mag
