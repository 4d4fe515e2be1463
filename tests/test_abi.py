"""The C-ABI library: it builds, loads, exports every declared entry point,
and rejects bad arguments on the host before touching the device.  Also the
byte-count pins of the format.  CPU only: no call here reaches a kernel."""
import ctypes
import json
import math
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4kv.h")
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "format_facts.json")))


@pytest.fixture(scope="module")
def api():
    from decode_attention_nvfp4_amd import api, build
    if not os.path.exists(build.LIB):
        build.build()
    api.lib()
    return api


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("nvfp4_kv_append", "nvfp4_kv_dequant", "nvfp4_decode_attn", "nvfp4_prefill_attn"):
        assert n in names


def test_library_exports_every_declared_symbol(api):
    from decode_attention_nvfp4_amd import build
    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (nvfp4_[a-z0-9_]+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    assert set(api.EXPORTS) == set(declared_functions())


def test_status_strings(api):
    L = api.lib()
    for code, word in ((0, b"ok"), (1, b"invalid"), (2, b"unsupported"), (3, b"workspace"), (4, b"HIP")):
        assert word in L.nvfp4_status_string(code)


def _fake_cache(api, **kw):
    c = api.CacheStruct(0x10000, 0x20000, 0x30000, 0x40000, 0.01, 0.02, 64, 8, 16, 128)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


FAKE = ctypes.c_void_p(0x50000)


def _append(api, cache, dtype=1, n_tok=4, max_pages=8, ptrs=True, name="nvfp4_kv_append"):
    p = FAKE if ptrs else None
    return getattr(api.lib(), name)(ctypes.byref(cache), p, p, dtype, n_tok, p, p, p, max_pages, None)


@pytest.mark.parametrize("name", ["nvfp4_kv_append", "nvfp4_kv_append_mse"])
def test_append_rejects_bad_arguments(api, name):
    L = api.lib()
    assert getattr(L, name)(None, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, None) == 1

    def ap(cache, **kw):
        return _append(api, cache, name=name, **kw)
    assert ap(_fake_cache(api, head_dim=64)) == 2
    assert ap(_fake_cache(api, page_size=32)) == 2
    assert ap(_fake_cache(api, k_tensor_scale=0.0)) == 1
    assert ap(_fake_cache(api, v_tensor_scale=-1.0)) == 1
    assert ap(_fake_cache(api, k_tensor_scale=float("nan"))) == 1
    assert ap(_fake_cache(api, k_tensor_scale=float("inf"))) == 1
    assert ap(_fake_cache(api, k_codes=0x10008)) == 1        # misaligned plane
    assert ap(_fake_cache(api, v_scales=None)) == 1
    assert ap(_fake_cache(api, num_pages=0)) == 1
    assert ap(_fake_cache(api), dtype=7) == 2
    assert ap(_fake_cache(api), n_tok=-1) == 1
    assert ap(_fake_cache(api), max_pages=0) == 1
    assert ap(_fake_cache(api), ptrs=False) == 1
    assert ap(_fake_cache(api), n_tok=0, ptrs=False) == 0     # empty append: no-op


def test_to_fp8_rejects_bad_arguments(api):
    L = api.lib()

    def tf(n=64, g=100.0, s8=0.06, codes=FAKE, scales=FAKE, out=FAKE):
        return L.nvfp4_to_fp8(codes, scales, n, g, s8, out, None)
    assert tf(n=-16) == 1
    assert tf(n=40) == 1
    assert tf(g=0.0) == 1
    assert tf(g=float("nan")) == 1
    assert tf(s8=float("inf")) == 1
    assert tf(s8=-1.0) == 1
    assert tf(codes=None) == 1
    assert tf(scales=None) == 1
    assert tf(codes=ctypes.c_void_p(0x50008)) == 1        # misaligned
    assert tf(out=ctypes.c_void_p(0x50004)) == 1
    assert tf(n=0, codes=None, scales=None, out=None) == 0
    assert tf(n=40) == 1 and b"multiple of 16" in L.nvfp4_last_error()


def test_mx_sizes_offsets_and_bad_arguments(api):
    L = api.lib()
    assert api.mx_plane_bytes(10, 8, 0) == 10 * 8 * 1024
    assert api.mx_plane_bytes(10, 8, 1) == 10 * 8 * 64
    assert api.mx_plane_bytes(10, 8, 4) == 0 and api.mx_plane_bytes(0, 8, 0) == 0
    # K + V per (token, head): 2 * (64 + 4) bytes, 0.53125 per element
    per = sum(api.mx_plane_bytes(1, 1, p) for p in range(4)) / 16
    assert per == 136 and per / 256 == 0.53125
    assert api.mx_exp_offset_from_amax(1.0) == -10
    assert api.mx_exp_offset_from_amax(1000.0) == 9 - 10
    assert api.mx_exp_offset_from_amax(0.0) == 0 and api.mx_exp_offset_from_amax(float("nan")) == 0

    def mx(**kw):
        c = api.MxCacheStruct(0x10000, 0x20000, 0x30000, 0x40000, -3, 2, 64, 8, 16, 128)
        for k, v in kw.items():
            setattr(c, k, v)
        return c
    p = FAKE
    assert L.nvfp4_mx_append(ctypes.byref(mx(head_dim=64)), p, p, 1, 4, p, p, p, 8, None) == 2
    assert L.nvfp4_mx_append(ctypes.byref(mx(k_exp_offset=-127)), p, p, 1, 4, p, p, p, 8, None) == 1
    assert L.nvfp4_mx_append(ctypes.byref(mx(v_scales=0x40008)), p, p, 1, 4, p, p, p, 8, None) == 1
    assert L.nvfp4_mx_append(ctypes.byref(mx()), p, p, 5, 4, p, p, p, 8, None) == 2
    assert L.nvfp4_mx_append(ctypes.byref(mx()), None, None, 1, 0, None, None, None, 8, None) == 0
    c = mx()
    assert L.nvfp4_mx_decode_attn(ctypes.byref(c), FAKE, 1, 2, 12, FAKE, 64, FAKE, 1000, 0.088, 0,
                                  FAKE, 1 << 30, FAKE, None) == 1          # 12 heads over 8 KV heads
    assert L.nvfp4_mx_decode_attn(ctypes.byref(c), FAKE, 1, 2, 32, FAKE, 64, FAKE, 1000, 0.088, 4,
                                  None, 0, FAKE, None) == 3
    assert api.mx_decode_workspace_bytes(2, 32, 8, 1000, 4) == api.decode_workspace_bytes(2, 32, 8, 1000, 4)

    # MXFP4 prefill: the nvfp4_prefill_attn checks; the workspace holds V~
    # only (half of the FP8 path's)
    def mpf(T=16, Hq=64, prefix=100, ws=FAKE, ws_bytes=1 << 30, q_dtype=1, cache=c):
        return L.nvfp4_mx_prefill_attn(ctypes.byref(cache), FAKE, q_dtype, T, Hq, FAKE, prefix, 1, 0.088, ws,
                                       ws_bytes, FAKE, None)
    assert mpf(Hq=60) == 1
    assert mpf(T=-1) == 1
    assert mpf(q_dtype=9) == 2
    assert mpf(ws=None, ws_bytes=0) == 3
    assert mpf(ws_bytes=100) == 3
    assert mpf(cache=mx(page_size=8)) == 2
    assert mpf(cache=mx(v_exp_offset=128)) == 1
    assert mpf(T=0) == 0
    assert L.nvfp4_mx_prefill_attn(ctypes.byref(c), FAKE, 1, 16, 64, FAKE, 100, 1, float("nan"), FAKE, 1 << 30,
                                   FAKE, None) == 1
    assert 2 * api.mx_prefill_workspace_bytes(2048, 64, 8, 32768) == api.prefill_workspace_bytes(2048, 64, 8, 32768, 0)
    assert api.mx_prefill_workspace_bytes(16, 8, 0, 10) == 0


def test_gather_probe_rejects_bad_arguments(api):
    L = api.lib()
    c = _fake_cache(api)

    def gp(B=2, maxp=64, max_len=1000, S=4, sink=FAKE, sink_bytes=1 << 20, cache=c):
        return L.nvfp4_decode_gather_probe(ctypes.byref(cache), B, FAKE, maxp, FAKE, max_len, S, sink, sink_bytes,
                                           None)
    assert gp(B=-1) == 1
    assert gp(S=-1) == 1
    assert gp(maxp=0) == 1
    assert gp(max_len=1025, maxp=64) == 1          # 65 pages > 64 per row
    assert gp(sink=None) == 1
    assert gp(sink_bytes=4 * 64 * 4 - 1) == 3      # 4 waves need 4 x 64 words
    assert gp(cache=_fake_cache(api, head_dim=64)) == 2
    assert gp(B=0, sink=None) == 0


def test_dequant_rejects_bad_arguments(api):
    L = api.lib()
    c = _fake_cache(api)
    assert L.nvfp4_kv_dequant(ctypes.byref(c), FAKE, -1, 4, FAKE, FAKE, 0, None) == 1
    assert L.nvfp4_kv_dequant(ctypes.byref(c), FAKE, 0, 4, FAKE, FAKE, 3, None) == 2
    assert L.nvfp4_kv_dequant(ctypes.byref(c), None, 0, 4, FAKE, FAKE, 0, None) == 1
    assert L.nvfp4_kv_dequant(ctypes.byref(c), FAKE, 0, 4, ctypes.c_void_p(0x50004), None, 0, None) == 1
    assert L.nvfp4_kv_dequant(ctypes.byref(c), None, 0, 0, None, None, 0, None) == 0


def _decode(api, cache, q_dtype=1, B=2, Hq=32, max_pages=64, max_len=1000, scale=0.088,
            splits=0, ws=FAKE, ws_bytes=1 << 30):
    return api.lib().nvfp4_decode_attn(ctypes.byref(cache), FAKE, q_dtype, B, Hq, FAKE, max_pages, FAKE,
                                       max_len, scale, splits, ws, ws_bytes, FAKE, None)


def test_decode_rejects_bad_arguments(api):
    c = _fake_cache(api)
    assert _decode(api, _fake_cache(api, head_dim=256)) == 2
    assert _decode(api, c, q_dtype=5) == 2
    assert _decode(api, c, Hq=12) == 1                  # not a multiple of Hkv = 8
    assert _decode(api, c, Hq=8 * 17) == 2              # more than 16 heads per KV head
    assert _decode(api, c, max_pages=10, max_len=1000) == 1
    assert _decode(api, c, scale=0.0) == 1
    assert _decode(api, c, scale=float("nan")) == 1
    assert _decode(api, c, B=-1) == 1
    assert _decode(api, c, splits=-2) == 1
    assert _decode(api, c, splits=4, ws=None, ws_bytes=0) == 3
    assert _decode(api, c, splits=4, ws_bytes=16) == 3
    assert _decode(api, c, splits=4, ws=ctypes.c_void_p(0x50010)) == 1   # workspace alignment
    assert _decode(api, c, B=0) == 0                    # empty batch: no-op


def test_decode_noalloc_rejects_bad_arguments_and_oversized_requests(api):
    """The no-allocation decode validates like nvfp4_decode_attn and refuses,
    before touching the device, a split whose partials exceed its fixed
    scratch (9000 waves x 2 pieces x 16 heads x 516 B > 40 MiB)."""
    L = api.lib()
    c = _fake_cache(api)

    def call(cache, B=2, Hq=32, max_pages=64, max_len=1000, scale=0.088, splits=0):
        return L.nvfp4_decode_attn_noalloc(ctypes.byref(cache), FAKE, 1, B, Hq, FAKE, max_pages, FAKE,
                                           max_len, scale, splits, FAKE, None)

    assert call(_fake_cache(api, head_dim=256)) == 2
    assert call(c, Hq=12) == 1
    assert call(c, scale=0.0) == 1
    assert call(c, B=0) == 0
    assert api.decode_workspace_bytes(2, 8 * 16, 8, 1000, 9000) > api.NOALLOC_SCRATCH_BYTES
    assert call(c, Hq=8 * 16, splits=9000) == 3
    assert b"fixed scratch" in L.nvfp4_last_error()


def test_prefill_rejects_bad_arguments(api):
    L = api.lib()
    c = _fake_cache(api)

    def pf(T=16, Hq=64, prefix=100, ws=FAKE, ws_bytes=1 << 30, q_dtype=1, cache=c, mode=0):
        return L.nvfp4_prefill_attn(ctypes.byref(cache), FAKE, q_dtype, T, Hq, FAKE, prefix, 1, mode, 0.088,
                                    ws, ws_bytes, FAKE, None)
    assert pf(Hq=60) == 1
    assert pf(T=-1) == 1
    assert pf(prefix=-5) == 1
    assert pf(q_dtype=9) == 2
    assert pf(ws=None, ws_bytes=0) == 3
    assert pf(ws_bytes=100) == 3
    assert pf(cache=_fake_cache(api, page_size=8)) == 2
    assert pf(mode=2) == 2
    assert pf(T=0) == 0
    # F16 operands need twice the FP8 workspace
    assert api.prefill_workspace_bytes(2048, 64, 8, 32768, 1) == 2 * api.prefill_workspace_bytes(2048, 64, 8, 32768, 0)
    assert api.prefill_workspace_bytes(16, 8, 2, 10, 5) == 0


def test_split_planner_and_workspace(api):
    """The decode work plan: W waves share the (sequence, KV head, page) work
    in equal contiguous ranges.  A requested W is used as given; 0 asks for
    one wave per resident wave slot of the device."""
    for B, Hkv, L in ((1, 1, 1024), (8, 8, 4097), (1, 8, 65536), (128, 8, 8192), (3, 2, 0), (4, 4, 17)):
        auto = api.decode_num_splits(B, Hkv, L, 0)
        units = B * Hkv * -(-L // 16)
        # at least 16 pages per wave, or for work that gives fewer than one
        # such wave per SIMD (4 x 256), up to one wave per SIMD with at least
        # 2 pages each; at most 128 waves per segment (but not below the CU
        # count) and 8 waves per CU
        want = -(-units // 16)
        if want < 4 * 256:
            want = min(4 * 256, -(-units // 2))
        want = min(want, max(256, 128 * B * Hkv))
        want = max(1, min(8 * 256, want))
        # a full launch (two waves per SIMD) gets 1024 small tail ranges that
        # the dispatcher hands to the first free slots
        assert auto == (want + 1024 if want == 2 * 4 * 256 else want)
        for req in (1, 2, 7, 64):
            assert api.decode_num_splits(B, Hkv, L, req) == req
        for G in (1, 4, 8):
            for req in (1, 7, 0):
                W = req or auto
                ws = api.decode_workspace_bytes(B, G * Hkv, Hkv, L, req)
                # two partial (o, lse) slots per wave and head, plus B + 1 prefix entries
                assert ws >= W * 2 * G * 129 * 4 + (B + 1) * 4
                assert ws % 256 == 0
    assert api.decode_num_splits(0, 8, 1024, 0) == 0
    assert api.decode_workspace_bytes(1, 6, 4, 1024, 0) == 0     # 6 % 4 != 0


def test_memory_footprint_matches_page_claims(api):
    """0.5625 bytes per element: 3.56x below FP16 (the page's "3.5x", ~71%)
    and 1.78x below FP8 (the page's "about 1.8x")."""
    facts = GOLD["memory_reduction"]
    for pages, hkv in ((1, 1), (64, 8), (2176, 8)):
        nbytes = api.kv_cache_bytes(pages, hkv)
        elems = 2 * pages * 16 * hkv * 128             # K and V
        assert nbytes == elems * 0.5625
        # the page's KV-memory formula, one layer: 2 * L * n_h * d_h * s * b * sizeof
        assert nbytes == 2 * 1 * hkv * 128 * (pages * 16) * 1 * 0.5625
    per = api.kv_cache_bytes(1, 1) / (2 * 16 * 128)
    vs16, vs8 = 2.0 / per, 1.0 / per
    assert abs(vs16 - facts["vs_fp16_factor"]) < 0.1
    assert abs(vs8 - facts["vs_fp8_factor"]) < 0.05
    assert abs(100 * (1 - per / 2.0) - facts["vs_fp16_percent"]) < 1.0
    # "about 50%" vs FP8 is a rounded headline: the format gives 43.75%
    assert abs(100 * (1 - per / 1.0) - facts["vs_fp8_percent"]) < 7.0
    for p in range(4):
        assert api.plane_bytes(3, 2, p) == 3 * 2 * (1024 if p in (0, 2) else 128)
    assert api.plane_bytes(3, 2, 4) == 0 and api.kv_cache_bytes(0, 2) == 0


def test_tensor_scale_matches_oracle(api, orc):
    from decode_attention_nvfp4_amd import workloads
    for seed in range(5):
        x = workloads.random_rows(seed, 50, "mixed")
        amax = float(np.abs(x).max())
        assert api.tensor_scale_from_amax(amax) == orc.tensor_scale(x)
    assert api.tensor_scale_from_amax(0.0) == 0.0
    assert api.tensor_scale_from_amax(float("inf")) == 0.0


def test_binding_refuses_host_tensors(api):
    import torch
    cache = type("C", (), {"num_kv_heads": 8})()
    with pytest.raises(ValueError):
        api.append(cache, torch.zeros(2, 8, 128), torch.zeros(2, 8, 128), torch.zeros(2, dtype=torch.int32),
                   torch.zeros(2, dtype=torch.int32), torch.zeros(1, 4, dtype=torch.int32))


# --------------------------------------------------- comparison KV formats

def _fake_cmp(api, **kw):
    c = api.CmpCacheStruct(0x10000, 0x20000, 0.01, 0.02, api.CMP_FP8, 64, 8, 16, 128)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_cmp_sizes_and_fp8_scale(api):
    L = api.lib()
    # 1 byte (FP8) or 2 bytes (BF16) per element, 16 tokens x 128 per (page, head)
    assert L.nvfp4_cmp_plane_bytes(10, 8, api.CMP_FP8) == 10 * 8 * 16 * 128
    assert L.nvfp4_cmp_plane_bytes(10, 8, api.CMP_BF16) == 2 * 10 * 8 * 16 * 128
    assert L.nvfp4_cmp_plane_bytes(10, 8, 0) == 0 and L.nvfp4_cmp_plane_bytes(0, 8, 1) == 0
    # NVFP4 against the comparison formats: 0.5625 vs 1 vs 2 bytes per element
    nv = L.nvfp4_kv_cache_bytes(10, 8)
    assert 2 * L.nvfp4_cmp_plane_bytes(10, 8, api.CMP_FP8) / nv == pytest.approx(1 / 0.5625)
    assert 2 * L.nvfp4_cmp_plane_bytes(10, 8, api.CMP_BF16) / nv == pytest.approx(2 / 0.5625)
    assert L.nvfp4_cmp_fp8_scale_from_amax(448.0) == 1.0
    assert L.nvfp4_cmp_fp8_scale_from_amax(3.0) == np.float32(3.0) / np.float32(448.0)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert L.nvfp4_cmp_fp8_scale_from_amax(bad) == 0.0


def test_cmp_append_and_decode_reject_bad_arguments(api):
    L = api.lib()

    def app(c, dtype=1, n_tok=4, ptrs=True):
        p = FAKE if ptrs else None
        return L.nvfp4_cmp_append(ctypes.byref(c), p, p, dtype, n_tok, p, p, p, 8, None)

    def dec(c, q_dtype=1, Hq=32, ws=FAKE, ws_bytes=1 << 30, splits=4, B=2):
        return L.nvfp4_cmp_decode_attn(ctypes.byref(c), FAKE, q_dtype, B, Hq, FAKE, 64, FAKE, 1000, 0.088,
                                       splits, ws, ws_bytes, FAKE, None)

    assert L.nvfp4_cmp_append(None, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 8, None) == 1
    assert app(_fake_cmp(api, format=0)) == 2
    assert app(_fake_cmp(api, format=3)) == 2
    assert app(_fake_cmp(api, head_dim=64)) == 2
    assert app(_fake_cmp(api, k=0x10008)) == 1                  # misaligned plane
    assert app(_fake_cmp(api, v=None)) == 1
    assert app(_fake_cmp(api, k_scale=0.0)) == 1                 # FP8 needs scales
    assert app(_fake_cmp(api, format=api.CMP_BF16, k_scale=0.0, v_scale=0.0), n_tok=0) == 0
    assert app(_fake_cmp(api), dtype=9) == 2
    assert app(_fake_cmp(api), ptrs=False) == 1
    assert app(_fake_cmp(api), n_tok=0, ptrs=False) == 0
    c = _fake_cmp(api)
    assert dec(_fake_cmp(api, format=5)) == 2
    assert dec(c, q_dtype=4) == 2
    assert dec(c, Hq=12) == 1
    assert dec(c, ws=None, ws_bytes=0) == 3
    assert dec(c, ws=ctypes.c_void_p(0x50010)) == 1
    assert dec(c, B=0) == 0
    assert L.nvfp4_cmp_decode_workspace_bytes(0, 2, 32, 8, 1000, 0) == 0
    assert L.nvfp4_cmp_decode_workspace_bytes(api.CMP_FP8, 2, 32, 8, 1000, 4) == \
        L.nvfp4_decode_workspace_bytes(2, 32, 8, 1000, 4)
