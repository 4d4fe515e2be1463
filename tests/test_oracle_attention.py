"""Pins for the oracle's attention over a dequantized cache (CPU only).

The oracle is checked against PyTorch's float64 softmax attention (a library
routine used as a second opinion) on small shapes, and against closed-form
special cases: one key, zero query, a dominant key, the first causal row and
the empty context.
"""
import numpy as np
import pytest
import torch

from decode_attention_nvfp4_amd import workloads

D = 128


def _cache(orc, L, Hkv, seed, dist="normal"):
    k = workloads.random_rows(seed, L * Hkv, dist).reshape(L, Hkv, D)
    v = workloads.random_rows(seed + 1000, L * Hkv, dist).reshape(L, Hkv, D)
    stk, stv = orc.tensor_scale(k), orc.tensor_scale(v)
    kc, ks = orc.quantize_rows(k, stk)
    vc, vs = orc.quantize_rows(v, stv)
    return kc, ks, stk, vc, vs, stv


def _torch_attention(q, kh, vh, Hkv, scale, causal_offset=None):
    """float64 softmax attention; q [n][Hq][D], kh/vh [L][Hkv][D]."""
    q = torch.from_numpy(q.astype(np.float64))
    kh = torch.from_numpy(kh.astype(np.float64))
    vh = torch.from_numpy(vh.astype(np.float64))
    n, Hq, _ = q.shape
    G = Hq // Hkv
    k = kh.repeat_interleave(G, dim=1).permute(1, 0, 2)     # [Hq][L][D]
    v = vh.repeat_interleave(G, dim=1).permute(1, 0, 2)
    s = torch.einsum("nhd,hld->hnl", q, k) * scale
    if causal_offset is not None:
        L = kh.shape[0]
        pos = torch.arange(n)[:, None] + causal_offset
        mask = torch.arange(L)[None, :] > pos
        s = s.masked_fill(mask[None], float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.einsum("hnl,hld->nhd", p, v).numpy()


@pytest.mark.parametrize("L,Hq,Hkv", [(1, 4, 1), (5, 8, 2), (37, 8, 2), (300, 4, 4), (129, 16, 2)])
def test_attend_matches_torch_float64(orc, L, Hq, Hkv):
    kc, ks, stk, vc, vs, stv = _cache(orc, L, Hkv, seed=L)
    q = workloads.random_rows(L + 77, Hq)
    out = orc.attend(q, Hkv, kc, ks, stk, vc, vs, stv)
    kh = orc.dequant_rows(kc, ks, stk)
    vh = orc.dequant_rows(vc, vs, stv)
    ref = _torch_attention(q[None], kh, vh, Hkv, 1.0 / np.sqrt(D))[0]
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_attend_outlier_channels_matches_torch(orc):
    L, Hq, Hkv = 200, 8, 2
    kc, ks, stk, vc, vs, stv = _cache(orc, L, Hkv, seed=3, dist="outlier")
    q = workloads.random_rows(99, Hq)
    out = orc.attend(q, Hkv, kc, ks, stk, vc, vs, stv, scale=0.3)
    ref = _torch_attention(q[None], orc.dequant_rows(kc, ks, stk), orc.dequant_rows(vc, vs, stv),
                           Hkv, 0.3)[0]
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_single_key_returns_its_value(orc):
    kc, ks, stk, vc, vs, stv = _cache(orc, 1, 2, seed=8)
    q = workloads.random_rows(1, 4)
    out = orc.attend(q, 2, kc, ks, stk, vc, vs, stv)
    vh = orc.dequant_rows(vc, vs, stv)
    for h in range(4):
        assert np.array_equal(out[h], vh[0, h // 2])


def test_zero_query_averages_values(orc):
    L = 50
    kc, ks, stk, vc, vs, stv = _cache(orc, L, 1, seed=9)
    out = orc.attend(np.zeros((2, D), np.float32), 1, kc, ks, stk, vc, vs, stv)
    vh = orc.dequant_rows(vc, vs, stv).astype(np.float64)
    np.testing.assert_allclose(out[0], vh[:, 0].mean(axis=0), rtol=1e-6, atol=1e-7)


def test_dominant_key_selects_its_value(orc):
    L = 64
    kc, ks, stk, vc, vs, stv = _cache(orc, L, 1, seed=10)
    kh = orc.dequant_rows(kc, ks, stk)
    vh = orc.dequant_rows(vc, vs, stv)
    j = 17
    q = (kh[j, 0] * 50.0).astype(np.float32)[None]
    out = orc.attend(q, 1, kc, ks, stk, vc, vs, stv)
    np.testing.assert_allclose(out[0], vh[j, 0], rtol=1e-5, atol=1e-5)


def test_empty_context_gives_zeros(orc):
    out = orc.attend(np.ones((4, D), np.float32), 2, np.zeros((0, 2, D), np.uint8),
                     np.zeros((0, 2, 8), np.uint8), 1.0, np.zeros((0, 2, D), np.uint8),
                     np.zeros((0, 2, 8), np.uint8), 1.0)
    assert np.all(out == 0)


def test_prefill_rows_match_torch_causal(orc):
    prefix, T, Hq, Hkv = 40, 24, 4, 2
    kc, ks, stk, vc, vs, stv = _cache(orc, prefix + T, Hkv, seed=11)
    q = workloads.random_rows(12, T * Hq).reshape(T, Hq, D)
    rows = np.arange(T)
    out = orc.prefill_rows(q, rows, Hkv, kc, ks, stk, vc, vs, stv, prefix)
    ref = _torch_attention(q, orc.dequant_rows(kc, ks, stk), orc.dequant_rows(vc, vs, stv), Hkv,
                           1.0 / np.sqrt(D), causal_offset=prefix)
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_first_causal_row_without_prefix_is_first_value(orc):
    kc, ks, stk, vc, vs, stv = _cache(orc, 16, 2, seed=13)
    q = workloads.random_rows(14, 3 * 4).reshape(3, 4, D)
    out = orc.prefill_rows(q[:1], [0], 2, kc, ks, stk, vc, vs, stv, prefix=0)
    vh = orc.dequant_rows(vc, vs, stv)
    for h in range(4):
        assert np.array_equal(out[0, h], vh[0, h // 2])


def test_decode_batch_threads_match_serial(orc):
    Hkv, Hq = 2, 4
    seqs = [_cache(orc, L, Hkv, seed=20 + L) for L in (3, 0, 40)]
    q = workloads.random_rows(5, 3 * Hq).reshape(3, Hq, D)
    # different tensor scales per sequence are not used by the batch API, so
    # requantize all three with one pair of scales
    stk, stv = 0.01, 0.02
    packed = []
    for kc, ks, _, vc, vs, _ in seqs:
        kh = orc.dequant_rows(kc, ks, seqs[0][2]) if kc.size else np.zeros((0, Hkv, D), np.float32)
        vh = orc.dequant_rows(vc, vs, seqs[0][5]) if vc.size else np.zeros((0, Hkv, D), np.float32)
        k2 = orc.quantize_rows(kh, stk)
        v2 = orc.quantize_rows(vh, stv)
        packed.append((k2[0], k2[1], v2[0], v2[1]))
    out = orc.decode_batch(q, packed, Hkv, stk, stv, threads=3)
    for b in range(3):
        ref = orc.attend(q[b], Hkv, packed[b][0], packed[b][1], stk, packed[b][2], packed[b][3], stv)
        assert np.array_equal(out[b], ref)
