"""Pins for the oracle's comparison KV formats (FP8 E4M3 with a tensor scale,
and BF16), CPU only.

The FP8 codes are tied to PyTorch's float8_e4m3fn cast (a library
round-to-nearest-even encoder) inside the finite range and to the stated
saturation outside it; the FP8 values to PyTorch's float8 decoder; the dense
attention to closed forms and to a float64 PyTorch softmax.
"""
import math

import numpy as np
import pytest
import torch

from decode_attention_nvfp4_amd import workloads

D = 128


def _e4m3_values():
    """The 127 finite non-negative E4M3FN values, from PyTorch's decoder."""
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def _torch_codes(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_fp8_codes_match_torch_on_values_midpoints_and_neighbours(orc):
    vals = _e4m3_values().astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (vals[:-1].astype(np.float64) + vals[1:]) / 2)
    pts = np.concatenate([vals, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    pts = pts[np.abs(pts) <= 448]
    np.testing.assert_array_equal(orc.fp8_codes(pts, 1.0), _torch_codes(pts))


def test_fp8_codes_match_torch_random_with_tensor_scale(orc):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-12, 4, 200000))).astype(np.float32)
    s_t = orc.fp8_tensor_scale(x)
    v = (x / np.float32(s_t)).astype(np.float32)       # the FP32 quotient (IEEE division)
    assert np.all(np.abs(v) <= 448.0)
    np.testing.assert_array_equal(orc.fp8_codes(x, s_t), _torch_codes(v))


def test_fp8_tensor_scale_maps_amax_to_448(orc):
    x = np.array([0.5, -3.0, 2.0], np.float32)
    s = orc.fp8_tensor_scale(x)
    assert s == np.float32(3.0) / np.float32(448.0)
    assert orc.fp8_code(-3.0, s) == 0xFE and orc.fp8_code(3.0, s) == 0x7E


@pytest.mark.parametrize("v", [464.0, 465.0, 500.0, 1e6, 3e38])
def test_fp8_saturates_at_448(orc, v):
    # above the finite range the stated rule clamps to 448 (PyTorch's cast
    # gives NaN there, so the pin is the rule itself)
    assert orc.fp8_code(v, 1.0) == 0x7E
    assert orc.fp8_code(-v, 1.0) == 0xFE


def test_fp8_signed_zero_and_underflow(orc):
    assert orc.fp8_code(0.0, 1.0) == 0x00
    assert orc.fp8_code(-0.0, 1.0) == 0x80
    smallest = 2.0 ** -9                                 # E4M3 subnormal step
    assert orc.fp8_code(smallest * 0.5, 1.0) == 0x00     # tie with 0: even code 0
    assert orc.fp8_code(smallest * 0.5000001, 1.0) == 0x01
    assert orc.fp8_code(-smallest * 1.5, 1.0) == 0x82    # tie 1 / 2: even code 2


def test_fp8_values_match_torch_decoder(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = orc.fp8_dequant(codes, 1.0)
    np.testing.assert_array_equal(got, ref)
    assert np.signbit(got[codes == 0x80]).all()
    # with a tensor scale: one rounding of the exact product
    s = np.float32(0.0371)
    got_s = orc.fp8_dequant(codes, float(s))
    np.testing.assert_array_equal(got_s, (ref.astype(np.float64) * float(s)).astype(np.float32))


def test_fp8_round_trip_error_bound(orc):
    # |x - dequant(code(x))| <= half an E4M3 step: 2^-4 relative for normals,
    # 2^-10 * s_t absolute in the subnormal range
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(50000) * 10).astype(np.float32)
    s = orc.fp8_tensor_scale(x)
    xh = orc.fp8_dequant(orc.fp8_codes(x, s), s).astype(np.float64)
    err = np.abs(xh - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(err <= bound)


# ------------------------------------------------------------ dense attention

def _torch_attention(q, kh, vh, Hkv, scale):
    q = torch.from_numpy(np.asarray(q, np.float64))
    k = torch.from_numpy(np.asarray(kh, np.float64))
    v = torch.from_numpy(np.asarray(vh, np.float64))
    G = q.shape[0] // Hkv
    k = k.repeat_interleave(G, dim=1).permute(1, 0, 2)   # [Hq][L][D]
    v = v.repeat_interleave(G, dim=1).permute(1, 0, 2)
    s = (q[:, None, :] * k).sum(-1) * scale
    p = torch.softmax(s, dim=-1)
    return (p[:, :, None] * v).sum(1).numpy()


@pytest.mark.parametrize("L,Hq,Hkv", [(1, 4, 1), (33, 8, 2), (200, 16, 4)])
def test_attend_dense_matches_torch_float64(orc, L, Hq, Hkv):
    rng = np.random.default_rng(L)
    kh = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    vh = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    q = workloads.random_rows(L + 3, Hq)
    out = orc.attend_dense(q, Hkv, kh, vh)
    ref = _torch_attention(q, kh, vh, Hkv, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_attend_dense_closed_forms(orc):
    rng = np.random.default_rng(2)
    v = rng.standard_normal((2, 1, D)).astype(np.float32)
    # identical keys: the mean of the values
    k = np.repeat(rng.standard_normal((1, 1, D)).astype(np.float32), 2, axis=0)
    q = rng.standard_normal((1, D)).astype(np.float32)
    np.testing.assert_allclose(orc.attend_dense(q, 1, k, v)[0], v.mean(axis=0)[0], rtol=1e-6, atol=1e-7)
    # two keys whose scores differ by delta: weights 1 / (1 + e^-delta)
    k = np.zeros((2, 1, D), np.float32)
    k[0, 0, 0] = 2.0
    q = np.zeros((1, D), np.float32)
    q[0, 0] = 1.5
    scale = 0.5
    w0 = 1.0 / (1.0 + math.exp(-(2.0 * 1.5 * scale)))
    np.testing.assert_allclose(orc.attend_dense(q, 1, k, v, scale=scale)[0],
                               w0 * v[0, 0] + (1 - w0) * v[1, 0], rtol=1e-6, atol=1e-7)
    # empty context: zeros
    assert not orc.attend_dense(q, 1, np.zeros((0, 1, D), np.float32), np.zeros((0, 1, D), np.float32)).any()


def test_decode_batch_dense_heads_and_sequences(orc):
    rng = np.random.default_rng(4)
    Hkv, G = 2, 3
    seqs = []
    for L in (5, 0, 17):
        seqs.append((rng.standard_normal((L, Hkv, D)).astype(np.float32),
                     rng.standard_normal((L, Hkv, D)).astype(np.float32)))
    q = rng.standard_normal((3, Hkv * G, D)).astype(np.float32)
    out = orc.decode_batch_dense(q, seqs, Hkv, threads=3)
    for b, (kh, vh) in enumerate(seqs):
        if kh.shape[0] == 0:
            assert not out[b].any()
            continue
        np.testing.assert_allclose(out[b], _torch_attention(q[b], kh, vh, Hkv, 1.0 / math.sqrt(D)),
                                   rtol=1e-6, atol=1e-7)
