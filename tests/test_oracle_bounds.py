"""The error model of attention on FP8 operands (oracle/bounds.py), checked
against a simulation of the rounding steps it models: Q, the dequantized K
and V, and the softmax weights each rounded to E4M3 by PyTorch's
float8_e4m3fn cast, then softmax attention in float64.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.bounds import fp8_attention_error_model

Z = 6.0


def e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def pow2_scaled(x: np.ndarray, target: float) -> np.ndarray:
    """E4M3 rounding of x after scaling by a power of two that puts max |x|
    near `target` (so the values stay in E4M3's normal range), scaled back."""
    m = float(np.abs(x).max())
    e = 0 if m == 0 else math.floor(math.log2(target / m))
    return e4m3(x * 2.0 ** e) / 2.0 ** e


def simulate(q, kh, vh, rows, prefix, causal, scale, v_slip=1.0):
    """Attention on E4M3 operands: per query row and head, Q scaled by a power
    of two; K and V as dequantized values scaled by a power of two; P =
    E4M3(2^(s - m + 4)) with m the row's max score in log2 units."""
    n, Hq, _ = q.shape
    Hkv = kh.shape[1]
    G = Hq // Hkv
    total = kh.shape[0]
    k8 = np.stack([pow2_scaled(kh[:, h], 256.0) for h in range(Hkv)], axis=1)
    v8 = np.stack([pow2_scaled(vh[:, h], 256.0) for h in range(Hkv)], axis=1) * v_slip
    out = np.zeros((n, Hq, 128))
    for r in range(n):
        lim = prefix + rows[r] if causal else total - 1
        for h in range(Hq):
            q8 = pow2_scaled(q[r, h], 256.0)
            s = (k8[:lim + 1, h // G] @ q8) * scale / math.log(2.0)   # log2 units
            p = e4m3(np.exp2(s - s.max() + 4.0))
            out[r, h] = (p @ v8[:lim + 1, h // G]) / p.sum()
    return out


def exact(q, kh, vh, rows, prefix, causal, scale):
    n, Hq, _ = q.shape
    G = Hq // kh.shape[1]
    out = np.zeros((n, Hq, 128))
    for r in range(n):
        lim = prefix + rows[r] if causal else kh.shape[0] - 1
        for h in range(Hq):
            s = (kh[:lim + 1, h // G].astype(np.float64) @ q[r, h].astype(np.float64)) * scale
            w = np.exp(s - s.max())
            out[r, h] = (w / w.sum()) @ vh[:lim + 1, h // G].astype(np.float64)
    return out


def case(seed, n, Hq, Hkv, prefix, causal, outliers=False, structured=False):
    """Seeded inputs.  structured: a tenth of the keys lie along a direction u
    that the queries share (they take most of the weight) and carry values
    near +2, the others near -2, so the output depends visibly on how the
    weight splits and on the value scale."""
    rng = np.random.default_rng(seed)
    total = prefix + n
    k = rng.standard_normal((total, Hkv, 128)).astype(np.float32)
    v = rng.standard_normal((total, Hkv, 128)).astype(np.float32)
    if structured:
        u = rng.standard_normal(128).astype(np.float32)
        u /= np.linalg.norm(u)
        hot = rng.random(total) < 0.1
        k[hot] += 3.0 * math.sqrt(128) * 0.25 * u
        v += np.where(hot, 2.0, -2.0)[:, None, None].astype(np.float32)
        q_dir = u
    if outliers:
        k[:, :, :4] *= 20.0
        v[:, :, 5:9] *= 20.0
    q = rng.standard_normal((n, Hq, 128)).astype(np.float32)
    if structured:
        q = (0.5 * q + 2.0 * math.sqrt(128) * 0.25 * q_dir).astype(np.float32)
    kh = oracle.dequant_rows(*oracle.quantize_rows(k, oracle.tensor_scale(k)), oracle.tensor_scale(k))
    vh = oracle.dequant_rows(*oracle.quantize_rows(v, oracle.tensor_scale(v)), oracle.tensor_scale(v))
    return q, kh, vh, np.arange(n)


CASES = [(1, 24, 4, 2, 0, True, False, False), (2, 16, 4, 1, 300, True, False, False),
         (3, 12, 8, 2, 100, False, False, False), (4, 20, 4, 2, 50, True, True, False),
         (7, 24, 4, 2, 400, True, False, True)]


@pytest.mark.parametrize("c", CASES)
def test_model_bounds_the_simulated_fp8_attention(c):
    seed, n, Hq, Hkv, prefix, causal, outl, structured = c
    q, kh, vh, rows = case(seed, n, Hq, Hkv, prefix, causal, outl, structured)
    scale = 1.0 / math.sqrt(128)
    ref = exact(q, kh, vh, rows, prefix, causal, scale)
    sim = simulate(q, kh, vh, rows, prefix, causal, scale)
    sigma, floor = fp8_attention_error_model(q, rows, Hkv, kh, vh, prefix, causal, scale)
    # the model's mean is the exact attention
    err = np.abs(sim - ref)
    assert np.all(err <= Z * sigma + floor + 1e-9), float((err / (Z * sigma + floor)).max())
    rms = float(np.sqrt(np.mean((err / np.maximum(sigma, 1e-300)) ** 2)))
    # the model is an upper estimate of the spread, and not a loose one
    assert 0.15 <= rms <= 1.2, rms


@pytest.mark.parametrize("which", ["v", "k"])
def test_model_catches_an_operand_scale_slip(which):
    """On inputs whose output depends visibly on the value scale and on how
    the weight splits (structured keys and values), V or K off by 3% (a
    slipped operand scale) stops looking like rounding noise: the RMS gate
    the GPU tests apply (2) fails, while the correct rounding passes it."""
    q, kh, vh, rows = case(5, 24, 4, 2, 400, True, structured=True)
    scale = 1.0 / math.sqrt(128)
    ref = exact(q, kh, vh, rows, 400, True, scale)
    sigma, _ = fp8_attention_error_model(q, rows, 2, kh, vh, 400, True, scale)
    good = simulate(q, kh, vh, rows, 400, True, scale)
    if which == "v":
        bad = simulate(q, kh, vh, rows, 400, True, scale, v_slip=1.03)
    else:
        bad = simulate(q, kh * np.float32(1.03), vh, rows, 400, True, scale)
    rms = lambda o: float(np.sqrt(np.mean((np.abs(o - ref) / np.maximum(sigma, 1e-300)) ** 2)))  # noqa: E731
    assert rms(good) <= 2.0
    assert rms(bad) > 2.0, rms(bad)


def test_single_key_row_is_the_value_rounding():
    """A row that sees one key returns that key's value: the only error is the
    E4M3 rounding of V (at most 2^-4 relative), inside 6 sigma of the model."""
    q, kh, vh, rows = case(6, 1, 2, 1, 0, True)
    scale = 1.0 / math.sqrt(128)
    sigma, floor = fp8_attention_error_model(q, rows, 1, kh, vh, 0, True, scale)
    np.testing.assert_allclose(sigma[0, 0], (2.0 ** -3 / math.sqrt(12.0)) * np.abs(vh[0, 0]), rtol=1e-6, atol=1e-12)
    assert np.all(Z * sigma[0, 0] >= 2.0 ** -4 * np.abs(vh[0, 0]))
