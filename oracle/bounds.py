"""Error model of attention on FP8 (E4M3) operands, for comparing the FP8
prefill path with the exact oracle.

Test infrastructure, like the rest of oracle/: the product library never
imports or calls it.

The pages' prefill flow dequantizes the NVFP4 cache to FP8 and runs the
attention products on FP8 operands with an FP32 accumulator ("NVIDIA解説:
NVFP4 KV Cacheで長コンテキストLLM推論を最適化", section 量子化・逆量子化フロー).
Each of the four operands (Q, the dequantized K and V, and the softmax
weights P) is then rounded to nearest E4M3, whose 3 mantissa bits give a
rounding error of at most half an ulp: 2^-4 relative at the bottom of a
binade.  Modelled as independent uniform errors, each has a relative
standard deviation of at most 2^-3 / sqrt(12) (SIGMA_E4M3).

First order, for one query row and head with exact scores s_t (natural log
units), weights w_t = softmax(s)_t and output o = sum_t w_t v_t:
  * Q and K rounding move score t by sum_d q_d k_td (dq_d + dk_td) * scale,
    of variance sigma_s_t^2 = 2 SIGMA_E4M3^2 scale^2 sum_d q_d^2 k_td^2;
  * P rounding multiplies weight t by (1 + dp_t);
  * a relative perturbation e_t of weight t moves output element d by
    w_t e_t (v_td - o_d) (the normalisation takes out the mean);
  * V rounding moves it by w_t v_td dv_td.
So var_d = sum_t w_t^2 [(sigma_s_t^2 + SIGMA_E4M3^2)(v_td - o_d)^2 +
SIGMA_E4M3^2 v_td^2].  Weights far below the row's largest fall into E4M3's
subnormals or under its smallest value (the kernel's P is at most 2^8 and
its smallest E4M3 step is 2^-9): each weight's absolute error is then at
most 2^-14 of the largest weight, which adds at most
2^-14 w_max sum_t |v_td - o_d| (counted twice below).
"""
from __future__ import annotations

import math

import numpy as np

SIGMA_E4M3 = 2.0 ** -3 / math.sqrt(12.0)
D = 128


def fp8_attention_error_model(q_rows, rows, Hkv, kh, vh, prefix, causal=True, scale=None):
    """(sigma, floor) per output element of the rows' attention on FP8
    operands: sigma [n][Hq][128] the model's standard deviation, floor
    [n][Hq][128] the subnormal / underflow allowance.

    q_rows: [n][Hq][128] queries of the selected chunk rows; rows: their
    indices in the chunk (query i sits at absolute position prefix + i);
    kh, vh: the dequantized cache values [Ltot][Hkv][128]."""
    q_rows = np.asarray(q_rows, np.float64)
    rows = np.asarray(rows)
    kh = np.asarray(kh, np.float64)
    vh = np.asarray(vh, np.float64)
    n, Hq = q_rows.shape[:2]
    G = Hq // Hkv
    total = kh.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    sigma = np.zeros((n, Hq, D))
    floor = np.zeros((n, Hq, D))
    keys = np.arange(total)
    for h in range(Hq):
        k = kh[:, h // G, :]
        v = vh[:, h // G, :]
        q = q_rows[:, h, :]
        s = (q @ k.T) * scale                                   # [n][total]
        if causal:
            lim = prefix + rows                                 # last visible key
            s = np.where(keys[None, :] <= lim[:, None], s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        o = w @ v                                               # [n][128]
        var_s = 2.0 * SIGMA_E4M3 ** 2 * scale ** 2 * ((q * q) @ (k * k).T)
        a = w * w * (var_s + SIGMA_E4M3 ** 2)                   # weight part
        b = w * w * SIGMA_E4M3 ** 2                             # value part
        # sum_t a_t (v_td - o_d)^2 = a.v^2 - 2 o a.v + o^2 sum a
        var = a @ (v * v) - 2.0 * o * (a @ v) + o * o * a.sum(axis=1, keepdims=True) + b @ (v * v)
        sigma[:, h, :] = np.sqrt(np.maximum(var, 0.0))
        wmax = w.max(axis=1, keepdims=True)
        vis = (w > 0).astype(np.float64)
        # sum_t |v_td - o_d| over the visible keys, bounded by sum |v| + n |o|
        dev_sum = vis @ np.abs(v) + vis.sum(axis=1, keepdims=True) * np.abs(o)
        floor[:, h, :] = 2.0 * 2.0 ** -14 * wmax * dev_sum
    return sigma, floor
