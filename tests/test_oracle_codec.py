"""Pins for the oracle's NVFP4 codec (CPU only).

Each check ties the oracle to something other than itself: the facts the
pages print (tests/golden/format_facts.json), a library decoder (PyTorch's
float8_e4m3fn and bfloat16 casts), brute-force nearest-value search in exact
rational arithmetic (fractions.Fraction) or in numpy over dense FP32 sweeps,
and closed-form error bounds.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from decode_attention_nvfp4_amd import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "format_facts.json")))


# ------------------------------------------------------------- E2M1 decode

def _e2m1_from_bits(code):
    """E2M1 value from its bit fields: exponent bias 1, field 0 subnormal."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    v = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -v if s else v


def test_e2m1_decode_matches_bit_layout_and_page_range(orc):
    facts = GOLD["e2m1"]
    assert facts["sign_bits"] + facts["exponent_bits"] + facts["mantissa_bits"] == 4
    vals = [orc.e2m1_value(c) for c in range(16)]
    assert vals == [_e2m1_from_bits(c) for c in range(16)]
    mags = sorted(set(abs(v) for v in vals))
    assert max(mags) == facts["range_max"]          # page: range about [-6, +6]
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert len(mags) == 8                           # 3 magnitude bits
    # codes 8..15 are the negatives of 0..7 (1 sign bit); 0x8 is -0
    for c in range(8):
        assert vals[c + 8] == -vals[c]
    assert math.copysign(1.0, vals[8]) == -1.0


# ------------------------------------------------------------- E4M3 decode

def test_e4m3_decode_all_256_codes_match_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for b in range(256):
        v = orc.e4m3_value(b)
        r = float(ref[b])
        if math.isnan(r):
            assert math.isnan(v), b
        else:
            assert v == r, (b, v, r)
            assert math.copysign(1, v) == math.copysign(1, r)
    assert orc.e4m3_value(0x7E) == GOLD["e4m3fn_max_finite"]["value"]
    assert math.isnan(orc.e4m3_value(0x7F))


# ------------------------------------------------------------ block scale

E4M3_VALUES = [Fraction(torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).item())
               for b in range(127)]


def _brute_block_scale(a: float, s_t: float) -> int:
    """Nearest of the 127 non-negative finite E4M3 values to a / (6 s_t),
    exact rationals; ties to the even code; above 448 clamps to 0x7E."""
    q = Fraction(a) / (6 * Fraction(s_t))
    if q >= E4M3_VALUES[126]:
        return 126
    best = min(abs(q - v) for v in E4M3_VALUES)
    cands = [k for k, v in enumerate(E4M3_VALUES) if abs(q - v) == best]
    if len(cands) == 1:
        return cands[0]
    assert len(cands) == 2
    return cands[0] if cands[0] % 2 == 0 else cands[1]


def _near(x, k):
    """k-th float32 neighbour of x (k may be negative)."""
    x = np.float32(x)
    for _ in range(abs(k)):
        x = np.nextafter(x, np.float32(np.inf if k > 0 else 0), dtype=np.float32)
    return float(x)


def test_block_scale_bruteforce_random_and_midpoints(orc):
    rng = np.random.default_rng(1)
    cases = []
    for s_t in [1.0, 4.5 / 2688, 1.0 / 3.0, 2.0 ** -20, 123.456, 7.0e-3]:
        s_t = float(np.float32(s_t))
        for a in rng.standard_normal(200).astype(np.float32):
            cases.append((abs(float(a)) * 3.0, s_t))
        # exactly on, and one ulp around, every midpoint between E4M3 codes
        for k in range(0, 126, 3):
            mid = (E4M3_VALUES[k] + E4M3_VALUES[k + 1]) / 2
            a0 = float(np.float32(float(mid * 6 * Fraction(s_t))))
            for j in (-1, 0, 1):
                cases.append((_near(a0, j), s_t))
    for a, s_t in cases:
        assert orc.block_scale_code(a, s_t) == _brute_block_scale(a, s_t), (a, s_t)


def test_block_scale_saturates_at_448(orc):
    s_t = float(np.float32(1.0 / 64))
    six = 6 * Fraction(s_t)
    for q in [448, 449, 464, 465, 1000, 3.0e5]:
        a = float(np.float32(float(q * six)))
        assert orc.block_scale_code(a, s_t) == 0x7E
    assert orc.block_scale_code(float(np.float32(3.4e38)), 1e-30) == 0x7E
    # the tensor's own amax maps onto 448 by construction of s_t
    x = workloads.random_rows(3, 64)
    st = orc.tensor_scale(x)
    assert orc.block_scale_code(float(np.abs(x).max()), st) == 0x7E


def test_block_scale_subnormals_and_zero(orc):
    s_t = 1.0
    six = Fraction(6)
    # smallest subnormal 2^-9; half of it ties to 0 (even); 3/4 of it -> 1
    assert orc.block_scale_code(float(six * Fraction(1, 2 ** 10)), s_t) == 0
    assert orc.block_scale_code(float(six * Fraction(3, 2 ** 11)), s_t) == 1
    assert orc.block_scale_code(float(six * Fraction(3, 2 ** 10)), s_t) == 2   # 1.5 * 2^-9: tie -> even 2
    assert orc.block_scale_code(0.0, s_t) == 0
    # torch's nearest-even cast agrees wherever the quotient a / 6 is an FP32
    # value q (s_t = 1, a = 6 q exact in FP32)
    qs = (np.random.default_rng(5).random(2000) * 440).astype(np.float32)
    qs = np.concatenate([qs, np.float32(2.0) ** -np.arange(0, 12, dtype=np.float32)])
    ref = torch.from_numpy(qs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for q, r in zip(qs, ref):
        a = float(np.float32(q) * np.float32(6.0))
        if Fraction(a) != Fraction(float(q)) * 6:
            continue
        assert orc.block_scale_code(a, 1.0) == int(r), (q, r)


# ------------------------------------------------------------- element codes

GRID = [Fraction(v) for v in (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)]


def _brute_element_code(x: float, sb_code: int, s_t: float) -> int:
    sign = 8 if math.copysign(1.0, x) < 0 else 0
    d = E4M3_VALUES[sb_code] * Fraction(s_t)
    if d == 0:
        return sign
    v = abs(Fraction(x)) / d
    dist = [abs(v - g) for g in GRID]
    best = min(dist)
    cands = [k for k in range(8) if dist[k] == best]
    m = cands[0] if len(cands) == 1 or cands[0] % 2 == 0 else cands[1]
    return sign | m


def _np_brute_codes(x: np.ndarray) -> np.ndarray:
    """Nearest-grid magnitude code for d == 1, ties to the even code (numpy,
    exact in double since x is FP32 and the grid values are short)."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    # anything above 6 is nearest to 6; clamping keeps the double distances exact
    ax = np.minimum(np.abs(x.astype(np.float64)), 7.0)
    dist = np.abs(ax[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    is_best = dist == best
    # among tied candidates prefer an even code
    even_best = is_best & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even_best.any(axis=1), even_best.argmax(axis=1), is_best.argmax(axis=1))
    sign = np.signbit(x).astype(np.uint8) << 3
    return (pick.astype(np.uint8) | sign)


def test_element_code_dense_sweep_d_equals_one(orc):
    """Every FP32 value in [0, 8) on a stride-16 lattice, plus every FP32
    value within 64 ulps of each grid point and each midpoint, both signs;
    block scale 1.0 (0x38) and s_t = 1 so x / d = x."""
    lo = np.float32(0.0).view(np.uint32)
    hi = np.float32(8.0).view(np.uint32)
    lattice = np.arange(lo, hi, 16, dtype=np.uint32).view(np.float32)
    pts = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0]
    near = []
    for p in pts:
        u = np.float32(p).view(np.uint32).astype(np.int64)
        near.append(np.clip(np.arange(u - 64, u + 65), 0, None).astype(np.uint32).view(np.float32))
    xs = np.concatenate([lattice] + near + [np.array([1e30, 3.4e38], np.float32)])
    xs = np.concatenate([xs, -xs])
    assert orc.e4m3_value(0x38) == 1.0
    step = 1 << 21
    for i in range(0, xs.size, step):
        chunk = np.ascontiguousarray(xs[i:i + step])
        got = orc.element_codes(chunk, 0x38, 1.0)
        exp = _np_brute_codes(chunk)
        bad = np.nonzero(got != exp)[0]
        assert bad.size == 0, (chunk[bad[:5]], got[bad[:5]], exp[bad[:5]])


def test_element_code_bruteforce_general_scales(orc):
    rng = np.random.default_rng(7)
    mids = [Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4),
            Fraction(5, 2), Fraction(7, 2), Fraction(5)]
    n = 0
    for _ in range(60):
        sb = int(rng.integers(1, 127))
        s_t = float(np.float32(np.exp(rng.uniform(-30, 10))))
        d = E4M3_VALUES[sb] * Fraction(s_t)
        for c in mids:
            x0 = float(np.float32(float(c * d)))
            for j in (-2, -1, 0, 1, 2):
                x = _near(x0, j)
                for sx in (x, -x):
                    assert orc.element_code(sx, sb, s_t) == _brute_element_code(sx, sb, s_t), (sx, sb, s_t)
                    n += 1
        for x in (rng.standard_normal(20) * float(d) * 3).astype(np.float32):
            assert orc.element_code(float(x), sb, s_t) == _brute_element_code(float(x), sb, s_t)
            n += 1
    assert n > 3000


def test_element_code_special_cases(orc):
    assert orc.element_code(0.0, 0x38, 1.0) == 0x0
    assert orc.element_code(-0.0, 0x38, 1.0) == 0x8
    assert orc.element_code(-0.1, 0x38, 1.0) == 0x8          # rounds to -0, sign kept
    assert orc.element_code(0.25, 0x38, 1.0) == 0            # tie 0 / 0.5 -> even code 0
    assert orc.element_code(0.75, 0x38, 1.0) == 2            # tie 0.5 / 1 -> even code 2
    assert orc.element_code(5.0, 0x38, 1.0) == 6             # tie 4 / 6 -> even code 6
    assert orc.element_code(100.0, 0x38, 1.0) == 7           # saturates at 6
    assert orc.element_code(-100.0, 0x38, 1.0) == 15
    assert orc.element_code(5.0, 0x00, 1.0) == 0             # zero block scale -> magnitude 0
    assert orc.element_code(-5.0, 0x00, 1.0) == 8


# ------------------------------------------------------------- whole rows

def test_quantize_rows_block_locality(orc):
    """One scale per 16 elements: changing one element changes only its own
    block's scale and codes."""
    x = workloads.random_rows(11, 32)
    st = orc.tensor_scale(x) * 2   # keep headroom so the tensor scale is fixed
    c0, s0 = orc.quantize_rows(x, st)
    rng = np.random.default_rng(2)
    for r in range(32):
        e = int(rng.integers(0, 128))
        y = x.copy()
        y[r, e] = np.float32(y[r, e] * -3.0 + 0.7)
        c1, s1 = orc.quantize_rows(y, st)
        blk = e // 16
        diff_rows = np.nonzero((c0 != c1).any(axis=1) | (s0 != s1).any(axis=1))[0]
        assert set(diff_rows.tolist()) <= {r}
        changed_codes = np.nonzero(c0[r] != c1[r])[0]
        assert all(i // 16 == blk for i in changed_codes)
        assert all(j == blk for j in np.nonzero(s0[r] != s1[r])[0])
    assert GOLD["two_level_scaling"]["block_size"] == 16


def test_two_level_roundtrip_error_bound(orc):
    """|x - x_hat| <= half the local grid gap times sb * s_t (plus one FP32
    rounding of x_hat) whenever the element is not clipped."""
    gaps = {0: 0.5, 1: 0.5, 2: 0.5, 3: 0.5, 4: 1.0, 5: 1.0, 6: 2.0, 7: 2.0}
    for dist in ("normal", "outlier", "mixed"):
        x = workloads.random_rows(21, 256, dist)
        st = orc.tensor_scale(x)
        codes, scales = orc.quantize_rows(x, st)
        xh = orc.dequant_rows(codes, scales, st)
        sb = np.array([[orc.e4m3_value(int(b)) for b in row] for row in scales])
        d = np.repeat(sb, 16, axis=1) * st
        m = codes & 7
        gap = np.vectorize(gaps.get)(m)
        bound = 0.5 * gap * d + np.abs(xh) * 2.0 ** -24
        # a zero block scale means the block's amax is at most half the
        # smallest E4M3 subnormal (2^-10) times 6 s_t; every element flushes to 0
        bound = np.where(d == 0, 6.0 * st * 2.0 ** -10, bound)
        clipped = (m == 7) & (np.abs(x) > 6 * d)
        err = np.abs(x.astype(np.float64) - xh.astype(np.float64))
        assert np.all(err[~clipped] <= bound[~clipped] * (1 + 1e-12))
        # clipped elements sit at +-6 sb s_t, and only by the E4M3 rounding of
        # the block scale: |x| <= 6 s_t (sb + next(sb)) / 2
        sb_next = np.array([[orc.e4m3_value(min(int(b) + 1, 126)) for b in row] for row in scales])
        lim = 6.0 * st * (np.repeat(sb, 16, axis=1) + np.repeat(sb_next, 16, axis=1)) / 2
        lim = np.where(np.repeat(scales, 16, axis=1) == 0x7E, np.inf, lim)   # saturated scale
        assert np.all(np.abs(x)[clipped] <= lim[clipped] * (1 + 1e-12))
        assert np.allclose(np.abs(xh)[clipped], 6.0 * d[clipped], rtol=2.0 ** -23, atol=0)


def test_exact_grid_points_roundtrip_exactly(orc):
    """x = e2m1 * sb * s_t, representable in FP32 (s_t a power of two),
    comes back unchanged."""
    st = 2.0 ** -9
    rng = np.random.default_rng(4)
    for _ in range(50):
        sb_code = int(rng.integers(8, 127))
        sb = orc.e4m3_value(sb_code)
        mags = rng.integers(0, 8, 16)
        mags[0] = 7   # block max on 6 so the block scale is exactly sb
        signs = rng.integers(0, 2, 16)
        vals = np.array([(-1) ** s * orc.e2m1_value(int(m)) * sb * st for m, s in zip(mags, signs)])
        x = vals.astype(np.float32)
        assert np.all(x.astype(np.float64) == vals)       # representable
        row = np.zeros((1, 128), np.float32)
        row[0, :16] = x
        codes, scales = orc.quantize_rows(row, st)
        assert scales[0, 0] == sb_code
        assert np.all((codes[0, :16] & 7) == mags)
        xh = orc.dequant_rows(codes, scales, st)
        assert np.array_equal(xh[0, :16], x)


def test_dequant_divides_by_global_scale(orc):
    """Dequantization multiplies by s_t == divides by the global encode scale
    g = 1/s_t; the multiply-by-g variant is off by g^2 and overflows FP16."""
    assert "divide" in GOLD["dequant_rule"]["rule"]
    x = workloads.random_rows(5, 64)
    x[0, 0] = np.float32(4.5)
    st = orc.tensor_scale(x)
    g = 1.0 / st
    codes, scales = orc.quantize_rows(x, st)
    xh = orc.dequant_rows(codes, scales, st).astype(np.float64)
    vals = np.array([[orc.e2m1_value(int(c)) for c in row] for row in codes])
    sb = np.array([[orc.e4m3_value(int(b)) for b in row] for row in scales])
    prod = vals * np.repeat(sb, 16, axis=1)
    divided = prod / g
    assert np.allclose(xh, divided, rtol=2 ** -23, atol=0)
    wrong = prod * g
    ratio = np.abs(wrong[prod != 0] / xh[prod != 0])
    assert np.allclose(ratio, g * g, rtol=1e-5)
    assert g * g > 3.0e5
    assert np.abs(wrong).max() > 65504.0                  # FP16 overflow
    assert np.abs(xh).max() <= 4.5 * (1 + 2 ** -20)


def test_bruteforce_tiny_blocks(orc):
    """Blocks of 16 drawn from a small value set (zeros, equal values, one
    outlier, exact grid points): every scale and code is the exact nearest
    choice, checked with rationals."""
    rng = np.random.default_rng(12)
    pool = np.array([0.0, -0.0, 0.1, -0.1, 0.25, 1.0, -1.0, 1.5, 3.0, -3.0, 7.5, 100.0, -100.0,
                     1e-6, 5.0, 6.0], np.float32)
    st = float(np.float32(100.0 / 2688))
    for _ in range(300):
        blk = rng.choice(pool, 16)
        if rng.random() < 0.2:
            blk[:] = blk[0]
        row = np.zeros((1, 128), np.float32)
        row[0, 16:32] = blk
        codes, scales = orc.quantize_rows(row, st)
        amax = float(np.max(np.abs(blk)))
        assert scales[0, 1] == _brute_block_scale(amax, st)
        for i in range(16):
            assert codes[0, 16 + i] == _brute_element_code(float(blk[i]), int(scales[0, 1]), st)
        # untouched all-zero blocks: scale 0, codes +0
        assert scales[0, 0] == 0 and np.all(codes[0, :16] == 0)


def test_tensor_scale_maps_amax_onto_largest_code(orc):
    for seed in range(4):
        x = workloads.random_rows(seed, 100, "mixed")
        st = orc.tensor_scale(x)
        amax = float(np.abs(x).max())
        assert st == float(np.float32(amax) / np.float32(2688.0))
        codes, scales = orc.quantize_rows(x, st)
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert scales[r, c // 16] == 0x7E and (codes[r, c] & 7) == 7


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1000,
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.4e38, 1e-40, -1e-40], np.float32)])
    got = orc.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert np.array_equal(workloads.round_bf16(x).view(np.uint32) >> 16, ref.astype(np.uint32))


def test_mse_ordering_nvfp4_below_mxfp4(orc):
    """The page's MSE example (0.08 vs 0.72) gives no distribution, so only
    the ordering is checkable: NVFP4 (E4M3 scale per 16) beats an MXFP4-style
    power-of-two scale per 32 on N(0,1) data.  The MXFP4 side here is a plain
    nearest-grid quantizer with the OCP shared exponent floor(log2 amax) - 2."""
    facts = GOLD["mxfp4_comparison"]
    assert facts["mse_nvfp4"] < facts["mse_mxfp4"]
    x = workloads.random_rows(30, 2048, dtype="f32")
    st = orc.tensor_scale(x)
    codes, scales = orc.quantize_rows(x, st)
    mse_nv = float(np.mean((orc.dequant_rows(codes, scales, st).astype(np.float64) - x) ** 2))
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    xb = x.reshape(-1, 32).astype(np.float64)
    e = np.floor(np.log2(np.abs(xb).max(axis=1, keepdims=True))) - 2
    v = np.abs(xb) / 2.0 ** e
    q = grid[np.abs(v[..., None] - grid).argmin(axis=-1)] * np.sign(xb) * 2.0 ** e
    mse_mx = float(np.mean((q - xb) ** 2))
    assert mse_nv < mse_mx
