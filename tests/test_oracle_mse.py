"""Pins for the oracle's MSE-searched block scale, CPU only.

The search is pinned to an independent brute force in exact rational
arithmetic: E4M3 values from PyTorch's float8 decoder, E2M1 rounding to the
nearest grid value (ties to the even code, clamped to 6) done with Fractions,
and the block's squared error summed exactly.  Closed-form blocks pin the
tie rules (the candidate nearest the amax/6 code wins, then the smaller
code) and a block where a smaller scale that clips the maximum beats amax/6.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from decode_attention_nvfp4_amd import workloads

RADIUS = 8
GRID = [Fraction(v) for v in ("0", "0.5", "1", "1.5", "2", "3", "4", "6")]
E4M3 = [Fraction(float(v)) for v in
        torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()]


def _e2m1_mag(r: Fraction) -> int:
    best = 0
    for i, g in enumerate(GRID):
        dist, bdist = abs(r - g), abs(r - GRID[best])
        if dist < bdist or (dist == bdist and i % 2 == 0 and best % 2 == 1):
            best = i
    return best


def exact_sq_error(x16, sb: int, s_t: float) -> Fraction:
    """Exact squared error of a block under block-scale code sb."""
    step = E4M3[sb] * Fraction(float(s_t))
    err = Fraction(0)
    for v in x16:
        xv = Fraction(float(v))
        q = GRID[_e2m1_mag(abs(xv) / step)] * step if step else Fraction(0)
        err += (abs(xv) - q) ** 2
    return err


def _window(c0: int):
    return [c for c in range(c0 - RADIUS, c0 + RADIUS + 1) if 1 <= c <= 126]


def _blocks(seed, n):
    out = []
    for d in ("normal", "outlier", "mixed"):
        x = workloads.random_rows(seed, n, d, dtype="f32")
        out.append((x.reshape(-1, 16), float(np.abs(x).max()) / (6 * 448)))
    rng = np.random.default_rng(seed)
    u = rng.uniform(-1, 1, (n, 128)).astype(np.float32)
    out.append((u.reshape(-1, 16), float(np.abs(u).max()) / (6 * 448)))
    return out


def test_mse_search_matches_exact_brute_force(orc):
    checked = 0
    for blocks, _ in _blocks(3, 6):
        x_all = blocks.reshape(-1, 128)
        s_t = orc.tensor_scale(x_all)
        for b in blocks:
            c0 = orc.block_scale_code(float(np.abs(b).max()), s_t)
            got = orc.block_scale_code_mse(b, s_t)
            if c0 == 0:
                assert got == 0
                continue
            errs = {c: exact_sq_error(b, c, s_t) for c in _window(c0)}
            best = min(errs.values())
            # the oracle's criterion is double arithmetic: it must choose a
            # minimiser up to its rounding, and exactly the first minimiser in
            # the search order whenever the exact minimum is clear
            assert errs[got] <= best * (1 + Fraction(1, 10**12))
            order = sorted(errs, key=lambda c: (abs(c - c0), c))
            ranked = sorted(errs.values())
            if len(ranked) == 1 or ranked[1] > best * (1 + Fraction(1, 10**9)):
                assert got == next(c for c in order if errs[c] == best)
            # the criterion itself, against the exact sum
            for c in (c0, got):
                assert orc.block_sq_error(b, c, s_t) == pytest.approx(float(errs[c]), rel=1e-13, abs=1e-300)
            checked += 1
    assert checked > 150


def test_mse_never_worse_than_amax6_and_lower_on_average(orc):
    x = workloads.random_rows(7, 64, "normal", dtype="f32")
    s_t = orc.tensor_scale(x)
    c_a, sc_a = orc.quantize_rows(x, s_t)
    c_m, sc_m = orc.quantize_rows_mse(x, s_t)
    e_a = (orc.dequant_rows(c_a, sc_a, s_t).astype(np.float64) - x) ** 2
    e_m = (orc.dequant_rows(c_m, sc_m, s_t).astype(np.float64) - x) ** 2
    per_a = e_a.reshape(-1, 16).sum(1)
    per_m = e_m.reshape(-1, 16).sum(1)
    assert np.all(per_m <= per_a * (1 + 1e-6) + 1e-30)
    # on N(0,1) rows the search removes about a quarter of the error
    assert e_m.mean() < 0.8 * e_a.mean()
    assert np.mean(sc_m != sc_a) > 0.3


def test_mse_rows_are_blockwise_search_then_element_codes(orc):
    x = workloads.random_rows(11, 8, "mixed", dtype="f32")
    s_t = orc.tensor_scale(x)
    codes, scales = orc.quantize_rows_mse(x, s_t)
    for r in range(x.shape[0]):
        for blk in range(8):
            b = x[r, 16 * blk:16 * blk + 16]
            sb = orc.block_scale_code_mse(b, s_t)
            assert scales[r, blk] == sb
            np.testing.assert_array_equal(codes[r, 16 * blk:16 * blk + 16], orc.element_codes(b, sb, s_t))


def test_mse_zero_block_keeps_zero_scale(orc):
    z = np.zeros(16, np.float32)
    assert orc.block_scale_code_mse(z, 1.0) == 0
    z[3] = -0.0
    assert orc.block_scale_code_mse(z, 1.0) == 0


def test_mse_tie_goes_to_the_amax6_code(orc):
    # s_t = 1, block [6, 0, ...]: the amax/6 code is 1.0 (0x38); 1.5 (0x3C,
    # 6 -> 4) and 2.0 (0x40, 6 -> 3) represent the block exactly as well;
    # all three have zero error and the amax/6 code is kept
    b = np.zeros(16, np.float32)
    b[0] = 6.0
    assert orc.block_scale_code(6.0, 1.0) == 0x38
    for c in (0x38, 0x3C, 0x40):
        assert exact_sq_error(b, c, 1.0) == 0
    assert orc.block_scale_code_mse(b, 1.0) == 0x38


def test_mse_smaller_clipping_scale_wins(orc):
    # s_t = 1, block [6, 4.9 x 15]: at the amax/6 scale 1.0 each 4.9 rounds
    # to 4 (error 15 * 0.81 = 12.15); at 0.9375 (0x37) the 6 clips to 5.625
    # and each 4.9 rounds to 6 * 0.9375 (error 0.375^2 + 15 * 0.725^2 ~ 8.02),
    # so the search must leave the amax/6 code
    b = np.full(16, 4.9, np.float32)
    b[0] = 6.0
    assert orc.block_scale_code(6.0, 1.0) == 0x38
    e0 = exact_sq_error(b, 0x38, 1.0)
    e1 = exact_sq_error(b, 0x37, 1.0)
    assert float(e0) == pytest.approx(15 * (float(np.float32(4.9)) - 4) ** 2)
    assert e1 < e0
    got = orc.block_scale_code_mse(b, 1.0)
    assert got != 0x38
    assert exact_sq_error(b, got, 1.0) == min(exact_sq_error(b, c, 1.0) for c in _window(0x38))


def test_mse_window_clamps_at_the_code_range(orc):
    # a block whose amax/6 code is the largest (448) searches only downwards;
    # one whose code is 1 only upwards (code 0 is never a candidate)
    b = np.linspace(-1, 1, 16).astype(np.float32)
    s_hi = float(np.float32(1.0) / np.float32(6 * 448))
    assert orc.block_scale_code(1.0, s_hi) == 0x7E
    got = orc.block_scale_code_mse(b, s_hi)
    assert 0x7E - RADIUS <= got <= 0x7E
    errs = {c: exact_sq_error(b, c, s_hi) for c in _window(0x7E)}
    assert errs[got] == min(errs.values())
    s_lo = float(np.float32(1.0) / np.float32(6 * 2.0 ** -9))
    assert orc.block_scale_code(1.0, s_lo) == 1
    got = orc.block_scale_code_mse(b, s_lo)
    assert 1 <= got <= 1 + RADIUS
    errs = {c: exact_sq_error(b, c, s_lo) for c in _window(1)}
    assert errs[got] == min(errs.values())


def test_mse_equal_distance_tie_goes_to_the_smaller_code(orc):
    # s_t = 1, block [6.0625, 3.5 x 6, 0 x 9] (every product exact in
    # double): the amax/6 code is 1.0 (0x38); 0.9375 (0x37) and 1.125 (0x39)
    # give the same, smaller error 0.56640625, and the smaller code is kept
    b = np.zeros(16, np.float32)
    b[0] = 6.0625
    b[1:7] = 3.5
    assert orc.block_scale_code(6.0625, 1.0) == 0x38
    e = {c: exact_sq_error(b, c, 1.0) for c in _window(0x38)}
    assert e[0x37] == e[0x39] == Fraction(145, 256) == min(e.values()) < e[0x38]
    assert orc.block_sq_error(b, 0x37, 1.0) == orc.block_sq_error(b, 0x39, 1.0) == 145 / 256
    assert orc.block_scale_code_mse(b, 1.0) == 0x37
