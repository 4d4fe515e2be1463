"""Pins for the oracle's NVFP4 -> FP8 conversion (dequantize dividing by the
global scale, then encode as E4M3 over an output scale), CPU only.

Every (E2M1 code, block scale) pair is checked against the same steps taken
with PyTorch's float32 division and float8_e4m3fn cast (an independent
encoder); the nibble order and block index against hand-built bytes; the
divide-by-global-scale rule against the oracle's own dequantization (which
multiplies by s_t = 1/g) within FP8's half-step bound, where the multiply
variant is off by g^2.
"""
import numpy as np
import pytest
import torch

from decode_attention_nvfp4_amd import workloads

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3(code):
    return float(torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32))


def _torch_steps(code, sb, g, s8):
    mag = E2M1[code & 7] * _e4m3(sb)
    v = torch.tensor([-mag if code & 8 else mag], dtype=torch.float32)
    xh = v / torch.tensor([g], dtype=torch.float32)
    q = (xh / torch.tensor([s8], dtype=torch.float32)).clamp(-448.0, 448.0)
    return int(q.to(torch.float8_e4m3fn).view(torch.uint8)[0])


@pytest.mark.parametrize("amax", [1.0, 3.7, 1e-3, 250.0])
@pytest.mark.parametrize("s8_rule", ["eight", "six", "odd"])
def test_every_code_and_scale_pair_matches_torch(orc, amax, s8_rule):
    g = float(np.float32(2688.0) / np.float32(amax))          # global encode scale
    s8 = {"eight": np.float32(8.0) / np.float32(g), "six": np.float32(6.0) / np.float32(g),
          "odd": np.float32(0.37) / np.float32(g)}[s8_rule]
    s8 = float(s8)
    for sb in range(0, 127):
        for code in range(16):
            assert orc.nvfp4_to_fp8_code(code, sb, g, s8) == _torch_steps(code, sb, g, s8), (code, sb)


def test_nibble_order_and_block_index(orc):
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0] = 0x71           # element 0: code 1 (0.5); element 1: code 7 (6)
    packed[0, 8] = 0xA3           # element 16: code 3 (1.5); element 17: code 0xA (-1)
    scales = np.array([[0x38, 0x40]], np.uint8)   # blocks 0 and 1: 1.0 and 2.0
    out = orc.nvfp4_to_fp8_packed(packed, scales, 1.0, 1.0)
    val = torch.from_numpy(out[0]).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert val[0] == 0.5 and val[1] == 6.0
    assert val[16] == 3.0 and val[17] == -2.0
    assert np.all(val[2:16] == 0) and np.all(val[18:] == 0)
    assert out[0, 2] == 0x00                       # +0 stays +0
    # a block scale byte with its sign bit set converts as the plain scale
    neg = orc.nvfp4_to_fp8_packed(packed, scales | 0x80, 1.0, 1.0)
    assert np.array_equal(neg, out)


def test_divides_by_the_global_scale(orc):
    x = workloads.random_rows(31, 64, "normal", dtype="f32")
    s_t = orc.tensor_scale(x)
    codes, scales = orc.quantize_rows(x, s_t)
    g = float(np.float32(1.0) / np.float32(s_t))
    s8 = float(np.float32(6.0) / np.float32(g))
    xh = orc.dequant_rows(codes, scales, s_t).astype(np.float64)
    fp8 = orc.nvfp4_to_fp8(codes, scales, g, s8)
    back = orc.fp8_dequant(fp8, s8).astype(np.float64)
    # half an E4M3 step (normal and subnormal), plus the FP32 roundings of
    # x / g against x * s_t
    bound = np.maximum(np.abs(xh) * 2.0 ** -4, 2.0 ** -10 * s8) + np.abs(xh) * 2.0 ** -22
    assert np.all(np.abs(back - xh) <= bound)
    # multiplying by the global scale instead is off by g^2 and saturates
    wrong = orc.fp8_dequant(orc.nvfp4_to_fp8(codes, scales, 1.0 / g, s8), s8).astype(np.float64)
    assert g > 100
    nz = xh != 0                                   # zeros stay zero either way
    assert np.mean((np.abs(wrong - xh) <= bound)[nz]) < 0.05
    assert np.mean(np.abs(wrong[nz]) == np.float32(448 * s8)) > 0.9


def test_power_of_two_scales_convert_exactly(orc):
    # g and s8 = 8 / g powers of two: v / g and the division by s8 are exact,
    # so every value whose significand fits E4M3's 4 bits and lies in its
    # normal range comes through unchanged
    g = 2.0 ** 7
    s8 = 8.0 / g
    n_exact = 0
    for sb in range(1, 127):
        for code in range(1, 8):
            v = E2M1[code] * _e4m3(sb)
            q = v / 8.0
            m, e = np.frexp(q)
            if q < 2.0 ** -6 or q > 448 or (m * 16) != np.floor(m * 16):
                continue
            got = orc.fp8_value(orc.nvfp4_to_fp8_code(code, sb, g, s8), s8)
            assert got == np.float32(v / g), (code, sb)
            n_exact += 1
    assert n_exact > 500
