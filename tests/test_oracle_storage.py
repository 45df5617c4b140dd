"""Pins of the oracle's storage widening (bf16 bits and fp32 to float64).

The bf16 branch is checked against torch's own bfloat16 dtype over every one of
the 65,536 bit patterns, and against values fixed by the bfloat16 format itself
(sign, 8-bit exponent with bias 127, 7-bit mantissa): 0x3F80 is 1.0, 0xC000 is
-2.0, 0x0001 the smallest subnormal 2^-133, 0x7F80 +inf, 0xFF80 -inf, 0x7F7F
the largest finite value (2 - 2^-7) * 2^127.  The input generator's rounding to
bf16 is checked against torch's float32 -> bfloat16 conversion.
"""
import numpy as np
import torch

from oracle import pkv_oracle as O
from pkv_workloads import f32_to_bf16_bits


def test_bf16_widening_matches_torch_bfloat16_on_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.storage_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_widening_of_fixed_patterns():
    cases = {
        0x3F80: 1.0,
        0xC000: -2.0,
        0x0001: 2.0 ** -133,
        0x8001: -(2.0 ** -133),
        0x0080: 2.0 ** -126,              # smallest normal
        0x7F80: np.inf,
        0xFF80: -np.inf,
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
        0x3FC0: 1.5,
        0x4049: 3.140625,                 # 1.5703125 * 2
        0x0000: 0.0,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = O.storage_to_f64(bits)
    for b, want, g in zip(cases, cases.values(), got):
        assert g == want, (hex(b), g, want)
    assert np.signbit(O.storage_to_f64(np.array([0x8000], np.uint16)))[0]
    assert np.isnan(O.storage_to_f64(np.array([0x7FC0, 0xFFC1], np.uint16))).all()


def test_fp32_widening_is_the_identity_in_float64():
    x = np.array([1.0, -0.0, 1e-45, 3.4028235e38, np.inf, 0.1], dtype=np.float32)
    got = O.storage_to_f64(x)
    assert np.array_equal(got, x.astype(np.float64))
    assert got.dtype == np.float64


def test_input_rounding_to_bf16_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200_000, dtype=np.float32),
                        rng.standard_normal(20_000, dtype=np.float32) * np.float32(1e30),
                        rng.standard_normal(20_000, dtype=np.float32) * np.float32(1e-38),
                        # exact ties: the halfway bit set, round to even either way
                        (np.arange(1 << 12, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    x = x[np.isfinite(x)]
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
