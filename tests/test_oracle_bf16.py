"""Pins for the oracle's bf16 rounding: torch's CPU float32 -> bfloat16 conversion
(round to nearest even, an independent library routine) on float32 values, plus
hand-built ties, subnormals, overflow, signed zero and NaN."""
import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, f64_to_bf16_rne


def torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_decode_all_patterns_roundtrip():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f64(bits)
    finite = np.isfinite(vals)
    back = f64_to_bf16_rne(vals)
    assert np.array_equal(back[finite], bits[finite])
    # infinities keep their sign, NaNs stay NaN
    inf = np.isinf(vals)
    assert np.array_equal(back[inf], bits[inf])
    assert np.all(np.isnan(bf16_to_f64(back[np.isnan(vals)])))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_f32_matches_torch(seed):
    rng = np.random.default_rng(seed)
    # random bit patterns cover every exponent, including subnormals
    raw = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x32 = raw.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    ours = f64_to_bf16_rne(x32.astype(np.float64))
    ref = torch_bf16_bits(x32)
    assert np.array_equal(ours, ref)


def test_ties_subnormals_overflow():
    cases = np.array([
        0x3F808000,  # exact midpoint 1 + 2^-8: ties to even -> 0x3F80
        0x3F818000,  # midpoint above an odd mantissa -> rounds up to 0x3F82
        0x3F808001,  # just above the midpoint -> up
        0x3F807FFF,  # just below -> down
        0x00008000,  # fp32 subnormal midpoint
        0x00018000,
        0x00000001,  # tiniest fp32 subnormal -> 0
        0x7F7FFFFF,  # fp32 max -> overflows to inf in bf16
        0x7F7F7FFF,  # just below the bf16 overflow midpoint -> bf16 max
        0x80000000,  # -0.0
        0xBF808000,  # negative tie
    ], dtype=np.uint32)
    x32 = cases.view(np.float32)
    assert np.array_equal(f64_to_bf16_rne(x32.astype(np.float64)), torch_bf16_bits(x32))
    assert f64_to_bf16_rne(np.array([np.nan]))[0] == 0x7FC0


def test_float64_tie_not_double_rounded():
    # 1 + 2^-8 + 2^-40 is above the bf16 midpoint but rounds to the midpoint in fp32;
    # direct rounding must go up, a double rounding would go down.
    x = 1.0 + 2.0**-8 + 2.0**-40
    assert f64_to_bf16_rne(np.array([x]))[0] == 0x3F81
