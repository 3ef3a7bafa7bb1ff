"""Pins for the oracle's number formats (bf16, fp16, OCP E4M3FN).

The oracle writes bf16 and E4M3FN from the format definitions; these tests
check them against torch's independent conversions and against hand-derived
values.  E4M3FN saturation above 448 is the oracle's reading of the pages
(P1, section "FP8 K 路径:不旋转,直接 cast" is silent on overflow).
"""

import numpy as np
import pytest
import torch

from oracle import fpfmt


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = fpfmt.bf16_bits_to_f32(b)
    keep = np.isfinite(x)
    return b[keep], x[keep]


def test_bf16_widening_is_exact():
    b, x = _all_finite_bf16()
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(t.view(np.uint32), x.view(np.uint32))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties
    base = rng.integers(0, 1 << 16, size=2000, dtype=np.uint64).astype(np.uint32) << 16
    extra = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base])
    u = np.concatenate([u, extra])
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    # keep away from overflow to inf (both agree but skip the edge)
    x = x[np.abs(x) < 3.0e38]
    ours = fpfmt.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_go_to_even_by_hand():
    # 1 + 2^-8 is halfway between bf16 1.0 (0x3F80) and 1 + 2^-7 (0x3F81) -> even 0x3F80
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    assert list(fpfmt.f32_to_bf16_bits(x)) == [0x3F80, 0x3F82]


def test_f16_by_hand():
    x = np.array([1e-8, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 1.0, -2.0],
                 dtype=np.float32)
    got = list(fpfmt.f32_to_f16_bits(x))
    # 1e-8 underflows to +0; 65520 is halfway to the next binade -> inf;
    # 2^-24 is the smallest subnormal; 2^-25 ties to even (0); 3*2^-25 ties to 2.
    assert got == [0x0000, 0x7C00, 0x0001, 0x0000, 0x0002, 0x3C00, 0xC000]


def test_e4m3_decode_all_patterns_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = fpfmt.e4m3fn_bits_to_f64(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2           # 0x7F and 0xFF only


def test_e4m3_encode_exhaustive_over_bf16():
    b, x = _all_finite_bf16()
    ours = fpfmt.f32_to_e4m3fn_bits(x)
    inr = np.abs(x) <= 448.0
    ref = torch.from_numpy(x[inr].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[inr], ref)
    # saturation reading: every finite |x| > 448 maps to +-448 (0x7E / 0xFE)
    big = ~inr
    assert np.all(ours[big] == np.where(x[big] > 0, 0x7E, 0xFE))


def test_e4m3_by_hand():
    x = np.array([448.0, 464.0, 1e30, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, -0.0,
                  1.0, 1.0625, 1.1875, np.nan, -np.inf], dtype=np.float32)
    got = [int(v) for v in fpfmt.f32_to_e4m3fn_bits(x)]
    # 448 = S.1111.110; 464 would round up to 480 (not representable) -> saturate;
    # 2^-9 is the smallest subnormal (0x01); 2^-10 ties between 0 and 2^-9 -> 0;
    # 3*2^-10 ties between 0x01 and 0x02 -> 0x02; -0 keeps its sign;
    # 1.0625 ties between 1.0 (0x38) and 1.125 (0x39) -> 0x38;
    # 1.1875 ties between 1.125 (0x39) and 1.25 (0x3A) -> 0x3A.
    assert got == [0x7E, 0x7E, 0x7E, 0x01, 0x00, 0x02, 0x80, 0x38, 0x38, 0x3A, 0x7F, 0xFE]
