"""Number formats used by the packed cache, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* bfloat16: the upper 16 bits of an IEEE binary32.  Widening is exact;
  narrowing rounds to nearest, ties to even.  K, V and q arrive as bf16 and
  the decode output leaves as bf16 (P1, section "后端能力声明" lists fp16 and
  bf16 as the supported activation dtypes).
* binary16 (fp16): the K norm, the V scale and the V zero are stored as fp16
  (P1, section "元数据为什么用 fp16 而不是 fp32").  Narrowing from fp32 is
  IEEE round-to-nearest-even with subnormals; overflow gives +-inf.  numpy's
  float16 conversion is that IEEE operation and is used as the primitive.
* OCP FP8 E4M3FN: the k8v4 preset stores K as one e4m3 byte per element
  (P1, section "FP8 K 路径:不旋转,直接 cast").  Bias 7, no infinities, the
  only NaN patterns are S.1111.111, largest finite 448.  The pages do not say
  what happens above 448; the reading taken here is saturation to +-448
  (the conversion the pages' store kernel relies on saturates on the GPUs it
  names), NaN stays NaN, and the sign of zero is kept.
"""

import numpy as np

# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------


def bf16_bits_to_f32(bits):
    """Exact widening: the bf16 pattern becomes the high half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """Round binary32 to bf16, nearest-even.  NaN becomes a quiet NaN.

    Written as the choice between the two bf16 neighbours of x: the value
    truncated toward zero (drop the low 16 bits) and the next pattern up in
    magnitude.  The low half decides: below 0x8000 keep the truncation,
    above it round up, exactly 0x8000 round to the even pattern.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    trunc = u >> np.uint64(16)
    low = u & np.uint64(0xFFFF)
    up = (low > 0x8000) | ((low == 0x8000) & ((trunc & np.uint64(1)) == 1))
    out = trunc + up.astype(np.uint64)
    nan = np.isnan(x)
    out = np.where(nan, (trunc | np.uint64(0x0040)), out)
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


# ----------------------------------------------------------------------------
# binary16
# ----------------------------------------------------------------------------


def f32_to_f16_bits(x):
    """IEEE binary32 -> binary16, round to nearest even (numpy primitive)."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        return x.astype(np.float16).view(np.uint16)


def f16_bits_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f16_bits_to_f32(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ----------------------------------------------------------------------------
# OCP FP8 E4M3FN
# ----------------------------------------------------------------------------


def e4m3fn_bits_to_f64(bits):
    """Decode E4M3FN bytes from the field definition.

    exponent field e (4 bits), mantissa m (3 bits), bias 7:
      e == 0          -> (-1)^s * m/8 * 2^(1-7)          (subnormal)
      e == 15, m == 7 -> NaN
      otherwise       -> (-1)^s * (1 + m/8) * 2^(e-7)
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** (1 - 7),
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# the 127 finite non-negative patterns 0x00..0x7E, in increasing order of value
_E4M3_POS_VALUES = e4m3fn_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
E4M3_MAX = 448.0


def f32_to_e4m3fn_bits(x):
    """Round to the nearest finite E4M3FN value, ties to the even pattern.

    Plain nearest-value search over the 127 non-negative finite values (the
    patterns are monotone in value, so a pattern is its index in the sorted
    list and "even pattern" is "even index").  |x| above 448 (inf included)
    saturates to 448; NaN gives the NaN pattern with x's sign.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    vals = _E4M3_POS_VALUES
    hi = np.searchsorted(vals, a, side="left")          # vals[hi] >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == vals[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)
