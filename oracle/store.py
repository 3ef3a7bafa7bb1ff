"""The store: quantise K and V of each (token, kv head) and write one slot.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

MSE-K path (presets with 3- or 4-bit K), after P1 sections "K 的归一化与旋转
为什么放在 kernel 外面", "二分查找", "位打包" and "向量范数的存储":
  1. x = f32(k)                                  (bf16 widening, exact)
  2. ss = sum of x_i * x_i as a balanced binary tree in index order
     (level by level, a'_i = a_{2i} + a_{2i+1})
  3. nrm = sqrt(ss)                              (correctly rounded)
  4. alpha = (1 / (nrm + 1e-8)) * r_d,  r_d = float32(1 / sqrt(d))
  5. u = s * x                                   (sign flips, exact)
  6. u = FWHT(u), stages h = 1, 2, ..., d/2, butterfly (a + b, a - b)
  7. y_j = u_j * alpha                           (= R k / (|k| + 1e-8))
  8. code_j = #{m : y_j >= mid_m}                (the binary search of the
     page with ">=", so a value equal to a boundary goes right; NaN -> 0)
  9. codes packed LSB-first: code j fills bits [j*b, j*b + b) of the code
     bytes (4-bit: even j in the low nibble; 3-bit: 8 codes -> 3 bytes)
 10. f16(nrm) after the codes (the raw norm: with the array-of-structures
     layout the norm correction is applied when reading)
Every operation above is one binary32 operation rounded to nearest even;
nothing is fused.  vLLM divides each element by (nrm + 1e-8) and rotates
with a GEMM whose summation order is not stated; this contract computes the
same quantities with one reciprocal and a fixed butterfly order, so it
differs from vLLM only in last-bit rounding, i.e. only at ties.

FP8-K path (k8v4; P1, section "FP8 K 路径"): byte_i = e4m3(f32(k_i)); no
norm, no rotation.

V path (P1, section "V 的 min/max 均匀量化"), with Q = 2^vb - 1:
  lo = min v, hi = max v
  sc = (hi - lo) / Q;  if not (sc > 1e-8): sc = 1e-8
  q_i = min(max(trunc((v_i - lo) * (1 / sc) + 0.5), 0), Q)
  codes packed like K codes, then f16(sc), f16(lo) ("zero" is the float
  minimum: a constant vector decodes to lo exactly).  The page divides per
  element; the contract multiplies by one reciprocal.
"""

import numpy as np

from . import fpfmt
from .rotation import fwht_f32_contract, rotation_matrix_f64

F32 = np.float32


def pairwise_sum_f32(a):
    """Balanced binary-tree sum along the last axis (length a power of two)."""
    a = np.asarray(a, dtype=F32)
    while a.shape[-1] > 1:
        a = (a[..., 0::2] + a[..., 1::2]).astype(F32)
    return a[..., 0]


def r_d(d):
    return F32(1.0 / np.sqrt(np.float64(d)))


def bucketize(y, midpoints):
    """code = number of boundaries m with y >= m (boundaries sorted)."""
    y = np.asarray(y, dtype=F32)
    mid = np.asarray(midpoints, dtype=F32)
    return (y[..., None] >= mid).sum(axis=-1).astype(np.int64)


def pack_codes(codes, bits):
    """LSB-first bit stream of b-bit codes along the last axis -> uint8 bytes."""
    codes = np.asarray(codes, dtype=np.int64)
    d = codes.shape[-1]
    nbytes = -(-d * bits // 8)
    out = np.zeros(codes.shape[:-1] + (nbytes,), dtype=np.int64)
    for j in range(d):
        for k in range(bits):
            pos = j * bits + k
            out[..., pos // 8] |= ((codes[..., j] >> k) & 1) << (pos % 8)
    return out.astype(np.uint8)


def unpack_codes(packed, bits, d):
    packed = np.asarray(packed, dtype=np.int64)
    codes = np.zeros(packed.shape[:-1] + (d,), dtype=np.int64)
    for j in range(d):
        for k in range(bits):
            pos = j * bits + k
            codes[..., j] |= ((packed[..., pos // 8] >> (pos % 8)) & 1) << k
    return codes


def quantize_k_contract(k_bits, signs, midpoints):
    """MSE-K steps 1-8 for bf16 K vectors [..., d].  Returns (codes, nrm, y).

    ``signs``: the d rotation signs (seeded-sign Hadamard), or a d x d float32
    matrix Q32 for the Haar rotation (``oracle/haar.py``): then steps 4-7 are
    y = rotate_contract(x, Q32) * (1 / (nrm + 1e-8))."""
    x = fpfmt.bf16_bits_to_f32(k_bits)
    d = x.shape[-1]
    ss = pairwise_sum_f32(x * x)
    nrm = np.sqrt(ss).astype(F32)
    if np.ndim(signs) == 2:
        from .haar import rotate_contract
        inv = (F32(1.0) / (nrm + F32(1e-8))).astype(F32)
        y = (rotate_contract(x, signs) * inv[..., None]).astype(F32)
        return bucketize(y, midpoints), nrm, y
    alpha = ((F32(1.0) / (nrm + F32(1e-8))).astype(F32) * r_d(d)).astype(F32)
    u = (x * np.asarray(signs, dtype=F32)).astype(F32)
    u = fwht_f32_contract(u)
    y = (u * alpha[..., None]).astype(F32)
    return bucketize(y, midpoints), nrm, y


def quantize_v_contract(v_bits, bits):
    """V steps for bf16 V vectors [..., d].  Returns (codes, sc_f32, lo_f32)."""
    v = fpfmt.bf16_bits_to_f32(v_bits)
    qmax = (1 << bits) - 1
    lo = v.min(axis=-1)
    hi = v.max(axis=-1)
    sc = ((hi - lo) / F32(qmax)).astype(F32)
    sc = np.where(sc > F32(1e-8), sc, F32(1e-8)).astype(F32)
    isc = (F32(1.0) / sc).astype(F32)
    t = ((v - lo[..., None]) * isc[..., None]).astype(F32)
    t = (t + F32(0.5)).astype(F32)
    q = np.trunc(t).astype(np.int64)
    q = np.minimum(np.maximum(q, 0), qmax)
    return q, sc, lo


def _u16_le(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return np.stack([(b & 0xFF).astype(np.uint8), (b >> 8).astype(np.uint8)], axis=-1)


def encode_slots(k_bits, v_bits, layout, signs, midpoints):
    """Slot bytes [..., slot_size_aligned] for K/V vectors [..., d]."""
    lead = np.asarray(k_bits).shape[:-1]
    out = np.zeros(lead + (layout.slot_size_aligned,), dtype=np.uint8)
    if layout.key_fp8:
        out[..., :layout.head_dim] = fpfmt.f32_to_e4m3fn_bits(fpfmt.bf16_bits_to_f32(k_bits))
    else:
        codes, nrm, _ = quantize_k_contract(k_bits, signs, midpoints)
        kb = layout.key_code_bytes
        out[..., :kb] = pack_codes(codes, layout.key_bits)
        out[..., kb:kb + 2] = _u16_le(fpfmt.f32_to_f16_bits(nrm))
    vq, sc, lo = quantize_v_contract(v_bits, layout.value_bits)
    o = layout.off_value
    out[..., o:o + layout.value_code_bytes] = pack_codes(vq, layout.value_bits)
    o = layout.off_value_scale
    out[..., o:o + 2] = _u16_le(fpfmt.f32_to_f16_bits(sc))
    out[..., o + 2:o + 4] = _u16_le(fpfmt.f32_to_f16_bits(lo))
    return out


def store_contract(cache, k_bits, v_bits, slot_mapping, layout, signs, midpoints):
    """Scatter the slots of N tokens into ``cache`` (modified in place).

    cache: uint8 [num_blocks, block_size, H, slot]; k_bits, v_bits: uint16
    [N, H, d]; slot_mapping: int [N].  A negative slot is a padding token and
    is skipped (P1, section "写入发生在 attention 之前"); a slot beyond the
    cache is skipped too.  Returns the number of out-of-range slots.
    """
    nb, bs, H, S = cache.shape
    sm = np.asarray(slot_mapping, dtype=np.int64)
    valid = (sm >= 0) & (sm < nb * bs)
    bad = int(((sm >= nb * bs)).sum())
    idx = np.nonzero(valid)[0]
    if len(idx):
        slots = encode_slots(np.asarray(k_bits)[idx], np.asarray(v_bits)[idx],
                             layout, signs, midpoints)
        s = sm[idx]
        cache[s // bs, s % bs] = slots
    return bad


# ----------------------------------------------------------------------------
# float64 reference quantities, for tie analysis
# ----------------------------------------------------------------------------


def rotate_unit_f64(k_bits, signs):
    """y64 = R k / (|k| + 1e-8) in float64 via the explicit rotation matrix
    (``signs`` as in quantize_k_contract)."""
    x = fpfmt.bf16_bits_to_f64(k_bits)
    nrm = np.sqrt((x * x).sum(axis=-1))
    R = rotation_matrix_f64(signs)
    return (x / (nrm + 1e-8)[..., None]) @ R.T


def k_near_tie_mask(y64, midpoints, eps=1e-6):
    """True where a float64 coordinate lies within eps of any boundary."""
    mid = np.asarray(midpoints, dtype=np.float64)
    return (np.abs(np.asarray(y64)[..., None] - mid) < eps).any(axis=-1)


def k_mismatch_is_tie(y64, code_a, code_b, midpoints, eps=1e-6):
    """A K code mismatch is tolerated only between neighbouring codes and only
    when the float64 coordinate is within eps of the boundary between them."""
    mid = np.asarray(midpoints, dtype=np.float64)
    a = np.asarray(code_a, dtype=np.int64)
    b = np.asarray(code_b, dtype=np.int64)
    lo = np.minimum(a, b)
    adj = np.abs(a - b) == 1
    m = mid[np.clip(lo, 0, len(mid) - 1)]
    return adj & (np.abs(np.asarray(y64) - m) < eps)


def v_unit_position_f64(v_bits, bits):
    """(v - lo) / ((hi - lo) / Q) in float64, in code units."""
    v = fpfmt.bf16_bits_to_f64(v_bits)
    qmax = (1 << bits) - 1
    lo = v.min(axis=-1, keepdims=True)
    hi = v.max(axis=-1, keepdims=True)
    sc = (hi - lo) / qmax
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(sc > 1e-8, (v - lo) / np.where(sc > 0, sc, 1.0), 0.0)
    return t


def v_mismatch_is_tie(t64, code_a, code_b, eps=1e-6):
    a = np.asarray(code_a, dtype=np.int64)
    b = np.asarray(code_b, dtype=np.int64)
    adj = np.abs(a - b) == 1
    half = np.minimum(a, b) + 0.5
    return adj & (np.abs(np.asarray(t64) - half) < eps)
