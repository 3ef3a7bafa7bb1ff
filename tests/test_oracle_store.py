"""Pins for the oracle's slot layout and store arithmetic.

* Slot sizes, byte map and page bytes: the pages' own numbers
  (tests/golden/slot_sizes.json; P1 sections "从 slot_size 的三项算术开始",
  "一个 slot 的字节图", "页内寻址"; P5 section "三、TurboQuant").
* Bit packing: the page's group formulas (P1, section "位打包") restated
  here and compared with the oracle's generic LSB-first bit stream.
* The fp32 contract against float64 mathematics: the rotated unit vector
  agrees to ~1e-7 and codes agree everywhere except at near-ties.
* Degenerate cases the pages fix: a constant V vector has scale 1e-8 and
  decodes to its minimum (P1, section "V 的 min/max 均匀量化"); a zero K
  vector lands on the central boundary, which sends it right.
"""

import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import fpfmt, layout, rotation
from oracle import store as st
from conftest import load_golden


def test_slot_sizes_match_pages():
    g = load_golden("slot_sizes.json")
    for name, row in g["presets"].items():
        lay = layout.slot_layout(name, g["head_dim"])
        assert lay.key_packed_size == row["key_data"] + row["key_meta"]
        assert lay.value_packed_size == row["value_data"] + row["value_meta"]
        assert lay.slot_size == row["slot"]
        assert lay.slot_size_aligned == row["slot_aligned"]


def test_k3v4_byte_map_matches_page():
    off = load_golden("slot_sizes.json")["k3v4_byte_map_offsets"]
    lay = layout.slot_layout("turboquant_k3v4_nc", 128)
    assert (0, lay.off_key_norm, lay.off_value, lay.off_value_scale, lay.off_value_zero,
            lay.slot_size) == (off["key_codes"], off["key_norm"], off["value_codes"],
                               off["value_scale"], off["value_zero"], off["end"])


def test_page_bytes_example():
    ex = load_golden("slot_sizes.json")["page_bytes_example"]
    lay = layout.slot_layout("turboquant_k3v4_nc", 128)
    assert layout.page_bytes(lay, ex["block_size"], ex["num_kv_heads"]) == ex["page_bytes"]
    assert ex["block_size"] * ex["num_kv_heads"] * 128 * 2 * 2 == ex["fp16_page_bytes"]


def test_slot_sizes_other_head_dims():
    # ceil(d*b/8) + 2 and ceil(d*b/8) + 4, rounded up to even
    for d in (64, 256):
        assert layout.slot_layout("turboquant_4bit_nc", d).slot_size_aligned == d // 2 + 2 + d // 2 + 4
        assert layout.slot_layout("turboquant_k3v4_nc", d).slot_size_aligned == 3 * d // 8 + 2 + d // 2 + 4
        assert layout.slot_layout("turboquant_k8v4", d).slot_size_aligned == d + d // 2 + 4


def test_pack_matches_page_group_formulas():
    rng = np.random.default_rng(0)
    c3 = rng.integers(0, 8, size=(40, 128))
    # 3-bit: 8 indices -> 24-bit integer sum(idx_k << 3k), then low/mid/high bytes
    grp = c3.reshape(40, 16, 8)
    p24 = (grp << (3 * np.arange(8))).sum(axis=-1)
    want3 = np.stack([p24 & 0xFF, (p24 >> 8) & 0xFF, (p24 >> 16) & 0xFF], axis=-1).reshape(40, 48)
    assert np.array_equal(st.pack_codes(c3, 3), want3.astype(np.uint8))
    # 4-bit: pairs, the first of each pair in the low nibble
    c4 = rng.integers(0, 16, size=(40, 128))
    want4 = (c4[:, 0::2] | (c4[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(st.pack_codes(c4, 4), want4)
    # the worked example of codes 0..7
    assert list(st.pack_codes(np.arange(8)[None], 3)[0]) == [0x88, 0xC6, 0xFA]
    for bits, c in ((3, c3), (4, c4)):
        assert np.array_equal(st.unpack_codes(st.pack_codes(c, bits), bits, 128), c)


def test_pairwise_sum_tree_shape():
    # the tree adds neighbours first: ((a0+a1)+(a2+a3)); with these values the
    # left-to-right order would lose the small terms
    a = np.array([1.0, 2.0 ** -24, 2.0 ** -24, 1.0], dtype=np.float32)
    assert st.pairwise_sum_f32(a[None])[0] == np.float32(2.0)
    b = np.array([2.0 ** -24, 2.0 ** -24, 1.0, 1.0], dtype=np.float32)
    assert st.pairwise_sum_f32(b[None])[0] == np.float32(2.0) + np.float32(2.0 ** -23)


def test_r_d_constant():
    assert st.r_d(128).view(np.uint32) == 0x3DB504F3


def _rand_keys(n, d, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float32)
    if outliers:
        x[:, rng.choice(d, 4, replace=False)] *= 20
        x *= np.exp(0.5 * rng.standard_normal(d)).astype(np.float32)
    return fpfmt.f32_to_bf16_bits(x)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_contract_agrees_with_float64_except_at_ties(bits, d):
    signs = rotation.rotation_signs(42, d)
    c, m = cb.codebook(d, bits)
    kb = _rand_keys(20000 if d == 128 else 6000, d, bits)
    codes, nrm, y32 = st.quantize_k_contract(kb, signs, m)
    y64 = st.rotate_unit_f64(kb, signs)
    assert np.max(np.abs(y32 - y64)) < 2e-7
    codes64 = np.searchsorted(m.astype(np.float64), y64, side="right")
    diff = codes != codes64
    assert np.all(st.k_mismatch_is_tie(y64[diff], codes[diff], codes64[diff], m))
    # the norm: correctly rounded fp32 of a fixed-tree sum, close to float64
    x64 = fpfmt.bf16_bits_to_f64(kb)
    n64 = np.sqrt((x64 * x64).sum(axis=1))
    assert np.max(np.abs(nrm - n64) / n64) < 1e-6


def test_near_tie_rate_is_small():
    d, bits = 128, 4
    c, m = cb.codebook(d, bits)
    kb = _rand_keys(50000, d, 9, outliers=False)
    y64 = st.rotate_unit_f64(kb, rotation.rotation_signs(1, d))
    rate = st.k_near_tie_mask(y64, m).mean()
    # density of N(0, 1/d) at the 15 boundaries times the 2e-6 window ~ 7.6e-5
    dens = sum(math.exp(-x * x * d / 2) * math.sqrt(d / (2 * math.pi)) for x in m.astype(float))
    assert rate < 5 * dens * 2e-6 + 1e-4


def test_zero_key_vector():
    d = 128
    c, m = cb.codebook(d, 4)
    lay = layout.slot_layout("turboquant_4bit_nc", d)
    z = np.zeros((1, d), np.uint16)
    v = fpfmt.f32_to_bf16_bits(np.linspace(-1, 1, d, dtype=np.float32))[None]
    slot = st.encode_slots(z, v, lay, rotation.rotation_signs(5, d), m)[0]
    # y = 0 >= +0.0 (the central boundary): code 8 everywhere -> bytes 0x88
    assert np.all(slot[:64] == 0x88)
    assert slot[64] == 0 and slot[65] == 0


def test_constant_value_vector():
    d = 128
    lay = layout.slot_layout("turboquant_4bit_nc", d)
    c, m = cb.codebook(d, 4)
    k = _rand_keys(1, d, 3)
    v = np.full((1, d), fpfmt.f32_to_bf16_bits(np.float32(0.7)), np.uint16)
    slot = st.encode_slots(k, v, lay, rotation.rotation_signs(5, d), m)[0]
    assert np.all(slot[66:130] == 0)
    sc = int(slot[130]) | int(slot[131]) << 8
    zr = int(slot[132]) | int(slot[133]) << 8
    assert sc == 0                      # f16(1e-8) underflows to +0
    assert fpfmt.f16_bits_to_f64(np.uint16(zr)) == np.float16(fpfmt.bf16_bits_to_f32(v[0, 0]))


@pytest.mark.parametrize("bits", [3, 4])
def test_value_reconstruction_error(bits):
    rng = np.random.default_rng(bits)
    v = fpfmt.f32_to_bf16_bits(rng.standard_normal((5000, 128)).astype(np.float32))
    q, sc, lo = st.quantize_v_contract(v, bits)
    x = fpfmt.bf16_bits_to_f64(v)
    rec = q * sc[:, None].astype(np.float64) + lo[:, None].astype(np.float64)
    assert np.all(np.abs(rec - x) <= sc[:, None] * (0.5 + 1e-5))
    assert q.min() == 0 and q.max() == (1 << bits) - 1


def test_value_rounding_follows_float64_except_at_ties():
    """Away from ties the contract rounds V exactly as float64 does."""
    rng = np.random.default_rng(11)
    v = fpfmt.f32_to_bf16_bits(rng.standard_normal((20000, 128)).astype(np.float32))
    q, _, _ = st.quantize_v_contract(v, 4)
    t = st.v_unit_position_f64(v, 4)
    q64 = np.clip(np.floor(t + 0.5), 0, 15).astype(np.int64)
    diff = q != q64
    # bf16 inputs sit on a coarse grid, so (v - lo) / sc lands exactly on k + 1/2
    # for ~0.2% of coordinates; the contract's last-bit rounding decides those,
    # and only those: every disagreement with float64 is such a tie.
    assert diff.any()
    assert np.all(st.v_mismatch_is_tie(t[diff], q[diff], q64[diff]))


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_key_direction_distortion(bits, d):
    """Reconstructing k / |k| as R^T c(code) gives the codebook's distortion
    (rotation makes every coordinate N(0, 1/d); P1, section "旋转的关键定理")."""
    signs = rotation.rotation_signs(77, d)
    c, m = cb.codebook(d, bits)
    kb = _rand_keys(4000, d, 21)
    codes, nrm, _ = st.quantize_k_contract(kb, signs, m)
    R = rotation.rotation_matrix_f64(signs)
    rec = c.astype(np.float64)[codes] @ R
    x = fpfmt.bf16_bits_to_f64(kb)
    unit = x / np.linalg.norm(x, axis=1, keepdims=True)
    nmse = ((rec - unit) ** 2).sum(axis=1).mean()
    assert nmse < math.sqrt(3) * math.pi / 2 * 2.0 ** (-2 * bits)
    assert abs(nmse - {3: 0.0345, 4: 0.0095}[bits]) < 0.15 * {3: 0.0345, 4: 0.0095}[bits]


def test_store_scatter_and_skip():
    d, H, bs, nb = 128, 2, 16, 4
    lay = layout.slot_layout("turboquant_4bit_nc", d)
    c, m = cb.codebook(d, 4)
    signs = rotation.rotation_signs(3, d)
    rng = np.random.default_rng(2)
    k = fpfmt.f32_to_bf16_bits(rng.standard_normal((5, H, d)).astype(np.float32))
    v = fpfmt.f32_to_bf16_bits(rng.standard_normal((5, H, d)).astype(np.float32))
    cache = np.full((nb, bs, H, lay.slot_size_aligned), 0xA5, np.uint8)
    sm = np.array([0, -1, 17, 63, 64])
    bad = st.store_contract(cache, k, v, sm, lay, signs, m)
    assert bad == 1
    slots = st.encode_slots(k, v, lay, signs, m)
    assert np.array_equal(cache[0, 0], slots[0])
    assert np.array_equal(cache[1, 1], slots[2])
    assert np.array_equal(cache[3, 15], slots[3])
    touched = np.zeros(cache.shape[:2], bool)
    touched[0, 0] = touched[1, 1] = touched[3, 15] = True
    assert np.all(cache[~touched] == 0xA5)
