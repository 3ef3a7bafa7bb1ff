"""Pins for the oracle's structure-of-arrays layout and folded norm.

* Page size (P1, section "AoS 与 SoA:两种页内布局"): the split page is as
  large as the AoS page, the page's 16 x 8 x 118 = 15104-byte example
  included, with a meta region of H x 3 x block_size fp16.
* Placement: every field an SoA store writes equals the field the AoS store
  (pinned on its own) writes for the same vector: data region = K codes then
  V codes, meta region = [H][norm, scale, zero][row].  With norm correction
  switched off the norm field is the AoS norm itself.
* Folded norm (P1, section "SoA 的另一项收益:把 norm correction 折进写入端"):
  against float64 |k| / |c| (within one fp16 rounding), and in closed form
  for a key along e_0 under the pure Hadamard rotation, where every
  coordinate is 1/sqrt(d) and all codes are the bucket of that value.
* Decode: equals a dense float64 attention over keys rebuilt in the original
  space as n R^T c and values code * scale + zero; and stays within the
  fp16 norm rounding of the AoS decode on the same inputs.
"""

import math
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import codebook as cb
from oracle import decode as dec
from oracle import fpfmt, layout, rotation, soa
from oracle import store as st
from packed_cache_decode_amd import synth

from conftest import load_golden

MSE_PRESETS = ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"]


@pytest.mark.parametrize("preset", MSE_PRESETS)
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bs,H", [(16, 1), (16, 8), (32, 4), (128, 2)])
def test_soa_page_is_aos_page_size(preset, d, bs, H):
    lay = layout.slot_layout(preset, d)
    assert soa.soa_page_bytes(lay, bs, H) == layout.page_bytes(lay, bs, H)
    assert soa.soa_page_bytes(lay, bs, H) - soa.meta_offset(lay, bs, H) == H * 3 * bs * 2


def test_soa_page_example():
    ex = load_golden("slot_sizes.json")["page_bytes_example"]
    lay = layout.slot_layout("turboquant_k3v4_nc", 128)
    assert soa.soa_page_bytes(lay, ex["block_size"], ex["num_kv_heads"]) == ex["page_bytes"]
    # data region 16 x 8 x (48 + 64), meta region 8 x 3 x 16 fp16
    assert soa.meta_offset(lay, 16, 8) == 16 * 8 * 112
    assert ex["page_bytes"] - soa.meta_offset(lay, 16, 8) == 768


def test_soa_rejects_fp8_keys():
    with pytest.raises(ValueError):
        soa.soa_page_bytes(layout.slot_layout("turboquant_k8v4", 128), 16, 8)


def _fill_both(preset, d=128, H=4, bs=16, seed=3, N=200, nc=True):
    w = synth.Workload("t", preset, batch=2, num_q_heads=2 * H, num_kv_heads=H, head_dim=d,
                       block_size=bs, seed=seed, len_range=(N // 2, N // 2))
    inp = synth.generate(w)
    lay = layout.slot_layout(preset, d)
    if not nc:
        lay = replace(lay, norm_correction=False)
    signs = rotation.rotation_signs(seed + 5, d)
    c, m = cb.codebook(d, lay.key_bits)
    aos = np.zeros((inp.num_blocks, bs, H, lay.slot_size_aligned), np.uint8)
    st.store_contract(aos, inp.k, inp.v, inp.slot_mapping, lay, signs, m)
    pages = np.zeros((inp.num_blocks, soa.soa_page_bytes(lay, bs, H)), np.uint8)
    soa.store_contract(pages, bs, inp.k, inp.v, inp.slot_mapping, lay, signs, m, c)
    return inp, lay, signs, c, m, aos, pages


def _u16(b):
    return b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)


@pytest.mark.parametrize("preset", MSE_PRESETS)
@pytest.mark.parametrize("nc", [True, False])
def test_soa_fields_match_aos_store(preset, nc):
    H, bs = 4, 16
    inp, lay, signs, c, m, aos, pages = _fill_both(preset, H=H, bs=bs, nc=nc)
    kd, vd = lay.key_code_bytes, lay.value_code_bytes
    mo = bs * H * (kd + vd)
    for s in inp.slot_mapping:
        p, r = divmod(int(s), bs)
        for h in range(H):
            slot = aos[p, r, h]
            data = pages[p, (r * H + h) * (kd + vd):(r * H + h + 1) * (kd + vd)]
            assert np.array_equal(data[:kd], slot[:kd])
            assert np.array_equal(data[kd:], slot[lay.off_value:lay.off_value + vd])
            meta = pages[p, mo:].view("<u2").reshape(H, 3, bs)
            assert meta[h, 1, r] == _u16(slot[lay.off_value_scale:lay.off_value_scale + 2])
            assert meta[h, 2, r] == _u16(slot[lay.off_value_zero:lay.off_value_zero + 2])
            if not nc:
                assert meta[h, 0, r] == _u16(slot[lay.off_key_norm:lay.off_key_norm + 2])
    # nothing outside the stored rows was written
    used = np.zeros(pages.shape, bool)
    for s in inp.slot_mapping:
        p, r = divmod(int(s), bs)
        used[p, r * H * (kd + vd):(r + 1) * H * (kd + vd)] = True
        for h in range(H):
            for f in range(3):
                o = mo + 2 * ((h * 3 + f) * bs + r)
                used[p, o:o + 2] = True
    assert not pages[~used].any()


@pytest.mark.parametrize("preset", MSE_PRESETS)
def test_folded_norm_against_float64(preset):
    d, H = 128, 8
    w = synth.Workload("t", preset, batch=4, num_q_heads=H, num_kv_heads=H, head_dim=d,
                       block_size=16, seed=21, len_range=(256, 256))
    inp = synth.generate(w)
    lay = layout.slot_layout(preset, d)
    signs = rotation.rotation_signs(9, d)
    c, m = cb.codebook(d, lay.key_bits)
    data, n16, _, _ = soa.encode_fields(inp.k, inp.v, lay, signs, m, c)
    codes = st.unpack_codes(data[..., :lay.key_code_bytes], lay.key_bits, d)
    x = fpfmt.bf16_bits_to_f64(inp.k)
    exact = np.sqrt((x * x).sum(-1)) / np.sqrt((c.astype(np.float64)[codes] ** 2).sum(-1))
    got = fpfmt.f16_bits_to_f64(n16)
    rel = np.abs(got - exact) / exact
    # one fp16 rounding (2^-11 relative) plus the fp32 steps before it
    assert rel.max() <= 2.0 ** -11 * (1 + 1e-4)
    same = got == fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(exact.astype(np.float32)))
    assert same.mean() > 0.999


@pytest.mark.parametrize("preset,code", [("turboquant_4bit_nc", 11), ("turboquant_k3v4_nc", 5),
                                         ("turboquant_3bit_nc", 5)])
def test_folded_norm_closed_form_e0(preset, code):
    # pure Hadamard, k = 3 e_0: y_j = 3 / (3 + 1e-8) / sqrt(128) ~ 0.0884 for every
    # j.  4 bits: 7 negative midpoints, then 0, 0.0228, 0.0462, 0.0707 lie at or
    # below it (0.0972 above): code 11.  3 bits: 3 negative midpoints, then 0 and
    # 0.0442 (0.0928 above): code 5.
    d = 128
    lay = layout.slot_layout(preset, d)
    c, m = cb.codebook(d, lay.key_bits)
    k = np.zeros((1, d), np.float32)
    k[0, 0] = 3.0
    kb = synth.f32_to_bf16_bits(k)
    v = synth.f32_to_bf16_bits(np.linspace(-1, 1, d, dtype=np.float32)[None])
    data, n16, _, _ = soa.encode_fields(kb, v, lay, np.ones(d), m, c)
    codes = st.unpack_codes(data[..., :lay.key_code_bytes], lay.key_bits, d)
    assert np.all(codes == code)
    want = 3.0 / (math.sqrt(d) * float(c[code]))
    got = float(fpfmt.f16_bits_to_f64(n16)[0])
    assert abs(got - want) <= want * 2.0 ** -11


def _dense_soa_reference(inp, lay, signs, c, m, sm_scale):
    """Dense attention over keys n R^T c and values code * scale + zero, in
    the original space, rebuilt from the store steps (not the page bytes)."""
    B, Hq, d = inp.q.shape
    H = inp.k.shape[1]
    G = Hq // H
    R = torch.from_numpy(rotation.rotation_matrix_f64(signs))
    q = torch.from_numpy(fpfmt.bf16_bits_to_f64(inp.q))
    offs = inp.token_offsets()
    out = torch.zeros(B, Hq, d, dtype=torch.float64)
    for b in range(B):
        a, e = offs[b], offs[b + 1]
        for g in range(H):
            codes, nrm, _ = st.quantize_k_contract(inp.k[a:e, g], signs, m)
            n = soa.folded_norm_contract(codes, nrm, c)
            n = torch.from_numpy(fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(n)))
            K = n[:, None] * (torch.from_numpy(c.astype(np.float64)[codes]) @ R)
            vq, sc, lo = st.quantize_v_contract(inp.v[a:e, g], lay.value_bits)
            sc16 = torch.from_numpy(fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(sc)))
            lo16 = torch.from_numpy(fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(lo)))
            V = torch.from_numpy(vq.astype(np.float64)) * sc16[:, None] + lo16[:, None]
            p = torch.softmax(q[b, g * G:(g + 1) * G] @ K.T * sm_scale, dim=-1)
            out[b, g * G:(g + 1) * G] = p @ V
    return out.numpy()


@pytest.mark.parametrize("preset", MSE_PRESETS)
def test_soa_decode_matches_dense_bruteforce(preset):
    H, bs = 2, 16
    w = synth.Workload("t", preset, batch=3, num_q_heads=4, num_kv_heads=H, head_dim=128,
                       block_size=bs, seed=4, len_range=(1, 77))
    inp = synth.generate(w)
    lay = layout.slot_layout(preset, 128)
    signs = rotation.rotation_signs(15, 128)
    c, m = cb.codebook(128, lay.key_bits)
    pages = np.zeros((inp.num_blocks, soa.soa_page_bytes(lay, bs, H)), np.uint8)
    soa.store_contract(pages, bs, inp.k, inp.v, inp.slot_mapping, lay, signs, m, c)
    got = soa.decode_f64(inp.q, pages, inp.block_table, inp.seq_lens, lay, signs, c, H, bs)
    ref = _dense_soa_reference(inp, lay, signs, c, m, 1 / math.sqrt(128))
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("preset", MSE_PRESETS)
def test_soa_decode_close_to_aos_decode(preset):
    H, bs = 4, 16
    inp, lay, signs, c, m, aos, pages = _fill_both(preset, H=H, bs=bs, N=300, seed=8)
    a = dec.decode_f64(inp.q, aos, inp.block_table, inp.seq_lens, lay, signs, c, H)
    s = soa.decode_f64(inp.q, pages, inp.block_table, inp.seq_lens, lay, signs, c, H, bs)
    # the two differ only in where the norm is rounded to fp16 (|k| before the
    # correction, or |k| / |c| after it): scores agree to ~2^-10 relative
    assert np.max(np.abs(a - s)) < 2e-2
    assert np.mean(np.abs(a - s)) < 2e-3
