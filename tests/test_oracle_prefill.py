"""Pins for the oracle's full dequantisation and continuation (chunked
prefill) attention, P1 sections "续写 prefill:小 chunk 走 decode,大 chunk 走
反量化" and "反量化 kernel:_tq_full_dequant_kv".

* Dequant, closed form: with the pure Hadamard rotation a key along e_0
  quantises to one code in every coordinate, and the norm-corrected
  dequantised key is that key again (up to the fp16 norm); FP8 keys come back
  as their E4M3 rounding.
* Dequant, statistics: the relative squared error of random keys is the
  codebook's distortion d * MSE (about 0.0095 at 4 bits, 0.035 at 3 bits),
  and every value lies within half a quantisation step of the original.
* Continuation: equals dense causal attention, with an explicit mask, over
  the dequantised keys and values of the whole sequence (slotted and split
  pages).
"""

import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import decode as dec
from oracle import fpfmt, layout, rotation, soa
from oracle import store as st
from packed_cache_decode_amd import synth


def _one_seq(preset, T, H, seed, bs=16, Hq=None):
    Hq = Hq or 2 * H
    w = synth.Workload("t", preset, batch=1, num_q_heads=Hq, num_kv_heads=H, head_dim=128,
                       block_size=bs, seed=seed, len_range=(T, T))
    inp = synth.generate(w)
    lay = layout.slot_layout(preset, 128)
    signs = rotation.rotation_signs(seed + 3, 128)
    kb = 4 if lay.key_fp8 else lay.key_bits
    c, m = cb.codebook(128, kb)
    cache = np.zeros((inp.num_blocks, bs, H, lay.slot_size_aligned), np.uint8)
    st.store_contract(cache, inp.k, inp.v, inp.slot_mapping, lay, signs, m)
    return inp, lay, signs, c, m, cache


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
def test_dequant_axis_key_closed_form(preset):
    d = 128
    lay = layout.slot_layout(preset, d)
    c, m = cb.codebook(d, lay.key_bits)
    k = np.zeros((1, 1, d), np.float32)
    k[0, 0, 0] = 3.0
    v = np.linspace(-1, 1, d, dtype=np.float32)[None, None]
    cache = np.zeros((1, 16, 1, lay.slot_size_aligned), np.uint8)
    st.store_contract(cache, synth.f32_to_bf16_bits(k), synth.f32_to_bf16_bits(v), np.array([0]),
                      lay, np.ones(d), m)
    K, V = dec.dequant_kv_f64(cache, np.array([0]), 1, lay, np.ones(d), c)
    want = np.zeros(d)
    want[0] = 3.0
    # every code is the same bucket; H applied to a constant vector is d e_0,
    # and the corrected norm |k| / (sqrt(d) c) undoes the centroid's size
    assert np.max(np.abs(K[0, 0] - want)) <= 3.0 * 2.0 ** -11
    assert np.max(np.abs(V[0, 0] - v[0, 0])) <= (2.0 / ((1 << lay.value_bits) - 1)) * 0.51


def test_dequant_fp8_keys_are_their_e4m3_rounding():
    inp, lay, signs, c, m, cache = _one_seq("turboquant_k8v4", 50, 2, 7)
    K, _ = dec.dequant_kv_f64(cache, inp.block_table[0], 50, lay, signs, c)
    want = fpfmt.e4m3fn_bits_to_f64(fpfmt.f32_to_e4m3fn_bits(fpfmt.bf16_bits_to_f32(inp.k)))
    assert np.array_equal(K, want)


@pytest.mark.parametrize("preset,dist", [("turboquant_4bit_nc", 0.0095), ("turboquant_k3v4_nc", 0.0346)])
def test_dequant_distortion_and_value_bound(preset, dist):
    T, H = 400, 4
    inp, lay, signs, c, m, cache = _one_seq(preset, T, H, 11)
    K, V = dec.dequant_kv_f64(cache, inp.block_table[0], T, lay, signs, c)
    k = fpfmt.bf16_bits_to_f64(inp.k)
    rel = ((K - k) ** 2).sum(-1) / (k ** 2).sum(-1)
    assert 0.7 * dist < rel.mean() < 1.3 * dist
    v = fpfmt.bf16_bits_to_f64(inp.v)
    step = (v.max(-1) - v.min(-1)) / 15
    assert np.all(np.abs(V - v) <= 0.5 * step[..., None] * 1.01 + 1e-3 * np.abs(v).max())


def _dense_causal(q_bits, K, V, q_len, sm_scale):
    """softmax(q K^T * scale + causal mask) V per query head; K, V [T, H, d]."""
    q = fpfmt.bf16_bits_to_f64(q_bits)                 # [q_len, Hq, d]
    T, H, d = K.shape
    G = q.shape[1] // H
    cached = T - q_len
    out = np.zeros(q.shape)
    mask = np.arange(T)[None, :] <= (cached + np.arange(q_len))[:, None]   # [q_len, T]
    for hq in range(q.shape[1]):
        g = hq // G
        s = q[:, hq] @ K[:, g].T * sm_scale
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        out[:, hq] = (p @ V[:, g]) / p.sum(-1, keepdims=True)
    return out


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_k8v4"])
def test_continuation_is_causal_attention_over_dequantised_cache(preset):
    T, H, q_len = 173, 2, 37
    inp, lay, signs, c, m, cache = _one_seq(preset, T, H, 5, Hq=8)
    rng = np.random.default_rng(1)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((q_len, 8, 128)).astype(np.float32))
    got = dec.decode_continuation_f64(qb, cache, inp.block_table[0], T, lay, signs, c, H)
    K, V = dec.dequant_kv_f64(cache, inp.block_table[0], T, lay, signs, c)
    ref = _dense_causal(qb, K, V, q_len, 1 / math.sqrt(128))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_continuation_split_page():
    preset, T, H, q_len, bs = "turboquant_4bit_nc", 150, 2, 20, 16
    w = synth.Workload("t", preset, batch=1, num_q_heads=4, num_kv_heads=H, head_dim=128,
                       block_size=bs, seed=2, len_range=(T, T))
    inp = synth.generate(w)
    lay = layout.slot_layout(preset, 128)
    signs = rotation.rotation_signs(4, 128)
    c, m = cb.codebook(128, 4)
    pages = np.zeros((inp.num_blocks, soa.soa_page_bytes(lay, bs, H)), np.uint8)
    soa.store_contract(pages, bs, inp.k, inp.v, inp.slot_mapping, lay, signs, m, c)
    rng = np.random.default_rng(3)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((q_len, 4, 128)).astype(np.float32))
    lens = T - q_len + 1 + np.arange(q_len)
    got = soa.decode_f64(qb, pages, np.repeat(inp.block_table[:1], q_len, 0), lens, lay, signs, c, H, bs)
    K, V = soa.dequant_kv_f64(pages, lay, bs, H, inp.block_table[0], T, signs, c)
    ref = _dense_causal(qb, K, V, q_len, 1 / math.sqrt(128))
    assert np.max(np.abs(got - ref)) < 1e-12
