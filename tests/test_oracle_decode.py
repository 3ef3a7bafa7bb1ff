"""Pins for the oracle's float64 paged decode attention.

* Rotated-domain identity (P1, section "分数计算"; P5, section "三、
  TurboQuant"): scoring the rotated query against centroids equals scoring
  the original query against the dequantised key n R^T c.
* Brute force: an independent dense attention (torch, float64) over K and V
  rebuilt from the store's codes (not from the cache bytes) agrees to 1e-12.
* The quantised attention approximates the unquantised one.
* Split-KV invariance of the LSE combine (P1, sections "读取内核", "在线
  softmax"), and the special cases T = 1, q = 0, empty sequence, and a key
  along e_0 with pure Hadamard where norm correction makes the score exact.
"""

import math

import numpy as np
import pytest
import torch

from oracle import codebook as cb
from oracle import decode as dec
from oracle import fpfmt, layout, rotation
from oracle import store as st
from packed_cache_decode_amd import synth


def _tiny_case(preset="turboquant_4bit_nc", T=77, H=2, Hq=4, seed=0, permute=True, d=128):
    w = synth.Workload("t", preset, batch=3, num_q_heads=Hq, num_kv_heads=H, head_dim=d,
                       block_size=16, seed=seed, len_range=(1, T), permute_pages=permute)
    inp = synth.generate(w)
    lay = layout.slot_layout(preset, d)
    signs = rotation.rotation_signs(seed + 11, d)
    kb = lay.key_bits if not lay.key_fp8 else 4
    c, m = cb.codebook(d, kb)
    cache = np.zeros((inp.num_blocks, 16, H, lay.slot_size_aligned), np.uint8)
    st.store_contract(cache, inp.k, inp.v, inp.slot_mapping, lay, signs, m)
    return inp, lay, signs, c, m, cache


def _dense_reference(inp, lay, signs, c, m, sm_scale):
    """Attention over K and V rebuilt from the store's own codes, in torch."""
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
            kb = inp.k[a:e, g]
            if lay.key_fp8:
                K = torch.from_numpy(fpfmt.e4m3fn_bits_to_f64(
                    fpfmt.f32_to_e4m3fn_bits(fpfmt.bf16_bits_to_f32(kb))))
            else:
                codes, nrm, _ = st.quantize_k_contract(kb, signs, m)
                ct = torch.from_numpy(c.astype(np.float64)[codes])
                n = torch.from_numpy(fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(nrm)))
                if lay.norm_correction:
                    n = n / torch.sqrt((ct * ct).sum(-1) + 1e-16)
                K = n[:, None] * (ct @ R)            # n R^T c, as rows
            vq, sc, lo = st.quantize_v_contract(inp.v[a:e, g], lay.value_bits)
            sc16 = torch.from_numpy(fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(sc)))
            lo16 = torch.from_numpy(fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(lo)))
            V = torch.from_numpy(vq.astype(np.float64)) * sc16[:, None] + lo16[:, None]
            qs = q[b, g * G:(g + 1) * G]
            p = torch.softmax(qs @ K.T * sm_scale, dim=-1)
            out[b, g * G:(g + 1) * G] = p @ V
    return out.numpy()


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_k8v4",
                                    "turboquant_3bit_nc"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode_matches_dense_bruteforce(preset, d):
    inp, lay, signs, c, m, cache = _tiny_case(preset, d=d)
    got = dec.decode_f64(inp.q, cache, inp.block_table, inp.seq_lens, lay, signs, c, 2)
    ref = _dense_reference(inp, lay, signs, c, m, 1 / math.sqrt(d))
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("preset,tol", [("turboquant_4bit_nc", 0.15), ("turboquant_k3v4_nc", 0.3),
                                        ("turboquant_k8v4", 0.1)])
def test_decode_approximates_unquantised_attention(preset, tol):
    inp, lay, signs, c, m, cache = _tiny_case(preset, T=200, seed=3)
    got = dec.decode_f64(inp.q, cache, inp.block_table, inp.seq_lens, lay, signs, c, 2)
    q = fpfmt.bf16_bits_to_f64(inp.q)
    offs = inp.token_offsets()
    errs = []
    for b in range(inp.q.shape[0]):
        a, e = offs[b], offs[b + 1]
        for h in range(4):
            K = fpfmt.bf16_bits_to_f64(inp.k[a:e, h // 2])
            V = fpfmt.bf16_bits_to_f64(inp.v[a:e, h // 2])
            s = K @ q[b, h] / math.sqrt(128)
            p = np.exp(s - s.max())
            o = p @ V / p.sum()
            errs.append(np.linalg.norm(got[b, h] - o) / max(np.linalg.norm(o), 1e-3))
    assert np.median(errs) < tol


def test_rotated_domain_identity():
    inp, lay, signs, c, m, cache = _tiny_case()
    slots = dec.gather_slots(cache, inp.block_table[0], int(inp.seq_lens[0]), 1)
    ct, n = dec.dequant_keys(slots, lay, c)
    R = rotation.rotation_matrix_f64(signs)
    q = fpfmt.bf16_bits_to_f64(inp.q[0, 2:4])
    s_rot = dec.scores_f64(q, (ct, n), lay, signs, 0.37)
    K = n[:, None] * (ct @ R)
    s_orig = 0.37 * q @ K.T
    assert np.max(np.abs(s_rot - s_orig)) < 1e-12 * max(1.0, np.abs(s_orig).max())


def test_split_invariance():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((3, 300)) * 4
    v = rng.standard_normal((300, 128))
    ref = dec.attend_f64(s, v)
    for bounds in ([(0, 300)], [(0, 7), (7, 7), (7, 150), (150, 300)],
                   [(i, min(i + 16, 300)) for i in range(0, 320, 16)]):
        got = dec.combine_partials(dec.split_partials(s, v, bounds))
        assert np.max(np.abs(got - ref)) < 1e-12


def test_single_token_and_zero_query():
    inp, lay, signs, c, m, cache = _tiny_case()
    T = int(inp.seq_lens[0])
    slots = dec.gather_slots(cache, inp.block_table[0], T, 0)
    vh = dec.dequant_values(slots, lay)
    # T = 1: the output is that token's dequantised value
    one = dec.decode_f64(inp.q, cache, inp.block_table, np.array([1, 0, 0]), lay, signs, c, 2)
    assert np.max(np.abs(one[0, 0] - vh[0])) < 1e-15
    # empty sequences give zeros
    assert np.all(one[1:] == 0)
    # q = 0: uniform weights, the mean of the values
    zq = np.zeros_like(inp.q)
    out = dec.decode_f64(zq, cache, inp.block_table, inp.seq_lens, lay, signs, c, 2)
    assert np.max(np.abs(out[0, 0] - vh.mean(axis=0))) < 1e-12


def test_axis_key_is_exact_with_norm_correction():
    """Pure Hadamard, K = a e_0: every rotated coordinate is 1/sqrt(d), all
    codes are equal, the normalised centroid vector is exactly R e_0, and the
    score is sm_scale * f16(a) * q_0 whatever the codebook."""
    d = 128
    lay = layout.slot_layout("turboquant_4bit_nc", d)
    signs = rotation.rotation_signs(0, d, sign_flip=False)
    c, m = cb.codebook(d, 4)
    a = [3.0, 5.0]
    k = np.zeros((2, 1, d), np.float32)
    k[0, 0, 0], k[1, 0, 0] = a
    kb = fpfmt.f32_to_bf16_bits(k)
    vb = fpfmt.f32_to_bf16_bits(np.stack([np.full((1, d), 1.0), np.full((1, d), -2.0)]).astype(np.float32))
    cache = np.zeros((1, 16, 1, lay.slot_size_aligned), np.uint8)
    st.store_contract(cache, kb, vb, np.array([0, 1]), lay, signs, m)
    codes = st.unpack_codes(cache[0, :2, 0, :64], 4, d)
    assert np.all(codes == codes[0, 0])
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 0.9
    q[0, 0, 5] = 7.0                     # orthogonal to both keys
    out = dec.decode_f64(fpfmt.f32_to_bf16_bits(q), cache, np.array([[0]]), np.array([2]),
                         lay, signs, c, 1)
    s = np.array(a) * fpfmt.bf16_bits_to_f64(fpfmt.f32_to_bf16_bits(np.float32(0.9))) / math.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    want = p[0] * 1.0 + p[1] * -2.0      # constant V vectors decode exactly
    assert np.max(np.abs(out[0, 0] - want)) < 1e-12
