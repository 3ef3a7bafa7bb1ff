"""Pins for the oracle's Haar rotation (``oracle/haar.py``).

* The Gaussian stream is standard normal (moments, Kolmogorov-Smirnov).
* Q is orthogonal (float64 to 1e-13, its float32 rounding to 1e-6) and
  reproducible from the seed.
* Haar law: the first coordinate of a fixed unit vector rotated by Q, over
  many seeds, follows the sphere marginal of dimension d (which fails without
  the sign correction of the QR factor).
* The fp32 rotation contract equals the float64 product within fp32 error,
  and the K codes it gives match float64 bucketing except at ties.
* Decode with the Haar rotation equals dense attention over keys rebuilt as
  n Q^T c.
"""

import math

import numpy as np
import pytest
from scipy import stats

from oracle import codebook as cb
from oracle import decode as dec
from oracle import fpfmt, haar, layout
from oracle import store as st
from packed_cache_decode_amd import synth


def test_gaussian_stream_is_standard_normal():
    g = haar.gaussian_stream(12345, 200000)
    assert abs(g.mean()) < 0.01
    assert abs(g.var() - 1.0) < 0.01
    assert stats.kstest(g, "norm").pvalue > 1e-3


def test_q_is_orthogonal_and_reproducible():
    Q = haar.haar_matrix_f64(7, 128)
    assert np.max(np.abs(Q.T @ Q - np.eye(128))) < 1e-13
    Q32 = haar.haar_matrix_f32(7, 128).astype(np.float64)
    assert np.max(np.abs(Q32.T @ Q32 - np.eye(128))) < 1e-6
    assert np.array_equal(haar.haar_matrix_f32(7, 128), haar.haar_matrix_f32(7, 128))
    assert not np.array_equal(haar.haar_matrix_f32(7, 128), haar.haar_matrix_f32(8, 128))


def test_haar_law_of_a_rotated_coordinate():
    d, n = 8, 3000
    x = np.array([haar.haar_matrix_f64(s, d)[0, 0] for s in range(n)])
    a = (d - 3) / 2.0
    # CDF of the sphere marginal: P(X <= t) = 1/2 + sign(t)/2 * I_{t^2}(1/2, a + 1)
    from scipy.special import betainc
    cdf = lambda t: 0.5 + 0.5 * np.sign(t) * betainc(0.5, a + 1.0, t * t)
    assert stats.kstest(x, cdf).pvalue > 1e-3


def test_rotation_contract_against_float64():
    rng = np.random.default_rng(0)
    Q32 = haar.haar_matrix_f32(3, 128)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    got = haar.rotate_contract(x, Q32).astype(np.float64)
    want = x.astype(np.float64) @ Q32.astype(np.float64).T
    assert np.max(np.abs(got - want)) < 1e-5 * np.abs(x).sum(-1).max() / 8


def test_haar_codes_match_float64_except_ties():
    w = synth.Workload("t", "turboquant_4bit_nc", batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128,
                       block_size=16, seed=5, len_range=(200, 200))
    inp = synth.generate(w)
    Q32 = haar.haar_matrix_f32(11, 128)
    c, m = cb.codebook(128, 4)
    codes, nrm, y = st.quantize_k_contract(inp.k, Q32, m)
    y64 = st.rotate_unit_f64(inp.k, Q32)
    c64 = st.bucketize(y64.astype(np.float32), m)
    diff = codes != c64
    if diff.any():
        assert st.k_mismatch_is_tie(y64[diff], codes[diff], c64[diff], m).all()
    assert np.abs(y - y64).max() < 1e-6


def test_haar_decode_matches_dense():
    import torch
    preset, H = "turboquant_k3v4_nc", 2
    w = synth.Workload("t", preset, batch=2, num_q_heads=4, num_kv_heads=H, head_dim=128,
                       block_size=16, seed=6, len_range=(1, 90))
    inp = synth.generate(w)
    lay = layout.slot_layout(preset, 128)
    Q32 = haar.haar_matrix_f32(21, 128)
    c, m = cb.codebook(128, 3)
    cache = np.zeros((inp.num_blocks, 16, H, lay.slot_size_aligned), np.uint8)
    st.store_contract(cache, inp.k, inp.v, inp.slot_mapping, lay, Q32, m)
    got = dec.decode_f64(inp.q, cache, inp.block_table, inp.seq_lens, lay, Q32, c, H)
    q = fpfmt.bf16_bits_to_f64(inp.q)
    offs = inp.token_offsets()
    Qd = Q32.astype(np.float64)
    for b in range(2):
        for g in range(H):
            kk = inp.k[offs[b]:offs[b + 1], g]
            codes, nrm, _ = st.quantize_k_contract(kk, Q32, m)
            ct = c.astype(np.float64)[codes]
            n = fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(nrm)) / np.sqrt((ct * ct).sum(-1) + 1e-16)
            K = n[:, None] * (ct @ Qd)                      # rows n Q^T c
            vq, sc, lo = st.quantize_v_contract(inp.v[offs[b]:offs[b + 1], g], lay.value_bits)
            V = vq * fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(sc))[:, None] + \
                fpfmt.f16_bits_to_f64(fpfmt.f32_to_f16_bits(lo))[:, None]
            for h in range(2 * g, 2 * g + 2):
                s = q[b, h] @ K.T / math.sqrt(128)
                p = np.exp(s - s.max())
                assert np.max(np.abs(got[b, h] - (p @ V) / p.sum())) < 1e-12
