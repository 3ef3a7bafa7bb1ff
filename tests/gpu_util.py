"""Helpers shared by the GPU parity tests (imported by tests only).

Inputs come from ``packed_cache_decode_amd.synth``; expected values come from
``oracle`` alone.  The HIP side is reached through the C ABI (the ctypes
binding and its thin torch wrapper).
"""

import math

import numpy as np

from oracle import codebook as cb
from oracle import decode as odec
from oracle import fpfmt, haar, layout, rotation
from oracle import store as ost

CANARY = 0xA5


def to_dev(a, dtype=None):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class OracleSide:
    """The oracle's own tables and layout for one context's parameters."""

    def __init__(self, preset, head_dim, rot_seed, sign_flip=True, codebook_mode="exact"):
        self.lay = layout.slot_layout(preset, head_dim)
        if sign_flip == "haar" and not self.lay.key_fp8:
            # the rotation is the oracle's own Haar matrix, passed where the signs go
            self.signs = haar.haar_matrix_f32(rot_seed, head_dim)
        else:
            self.signs = rotation.rotation_signs(rot_seed, head_dim, sign_flip not in (False, 0, "hadamard"))
        kb = 4 if self.lay.key_fp8 else self.lay.key_bits
        self.centroids, self.midpoints = cb.codebook(head_dim, kb, codebook_mode)

    def encode(self, k, v, chunk=65536):
        """Slot bytes [N, H, slot] in chunks (bounded memory)."""
        out = np.empty(k.shape[:-1] + (self.lay.slot_size_aligned,), np.uint8)
        for a in range(0, k.shape[0], chunk):
            out[a:a + chunk] = ost.encode_slots(k[a:a + chunk], v[a:a + chunk], self.lay,
                                                self.signs, self.midpoints)
        return out

    def store(self, cache, k, v, slot_mapping, chunk=65536):
        bad = 0
        for a in range(0, k.shape[0], chunk):
            bad += ost.store_contract(cache, k[a:a + chunk], v[a:a + chunk],
                                      slot_mapping[a:a + chunk], self.lay, self.signs, self.midpoints)
        return bad

    def decode(self, q, cache, block_table, seq_lens, num_kv_heads, sm_scale=None, heads=None):
        return odec.decode_f64(q, cache, block_table, seq_lens, self.lay, self.signs,
                               self.centroids, num_kv_heads, sm_scale, heads)


def compare_slots(got, want, k_bits, v_bits, ors):
    """Compare slot bytes [..., slot]; K/V code mismatches are tolerated only at
    ties (float64 value within 1e-6 of the boundary between the two codes).
    Returns a dict of counts; raises AssertionError on any other difference."""
    lay = ors.lay
    got = got.reshape(-1, lay.slot_size_aligned)
    want = want.reshape(-1, lay.slot_size_aligned)
    kb = k_bits.reshape(-1, lay.head_dim)
    vb = v_bits.reshape(-1, lay.head_dim)
    diff_rows = np.nonzero((got != want).any(axis=1))[0]
    res = dict(vectors=got.shape[0], coords=got.shape[0] * lay.head_dim * 2, rows_differing=len(diff_rows),
               k_tie_mismatch=0, v_tie_mismatch=0)
    if len(diff_rows) == 0:
        return res
    g, w = got[diff_rows], want[diff_rows]
    d = lay.head_dim
    # metadata and FP8 bytes must match exactly
    meta = np.ones(lay.slot_size_aligned, bool)
    if not lay.key_fp8:
        meta[:lay.key_code_bytes] = False
    meta[lay.off_value:lay.off_value + lay.value_code_bytes] = False
    assert np.array_equal(g[:, meta], w[:, meta]), "norm/scale/zero/fp8 bytes differ"
    if not lay.key_fp8:
        gc = ost.unpack_codes(g[:, :lay.key_code_bytes], lay.key_bits, d)
        wc = ost.unpack_codes(w[:, :lay.key_code_bytes], lay.key_bits, d)
        kd = gc != wc
        if kd.any():
            y64 = ost.rotate_unit_f64(kb[diff_rows], ors.signs)
            ok = ost.k_mismatch_is_tie(y64[kd], gc[kd], wc[kd], ors.midpoints)
            assert ok.all(), f"{int((~ok).sum())} K code mismatches away from ties"
            res["k_tie_mismatch"] = int(kd.sum())
    o = lay.off_value
    gv = ost.unpack_codes(g[:, o:o + lay.value_code_bytes], lay.value_bits, d)
    wv = ost.unpack_codes(w[:, o:o + lay.value_code_bytes], lay.value_bits, d)
    vd = gv != wv
    if vd.any():
        t64 = ost.v_unit_position_f64(vb[diff_rows], lay.value_bits)
        ok = ost.v_mismatch_is_tie(t64[vd], gv[vd], wv[vd])
        assert ok.all(), f"{int((~ok).sum())} V code mismatches away from ties"
        res["v_tie_mismatch"] = int(vd.sum())
    return res


def bf16_half_ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


DECODE_ABS_TOL = 2e-3


def check_decode(got, want, bf16_out):
    """max |got - want| <= 2e-3 (+ half a bf16 ulp of the reference when the
    output is bf16).  Returns the max-abs error."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    tol = DECODE_ABS_TOL + (bf16_half_ulp(want) if bf16_out else 0.0)
    bad = err > tol
    assert not bad.any(), (f"{int(bad.sum())} outputs beyond tolerance; max err "
                           f"{float(err.max()):.3e} at {np.unravel_index(np.argmax(err), err.shape)}")
    return float(err.max())
