"""The structure-of-arrays page layout, with the norm correction folded into
the store.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Layout (P1, section "AoS 与 SoA:两种页内布局"): a page is split in two.
  data region  [block_size][H][key code bytes + value code bytes]: the packed
               K codes of one (token, head) followed by its packed V codes;
  meta region  [H][3][block_size] of fp16, right after the data region: for
               every head, block_size K norms, then block_size V scales, then
               block_size V zeros.
The page keeps the AoS page's size, block_size * H * slot bytes, because an
unpadded slot is exactly the data bytes plus the three fp16 scalars (true at
every head_dim 64/128/256 and every preset with a K norm).  FP8 keys carry no
K norm, so this layout is defined here for the 3/4-bit key presets only.

Folded norm (P1, section "SoA 的另一项收益:把 norm correction 折进写入端"):
with norm correction on, the store keeps n = |k| / |c| in place of |k|,
where c is the vector of centroids the token's codes select; the decode then
multiplies by the stored value and never forms |c|.  As an fp32 contract
(the conventions of ``store.py``: single binary32 operations, nearest even):
  css = balanced tree, in index order, of c_j * c_j
  inv = 1 / sqrt(css + 1e-16)
  n   = nrm * inv            (nrm = the store's sqrt of its own tree sum)
  stored as f16(n).
The page computes the same three steps (sum of squares, reciprocal square
root with 1e-16, multiply) with an unstated summation order.
"""

import numpy as np

from . import fpfmt
from .decode import attend_f64, scores_f64
from .store import (pairwise_sum_f32, pack_codes, quantize_k_contract, quantize_v_contract,
                    unpack_codes)

F32 = np.float32
FIELDS = 3                      # K norm, V scale, V zero


def _check(layout):
    if layout.key_fp8:
        raise ValueError("the SoA layout holds a K norm: 3/4-bit key presets only")
    if layout.slot_size != layout.slot_size_aligned:
        raise ValueError("padded slot: SoA page would not match the AoS page size")


def data_bytes(layout):
    """Bytes of one (token, head) in the data region."""
    return layout.key_code_bytes + layout.value_code_bytes


def meta_offset(layout, block_size, num_kv_heads):
    """Byte offset of the meta region inside a page."""
    return block_size * num_kv_heads * data_bytes(layout)


def soa_page_bytes(layout, block_size, num_kv_heads):
    _check(layout)
    return meta_offset(layout, block_size, num_kv_heads) + num_kv_heads * FIELDS * block_size * 2


def folded_norm_contract(codes, nrm, centroids):
    """n = nrm * (1 / sqrt(sum c^2 + 1e-16)) in the fp32 contract; codes [..., d]."""
    c = np.asarray(centroids, dtype=F32)[np.asarray(codes, dtype=np.int64)]
    css = pairwise_sum_f32((c * c).astype(F32))
    inv = (F32(1.0) / np.sqrt((css + F32(1e-16)).astype(F32)).astype(F32)).astype(F32)
    return (np.asarray(nrm, dtype=F32) * inv).astype(F32)


def encode_fields(k_bits, v_bits, layout, signs, midpoints, centroids):
    """(data bytes [..., KD + VD], norm16, scale16, zero16) for vectors [..., d]."""
    _check(layout)
    codes, nrm, _ = quantize_k_contract(k_bits, signs, midpoints)
    n = folded_norm_contract(codes, nrm, centroids) if layout.norm_correction else nrm
    vq, sc, lo = quantize_v_contract(v_bits, layout.value_bits)
    data = np.concatenate([pack_codes(codes, layout.key_bits), pack_codes(vq, layout.value_bits)], axis=-1)
    return (data, fpfmt.f32_to_f16_bits(n), fpfmt.f32_to_f16_bits(sc), fpfmt.f32_to_f16_bits(lo))


def _meta_view(pages, layout, block_size, H):
    """The meta regions as a uint16 array [num_blocks, H, 3, block_size] (little-endian)."""
    mo = meta_offset(layout, block_size, H)
    raw = pages[:, mo:mo + H * FIELDS * block_size * 2]
    return raw.view("<u2").reshape(pages.shape[0], H, FIELDS, block_size)


def _data_view(pages, layout, block_size, H):
    mo = meta_offset(layout, block_size, H)
    return pages[:, :mo].reshape(pages.shape[0], block_size, H, data_bytes(layout))


def store_contract(pages, block_size, k_bits, v_bits, slot_mapping, layout, signs, midpoints,
                   centroids):
    """Scatter N tokens into ``pages`` (uint8 [num_blocks, page_bytes], in place).

    k_bits, v_bits: uint16 [N, H, d].  Negative slots are padding and slots
    beyond the cache are skipped, as in the AoS store.  Returns the number of
    out-of-range slots.
    """
    nb = pages.shape[0]
    N, H, _ = np.asarray(k_bits).shape
    bs = block_size
    assert pages.shape[1] == soa_page_bytes(layout, bs, H)
    sm = np.asarray(slot_mapping, dtype=np.int64)
    valid = (sm >= 0) & (sm < nb * bs)
    bad = int((sm >= nb * bs).sum())
    idx = np.nonzero(valid)[0]
    if len(idx):
        data, n16, s16, z16 = encode_fields(np.asarray(k_bits)[idx], np.asarray(v_bits)[idx],
                                            layout, signs, midpoints, centroids)
        s = sm[idx]
        page, row = s // bs, s % bs
        dv = _data_view(pages, layout, bs, H)
        mv = _meta_view(pages, layout, bs, H)
        dv[page, row] = data
        for h in range(H):
            mv[page, h, 0, row] = n16[:, h]
            mv[page, h, 1, row] = s16[:, h]
            mv[page, h, 2, row] = z16[:, h]
    return bad


def gather(pages, layout, block_size, H, block_table_row, seq_len, kv_head):
    """(data [T, KD + VD], norm16 [T], scale16 [T], zero16 [T]) of one sequence and head."""
    t = np.arange(seq_len)
    page = np.asarray(block_table_row, dtype=np.int64)[t // block_size]
    row = t % block_size
    data = _data_view(pages, layout, block_size, H)[page, row, kv_head]
    mv = _meta_view(pages, layout, block_size, H)
    return data, mv[page, kv_head, 0, row], mv[page, kv_head, 1, row], mv[page, kv_head, 2, row]


def dequant(pages, layout, block_size, H, block_table_row, seq_len, kv_head, centroids):
    """(c [T, d] float64, n [T] float64, v_hat [T, d] float64): the key is n R^T c.

    With norm correction the stored norm is already |k| / |c|, so n is the
    stored fp16 value itself (no division here)."""
    d = layout.head_dim
    data, n16, s16, z16 = gather(pages, layout, block_size, H, block_table_row, seq_len, kv_head)
    kc = unpack_codes(data[:, :layout.key_code_bytes], layout.key_bits, d)
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)[kc]
    n = fpfmt.f16_bits_to_f64(n16)
    vc = unpack_codes(data[:, layout.key_code_bytes:], layout.value_bits, d)
    sc = fpfmt.f16_bits_to_f64(s16)
    zr = fpfmt.f16_bits_to_f64(z16)
    return c, n, vc.astype(np.float64) * sc[:, None] + zr[:, None]


def decode_f64(q_bits, pages, block_table, seq_lens, layout, signs, centroids, num_kv_heads,
               block_size, sm_scale=None, heads=None):
    """Decode output [B, Hq, d] in float64 over an SoA cache (see
    ``decode.decode_f64`` for the attention itself)."""
    q = fpfmt.bf16_bits_to_f64(q_bits)
    B, Hq, d = q.shape
    G = Hq // num_kv_heads
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.full((B, Hq, d), np.nan)
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)
    for b in range(B):
        for g in range(num_kv_heads):
            hs = [h for h in range(g * G, (g + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            c, n, v_hat = dequant(pages, layout, block_size, num_kv_heads, block_table[b],
                                  int(seq_lens[b]), g, centroids)
            s = scores_f64(q[b, hs], (c, n), layout, signs, sm_scale)
            out[b, hs] = attend_f64(s, v_hat)
    return out


def dequant_kv_f64(pages, layout, block_size, H, block_table_row, seq_len, signs, centroids):
    """K and V [seq_len, H, d] of one sequence of a split-page cache, float64:
    the key is n R^T c with the stored (folded) norm n."""
    from .rotation import rotation_matrix_f64
    d = layout.head_dim
    R = rotation_matrix_f64(signs)
    K = np.zeros((seq_len, H, d))
    V = np.zeros((seq_len, H, d))
    for g in range(H):
        c, n, v_hat = dequant(pages, layout, block_size, H, block_table_row, seq_len, g, centroids)
        K[:, g] = n[:, None] * (c @ R)
        V[:, g] = v_hat
    return K, V
