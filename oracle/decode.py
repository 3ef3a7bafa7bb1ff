"""Paged decode attention over the packed cache, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

For sequence b, query head h and kv head g = h // (Hq / H) (P1, section
"程序入口:split 区间怎么算"), over tokens t in [0, seq_len[b]):
  * the token's slot is row t % bs of page block_table[b][t // bs]
    (P1, section "页内寻址");
  * MSE K (P1, section "分数计算:FP8 K 与 MSE K 的两条路径"): the codes
    index the float32 centroids (taken as exact float64 values), the norm is
    the stored fp16 value, and with norm correction the norm is divided by
    sqrt(sum_j c_j^2 + 1e-16); the query is rotated once with the same R as
    the store, q_rot = R q, and the score is sm_scale * n * (q_rot . c).
    The rotation is orthogonal, so this equals q . (n R^T c) -- the score
    against the dequantised key in the original space (P1, section "旋转前
    后的不变与改变"; P5, section "三、TurboQuant").
  * FP8 K: the score is sm_scale * (q . e4m3(k)); K was stored unrotated,
    so q is not rotated.
  * V (P1, section "V 的解包"): v_hat = code * f32(scale16) + f32(zero16).
  * softmax over the scores after subtracting their maximum, then the
    probability-weighted sum of v_hat (P1, section "在线 softmax").
  * sm_scale defaults to 1/sqrt(d) (same section of the score paths).
  * an empty sequence yields zeros (the pages are silent; this matches the
    page's rule that an empty split contributes nothing, lse = -inf).

``dequant_kv_f64`` expands one sequence back into K and V of the original
space, and ``decode_continuation_f64`` is the causal attention of a chunk of
new queries run as decode requests of growing length (P1, sections "反量化
kernel:_tq_full_dequant_kv" and "续写 prefill:小 chunk 走 decode,大 chunk 走反
量化").

``split_partials`` and ``combine_partials`` restate the split-KV scheme
(P1, sections "读取内核" and "在线 softmax"): each split keeps (max, sum,
acc), stores acc / sum and lse = max + log(sum); the combine weights each
split by exp(lse_s - max lse).
"""

import numpy as np

from . import fpfmt
from .rotation import rotation_matrix_f64
from .store import unpack_codes


def _u16(lo_byte, hi_byte):
    return (np.asarray(lo_byte, np.uint16) | (np.asarray(hi_byte, np.uint16) << 8)).astype(np.uint16)


def gather_slots(cache, block_table_row, seq_len, kv_head):
    """Slot bytes [seq_len, slot] of one sequence and one kv head."""
    nb, bs, H, S = cache.shape
    t = np.arange(seq_len)
    pages = np.asarray(block_table_row, dtype=np.int64)[t // bs]
    return cache[pages, t % bs, kv_head]


def dequant_keys(slots, layout, centroids):
    """Per token: (c [T, d] float64, n [T] float64) for MSE K, where the key is
    n * R^T c; for FP8 K, (k [T, d] float64, None)."""
    d = layout.head_dim
    if layout.key_fp8:
        return fpfmt.e4m3fn_bits_to_f64(slots[:, :d]), None
    codes = unpack_codes(slots[:, :layout.key_code_bytes], layout.key_bits, d)
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)[codes]
    o = layout.off_key_norm
    n = fpfmt.f16_bits_to_f64(_u16(slots[:, o], slots[:, o + 1]))
    if layout.norm_correction:
        n = n / np.sqrt((c * c).sum(axis=-1) + 1e-16)
    return c, n


def dequant_values(slots, layout):
    d = layout.head_dim
    o = layout.off_value
    codes = unpack_codes(slots[:, o:o + layout.value_code_bytes], layout.value_bits, d)
    o = layout.off_value_scale
    sc = fpfmt.f16_bits_to_f32(_u16(slots[:, o], slots[:, o + 1])).astype(np.float64)
    zr = fpfmt.f16_bits_to_f32(_u16(slots[:, o + 2], slots[:, o + 3])).astype(np.float64)
    return codes.astype(np.float64) * sc[:, None] + zr[:, None]


def scores_f64(q_f64, keys, layout, signs, sm_scale):
    """Scores [G, T] of G query vectors against the dequantised keys."""
    kc, n = keys
    if layout.key_fp8:
        return sm_scale * (q_f64 @ kc.T)
    R = rotation_matrix_f64(signs)
    q_rot = q_f64 @ R.T
    return sm_scale * n[None, :] * (q_rot @ kc.T)


def attend_f64(s, v_hat):
    """softmax(s) @ v_hat with the maximum subtracted; rows of s are heads."""
    if s.shape[-1] == 0:
        return np.zeros((s.shape[0], v_hat.shape[-1]))
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    return (p @ v_hat) / p.sum(axis=-1, keepdims=True)


def decode_f64(q_bits, cache, block_table, seq_lens, layout, signs, centroids,
               num_kv_heads, sm_scale=None, heads=None):
    """Decode output [B, Hq, d] in float64.

    q_bits: uint16 bf16 [B, Hq, d]; cache: uint8 [nb, bs, H, slot];
    block_table: int [B, max_blocks]; seq_lens: int [B].
    ``heads``: optional list of (b, h) pairs to compute (others stay NaN).
    """
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
            slots = gather_slots(cache, block_table[b], int(seq_lens[b]), g)
            keys = dequant_keys(slots, layout, centroids)
            v_hat = dequant_values(slots, layout)
            s = scores_f64(q[b, hs], keys, layout, signs, sm_scale)
            out[b, hs] = attend_f64(s, v_hat)
    return out


def split_partials(s, v_hat, bounds):
    """Per split [a, e): (o_s = acc/l, lse_s) with lse = -inf for an empty split."""
    parts = []
    for a, e in bounds:
        if e <= a:
            parts.append((np.zeros((s.shape[0], v_hat.shape[-1])), np.full(s.shape[0], -np.inf)))
            continue
        ss = s[:, a:e]
        m = ss.max(axis=-1)
        p = np.exp(ss - m[:, None])
        l = p.sum(axis=-1)
        parts.append(((p @ v_hat[a:e]) / l[:, None], m + np.log(l)))
    return parts


def combine_partials(parts):
    lses = np.stack([p[1] for p in parts])          # [S, G]
    outs = np.stack([p[0] for p in parts])          # [S, G, d]
    M = lses.max(axis=0)
    w = np.where(np.isfinite(lses), np.exp(lses - np.where(np.isfinite(M), M, 0.0)), 0.0)
    den = w.sum(axis=0)
    num = (w[..., None] * outs).sum(axis=0)
    return np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)


def dequant_kv_f64(cache, block_table_row, seq_len, layout, signs, centroids):
    """K and V [seq_len, H, d] of one sequence back in the original space, in
    float64 (P1, section "反量化 kernel:_tq_full_dequant_kv"): the key is
    n R^T c with the explicit rotation matrix (FP8 keys: the decoded bytes),
    the value code * scale + zero."""
    H = cache.shape[2]
    d = layout.head_dim
    K = np.zeros((seq_len, H, d))
    V = np.zeros((seq_len, H, d))
    R = None if layout.key_fp8 else rotation_matrix_f64(signs)
    for g in range(H):
        slots = gather_slots(cache, block_table_row, seq_len, g)
        kc, n = dequant_keys(slots, layout, centroids)
        K[:, g] = kc if layout.key_fp8 else n[:, None] * (kc @ R)
        V[:, g] = dequant_values(slots, layout)
    return K, V


def decode_continuation_f64(q_bits, cache, block_table_row, seq_len, layout, signs, centroids,
                            num_kv_heads, sm_scale=None):
    """Causal attention of a chunk of q_len queries (the last q_len of seq_len
    stored tokens), P1 section "续写 prefill:小 chunk 走 decode,大 chunk 走反量化":
    query i is a decode request of length seq_len - q_len + i + 1 over the
    sequence's block-table row."""
    q_len = np.asarray(q_bits).shape[0]
    cached = seq_len - q_len
    lens = cached + 1 + np.arange(q_len)
    table = np.repeat(np.asarray(block_table_row)[None], q_len, axis=0)
    return decode_f64(q_bits, cache, table, lens, layout, signs, centroids, num_kv_heads, sm_scale)
