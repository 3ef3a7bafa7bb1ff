"""Whole-output oracle parity at full size, with the oracle spread over a
process pool (imported by tests only).

The GPU side writes its whole cache and its decode outputs; the oracle side
encodes every token of the workload itself (``oracle.store`` /
``oracle.soa``), into a cache of its own, and decodes every (sequence, query
head) from that cache (``oracle.decode`` / ``oracle.soa``).  No oracle input
comes from the GPU: the GPU's arrays are only compared against.

Work units are independent, so they run in a pool of worker processes forked
from a server that never touched the GPU (``multiprocessing`` "forkserver",
started before any test initialises the device).  Large arrays travel as
``.npy`` files in a temporary directory, opened memory-mapped by the workers:
  k.npy, v.npy          bf16 bits [N, H, d]
  sm.npy                int64 slot mapping [N]
  q.npy, bt.npy, sl.npy decode inputs
  want_cache.npy        the oracle's cache, written by the store workers
Counts follow the store tie rule: a differing code is tolerated only when the
float64 value lies within 1e-6 of the boundary between the two codes, and
near-ties (within 1e-6 of any boundary) are counted and reported, not bounded.
"""

import os

import numpy as np

from oracle import codebook as cb
from oracle import fpfmt
from oracle import decode as odec
from oracle import haar, layout, rotation
from oracle import soa as osoa
from oracle import store as ost

CANARY = 0xA5
TIE_EPS = 1e-6

_tables = {}


def oracle_tables(preset, head_dim, rot_seed):
    """(layout, signs, centroids, midpoints) of a context's parameters, seeded
    Hadamard signs and the default codebook."""
    key = (preset, head_dim, rot_seed)
    if key not in _tables:
        lay = layout.slot_layout(preset, head_dim)
        signs = rotation.rotation_signs(rot_seed, head_dim, True)
        kb = 4 if lay.key_fp8 else lay.key_bits
        c, m = cb.codebook(head_dim, kb, "exact")
        _tables[key] = (lay, signs, c, m)
    return _tables[key]


def _load(d, name, mode="r"):
    return np.load(os.path.join(d, name + ".npy"), mmap_mode=mode)


def worker_count():
    """One worker per core available to this process, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def near_points(x, points, eps=TIE_EPS):
    """True where x lies within eps of one of the sorted points (the nearest
    point on either side of x, found by binary search)."""
    points = np.asarray(points, np.float64)
    i = np.searchsorted(points, x)
    lo = points[np.clip(i - 1, 0, len(points) - 1)]
    hi = points[np.clip(i, 0, len(points) - 1)]
    return np.minimum(np.abs(x - lo), np.abs(x - hi)) < eps


def near_tie_counts(k_bits, v_bits, lay, signs, midpoints):
    """(K coordinates within 1e-6 of a boundary, V coordinates within 1e-6 of
    a half-integer code position), both in float64."""
    k_near = 0
    if not lay.key_fp8:
        y64 = ost.rotate_unit_f64(k_bits, signs)
        k_near = int(near_points(y64, midpoints).sum())
    t64 = ost.v_unit_position_f64(v_bits, lay.value_bits)
    half = np.arange((1 << lay.value_bits) - 1) + 0.5
    v_near = int(near_points(t64, half).sum())
    return k_near, v_near


def store_chunk(job):
    """Encode tokens [a, e) with the oracle into want_cache; count near-ties."""
    d, a, e, preset, head_dim, rot_seed, block_size, soa = job
    lay, signs, c, m = oracle_tables(preset, head_dim, rot_seed)
    k = np.asarray(_load(d, "k")[a:e])
    v = np.asarray(_load(d, "v")[a:e])
    sm = np.asarray(_load(d, "sm")[a:e])
    want = _load(d, "want_cache", "r+")
    if soa:
        osoa.store_contract(want, block_size, k, v, sm, lay, signs, m, c)
    else:
        ost.store_contract(want, k, v, sm, lay, signs, m)
    want.flush()
    k_near, v_near = near_tie_counts(k, v, lay, signs, m)
    return dict(k_near=k_near, v_near=v_near, vectors=k.shape[0] * k.shape[1])


def decode_groups(job):
    """Oracle outputs of (sequence, kv head) groups from the oracle's cache:
    a list of (b, g, out [G, d] float64)."""
    d, groups, preset, head_dim, rot_seed, block_size, num_kv_heads, soa = job
    lay, signs, c, m = oracle_tables(preset, head_dim, rot_seed)
    cache = _load(d, "want_cache")
    q = _load(d, "q")
    bt = _load(d, "bt")
    sl = _load(d, "sl")
    G = q.shape[1] // num_kv_heads
    res = []
    for b, g in groups:
        heads = [(0, h) for h in range(g * G, (g + 1) * G)]
        qb = np.asarray(q[b:b + 1])
        btb = np.asarray(bt[b:b + 1])
        slb = np.asarray(sl[b:b + 1])
        if soa:
            o = osoa.decode_f64(qb, cache, btb, slb, lay, signs, c, num_kv_heads, block_size,
                                heads=heads)
        else:
            o = odec.decode_f64(qb, cache, btb, slb, lay, signs, c, num_kv_heads, heads=heads)
        res.append((b, g, o[0, g * G:(g + 1) * G]))
    return res


def soa_as_slots(pages, lay, bs, H, slots):
    """The fields of the given slots of a split-page cache, laid out as slotted
    slots [N, H, slot] (the norm field holds the stored folded norm)."""
    db = osoa.data_bytes(lay)
    mo = osoa.meta_offset(lay, bs, H)
    data = pages[:, :mo].reshape(pages.shape[0], bs, H, db)
    meta = pages[:, mo:mo + H * 3 * bs * 2].view("<u2").reshape(pages.shape[0], H, 3, bs)
    p, r = slots // bs, slots % bs
    dd = data[p, r]
    mm = meta[p, :, :, r]
    out = np.zeros(dd.shape[:2] + (lay.slot_size_aligned,), np.uint8)
    kc = lay.key_code_bytes

    def u16(x):
        return np.stack([(x & 0xFF).astype(np.uint8), (x >> 8).astype(np.uint8)], axis=-1)

    out[..., :kc] = dd[..., :kc]
    out[..., kc:kc + 2] = u16(mm[..., 0])
    out[..., lay.off_value:lay.off_value + lay.value_code_bytes] = dd[..., kc:]
    out[..., lay.off_value_scale:lay.off_value_scale + 2] = u16(mm[..., 1])
    out[..., lay.off_value_zero:lay.off_value_zero + 2] = u16(mm[..., 2])
    return out


def tie_alternative_codes(y64, codes, midpoints, mismatch):
    """The oracle's codes with each coordinate in ``mismatch`` moved across the
    boundary it lies on, where the float64 value is within 1e-6 of that
    boundary (a proven tie); other coordinates keep the oracle's code."""
    mid = np.asarray(midpoints, np.float64)
    alt = codes.copy()
    for idx in zip(*np.nonzero(mismatch)):
        y = y64[idx]
        c0 = int(codes[idx])
        for cand in (c0 - 1, c0 + 1):
            if 0 <= cand <= len(mid):
                bnd = mid[min(c0, cand)]
                if abs(y - bnd) < TIE_EPS:
                    alt[idx] = cand
    return alt


def compare_store(got, want, k_rows_of, v_rows_of, slot_rows, lay, signs, centroids, midpoints,
                  soa, bs, H):
    """Whole-cache comparison.  ``got``/``want``: the GPU's and the oracle's
    caches (same shape; the oracle's started from the same canary fill).
    ``slot_rows(slots)`` gives the token index of each slot.  Returns a dict
    of counts; raises AssertionError on a difference that is not a proven tie.
    """
    diff = got != want
    res = dict(bytes_differing=int(diff.sum()), k_tie_mismatch=0, v_tie_mismatch=0,
               slots_differing=0)
    if not diff.any():
        return res
    d = lay.head_dim
    if soa:
        # map differing bytes to the slots of their pages (all slots of a
        # differing page are checked)
        pages = np.nonzero(diff.any(axis=1))[0]
        slots = (pages[:, None] * bs + np.arange(bs)[None]).reshape(-1)
        g_sl = soa_as_slots(got, lay, bs, H, slots)
        w_sl = soa_as_slots(want, lay, bs, H, slots)
    else:
        rows = np.nonzero(diff.reshape(-1, bs, H * lay.slot_size_aligned).any(axis=2))
        slots = rows[0] * bs + rows[1]
        g_sl = got.reshape(-1, bs, H, lay.slot_size_aligned)[rows]
        w_sl = want.reshape(-1, bs, H, lay.slot_size_aligned)[rows]
    keep = (g_sl != w_sl).reshape(len(slots), -1).any(axis=1)
    slots, g_sl, w_sl = slots[keep], g_sl[keep], w_sl[keep]
    tok = slot_rows(slots)
    assert (tok >= 0).all(), "bytes differ in a slot no token addresses"
    k = k_rows_of(tok)
    v = v_rows_of(tok)
    g2 = g_sl.reshape(-1, lay.slot_size_aligned)
    w2 = w_sl.reshape(-1, lay.slot_size_aligned)
    kb = k.reshape(-1, d)
    vb = v.reshape(-1, d)
    drow = np.nonzero((g2 != w2).any(axis=1))[0]
    res["slots_differing"] = len(drow)
    g2, w2, kb, vb = g2[drow], w2[drow], kb[drow], vb[drow]
    meta = np.ones(lay.slot_size_aligned, bool)
    if not lay.key_fp8:
        meta[:lay.key_code_bytes] = False
        if soa and lay.norm_correction:
            meta[lay.off_key_norm:lay.off_key_norm + 2] = False      # checked below
    meta[lay.off_value:lay.off_value + lay.value_code_bytes] = False
    assert np.array_equal(g2[:, meta], w2[:, meta]), "norm/scale/zero/fp8 bytes differ"
    if not lay.key_fp8:
        gc = ost.unpack_codes(g2[:, :lay.key_code_bytes], lay.key_bits, d)
        wc = ost.unpack_codes(w2[:, :lay.key_code_bytes], lay.key_bits, d)
        kd = gc != wc
        y64 = ost.rotate_unit_f64(kb, signs)
        if kd.any():
            ok = ost.k_mismatch_is_tie(y64[kd], gc[kd], wc[kd], midpoints)
            assert ok.all(), f"{int((~ok).sum())} K code mismatches away from ties"
            res["k_tie_mismatch"] = int(kd.sum())
        if soa and lay.norm_correction:
            # the folded norm: the oracle's fold of its own codes, or -- only
            # on a vector whose codes differ at proven ties -- its fold of the
            # tie-alternative codes it derives itself
            o = lay.off_key_norm
            g16 = g2[:, o].astype(np.uint16) | (g2[:, o + 1].astype(np.uint16) << 8)
            w16 = w2[:, o].astype(np.uint16) | (w2[:, o + 1].astype(np.uint16) << 8)
            _, nrm, _ = ost.quantize_k_contract(kb, signs, midpoints)
            alt = tie_alternative_codes(y64, wc, midpoints, kd)
            a16 = fpfmt.f32_to_f16_bits(osoa.folded_norm_contract(alt, nrm, centroids))
            ok = (g16 == w16) | ((g16 == a16) & kd.any(axis=1))
            if not ok.all():
                bad = np.nonzero(~ok)[0][:6]
                c64 = np.asarray(centroids, np.float64)[wc[bad]]
                exact = nrm[bad].astype(np.float64) / np.sqrt((c64 * c64).sum(axis=-1) + 1e-16)
                detail = [dict(gpu=float(fpfmt.f16_bits_to_f64(g16[i])),
                               oracle=float(fpfmt.f16_bits_to_f64(w16[i])),
                               fold_f32=float(osoa.folded_norm_contract(wc[i], nrm[i], centroids)),
                               f64=float(e), codes_differ=bool(kd[i].any()))
                          for i, e in zip(bad, exact)]
                raise AssertionError(f"{int((~ok).sum())} of {len(ok)} folded norms differ from "
                                     f"the oracle's: {detail}")
    o = lay.off_value
    gv = ost.unpack_codes(g2[:, o:o + lay.value_code_bytes], lay.value_bits, d)
    wv = ost.unpack_codes(w2[:, o:o + lay.value_code_bytes], lay.value_bits, d)
    vd = gv != wv
    if vd.any():
        t64 = ost.v_unit_position_f64(vb, lay.value_bits)
        ok = ost.v_mismatch_is_tie(t64[vd], gv[vd], wv[vd])
        assert ok.all(), f"{int((~ok).sum())} V code mismatches away from ties"
        res["v_tie_mismatch"] = int(vd.sum())
    return res


def bf16_half_ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def decode_stats(got, want, bf16_out, abs_tol=2e-3):
    """max-abs, mean-abs and argmax of |got - want| over every output, and
    the count beyond 2e-3 (+ half a bf16 ulp of the reference for bf16)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    tol = abs_tol + (bf16_half_ulp(want) if bf16_out else 0.0)
    am = np.unravel_index(int(np.argmax(err)), err.shape)
    return dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                argmax=tuple(int(i) for i in am), beyond=int((err > tol).sum()),
                outputs=int(err.size))
