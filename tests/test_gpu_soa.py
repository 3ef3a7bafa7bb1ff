"""GPU parity of the split page layout (data region + meta region, folded K
norm) against the oracle (``oracle/soa.py``).

Store: the whole cache is compared with the oracle's bytes, starting from a
canary fill.  A K or V code may differ only at a tie (the rule of the slotted
store tests); where a K code differs at a proven tie, the folded norm may be
the oracle's fold of the tie-alternative codes it derives itself.  Decode:
the GPU decode of an oracle-written cache against the oracle's float64
attention, max-abs 2e-3 (fp32 output), through the ring kernel (3/4-bit
keys, in passes of up to 8 query heads per kv head) and the general kernel
(other head dims).  The full-size workloads in this layout
are compared output by output in test_gpu_fullsize.py.
"""

import numpy as np
import pytest

import fullsize_oracle as fo
from gpu_util import CANARY, OracleSide, check_decode, compare_slots, to_dev
from oracle import fpfmt
from oracle import soa as osoa
from oracle import store as ost
from packed_cache_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MSE = ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"]


def _views(pages, lay, bs, H):
    """(data [nb, bs, H, DB], meta [nb, H, 3, bs] uint16) views of the pages."""
    db = osoa.data_bytes(lay)
    mo = osoa.meta_offset(lay, bs, H)
    data = pages[:, :mo].reshape(pages.shape[0], bs, H, db)
    meta = pages[:, mo:mo + H * 3 * bs * 2].view("<u2").reshape(pages.shape[0], H, 3, bs)
    return data, meta


def _as_slots(pages, lay, bs, H, slots):
    """The fields of the given slots, laid out as slotted-page slots [N, H, slot]."""
    data, meta = _views(pages, lay, bs, H)
    p, r = slots // bs, slots % bs
    d = data[p, r]                                   # [N, H, DB]
    m = meta[p, :, :, r]                             # [N, H, 3]
    out = np.zeros(d.shape[:2] + (lay.slot_size_aligned,), np.uint8)
    kc = lay.key_code_bytes

    def u16(x):
        return np.stack([(x & 0xFF).astype(np.uint8), (x >> 8).astype(np.uint8)], axis=-1)

    out[..., :kc] = d[..., :kc]
    out[..., kc:kc + 2] = u16(m[..., 0])
    out[..., lay.off_value:lay.off_value + lay.value_code_bytes] = d[..., kc:]
    out[..., lay.off_value_scale:lay.off_value_scale + 2] = u16(m[..., 1])
    out[..., lay.off_value_zero:lay.off_value_zero + 2] = u16(m[..., 2])
    return out


def _store(w, seed=77, extra_blocks=2, slot_mapping=None):
    from packed_cache_decode_amd.runtime import PackedKVCache
    inp = synth.generate(w)
    sm = inp.slot_mapping if slot_mapping is None else slot_mapping
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, seed, layout="soa")
    cache = tq.new_cache(inp.num_blocks + extra_blocks, CANARY)
    tq.store(to_dev(inp.k), to_dev(inp.v), to_dev(sm), cache)
    torch.cuda.synchronize()
    err = tq.device_error()
    got = cache.cpu().numpy()
    tq.close()
    ors = OracleSide(w.preset, w.head_dim, seed)
    want = np.full_like(got, CANARY)
    osoa.store_contract(want, w.block_size, inp.k, inp.v, sm, ors.lay, ors.signs, ors.midpoints,
                        ors.centroids)
    return inp, sm, got, want, ors, err


def _assert_store_parity(w, inp, sm, got, want, ors):
    lay, bs, H = ors.lay, w.block_size, w.num_kv_heads
    keep = (sm >= 0) & (sm < got.shape[0] * bs)
    slots = sm[keep]
    g_sl = _as_slots(got, lay, bs, H, slots)
    w_sl = _as_slots(want, lay, bs, H, slots)
    k, v = inp.k[keep], inp.v[keep]
    # A vector whose K codes differ from the oracle's at a proven tie may
    # carry either fold of the norm: the oracle's fold of its own codes, or
    # its fold of the tie-alternative codes it derives itself (each tied
    # coordinate moved across the boundary it lies on).  compare_slots then
    # checks that every differing code is such a tie.
    d = lay.head_dim
    gc = ost.unpack_codes(g_sl[..., :lay.key_code_bytes], lay.key_bits, d)
    wc = ost.unpack_codes(w_sl[..., :lay.key_code_bytes], lay.key_bits, d)
    kd = gc != wc
    rows = kd.any(-1)
    if rows.any():
        y64 = ost.rotate_unit_f64(k[rows], ors.signs)
        alt = fo.tie_alternative_codes(y64, wc[rows], ors.midpoints, kd[rows])
        _, nrm, _ = ost.quantize_k_contract(k[rows], ors.signs, ors.midpoints)
        a16 = fpfmt.f32_to_f16_bits(osoa.folded_norm_contract(alt, nrm, ors.centroids))
        o = lay.off_key_norm
        g16 = g_sl[rows, o].astype(np.uint16) | (g_sl[rows, o + 1].astype(np.uint16) << 8)
        w16 = w_sl[rows, o].astype(np.uint16) | (w_sl[rows, o + 1].astype(np.uint16) << 8)
        assert np.all((g16 == w16) | (g16 == a16)), "folded norm is neither of the oracle's folds"
        w_sl[rows, o] = g_sl[rows, o]
        w_sl[rows, o + 1] = g_sl[rows, o + 1]
    res = compare_slots(g_sl, w_sl, k, v, ors)
    assert res["k_tie_mismatch"] + res["v_tie_mismatch"] <= 1e-5 * res["coords"]
    # nothing outside the addressed fields changed
    fixed = got.copy()
    fd, fm = _views(fixed, lay, bs, H)
    wd, wm = _views(want, lay, bs, H)
    p, r = slots // bs, slots % bs
    fd[p, r] = wd[p, r]
    for h in range(H):
        fm[p, h, :, r] = wm[p, h, :, r]
    assert np.array_equal(fixed, want), "bytes outside the stored fields differ"
    return res


def _wl(preset, H=8, Hq=8, d=128, bs=16, seed=5, lens=(1, 90), B=3):
    return synth.Workload(f"soa_{preset}", preset, batch=B, num_q_heads=Hq, num_kv_heads=H,
                          head_dim=d, block_size=bs, seed=seed, len_range=lens)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("H,bs,d", [(8, 16, 128), (4, 32, 128), (2, 128, 128), (3, 16, 128),
                                    (4, 16, 64), (4, 16, 256), (1, 64, 256)])
def test_soa_store_parity(preset, H, bs, d):
    w = _wl(preset, H=H, Hq=H, d=d, bs=bs, lens=(1, 300), seed=bs + d + H)
    inp, sm, got, want, ors, err = _store(w)
    assert err == 0
    res = _assert_store_parity(w, inp, sm, got, want, ors)
    assert res["rows_differing"] == 0, res


@pytest.mark.parametrize("preset", MSE)
def test_soa_store_padding_slots_and_degenerate_vectors(preset):
    w = _wl(preset, H=4, Hq=4, lens=(40, 80), seed=9)
    inp = synth.generate(w)
    sm = inp.slot_mapping.copy()
    sm[::7] = -1                                     # padding tokens are skipped
    inp.k[3] = 0                                     # zero K: codes of 0, norm 0
    inp.v[5] = inp.v[5, :, :1]                       # constant V: codes 0, scale 0
    from packed_cache_decode_amd.runtime import PackedKVCache
    seed = 77
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, seed, layout="soa")
    cache = tq.new_cache(inp.num_blocks + 1, CANARY)
    tq.store(to_dev(inp.k), to_dev(inp.v), to_dev(sm), cache)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    got = cache.cpu().numpy()
    tq.close()
    ors = OracleSide(w.preset, w.head_dim, seed)
    want = np.full_like(got, CANARY)
    osoa.store_contract(want, w.block_size, inp.k, inp.v, sm, ors.lay, ors.signs, ors.midpoints,
                        ors.centroids)
    _assert_store_parity(w, inp, sm, got, want, ors)


def test_soa_rejects_fp8_keys():
    from packed_cache_decode_amd import _lib
    with pytest.raises(_lib.TQError):
        _lib.tq_codebook_init_layout("turboquant_k8v4", 128, 8, 16, 1, layout="soa")


def _decode_soa(w, seed=11, out_fp32=True, lens=None, opts=None):
    from packed_cache_decode_amd.runtime import PackedKVCache
    inp = synth.generate(w)
    if lens is not None:
        inp.seq_lens = np.minimum(np.asarray(lens, np.int32), inp.seq_lens)
    ors = OracleSide(w.preset, w.head_dim, seed)
    pages = np.zeros((inp.num_blocks, osoa.soa_page_bytes(ors.lay, w.block_size, w.num_kv_heads)),
                     np.uint8)
    osoa.store_contract(pages, w.block_size, inp.k, inp.v, inp.slot_mapping, ors.lay, ors.signs,
                        ors.midpoints, ors.centroids)
    want = osoa.decode_f64(inp.q, pages, inp.block_table, inp.seq_lens, ors.lay, ors.signs,
                           ors.centroids, w.num_kv_heads, w.block_size)
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, seed, layout="soa")
    if opts:
        tq.set_decode_options(**opts)
    max_len = int(max(1, inp.seq_lens.max()))
    out = tq.decode(to_dev(inp.q), to_dev(pages), to_dev(inp.block_table), to_dev(inp.seq_lens),
                    max_len, out_fp32=out_fp32)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    return out.float().cpu().numpy(), want


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("G,H", [(1, 1), (4, 2), (8, 2), (4, 8), (2, 3)])
def test_soa_decode_ring(preset, G, H):
    got, want = _decode_soa(_wl(preset, H=H, Hq=G * H, lens=(1, 700), B=4, seed=G + H))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("bs", [32, 64, 128])
def test_soa_decode_block_sizes(preset, bs):
    got, want = _decode_soa(_wl(preset, H=2, Hq=8, bs=bs, lens=(1, 900), B=3, seed=bs))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("G,H", [(16, 1), (12, 2), (24, 1)])
def test_soa_decode_query_head_passes(preset, G, H):
    # more than 8 query heads per kv head: the ring kernel in passes of 8 (the
    # last one short), one merge for every head; empty and multi-split lengths
    w = _wl(preset, H=H, Hq=G * H, lens=(20000, 20000), B=3, seed=G + 3 * H)
    got, want = _decode_soa(w, lens=[0, 700, 20000])
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("G,H,d", [(4, 2, 64), (4, 2, 256), (3, 2, 64), (7, 1, 256), (12, 1, 64)])
def test_soa_decode_general_kernel(preset, G, H, d):
    # other head dims on the split page: the general kernel, built for the
    # next power of two of the query heads per kv head
    got, want = _decode_soa(_wl(preset, H=H, Hq=G * H, d=d, lens=(1, 500), B=3, seed=G + d))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", MSE)
def test_soa_decode_bf16_ragged_and_long(preset):
    # lengths from 0 up to past one workgroup split of the ring kernel
    # (1024 slabs), with bf16 output
    w = _wl(preset, H=2, Hq=8, lens=(20000, 20000), B=5, seed=3)
    got, want = _decode_soa(w, out_fp32=False, lens=[0, 1, 17, 16400, 20000])
    check_decode(got, want, bf16_out=True)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("waves", ["8", "16"])
def test_soa_decode_ring_workgroup_sizes(preset, waves):
    w = _wl(preset, H=2, Hq=16, lens=(20000, 20000), B=5, seed=7)
    for dyn in (False, True):
        got, want = _decode_soa(w, lens=[0, 3, 700, 16400, 20000],
                                opts=dict(ring_waves=int(waves), dynamic_claims=dyn))
        check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", MSE)
def test_soa_decode_ring_length_order(preset):
    # more (sequence, kv head) pairs than compute units, ragged lengths: the
    # length-ordered dispatch on the split page
    rng = np.random.default_rng(19)
    lens = [int(x) for x in rng.integers(0, 1200, size=36)]
    lens[:3] = [0, 1, 1199]
    w = _wl(preset, H=8, Hq=32, lens=(1200, 1200), B=36, seed=75)
    got, want = _decode_soa(w, lens=lens)
    check_decode(got, want, bf16_out=False)
    # two whole layers of 8-wavefront workgroups per XCD (long and short
    # sequences paired on each CU), some XCDs one sequence short
    lens = [int(x) for x in rng.integers(0, 400, size=61)]
    lens[:3] = [0, 1, 399]
    w = _wl(preset, H=8, Hq=16, lens=(400, 400), B=61, seed=77)
    got, want = _decode_soa(w, lens=lens, opts=dict(ring_waves=8))
    check_decode(got, want, bf16_out=False)
