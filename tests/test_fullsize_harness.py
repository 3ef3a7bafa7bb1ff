"""CPU checks of the full-size parity harness (``fullsize_oracle``): with the
oracle's own cache and outputs standing in for the GPU's it reports no
difference, and a planted difference (a code away from a tie, a scale byte,
a byte outside the addressed slots, a decode output) is caught.  The planted
bytes are changed in the stand-in arrays on the host; nothing runs on a GPU.
"""

import os
import shutil
import tempfile

import numpy as np
import pytest

import fullsize_oracle as fo
from oracle import store as ost
from packed_cache_decode_amd import synth

SEED = 99


def _small(preset, B=3, H=2, Hq=4, lens=(1, 70)):
    return synth.Workload(f"harness_{preset}", preset, batch=B, num_q_heads=Hq, num_kv_heads=H,
                          head_dim=128, block_size=16, seed=7, len_range=lens)


def _oracle_side(w, soa):
    """The harness's oracle cache and outputs, computed in this process."""
    inp = synth.generate(w)
    tmp = tempfile.mkdtemp(prefix="tq_harness_")
    try:
        for key, arr in (("k", inp.k), ("v", inp.v), ("sm", inp.slot_mapping), ("q", inp.q),
                         ("bt", inp.block_table), ("sl", inp.seq_lens)):
            np.save(os.path.join(tmp, key + ".npy"), arr)
        lay, signs, c, m = fo.oracle_tables(w.preset, 128, SEED)
        if soa:
            from oracle import soa as osoa
            shape = (inp.num_blocks + 2, osoa.soa_page_bytes(lay, w.block_size, w.num_kv_heads))
        else:
            shape = (inp.num_blocks + 2, w.block_size, w.num_kv_heads, lay.slot_size_aligned)
        want = np.lib.format.open_memmap(os.path.join(tmp, "want_cache.npy"), mode="w+",
                                         dtype=np.uint8, shape=shape)
        want[:] = fo.CANARY
        want.flush()
        del want
        N = inp.num_tokens
        st = [fo.store_chunk((tmp, a, min(N, a + 50), w.preset, 128, SEED, w.block_size, soa))
              for a in range(0, N, 50)]
        cache = np.array(np.load(os.path.join(tmp, "want_cache.npy")))
        groups = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
        out = np.full((w.batch, w.num_q_heads, 128), np.nan)
        G = w.gqa
        for b, g, o in fo.decode_groups((tmp, groups, w.preset, 128, SEED, w.block_size,
                                         w.num_kv_heads, soa)):
            out[b, g * G:(g + 1) * G] = o
        return inp, cache, out, st
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _compare(w, inp, got, want, soa):
    lay, signs, c, m = fo.oracle_tables(w.preset, 128, SEED)
    nslots = got.shape[0] * w.block_size
    inv = np.full(nslots, -1, np.int64)
    inv[inp.slot_mapping] = np.arange(inp.num_tokens)
    return fo.compare_store(got, want, lambda t: inp.k[t], lambda t: inp.v[t], lambda s: inv[s],
                            lay, signs, c, m, soa, w.block_size, w.num_kv_heads)


@pytest.mark.parametrize("preset,soa", [("turboquant_4bit_nc", False), ("turboquant_k3v4_nc", False),
                                        ("turboquant_k8v4", False), ("turboquant_4bit_nc", True)])
def test_harness_accepts_the_oracle_and_catches_planted_differences(preset, soa):
    w = _small(preset)
    inp, want, out, st = _oracle_side(w, soa)
    assert sum(r["vectors"] for r in st) == inp.num_tokens * w.num_kv_heads
    res = _compare(w, inp, want.copy(), want, soa)
    assert res["bytes_differing"] == 0
    assert fo.decode_stats(out, out, bf16_out=False)["beyond"] == 0

    lay = fo.oracle_tables(preset, 128, SEED)[0]
    s0 = int(inp.slot_mapping[5])
    p, r = s0 // w.block_size, s0 % w.block_size
    # a byte outside every addressed slot (a spare page)
    got = want.copy()
    got[-1].reshape(-1)[3] ^= 1
    with pytest.raises(AssertionError):
        _compare(w, inp, got, want, soa)
    # the V scale of one vector
    if not soa:
        got = want.copy()
        got[p, r, 1, lay.off_value_scale] ^= 0x10
        with pytest.raises(AssertionError, match="bytes differ"):
            _compare(w, inp, got, want, soa)
    # one K code moved by two levels (never a tie)
    if not lay.key_fp8:
        got = want.copy()
        if soa:
            from oracle import soa as osoa
            db = osoa.data_bytes(lay)
            byte = got[p].reshape(-1)[(r * w.num_kv_heads + 1) * db:][:1]
            got[p].reshape(-1)[(r * w.num_kv_heads + 1) * db] = byte[0] ^ 0x02
        else:
            got[p, r, 1, 0] ^= 0x02
        with pytest.raises(AssertionError):
            _compare(w, inp, got, want, soa)
    # a decode output 3e-3 away
    bad = out.copy()
    bad[1, 2, 7] += 3e-3
    s = fo.decode_stats(bad, out, bf16_out=False)
    assert s["beyond"] == 1 and s["argmax"] == (1, 2, 7)


def test_tie_alternative_codes_moves_only_proven_ties():
    mid = np.array([-0.1, 0.0, 0.1], np.float32)
    y = np.array([[0.1 + 5e-7, 0.05, -0.1 - 2e-6]])
    codes = ost.bucketize(y.astype(np.float32), mid)
    alt = fo.tie_alternative_codes(y, codes, mid, np.ones_like(codes, bool))
    assert alt.tolist() == [[2, 2, 0]] and codes.tolist() == [[3, 2, 0]]


def test_near_points_equals_the_all_pairs_test():
    rng = np.random.default_rng(3)
    mids = np.sort(rng.normal(0, 0.1, 15))
    x = np.concatenate([rng.normal(0, 0.1, 5000), mids + rng.uniform(-2e-6, 2e-6, 15),
                        [-10.0, 10.0, mids[0], mids[-1]]])
    want = ost.k_near_tie_mask(x, mids, 1e-6)
    assert np.array_equal(fo.near_points(x, mids), want)
    assert want.sum() >= 4
