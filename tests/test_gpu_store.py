"""GPU parity of tq_store against the oracle's fp32 contract (bit-exact bytes).

Every case starts from a canary-filled cache and compares the whole cache,
so a byte written outside the addressed slots fails too.  A code mismatch is
tolerated only at a tie (float64 value within 1e-6 of the boundary between
the two codes) and the tolerated count must stay below 1e-5 of the
coordinates; the expected count is 0.
"""

import numpy as np
import pytest

from gpu_util import CANARY, OracleSide, compare_slots, to_dev
from oracle import fpfmt
from packed_cache_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PRESETS = ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_k8v4", "turboquant_3bit_nc"]


def _run_store(w, seed=77, sign_flip=True, mode="exact", extra_blocks=2, inp=None,
               slot_mapping=None):
    from packed_cache_decode_amd.runtime import PackedKVCache
    inp = inp or synth.generate(w)
    sm = inp.slot_mapping if slot_mapping is None else slot_mapping
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, seed, sign_flip, mode)
    nb = inp.num_blocks + extra_blocks
    cache = tq.new_cache(nb, CANARY)
    tq.store(to_dev(inp.k), to_dev(inp.v), to_dev(sm), cache)
    torch.cuda.synchronize()
    err = tq.device_error()
    got = cache.cpu().numpy()
    tq.close()
    ors = OracleSide(w.preset, w.head_dim, seed, sign_flip, mode)
    want = np.full_like(got, CANARY)
    ors.store(want, inp.k, inp.v, sm)
    return inp, got, want, ors, err


def _assert_parity(inp, got, want, ors, sm=None):
    sm = inp.slot_mapping if sm is None else sm
    nb, bs, H, S = got.shape
    keep = (sm >= 0) & (sm < nb * bs)
    slots = sm[keep]
    # outside the addressed slots nothing changed
    touched = np.zeros((nb * bs,), bool)
    touched[slots] = True
    touched = touched.reshape(nb, bs)
    assert np.all(got[~touched] == CANARY)
    res = compare_slots(got[slots // bs, slots % bs], want[slots // bs, slots % bs],
                        inp.k[keep], inp.v[keep], ors)
    tol = res["k_tie_mismatch"] + res["v_tie_mismatch"]
    assert tol <= 1e-5 * res["coords"]
    return res


def _small(preset, H=8, Hq=8, d=128, bs=16, seed=5, lens=(1, 90), B=3):
    return synth.Workload(f"small_{preset}", preset, batch=B, num_q_heads=Hq, num_kv_heads=H,
                          head_dim=d, block_size=bs, seed=seed, len_range=lens)


@pytest.mark.parametrize("preset", PRESETS)
def test_store_small_parity(preset):
    inp, got, want, ors, err = _run_store(_small(preset))
    assert err == 0
    res = _assert_parity(inp, got, want, ors)
    assert res["rows_differing"] == 0, res


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("bs,d", [(32, 128), (64, 128), (128, 128), (16, 64), (16, 256)])
def test_store_block_sizes_and_head_dims(preset, bs, d):
    inp, got, want, ors, err = _run_store(_small(preset, H=4, d=d, bs=bs, lens=(1, 300), seed=bs + d))
    assert err == 0
    assert _assert_parity(inp, got, want, ors)["rows_differing"] == 0


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("H", [1, 3, 8])
def test_store_head_dims_64_256(preset, d, H):
    # head dims 64 and 256 take the four-lanes-per-vector kernel (16 or 64
    # coordinates per lane): rows assembled in LDS (8 kv heads) or written
    # per lane (1 and 3), against the oracle byte for byte
    inp, got, want, ors, err = _run_store(_small(preset, H=H, d=d, lens=(1, 200), B=4, seed=d + H))
    assert err == 0
    assert _assert_parity(inp, got, want, ors)["rows_differing"] == 0


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
def test_store_pure_hadamard_and_page_codebook(preset):
    w = _small(preset, seed=9)
    for flip, mode in ((False, "exact"), (True, "page_trapz"), (True, "beta")):
        inp, got, want, ors, err = _run_store(w, seed=123, sign_flip=flip, mode=mode)
        assert _assert_parity(inp, got, want, ors)["rows_differing"] == 0


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("d", [128, 64, 256])
def test_store_degenerate_vectors(preset, d):
    """zero K, constant V, K beyond the e4m3 range, tiny and huge magnitudes,
    and padding tokens (slot < 0) that must be skipped."""
    w = _small(preset, H=2, d=d, lens=(40, 40), B=1, seed=3)
    inp = synth.generate(w)
    k = fpfmt.bf16_bits_to_f32(inp.k).copy()
    v = fpfmt.bf16_bits_to_f32(inp.v).copy()
    k[0] = 0.0                          # zero key -> codes at the central boundary
    v[1] = 0.625                        # constant value -> scale 1e-8 -> stored 0
    k[2, 0, :8] = [500.0, -600.0, 448.0, 464.0, -1e30, 2.0 ** -12, 3 * 2.0 ** -10, 1.0625]
    k[3] *= 1e-30                       # tiny but nonzero key
    k[4] *= 1e4                         # large key (norm in the fp16 range)
    k[5] *= 1e6                         # norm overflows fp16 -> inf
    v[6, 1] = -v[6, 1]
    inp.k = fpfmt.f32_to_bf16_bits(k)
    inp.v = fpfmt.f32_to_bf16_bits(v)
    sm = inp.slot_mapping.copy()
    sm[7] = -1
    sm[11] = -5
    got_inp, got, want, ors, err = _run_store(w, inp=inp, slot_mapping=sm)
    assert err == 0
    assert _assert_parity(inp, got, want, ors, sm)["rows_differing"] == 0


@pytest.mark.parametrize("d", [128, 64, 256])
def test_store_out_of_range_slot_sets_error_and_skips(d):
    w = _small("turboquant_4bit_nc", H=2, d=d, lens=(20, 20), B=1)
    inp = synth.generate(w)
    sm = inp.slot_mapping.copy()
    sm[3] = (inp.num_blocks + 2) * 16 + 5      # beyond the cache (which has 2 spare pages)
    got_inp, got, want, ors, err = _run_store(w, inp=inp, slot_mapping=sm)
    assert err == 1
    assert _assert_parity(inp, got, want, ors, sm)["rows_differing"] == 0


def test_store_zero_tokens_is_noop():
    from packed_cache_decode_amd import _lib
    from packed_cache_decode_amd.runtime import PackedKVCache
    tq = PackedKVCache("turboquant_4bit_nc", 128, 8, 16, 1)
    cache = tq.new_cache(2, CANARY)
    _lib.tq_store(tq.ctx, 0, 0, 1024, 0, 0, cache, 2)
    torch.cuda.synchronize()
    assert bool((cache == CANARY).all())
    tq.close()


def test_store_deterministic():
    w = _small("turboquant_k3v4_nc", seed=31)
    a = _run_store(w)[1]
    b = _run_store(w)[1]
    assert np.array_equal(a, b)
