"""GPU parity with the Haar rotation (TQ_ROTATION_HAAR) against the oracle,
which draws its own Haar matrix from the same seed (``oracle/haar.py``).

Store: whole-cache comparison from a canary fill, codes tolerated only at ties
(the store's rule).  Decode (the general kernel), dequantisation and the
continuation: the float tolerances of their own tests.
"""

import numpy as np
import pytest

from gpu_util import CANARY, OracleSide, check_decode, compare_slots, to_dev
from oracle import decode as odec
from oracle import soa as osoa
from packed_cache_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MSE = ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"]


def _wl(preset, H=4, Hq=8, d=128, bs=16, seed=5, lens=(1, 300), B=3):
    return synth.Workload(f"haar_{preset}", preset, batch=B, num_q_heads=Hq, num_kv_heads=H,
                          head_dim=d, block_size=bs, seed=seed, len_range=lens)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("d", [64, 128, 256])
def test_haar_store_parity(preset, d):
    from packed_cache_decode_amd.runtime import PackedKVCache
    w = _wl(preset, d=d, seed=d)
    inp = synth.generate(w)
    seed = 404
    tq = PackedKVCache(preset, d, w.num_kv_heads, 16, seed, sign_flip="haar")
    cache = tq.new_cache(inp.num_blocks + 1, CANARY)
    tq.store(to_dev(inp.k), to_dev(inp.v), to_dev(inp.slot_mapping), cache)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    got = cache.cpu().numpy()
    tq.close()
    ors = OracleSide(preset, d, seed, "haar")
    want = np.full_like(got, CANARY)
    ors.store(want, inp.k, inp.v, inp.slot_mapping)
    sm = inp.slot_mapping
    bs = w.block_size
    touched = np.zeros(got.shape[0] * bs, bool)
    touched[sm] = True
    assert np.all(got[~touched.reshape(-1, bs)] == CANARY)
    res = compare_slots(got[sm // bs, sm % bs], want[sm // bs, sm % bs], inp.k, inp.v, ors)
    assert res["k_tie_mismatch"] + res["v_tie_mismatch"] <= 1e-5 * res["coords"]


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("G,d", [(4, 128), (8, 64), (2, 256)])
def test_haar_decode_parity(preset, G, d):
    from packed_cache_decode_amd.runtime import PackedKVCache
    H, seed = 2, 77
    w = _wl(preset, H=H, Hq=G * H, d=d, seed=G + d, lens=(1, 700))
    inp = synth.generate(w)
    ors = OracleSide(preset, d, seed, "haar")
    cache = np.zeros((inp.num_blocks, 16, H, ors.lay.slot_size_aligned), np.uint8)
    ors.store(cache, inp.k, inp.v, inp.slot_mapping)
    want = ors.decode(inp.q, cache, inp.block_table, inp.seq_lens, H)
    tq = PackedKVCache(preset, d, H, 16, seed, sign_flip="haar")
    out = tq.decode(to_dev(inp.q), to_dev(cache), to_dev(inp.block_table), to_dev(inp.seq_lens),
                    int(inp.seq_lens.max()), out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    check_decode(out.cpu().numpy(), want, bf16_out=False)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("kernel", ["ring", "page", "staged", "direct", "general"])
def test_haar_decode_matrix_core_kernels(preset, kernel):
    # head_dim 128 with the Haar rotation runs on the matrix-core kernels
    # (the queries rotated once by a small kernel into the workspace): each
    # of them on a ragged batch, 8 query heads per kv head (16 for the
    # per-head kernels), fp32 and bf16 outputs; and, when asked for, on the
    # general fp32 kernel (its own dense rotation)
    from packed_cache_decode_amd.runtime import PackedKVCache
    H, seed = 2, 79
    G = 8 if kernel in ("ring", "page") else 16
    w = _wl(preset, H=H, Hq=G * H, d=128, seed=5, lens=(1, 900), B=5)
    inp = synth.generate(w)
    inp.seq_lens[0] = 0
    ors = OracleSide(preset, 128, seed, "haar")
    cache = np.zeros((inp.num_blocks, 16, H, ors.lay.slot_size_aligned), np.uint8)
    ors.store(cache, inp.k, inp.v, inp.slot_mapping)
    want = ors.decode(inp.q, cache, inp.block_table, inp.seq_lens, H)
    tq = PackedKVCache(preset, 128, H, 16, seed, sign_flip="haar")
    tq.set_decode_options(kernel=kernel)
    args = (to_dev(inp.q), to_dev(cache), to_dev(inp.block_table), to_dev(inp.seq_lens),
            int(max(1, inp.seq_lens.max())))
    out32 = tq.decode(*args, out_fp32=True)
    out16 = tq.decode(*args, out_fp32=False)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    check_decode(out32.cpu().numpy(), want, bf16_out=False)
    check_decode(out16.float().cpu().numpy(), want, bf16_out=True)


@pytest.mark.parametrize("preset", MSE)
@pytest.mark.parametrize("kernel,d", [("", 128), ("direct", 128), ("", 64), ("", 256)])
def test_haar_decode_query_head_passes(preset, kernel, d):
    # 24 query heads per kv head: the per-head kernels in passes of 16, the
    # queries of each pass rotated into the workspace before it (head dims
    # 64 and 256: the direct kernel at those dims)
    from packed_cache_decode_amd.runtime import PackedKVCache
    H, G, seed = 2, 24, 81
    w = _wl(preset, H=H, Hq=G * H, d=d, seed=6, lens=(1, 700), B=3)
    inp = synth.generate(w)
    ors = OracleSide(preset, d, seed, "haar")
    cache = np.zeros((inp.num_blocks, 16, H, ors.lay.slot_size_aligned), np.uint8)
    ors.store(cache, inp.k, inp.v, inp.slot_mapping)
    want = ors.decode(inp.q, cache, inp.block_table, inp.seq_lens, H)
    tq = PackedKVCache(preset, d, H, 16, seed, sign_flip="haar")
    tq.set_decode_options(kernel=kernel)
    out = tq.decode(to_dev(inp.q), to_dev(cache), to_dev(inp.block_table), to_dev(inp.seq_lens),
                    int(max(1, inp.seq_lens.max())), out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    check_decode(out.cpu().numpy(), want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_3bit_nc"])
def test_haar_split_page_store_decode_dequant(preset):
    from packed_cache_decode_amd.runtime import PackedKVCache
    H, G, T, seed, bs = 2, 4, 333, 9, 16
    w = _wl(preset, H=H, Hq=G * H, seed=3, lens=(T, T), B=1)
    inp = synth.generate(w)
    ors = OracleSide(preset, 128, seed, "haar")
    pages = np.zeros((inp.num_blocks, osoa.soa_page_bytes(ors.lay, bs, H)), np.uint8)
    osoa.store_contract(pages, bs, inp.k, inp.v, inp.slot_mapping, ors.lay, ors.signs, ors.midpoints,
                        ors.centroids)
    tq = PackedKVCache(preset, 128, H, bs, seed, sign_flip="haar", layout="soa")
    out = tq.decode(to_dev(inp.q), to_dev(pages), to_dev(inp.block_table), to_dev(inp.seq_lens), T,
                    out_fp32=True)
    k, v = tq.dequant(to_dev(pages), to_dev(inp.block_table[0].copy()), T, out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    want = osoa.decode_f64(inp.q, pages, inp.block_table, inp.seq_lens, ors.lay, ors.signs, ors.centroids,
                           H, bs)
    check_decode(out.cpu().numpy(), want, bf16_out=False)
    K, V = osoa.dequant_kv_f64(pages, ors.lay, bs, H, inp.block_table[0], T, ors.signs, ors.centroids)
    scale = np.abs(K).max(axis=-1, keepdims=True)
    assert np.all(np.abs(k.cpu().numpy() - K) <= 1e-5 * scale)
    assert np.all(np.abs(v.cpu().numpy() - V) <= 1e-5 * np.abs(V).max(axis=-1, keepdims=True))


def test_haar_dequant_and_continuation():
    from packed_cache_decode_amd.runtime import PackedKVCache
    preset, H, G, T, q_len, seed = "turboquant_k3v4_nc", 2, 4, 400, 40, 12
    w = _wl(preset, H=H, Hq=G * H, seed=8, lens=(T, T), B=1)
    inp = synth.generate(w)
    ors = OracleSide(preset, 128, seed, "haar")
    cache = np.zeros((inp.num_blocks, 16, H, ors.lay.slot_size_aligned), np.uint8)
    ors.store(cache, inp.k, inp.v, inp.slot_mapping)
    rng = np.random.default_rng(2)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((q_len, G * H, 128)).astype(np.float32))
    tq = PackedKVCache(preset, 128, H, 16, seed, sign_flip="haar")
    k, v = tq.dequant(to_dev(cache), to_dev(inp.block_table[0].copy()), T, out_fp32=True)
    out = tq.decode_continuation(to_dev(qb), to_dev(cache), to_dev(inp.block_table[0].copy()), T,
                                 out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    K, V = odec.dequant_kv_f64(cache, inp.block_table[0], T, ors.lay, ors.signs, ors.centroids)
    assert np.all(np.abs(k.cpu().numpy() - K) <= 1e-5 * np.abs(K).max(axis=-1, keepdims=True))
    want = odec.decode_continuation_f64(qb, cache, inp.block_table[0], T, ors.lay, ors.signs, ors.centroids, H)
    check_decode(out.cpu().numpy(), want, bf16_out=False)
