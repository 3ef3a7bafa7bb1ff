"""GPU parity of the two chunked-prefill helpers against the oracle:
tq_dequant (full dequantisation back to the original space) and
tq_decode_continuation (a chunk of queries run as decode requests of growing
length).  Both read a cache the oracle wrote.

Tolerances: dequant with fp32 output within 1e-5 of each row's largest
|value| (the fp32 butterflies and norm factor against float64); with bf16
output, half a bf16 ulp more.  Continuation: the decode bound, max-abs 2e-3.
"""

import numpy as np
import pytest

from gpu_util import OracleSide, bf16_half_ulp, check_decode, to_dev
from oracle import decode as odec
from oracle import soa as osoa
from packed_cache_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PRESETS = ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_k8v4", "turboquant_3bit_nc"]


def _seq(preset, T, H, d=128, bs=16, seed=3, Hq=None):
    w = synth.Workload("pf", preset, batch=1, num_q_heads=Hq or 2 * H, num_kv_heads=H, head_dim=d,
                       block_size=bs, seed=seed, len_range=(T, T))
    return w, synth.generate(w)


def _oracle_cache(w, inp, ors, layout_name):
    if layout_name == "soa":
        pages = np.zeros((inp.num_blocks, osoa.soa_page_bytes(ors.lay, w.block_size, w.num_kv_heads)), np.uint8)
        osoa.store_contract(pages, w.block_size, inp.k, inp.v, inp.slot_mapping, ors.lay, ors.signs,
                            ors.midpoints, ors.centroids)
        return pages
    cache = np.zeros((inp.num_blocks, w.block_size, w.num_kv_heads, ors.lay.slot_size_aligned), np.uint8)
    ors.store(cache, inp.k, inp.v, inp.slot_mapping)
    return cache


def _want_kv(w, inp, ors, cache, layout_name, T):
    if layout_name == "soa":
        return osoa.dequant_kv_f64(cache, ors.lay, w.block_size, w.num_kv_heads, inp.block_table[0], T,
                                   ors.signs, ors.centroids)
    return odec.dequant_kv_f64(cache, inp.block_table[0], T, ors.lay, ors.signs, ors.centroids)


def _check_kv(got, want, bf16):
    scale = np.abs(want).max(axis=-1, keepdims=True)
    tol = 1e-5 * scale + (2 * bf16_half_ulp(want) if bf16 else 0.0)
    err = np.abs(np.asarray(got, np.float64) - want)
    assert np.all(err <= tol), f"max err {err.max():.3e}"


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("d,bs,H", [(128, 16, 8), (128, 32, 3), (64, 16, 2), (256, 64, 2)])
def test_dequant_parity(preset, d, bs, H):
    from packed_cache_decode_amd.runtime import PackedKVCache
    T = 301
    w, inp = _seq(preset, T, H, d=d, bs=bs, seed=d + bs + H)
    seed = 21
    ors = OracleSide(preset, d, seed)
    cache = _oracle_cache(w, inp, ors, "aos")
    tq = PackedKVCache(preset, d, H, bs, seed)
    bt = to_dev(inp.block_table[0].copy())
    for fp32 in (True, False):
        k, v = tq.dequant(to_dev(cache), bt, T, out_fp32=fp32)
        torch.cuda.synchronize()
        K, V = _want_kv(w, inp, ors, cache, "aos", T)
        _check_kv(k.float().cpu().numpy(), K, not fp32)
        _check_kv(v.float().cpu().numpy(), V, not fp32)
    assert tq.device_error() == 0
    tq.close()


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
@pytest.mark.parametrize("d,bs", [(128, 16), (64, 32)])
def test_dequant_parity_split_page(preset, d, bs):
    from packed_cache_decode_amd.runtime import PackedKVCache
    T, H, seed = 257, 4, 5
    w, inp = _seq(preset, T, H, d=d, bs=bs, seed=9)
    ors = OracleSide(preset, d, seed)
    pages = _oracle_cache(w, inp, ors, "soa")
    tq = PackedKVCache(preset, d, H, bs, seed, layout="soa")
    k, v = tq.dequant(to_dev(pages), to_dev(inp.block_table[0].copy()), T, out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    K, V = _want_kv(w, inp, ors, pages, "soa", T)
    _check_kv(k.cpu().numpy(), K, False)
    _check_kv(v.cpu().numpy(), V, False)


def test_dequant_bad_page_writes_zeros_and_flags():
    from packed_cache_decode_amd.runtime import PackedKVCache
    preset, T, H, seed = "turboquant_4bit_nc", 64, 2, 1
    w, inp = _seq(preset, T, H, seed=4)
    ors = OracleSide(preset, 128, seed)
    cache = _oracle_cache(w, inp, ors, "aos")
    bt = inp.block_table[0].copy()
    bt[1] = inp.num_blocks + 5                       # tokens 16..31 point outside the cache
    tq = PackedKVCache(preset, 128, H, 16, seed)
    k, v = tq.dequant(to_dev(cache), to_dev(bt), T, out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 2
    tq.close()
    k, v = k.cpu().numpy(), v.cpu().numpy()
    assert np.all(k[16:32] == 0) and np.all(v[16:32] == 0)
    K, V = _want_kv(w, inp, ors, cache, "aos", T)
    _check_kv(k[:16], K[:16], False)
    _check_kv(k[32:], K[32:], False)


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("T,q_len,G", [(300, 37, 4), (129, 128, 8), (1000, 1, 4), (2100, 64, 2)])
def test_decode_continuation_parity(preset, T, q_len, G):
    _continuation_case(preset, T, q_len, G)


def _continuation_case(preset, T, q_len, G, kernel=""):
    from packed_cache_decode_amd.runtime import PackedKVCache
    H, seed = 2, 8
    w, inp = _seq(preset, T, H, Hq=G * H, seed=T + q_len)
    ors = OracleSide(preset, 128, seed)
    cache = _oracle_cache(w, inp, ors, "aos")
    rng = np.random.default_rng(q_len)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((q_len, G * H, 128)).astype(np.float32))
    want = odec.decode_continuation_f64(qb, cache, inp.block_table[0], T, ors.lay, ors.signs,
                                        ors.centroids, H)
    tq = PackedKVCache(preset, 128, H, 16, seed)
    tq.set_decode_options(kernel=kernel)
    out = tq.decode_continuation(to_dev(qb), to_dev(cache), to_dev(inp.block_table[0].copy()), T,
                                 out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    check_decode(out.cpu().numpy(), want, bf16_out=False)


@pytest.mark.parametrize("kernel", ["ring", "page", "staged", "direct"])
def test_decode_continuation_each_kernel(kernel):
    """Short sequences with peaked softmax (the case that exposed an
    accumulation that lost precision) through each decode kernel."""
    _continuation_case("turboquant_k3v4_nc", 300, 37, 4, kernel)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_3bit_nc"])
def test_decode_continuation_split_page(preset):
    from packed_cache_decode_amd.runtime import PackedKVCache
    T, q_len, H, G, bs, seed = 700, 50, 2, 4, 16, 6
    w, inp = _seq(preset, T, H, Hq=G * H, seed=12)
    ors = OracleSide(preset, 128, seed)
    pages = _oracle_cache(w, inp, ors, "soa")
    rng = np.random.default_rng(5)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((q_len, G * H, 128)).astype(np.float32))
    lens = T - q_len + 1 + np.arange(q_len)
    want = osoa.decode_f64(qb, pages, np.repeat(inp.block_table[:1], q_len, 0), lens, ors.lay, ors.signs,
                           ors.centroids, H, bs)
    tq = PackedKVCache(preset, 128, H, bs, seed, layout="soa")
    out = tq.decode_continuation(to_dev(qb), to_dev(pages), to_dev(inp.block_table[0].copy()), T)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    check_decode(out.float().cpu().numpy(), want, bf16_out=True)
