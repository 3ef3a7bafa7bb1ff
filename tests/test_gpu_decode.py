"""GPU parity of tq_decode against the oracle's float64 attention over the
dequantised cache: max-abs 2e-3 with fp32 output, plus half a bf16 ulp of
the reference with bf16 output (rounding to bf16 alone can exceed 2e-3 for
|o| >= 1).

Small cases decode a cache written by the oracle (so the decode is tested on
its own); full-size cases decode the cache the GPU store wrote, and compare
sampled (sequence, head) outputs with the oracle, which encodes those
sequences itself.
"""

import numpy as np
import pytest

from gpu_util import OracleSide, check_decode, to_dev
from packed_cache_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _decode_from_oracle_cache(w, seed=11, sign_flip=True, lens=None, sm_scale=None, zero_q=False,
                              out_fp32=True, mode="exact"):
    from packed_cache_decode_amd.runtime import PackedKVCache
    inp = synth.generate(w)
    if lens is not None:
        inp.seq_lens = np.minimum(np.asarray(lens, np.int32), inp.seq_lens)
    if zero_q:
        inp.q = np.zeros_like(inp.q)
    ors = OracleSide(w.preset, w.head_dim, seed, sign_flip, mode)
    cache = np.zeros((inp.num_blocks, w.block_size, w.num_kv_heads, ors.lay.slot_size_aligned), np.uint8)
    ors.store(cache, inp.k, inp.v, inp.slot_mapping)
    want = ors.decode(inp.q, cache, inp.block_table, inp.seq_lens, w.num_kv_heads, sm_scale)
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, seed, sign_flip, mode)
    max_len = int(max(1, inp.seq_lens.max()))
    out = tq.decode(to_dev(inp.q), to_dev(cache), to_dev(inp.block_table), to_dev(inp.seq_lens),
                    max_len, out_fp32=out_fp32, sm_scale=sm_scale or 0.0)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
    got = out.float().cpu().numpy()
    return got, want


def _wl(preset, G=4, H=2, d=128, bs=16, lens=(1, 700), B=4, seed=1):
    return synth.Workload(f"dec_{preset}", preset, batch=B, num_q_heads=G * H, num_kv_heads=H,
                          head_dim=d, block_size=bs, seed=seed, len_range=lens)


PRESETS = ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_k8v4", "turboquant_3bit_nc"]


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_small_parity_fp32(preset, G):
    got, want = _decode_from_oracle_cache(_wl(preset, G=G, seed=G))
    err = check_decode(got, want, bf16_out=False)
    print(f"{preset} G={G}: max abs {err:.2e}")


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("G,H", [(4, 3), (12, 2), (16, 1)])
def test_decode_per_head_kernel_shapes(preset, G, H):
    # odd kv-head counts and more than 8 query heads per kv head take the
    # per-head matrix-core kernel instead of the page-cooperative one
    got, want = _decode_from_oracle_cache(_wl(preset, G=G, H=H, B=3, seed=G + H))
    check_decode(got, want, bf16_out=False)


# TQ_DECODE_KERNEL forces one matrix-core kernel where it applies ("" picks
# by key type: page-cooperative for FP8 keys, staged for 4-bit keys with an
# even number of kv heads, direct otherwise)
KERNELS = ["", "page", "staged", "direct", "ring"]


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("H", [1, 4, 8])
@pytest.mark.parametrize("kernel", KERNELS)
def test_decode_kernels_head_counts(preset, H, kernel, monkeypatch):
    monkeypatch.setenv("TQ_DECODE_KERNEL", kernel)
    got, want = _decode_from_oracle_cache(_wl(preset, G=8 if H < 8 else 4, H=H, B=3, lens=(1, 300), seed=30 + H))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("group", ["1", "2", "4"])
def test_decode_page_kernel_head_groups(preset, group, monkeypatch):
    # the page kernel with a workgroup per part of a page row's kv heads
    monkeypatch.setenv("TQ_DECODE_KERNEL", "page")
    monkeypatch.setenv("TQ_DECODE_PAGE_HEADS", group)
    got, want = _decode_from_oracle_cache(_wl(preset, G=4, H=8, B=3, lens=(1, 300), seed=50))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_4bit_nc"])
def test_decode_sixteen_kv_heads(preset):
    # 16 kv heads per row: FP8 keys take the page kernel in groups of 8 heads
    got, want = _decode_from_oracle_cache(_wl(preset, G=2, H=16, B=2, lens=(1, 200), seed=51))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
@pytest.mark.parametrize("kernel", ["page", "staged", "direct", "ring"])
def test_decode_kernels_mse_ragged(preset, kernel, monkeypatch):
    monkeypatch.setenv("TQ_DECODE_KERNEL", kernel)
    w = _wl(preset, G=4, H=2, B=7, lens=(600, 600), seed=9)
    got, want = _decode_from_oracle_cache(w, lens=[0, 1, 15, 16, 17, 257, 600])
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
def test_decode_ring_workgroup_splits(preset, monkeypatch):
    # sequences longer than one ring workgroup split (1024 slabs) take several
    # workgroups and the merge kernel; the short one fits one split, and the
    # splits past it have nothing to do
    monkeypatch.setenv("TQ_DECODE_KERNEL", "ring")
    w = _wl(preset, G=4, H=2, B=3, lens=(100, 20000), seed=41)
    got, want = _decode_from_oracle_cache(w, lens=[100, 16400, 20000])
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
@pytest.mark.parametrize("waves", ["8", "16"])
def test_decode_ring_workgroup_sizes(preset, waves, monkeypatch):
    # the ring kernel's two workgroup shapes (8 wavefronts two per CU, 16 one
    # per CU) on empty, ragged and multi-split sequences
    monkeypatch.setenv("TQ_DECODE_KERNEL", "ring")
    monkeypatch.setenv("TQ_DECODE_RING_WAVES", waves)
    w = _wl(preset, G=8, H=2, B=6, lens=(20000, 20000), seed=43)
    got, want = _decode_from_oracle_cache(w, lens=[0, 1, 17, 600, 16400, 20000])
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("waves", ["8", "16"])
def test_decode_ring_deterministic_each_workgroup_size(waves, monkeypatch):
    monkeypatch.setenv("TQ_DECODE_KERNEL", "ring")
    monkeypatch.setenv("TQ_DECODE_RING_WAVES", waves)
    monkeypatch.setenv("TQ_DECODE_DETERMINISTIC", "1")
    w = _wl("turboquant_k3v4_nc", G=4, seed=5, lens=(100, 5000))
    a, want = _decode_from_oracle_cache(w)
    b, _ = _decode_from_oracle_cache(w)
    assert np.array_equal(a, b)
    check_decode(a, want, bf16_out=False)


@pytest.mark.parametrize("preset", PRESETS)
def test_decode_small_parity_bf16(preset):
    got, want = _decode_from_oracle_cache(_wl(preset, G=4, seed=21), out_fp32=False)
    check_decode(got, want, bf16_out=True)


@pytest.mark.parametrize("preset", PRESETS)
def test_decode_ragged_and_tiny_lengths(preset):
    # 0, 1, a page minus one, a page, a page plus one, several chunks + tail
    w = _wl(preset, G=2, B=7, lens=(600, 600), seed=5)
    got, want = _decode_from_oracle_cache(w, lens=[0, 1, 15, 16, 17, 257, 600])
    check_decode(got, want, bf16_out=False)
    assert np.all(got[0] == 0.0)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_3bit_nc"])
@pytest.mark.parametrize("bs,d", [(32, 128), (128, 128), (16, 64), (16, 256)])
def test_decode_block_sizes_and_head_dims(bs, d, preset):
    got, want = _decode_from_oracle_cache(_wl(preset, G=4, d=d, bs=bs, seed=bs + d))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
def test_decode_beta_codebook(preset):
    got, want = _decode_from_oracle_cache(_wl(preset, G=4, seed=31), mode="beta")
    check_decode(got, want, bf16_out=False)


def test_decode_pure_hadamard_custom_scale_zero_query():
    w = _wl("turboquant_k3v4_nc", G=4, seed=8)
    got, want = _decode_from_oracle_cache(w, sign_flip=False, sm_scale=0.05)
    check_decode(got, want, bf16_out=False)
    got, want = _decode_from_oracle_cache(w, zero_q=True)
    check_decode(got, want, bf16_out=False)


def test_decode_bad_page_id_sets_error():
    from packed_cache_decode_amd.runtime import PackedKVCache
    w = _wl("turboquant_4bit_nc", G=1, H=1, B=1, lens=(40, 40))
    inp = synth.generate(w)
    tq = PackedKVCache(w.preset, 128, 1, 16, 3)
    cache = tq.new_cache(inp.num_blocks)
    bt = inp.block_table.copy()
    bt[0, 1] = inp.num_blocks + 7
    tq.decode(to_dev(inp.q), cache, to_dev(bt), to_dev(inp.seq_lens), 40, out_fp32=True)
    torch.cuda.synchronize()
    assert tq.device_error() == 2
    tq.close()


@pytest.mark.parametrize("kernel", ["ring", "page", "staged", "direct"])
def test_decode_deterministic(kernel, monkeypatch):
    """With TQ_DECODE_DETERMINISTIC=1 every kernel gives the same bits on
    every run (the ring kernel deals its slabs out in a fixed order)."""
    monkeypatch.setenv("TQ_DECODE_KERNEL", kernel)
    monkeypatch.setenv("TQ_DECODE_DETERMINISTIC", "1")
    w = _wl("turboquant_4bit_nc", G=4, seed=2)
    a, _ = _decode_from_oracle_cache(w)
    b, _ = _decode_from_oracle_cache(w)
    assert np.array_equal(a, b)


def test_decode_dynamic_claims_agree_with_fixed_shares(monkeypatch):
    """The ring kernel's default (slabs claimed from a shared counter) sums in
    a run-dependent order: its results agree with the fixed-order mode to
    rounding, and both meet the oracle bound."""
    w = _wl("turboquant_4bit_nc", G=4, seed=2, lens=(3000, 9000))
    a, want = _decode_from_oracle_cache(w)
    monkeypatch.setenv("TQ_DECODE_DETERMINISTIC", "1")
    b, _ = _decode_from_oracle_cache(w)
    check_decode(a, want, bf16_out=False)
    check_decode(b, want, bf16_out=False)
    # the two orders differ by rounding only: each wavefront's running max
    # (and so the f16 hi/lo split of its weights) and the order of the fp32
    # sums follow which slabs it took.  Random rounding over n = 9000 tokens
    # moves a result by about sqrt(n) * 2^-24 * max|V| ~ 2.5e-5 (|V| < 4);
    # the bound is four times that, far inside the oracle bound of 2e-3
    assert np.max(np.abs(a - b)) < 1e-4


FULL = ["tiny", "llama3_8b", "k3v4_gqa8", "k8v4_32k", "long_131k"]


@pytest.mark.parametrize("name", FULL)
def test_decode_full_size_sampled(name):
    """Full-size workload: GPU store, then GPU decode with bf16 output (the
    configuration the benchmark times); sampled (sequence, kv head) groups are
    compared with the oracle, which encodes those sequences itself."""
    from packed_cache_decode_amd.runtime import PackedKVCache
    w = synth.WORKLOADS[name]
    print(f"[decode full] {name}: generating", flush=True)
    inp = synth.generate(w)
    seed = 777
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, seed)
    cache = tq.new_cache(inp.num_blocks)
    tq.store(to_dev(inp.k), to_dev(inp.v), to_dev(inp.slot_mapping), cache)
    max_len = int(inp.seq_lens.max())
    out = tq.decode(to_dev(inp.q), cache, to_dev(inp.block_table), to_dev(inp.seq_lens), max_len)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    got = out.float().cpu().numpy()
    tq.close()
    del cache
    ors = OracleSide(w.preset, w.head_dim, seed)
    rng = np.random.default_rng(1)
    B, H, G = w.batch, w.num_kv_heads, w.gqa
    picks = [(int(b), int(g)) for b, g in zip(rng.choice(B, size=min(B, 3), replace=False),
                                              rng.integers(0, H, size=min(B, 3)))]
    offs = inp.token_offsets()
    worst = 0.0
    for b, g in picks:
        T = int(inp.seq_lens[b])
        kk = inp.k[offs[b]:offs[b] + T, g:g + 1]
        vv = inp.v[offs[b]:offs[b] + T, g:g + 1]
        slots = ors.encode(kk, vv)                         # [T, 1, slot]
        npages = -(-T // w.block_size)
        local = np.zeros((npages, w.block_size, 1, slots.shape[-1]), np.uint8)
        t = np.arange(T)
        local[t // w.block_size, t % w.block_size] = slots
        qb = inp.q[b:b + 1, g * G:(g + 1) * G]
        want = ors.decode(qb, local, np.arange(npages)[None], np.array([T]), 1)
        worst = max(worst, check_decode(got[b:b + 1, g * G:(g + 1) * G], want, bf16_out=True))
    print(f"[decode full] {name}: sampled {picks}, max abs err {worst:.2e}", flush=True)


@pytest.mark.parametrize("preset,kernel", [("turboquant_k8v4", ""), ("turboquant_4bit_nc", "page"),
                                           ("turboquant_4bit_nc", "staged"), ("turboquant_k3v4_nc", "ring")])
def test_decode_workspace_reuse_across_shapes(preset, kernel, monkeypatch):
    """One context, one workspace, several calls of different batch and
    length (the workspace is reused as the split count changes): each result
    matches the oracle."""
    from packed_cache_decode_amd.runtime import PackedKVCache
    monkeypatch.setenv("TQ_DECODE_KERNEL", kernel)
    seed = 13
    tq = PackedKVCache(preset, 128, 2, 16, seed)
    ors = OracleSide(preset, 128, seed)
    for B, lens, wseed in [(7, (1, 900), 3), (3, (300, 2000), 4), (9, (1, 64), 5), (7, (1, 900), 3)]:
        w = _wl(preset, G=4, H=2, B=B, lens=lens, seed=wseed)
        inp = synth.generate(w)
        cache = np.zeros((inp.num_blocks, 16, 2, ors.lay.slot_size_aligned), np.uint8)
        ors.store(cache, inp.k, inp.v, inp.slot_mapping)
        want = ors.decode(inp.q, cache, inp.block_table, inp.seq_lens, 2)
        out = tq.decode(to_dev(inp.q), to_dev(cache), to_dev(inp.block_table), to_dev(inp.seq_lens),
                        int(inp.seq_lens.max()), out_fp32=True)
        torch.cuda.synchronize()
        check_decode(out.cpu().numpy(), want, bf16_out=False)
    assert tq.device_error() == 0
    tq.close()


@pytest.mark.parametrize("preset,H,kernel", [("turboquant_k8v4", 1, ""), ("turboquant_4bit_nc", 2, ""),
                                             ("turboquant_4bit_nc", 2, "ring")])
def test_decode_many_short_sequences(preset, H, kernel, monkeypatch):
    """4100 short sequences (0 to 40 tokens): a single token often dominates
    the softmax, which is where the P.V weights need more than one f16."""
    monkeypatch.setenv("TQ_DECODE_KERNEL", kernel)
    w = _wl(preset, G=1, H=H, B=4100, lens=(0, 40), seed=17)
    got, want = _decode_from_oracle_cache(w)
    check_decode(got, want, bf16_out=False)
