"""GPU parity of tq_decode against the oracle's float64 attention over the
dequantised cache: max-abs 2e-3 with fp32 output, plus half a bf16 ulp of
the reference with bf16 output (rounding to bf16 alone can exceed 2e-3 for
|o| >= 1).

Every case decodes a cache written by the oracle, so the decode is tested on
its own; the full-size workloads, decoding the cache the GPU store wrote,
are compared output by output in test_gpu_fullsize.py.
"""

import numpy as np
import pytest

from gpu_util import OracleSide, check_decode, to_dev
from packed_cache_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _decode_from_oracle_cache(w, seed=11, sign_flip=True, lens=None, sm_scale=None, zero_q=False,
                              out_fp32=True, mode="exact", opts=None):
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
    if opts:
        tq.set_decode_options(**opts)
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


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("G,H", [(24, 2), (40, 1)])
def test_decode_query_head_passes(preset, G, H):
    # more query heads per kv head than one pass of a per-head matrix-core
    # kernel takes (16): passes of 16 (the last one short) over the cache,
    # one merge for every head; empty, one-token and multi-split lengths
    w = _wl(preset, G=G, H=H, B=4, lens=(3000, 3000), seed=G + H)
    got, want = _decode_from_oracle_cache(w, lens=[0, 1, 1500, 3000])
    check_decode(got, want, bf16_out=False)
    got16, want16 = _decode_from_oracle_cache(w, lens=[0, 1, 1500, 3000], out_fp32=False)
    check_decode(got16, want16, bf16_out=True)


def test_decode_more_than_16_query_heads_general_kernel_refuses():
    # the general kernel takes at most 16 query heads per kv head
    from packed_cache_decode_amd import _lib
    w = _wl("turboquant_4bit_nc", G=24, H=1, d=64, B=1, lens=(20, 20), seed=3)
    with pytest.raises(_lib.TQError, match="UNSUPPORTED"):
        _decode_from_oracle_cache(w, opts=dict(kernel="general"))


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("d", [64, 256])
def test_decode_head_dims_64_256_query_head_passes(preset, d):
    # more than 16 query heads per kv head at head dims 64 and 256: the
    # direct kernel in passes of 16 (the last one short), one merge for all
    w = _wl(preset, G=24, H=2, d=d, B=4, lens=(900, 900), seed=d + 7)
    got, want = _decode_from_oracle_cache(w, lens=[0, 1, 450, 900])
    check_decode(got, want, bf16_out=False)


# the context's decode options force one kernel where it applies ("" picks by
# key type and shape: page-cooperative for FP8 keys, ring for 3/4-bit keys
# with up to 8 query heads per kv head, staged or direct otherwise; "general"
# is the fp32 vector-ALU kernel)
KERNELS = ["", "page", "staged", "direct", "ring", "general"]


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("H", [1, 4, 8])
@pytest.mark.parametrize("kernel", KERNELS)
def test_decode_kernels_head_counts(preset, H, kernel):
    got, want = _decode_from_oracle_cache(_wl(preset, G=8 if H < 8 else 4, H=H, B=3, lens=(1, 300), seed=30 + H),
                                          opts=dict(kernel=kernel))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("group", ["1", "2", "4"])
def test_decode_page_kernel_head_groups(preset, group):
    # the page kernel with a workgroup per part of a page row's kv heads
    got, want = _decode_from_oracle_cache(_wl(preset, G=4, H=8, B=3, lens=(1, 300), seed=50),
                                          opts=dict(kernel="page", page_heads=int(group)))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_k8v4", "turboquant_4bit_nc"])
def test_decode_sixteen_kv_heads(preset):
    # 16 kv heads per row: FP8 keys take the page kernel in groups of 8 heads
    got, want = _decode_from_oracle_cache(_wl(preset, G=2, H=16, B=2, lens=(1, 200), seed=51))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
@pytest.mark.parametrize("kernel", ["page", "staged", "direct", "ring", "general"])
def test_decode_kernels_mse_ragged(preset, kernel):
    w = _wl(preset, G=4, H=2, B=7, lens=(600, 600), seed=9)
    got, want = _decode_from_oracle_cache(w, lens=[0, 1, 15, 16, 17, 257, 600], opts=dict(kernel=kernel))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
def test_decode_ring_workgroup_splits(preset):
    # sequences longer than one ring workgroup split (1024 slabs) take several
    # workgroups and the merge kernel; the short one fits one split, and the
    # splits past it have nothing to do
    w = _wl(preset, G=4, H=2, B=3, lens=(100, 20000), seed=41)
    got, want = _decode_from_oracle_cache(w, lens=[100, 16400, 20000], opts=dict(kernel="ring"))
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc"])
@pytest.mark.parametrize("waves", ["8", "16"])
def test_decode_ring_length_order(preset, waves):
    # more (sequence, kv head) pairs than compute units: the ring workgroups
    # are dispatched in the order of a device-side ranking of the lengths
    # (ragged, with empty, one-token and equal lengths)
    rng = np.random.default_rng(17)
    lens = [int(x) for x in rng.integers(0, 1500, size=40)]
    lens[:5] = [0, 1, 700, 700, 1499]
    w = _wl(preset, G=2, H=8, B=40, lens=(1500, 1500), seed=67)
    got, want = _decode_from_oracle_cache(w, lens=lens, opts=dict(kernel="ring", ring_waves=int(waves)))
    check_decode(got, want, bf16_out=False)
    # a larger batch (150 sequences, more ranks than one wavefront holds)
    lens = [int(x) for x in rng.integers(0, 500, size=150)]
    lens[:3] = [0, 499, 499]
    w = _wl(preset, G=4, H=2, B=150, lens=(500, 500), seed=69)
    got, want = _decode_from_oracle_cache(w, lens=lens, opts=dict(kernel="ring", ring_waves=int(waves)))
    check_decode(got, want, bf16_out=False)
    # at least two whole layers of workgroups per XCD (the 8-wavefront
    # workgroups then pair long with short sequences on each CU): 61
    # sequences x 8 kv heads (some XCDs one sequence short), and 150 x 4
    # (more layers than the two resident ones)
    for B, H, seed in ((61, 8, 71), (150, 4, 73)):
        lens = [int(x) for x in rng.integers(0, 400, size=B)]
        lens[:4] = [0, 1, 399, 399]
        w = _wl(preset, G=2, H=H, B=B, lens=(400, 400), seed=seed)
        got, want = _decode_from_oracle_cache(w, lens=lens, opts=dict(kernel="ring", ring_waves=int(waves)))
        check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("preset", ["turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"])
@pytest.mark.parametrize("waves", ["8", "16"])
def test_decode_ring_workgroup_sizes(preset, waves):
    # the ring kernel's two workgroup shapes (8 wavefronts two per CU, 16 one
    # per CU) on empty, ragged and multi-split sequences, with fixed and with
    # dynamic slab claims
    w = _wl(preset, G=8, H=2, B=6, lens=(20000, 20000), seed=43)
    for dyn in (False, True):
        got, want = _decode_from_oracle_cache(w, lens=[0, 1, 17, 600, 16400, 20000],
                                              opts=dict(kernel="ring", ring_waves=int(waves),
                                                        dynamic_claims=dyn))
        check_decode(got, want, bf16_out=False)
    check_decode(got, want, bf16_out=False)


@pytest.mark.parametrize("waves", ["8", "16"])
def test_decode_ring_deterministic_each_workgroup_size(waves):
    opts = dict(kernel="ring", ring_waves=int(waves))
    w = _wl("turboquant_k3v4_nc", G=4, seed=5, lens=(100, 5000))
    a, want = _decode_from_oracle_cache(w, opts=opts)
    b, _ = _decode_from_oracle_cache(w, opts=opts)
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


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("G,H,bs", [(1, 3, 16), (7, 2, 32), (16, 1, 16)])
@pytest.mark.parametrize("kernel", ["", "general"])
def test_decode_head_dims_64_256(preset, d, G, H, bs, kernel):
    # head dims 64 and 256 on the slotted page take the direct matrix-core
    # kernel at those dims (queries rotated into the workspace, D/32 score
    # steps, D/16 value tiles, its own merge); the general fp32 kernel on the
    # same inputs when asked.  Empty, one-token, page-edge and multi-split
    # lengths; fp32 and bf16 outputs.
    w = _wl(preset, G=G, H=H, d=d, bs=bs, B=6, lens=(1200, 1200), seed=G + H + d)
    lens = [0, 1, 15, 16, 33, 1200]
    got, want = _decode_from_oracle_cache(w, lens=lens, opts=dict(kernel=kernel))
    check_decode(got, want, bf16_out=False)
    assert np.all(got[0] == 0.0)
    got16, want16 = _decode_from_oracle_cache(w, lens=lens, out_fp32=False, opts=dict(kernel=kernel))
    check_decode(got16, want16, bf16_out=True)


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
def test_decode_deterministic(kernel):
    """With the default options every kernel gives the same bits on every run
    (the ring kernel deals its slabs out in a fixed order)."""
    w = _wl("turboquant_4bit_nc", G=4, seed=2)
    a, _ = _decode_from_oracle_cache(w, opts=dict(kernel=kernel))
    b, _ = _decode_from_oracle_cache(w, opts=dict(kernel=kernel))
    assert np.array_equal(a, b)


def test_decode_dynamic_claims_agree_with_fixed_shares():
    """The ring kernel's dynamic claims (slabs claimed from a shared counter)
    sum in a run-dependent order: its results agree with the default fixed
    order to rounding, and both meet the oracle bound."""
    w = _wl("turboquant_4bit_nc", G=4, seed=2, lens=(3000, 9000))
    a, want = _decode_from_oracle_cache(w, opts=dict(dynamic_claims=True))
    b, _ = _decode_from_oracle_cache(w)
    check_decode(a, want, bf16_out=False)
    check_decode(b, want, bf16_out=False)
    # the two orders differ by rounding only: each wavefront's running max
    # (and so the f16 hi/lo split of its weights) and the order of the fp32
    # sums follow which slabs it took.  Random rounding over n = 9000 tokens
    # moves a result by about sqrt(n) * 2^-24 * max|V| ~ 2.5e-5 (|V| < 4);
    # the bound is four times that, far inside the oracle bound of 2e-3
    assert np.max(np.abs(a - b)) < 1e-4


@pytest.mark.parametrize("preset,kernel", [("turboquant_k8v4", ""), ("turboquant_4bit_nc", "page"),
                                           ("turboquant_4bit_nc", "staged"), ("turboquant_k3v4_nc", "ring")])
def test_decode_workspace_reuse_across_shapes(preset, kernel):
    """One context, one workspace, several calls of different batch and
    length (the workspace is reused as the split count changes): each result
    matches the oracle."""
    from packed_cache_decode_amd.runtime import PackedKVCache
    seed = 13
    tq = PackedKVCache(preset, 128, 2, 16, seed)
    tq.set_decode_options(kernel=kernel)
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
def test_decode_many_short_sequences(preset, H, kernel):
    """4100 short sequences (0 to 40 tokens): a single token often dominates
    the softmax, which is where the P.V weights need more than one f16."""
    w = _wl(preset, G=1, H=H, B=4100, lens=(0, 40), seed=17)
    got, want = _decode_from_oracle_cache(w, opts=dict(kernel=kernel))
    check_decode(got, want, bf16_out=False)


def test_decode_options_round_trip_and_validation():
    """Options set through the ABI are read back; values outside the
    documented ones are rejected and leave the context unchanged."""
    from packed_cache_decode_amd import _lib
    from packed_cache_decode_amd.runtime import PackedKVCache
    tq = PackedKVCache("turboquant_4bit_nc", 128, 2, 16, 1)
    assert _lib.tq_get_decode_options(tq.ctx) == dict(kernel=0, dynamic_claims=0, ring_waves=0,
                                                      page_heads=0)
    tq.set_decode_options(kernel="page", dynamic_claims=True, ring_waves=8, page_heads=2)
    want = dict(kernel=2, dynamic_claims=1, ring_waves=8, page_heads=2)
    assert _lib.tq_get_decode_options(tq.ctx) == want
    tq.set_decode_options(kernel="general")
    assert _lib.tq_get_decode_options(tq.ctx)["kernel"] == 5
    tq.set_decode_options(kernel="page", dynamic_claims=True, ring_waves=8, page_heads=2)
    for bad in (dict(kernel=6), dict(kernel=-1), dict(ring_waves=12), dict(page_heads=3)):
        with pytest.raises(_lib.TQError):
            _lib.tq_set_decode_options(tq.ctx, **bad)
        assert _lib.tq_get_decode_options(tq.ctx) == want
    _lib.tq_set_decode_options(tq.ctx)
    assert _lib.tq_get_decode_options(tq.ctx)["kernel"] == 0
    tq.close()


def test_device_error_read_on_a_side_stream():
    """The sticky error word is read after the given stream's work only."""
    from packed_cache_decode_amd.runtime import PackedKVCache
    w = _wl("turboquant_4bit_nc", G=1, H=1, B=1, lens=(40, 40))
    inp = synth.generate(w)
    tq = PackedKVCache(w.preset, 128, 1, 16, 3)
    cache = tq.new_cache(inp.num_blocks)
    bt = inp.block_table.copy()
    bt[0, 0] = -3
    side = torch.cuda.Stream()
    q, btd, sl = to_dev(inp.q), to_dev(bt), to_dev(inp.seq_lens)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tq.decode(q, cache, btd, sl, 40, out_fp32=True, stream=side)
        assert tq.device_error(stream=side) == 2
        assert tq.device_error(stream=side) == 0
    tq.close()
