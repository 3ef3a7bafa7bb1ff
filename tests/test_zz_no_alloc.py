"""The allocation-free decode entry point (tq_decode_noalloc) against tq_decode:
two calls in a row on one context, the second with a smaller input, each
equal bit for bit to tq_decode's output on the same inputs (the same
kernels and plan; the partials go to the library's scratch array instead
of the caller's workspace), and a shape that needs more scratch than the
array holds refused before anything is enqueued.
"""

import numpy as np
import pytest

from gpu_util import to_dev
from packed_cache_decode_amd import _lib, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(tq, w, out_fp32):
    inp = synth.generate(w)
    cache = tq.new_cache(inp.num_blocks)
    tq.store(to_dev(inp.k), to_dev(inp.v), to_dev(inp.slot_mapping), cache)
    q, bt, sl = to_dev(inp.q), to_dev(inp.block_table), to_dev(inp.seq_lens)
    max_len = int(inp.seq_lens.max())
    want = tq.decode(q, cache, bt, sl, max_len, out_fp32=out_fp32)
    dt = torch.float32 if out_fp32 else torch.bfloat16
    got = torch.full_like(want, float("nan"))
    _lib.tq_decode_noalloc(tq.ctx, q, cache, cache.shape[0], bt, bt.shape[1], sl, w.batch,
                           w.num_q_heads, max_len, 0.0, got, got.dtype == torch.float32)
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    assert got.dtype == dt
    return got.view(torch.int16 if not out_fp32 else torch.int32).cpu().numpy(), \
        want.view(torch.int16 if not out_fp32 else torch.int32).cpu().numpy(), \
        _lib.tq_decode_workspace_bytes(tq.ctx, w.batch, w.num_q_heads, max_len)


@pytest.mark.parametrize("preset,kernel", [("turboquant_4bit_nc", ""), ("turboquant_k8v4", ""),
                                           ("turboquant_k3v4_nc", "staged")])
def test_noalloc_equals_decode_on_two_calls(preset, kernel):
    from packed_cache_decode_amd.runtime import PackedKVCache
    tq = PackedKVCache(preset, 128, 8, 16, 5)
    tq.set_decode_options(kernel=kernel)
    big = synth.Workload("noalloc_big", preset, batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         block_size=16, seed=3, len_range=(20000, 40000))
    small = synth.Workload("noalloc_small", preset, batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=16, seed=4, len_range=(1, 9000))
    got, want, ws_big = _case(tq, big, out_fp32=False)
    assert ws_big > 0                       # the call used the scratch array
    assert np.array_equal(got, want)
    got, want, _ = _case(tq, small, out_fp32=True)
    assert np.array_equal(got, want)
    tq.close()


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    from packed_cache_decode_amd.runtime import PackedKVCache
    tq = PackedKVCache("turboquant_4bit_nc", 128, 8, 16, 5)
    limit = _lib.tq_decode_noalloc_max_bytes()
    assert limit == 32 << 20
    # a declared shape (never launched) whose partials exceed the array
    B, Hq, T = 4096, 64, 1 << 20
    assert _lib.tq_decode_workspace_bytes(tq.ctx, B, Hq, T) > limit
    small = torch.zeros(256, dtype=torch.int32, device="cuda")
    st = _lib.load().tq_decode_noalloc(tq.ctx, small.data_ptr(), small.data_ptr(), 1, small.data_ptr(),
                                       T // 16, small.data_ptr(), B, Hq, T, 0.0, small.data_ptr(), 1,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == -4                         # TQ_ERR_WORKSPACE, nothing enqueued
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    tq.close()
