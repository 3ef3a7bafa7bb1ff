"""Whole-output parity at full size: every addressed slot of the cache the GPU
store wrote, and every (sequence, query head) output of the GPU decode, on
the five workloads at their full sizes and in the launch configuration the
benchmark times (the default decode options), against the oracle.

The oracle encodes every token itself and decodes from its own cache, in a
pool of worker processes (``fullsize_oracle``).  Store: byte-exact except at
proven ties (float64 value within 1e-6 of the boundary between the two
codes), tolerated mismatches below 1e-5 of the coordinates, nothing written
outside the addressed slots (both caches start from the same canary fill and
have two spare pages).  Decode: max-abs 2e-3 with fp32 output, and 2e-3 plus
half a bf16 ulp of the reference with bf16 output.  Each case prints its
counts: tolerated tie mismatches, near-ties, max-abs, mean-abs and the
location of the largest error.
"""

import multiprocessing as mp
import os
import shutil
import tempfile
import time

import numpy as np
import pytest

import fullsize_oracle as fo
from gpu_util import to_dev
from packed_cache_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FULL = ["tiny", "llama3_8b", "k3v4_gqa8", "k8v4_32k", "long_131k"]
MEAN_GUARD = 5e-6
SEED = 4242


def _log(name, msg):
    print(f"[full {name}] {msg}", flush=True)


@pytest.fixture(scope="module")
def pool():
    ctx = mp.get_context("forkserver")
    with ctx.Pool(fo.worker_count()) as p:
        yield p


def _imap(pool, fn, jobs, name, what):
    out, n, t0 = [], len(jobs), time.time()
    step = max(1, n // 8)
    for i, r in enumerate(pool.imap_unordered(fn, jobs), 1):
        out.append(r)
        if i % step == 0 or i == n:
            _log(name, f"{what}: {i}/{n} units, {time.time() - t0:.1f} s")
    return out


def run_full(name, layout, pool):
    from packed_cache_decode_amd.runtime import PackedKVCache
    w = synth.WORKLOADS[name]
    soa = layout == "soa"
    _log(name, f"layout {layout}: generating inputs")
    inp = synth.generate(w)
    tmp = tempfile.mkdtemp(prefix=f"tq_full_{name}_")
    try:
        for key, arr in (("k", inp.k), ("v", inp.v), ("sm", inp.slot_mapping), ("q", inp.q),
                         ("bt", inp.block_table), ("sl", inp.seq_lens)):
            np.save(os.path.join(tmp, key + ".npy"), arr)

        # ---- GPU: store every token, then decode (bf16 and fp32 output) ----
        _log(name, "GPU store + decode")
        tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, SEED, layout=layout)
        cache = tq.new_cache(inp.num_blocks + 2, fo.CANARY)
        tq.store(to_dev(inp.k), to_dev(inp.v), to_dev(inp.slot_mapping), cache)
        max_len = int(max(1, inp.seq_lens.max()))
        q, bt, sl = to_dev(inp.q), to_dev(inp.block_table), to_dev(inp.seq_lens)
        out16 = tq.decode(q, cache, bt, sl, max_len)
        out32 = tq.decode(q, cache, bt, sl, max_len, out_fp32=True)
        torch.cuda.synchronize()
        err = tq.device_error()
        got_cache = cache.cpu().numpy()
        got16 = out16.float().cpu().numpy()
        got32 = out32.cpu().numpy()
        tq.close()
        del cache, q, bt, sl, out16, out32
        assert err == 0, f"device error word {err}"

        # ---- oracle store into its own canary-filled cache ----
        want = np.lib.format.open_memmap(os.path.join(tmp, "want_cache.npy"), mode="w+",
                                         dtype=np.uint8, shape=got_cache.shape)
        want[:] = fo.CANARY
        want.flush()
        del want
        N = inp.num_tokens
        chunk = int(min(4096, max(512, N // (4 * fo.worker_count()))))
        jobs = [(tmp, a, min(N, a + chunk), w.preset, w.head_dim, SEED, w.block_size, soa)
                for a in range(0, N, chunk)]
        st = _imap(pool, fo.store_chunk, jobs, name, "oracle store")
        k_near = sum(r["k_near"] for r in st)
        v_near = sum(r["v_near"] for r in st)
        vectors = sum(r["vectors"] for r in st)
        want = np.load(os.path.join(tmp, "want_cache.npy"), mmap_mode="r")
        lay, signs, c, m = fo.oracle_tables(w.preset, w.head_dim, SEED)
        nslots = got_cache.shape[0] * w.block_size
        sm = inp.slot_mapping
        valid = (sm >= 0) & (sm < nslots)
        inv = np.full(nslots, -1, np.int64)
        inv[sm[valid]] = np.nonzero(valid)[0]
        res = fo.compare_store(got_cache, np.asarray(want), lambda t: inp.k[t], lambda t: inp.v[t],
                               lambda s: inv[s], lay, signs, c, m, soa, w.block_size,
                               w.num_kv_heads)
        coords = vectors * w.head_dim * (1 if lay.key_fp8 else 2)
        tolerated = res["k_tie_mismatch"] + res["v_tie_mismatch"]
        _log(name, f"store: {vectors} vectors, {res['bytes_differing']} bytes differ, "
                   f"tolerated tie mismatches K {res['k_tie_mismatch']} V {res['v_tie_mismatch']} "
                   f"({tolerated / coords:.2e} of coordinates), near-ties K {k_near} "
                   f"({k_near / max(1, vectors * w.head_dim):.2e}) V {v_near}")
        assert tolerated < 1e-5 * coords
        del want

        # ---- oracle decode of every (sequence, kv head) from its own cache ----
        B, H, G = w.batch, w.num_kv_heads, w.gqa
        groups = [(b, g) for b in range(B) for g in range(H)]
        per_job = max(1, len(groups) // (4 * fo.worker_count()))
        jobs = [(tmp, groups[i:i + per_job], w.preset, w.head_dim, SEED, w.block_size, H, soa)
                for i in range(0, len(groups), per_job)]
        want_out = np.full((B, H * G, w.head_dim), np.nan)
        for part in _imap(pool, fo.decode_groups, jobs, name, "oracle decode"):
            for b, g, o in part:
                want_out[b, g * G:(g + 1) * G] = o
        assert not np.isnan(want_out).any()
        s32 = fo.decode_stats(got32, want_out, bf16_out=False)
        s16 = fo.decode_stats(got16, want_out, bf16_out=True)
        for tag, s in (("fp32 out", s32), ("bf16 out", s16)):
            _log(name, f"decode {tag}: {s['outputs']} outputs, max-abs {s['max_abs']:.3e} at "
                       f"(sequence, head, coordinate) {s['argmax']}, mean-abs {s['mean_abs']:.3e}, "
                       f"beyond tolerance {s['beyond']}")
        assert s32["beyond"] == 0 and s16["beyond"] == 0
        # A guard on the arithmetic itself, beside the 2e-3 parity bound:
        # scores and weights carried as f16 hi + lo pairs (about 2^-20 of
        # each) and fp32 sums leave a mean error of a few 1e-7 on these
        # unit-scale outputs.  A lossy change that still passes 2e-3 shows
        # here (V codes fed to the matrix cores as f16 subnormals, whose
        # products are not summed exactly, put the mean near 2e-5).
        assert s32["mean_abs"] < MEAN_GUARD, s32
        return res, s32, s16
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_output(name, pool):
    run_full(name, "aos", pool)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama3_8b", "k3v4_gqa8", "long_131k"])
def test_full_size_whole_output_split_page(name, pool):
    run_full(name, "soa", pool)
