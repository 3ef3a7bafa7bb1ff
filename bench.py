"""Benchmark of the packed KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3_8b]

One step = the whole hot path over one batch of the workload: tq_store of
every (token, kv head) of the batch into the paged cache, then one tq_decode
step for every sequence.  Inputs (bf16 K/V/q, slot mapping, block tables) are
seeded synthetic data of the workload's shape, resident in HBM before timing.
Before each kernel a 1 GiB buffer is read (outside the event-timed
intervals) so neither call is served from L2 or the 256 MB Infinity Cache;
reading, unlike writing, leaves no dirty lines to be written back during the
timed kernel.

Printed: one JSON line.  `value` is decode HBM throughput in GB/s: the
algorithmic bytes of one decode (packed cache of every token and kv head,
q, output, block-table entries, seq_lens) divided by the event-timed
duration of tq_decode (its split kernel and its combine kernel), averaged
over the K timed steps.  The store's tokens/s comes from the same steps.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# kernel sources whose counter-measured HBM traffic profiles/ records
KERNEL_SOURCES = {
    "decode": ("packed_cache_decode_amd/csrc/tq_decode.hip", "packed_cache_decode_amd/csrc/tq_decode_mfma.hip",
               "packed_cache_decode_amd/csrc/tq_internal.h"),
    "store": ("packed_cache_decode_amd/csrc/tq_store.hip", "packed_cache_decode_amd/csrc/tq_internal.h"),
}


def sources_sha256(kind):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(kind, workload, layout="aos"):
    """HBM bytes per launch of the store or decode on `workload`, as rocprofv3's
    FETCH_SIZE + WRITE_SIZE counters read them (calibrated against plain
    streaming kernels of known size), from the summary under profiles/; None
    when there is no summary taken on the current kernel sources."""
    suffix = "" if layout == "aos" else f"_{layout}"
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}{suffix}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_sources_sha256") != sources_sha256(kind) or "hbm_bytes_per_launch" not in rec:
        return None
    return int(float(rec["hbm_bytes_per_launch"]))


def decode_alg_bytes(inp, slot):
    w = inp.w
    T = inp.seq_lens.astype(int)
    pages = -(-T // w.block_size)
    return int(T.sum() * w.num_kv_heads * slot + 2 * w.batch * w.num_q_heads * w.head_dim * 2
               + 4 * pages.sum() + 4 * w.batch)


def store_alg_bytes_per_token(w, slot):
    return w.num_kv_heads * (2 * w.head_dim * 2 + slot) + 8


def cpu_baseline(inp, slot, budget_s=12.0):
    """Time the CPU oracle (as it is) on a bounded sample of the workload."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:           # pragma: no cover
        threadpool_limits = None
    import numpy as np

    from oracle import codebook as cb
    from oracle import decode as odec
    from oracle import layout, rotation
    from oracle import store as ost

    w = inp.w
    lay = layout.slot_layout(w.preset, w.head_dim)
    signs = rotation.rotation_signs(99, w.head_dim)
    kb = 4 if lay.key_fp8 else lay.key_bits
    c, m = cb.codebook(w.head_dim, kb)
    import contextlib
    lim = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    with lim:
        # store: encode tokens of sequence 0 until half the budget is spent
        n_store, t_store = 0, 0.0
        while t_store < budget_s / 2 and n_store < inp.num_tokens:
            step = min(1024, inp.num_tokens - n_store)
            t0 = time.perf_counter()
            ost.encode_slots(inp.k[n_store:n_store + step], inp.v[n_store:n_store + step], lay, signs, m)
            t_store += time.perf_counter() - t0
            n_store += step
        # decode: whole (sequence, kv head) groups until the other half is spent
        offs = inp.token_offsets()
        G = w.gqa
        n_groups, dec_bytes, t_dec = 0, 0, 0.0
        for b in range(w.batch):
            for g in range(w.num_kv_heads):
                if t_dec >= budget_s / 2:
                    break
                T = int(inp.seq_lens[b])
                slots = ost.encode_slots(inp.k[offs[b]:offs[b] + T, g:g + 1],
                                         inp.v[offs[b]:offs[b] + T, g:g + 1], lay, signs, m)
                npg = -(-T // w.block_size)
                local = np.zeros((npg, w.block_size, 1, slot), np.uint8)
                t = np.arange(T)
                local[t // w.block_size, t % w.block_size] = slots
                t0 = time.perf_counter()
                odec.decode_f64(inp.q[b:b + 1, g * G:(g + 1) * G], local, np.arange(npg)[None],
                                np.array([T]), lay, signs, c, 1)
                t_dec += time.perf_counter() - t0
                n_groups += 1
                dec_bytes += T * slot + 2 * G * w.head_dim * 2 + 4 * npg + 4
    return dict(
        value=round(dec_bytes / t_dec / 1e9, 6), unit="GB/s", cores=1, kind="oracle",
        sample=(f"float64 decode oracle on {n_groups} (sequence, kv head) groups of this workload "
                f"({dec_bytes} algorithmic bytes, {t_dec:.1f} s); fp32-contract store oracle on "
                f"{n_store} tokens x {w.num_kv_heads} heads ({t_store:.1f} s); one thread"),
        store_tokens_per_s=round(n_store / t_store, 1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--layout", choices=["aos", "soa"], default="aos",
                    help="page layout: slots back to back (default), or the split page "
                         "(data region + fp16 meta region, K norm folded at store time)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="how caches are evicted before each timed kernel: read a 1 GiB buffer "
                         "(default; leaves no dirty lines), write it, or not at all")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from packed_cache_decode_amd import synth
    from packed_cache_decode_amd.runtime import PackedKVCache

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    inp = synth.generate(w)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    k, v, q = up(inp.k), up(inp.v), up(inp.q)
    sm, bt, sl = up(inp.slot_mapping), up(inp.block_table), up(inp.seq_lens)
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, rot_seed=2024,
                       device=dev, layout=args.layout)
    cache = tq.new_cache(inp.num_blocks)
    max_len = int(inp.seq_lens.max())
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    tq.workspace(w.batch, w.num_q_heads, max_len)
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)      # 1 GiB
    sink = torch.empty((), dtype=torch.int32, device=dev)

    def do_flush():
        if args.flush == "read":
            torch.amax(flush, dim=0, out=sink)
        elif args.flush == "write":
            flush.fill_(1)

    def step(evs=None):
        do_flush()
        if evs:
            evs[0].record()
        tq.store(k, v, sm, cache)
        if evs:
            evs[1].record()
        do_flush()
        if evs:
            evs[2].record()
        tq.decode(q, cache, bt, sl, max_len, out=out)
        if evs:
            evs[3].record()

    # plain streaming probes of the same session: the read used as the cache
    # flush (1 GiB) and a device copy (256 MiB read + 256 MiB written)
    def probe(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3

    copy_src = torch.ones(1 << 26, dtype=torch.int32, device=dev)
    copy_dst = torch.empty_like(copy_src)
    t_read = probe(lambda: torch.amax(flush, dim=0, out=sink))
    t_copy = probe(lambda: copy_dst.copy_(copy_src))
    hbm_probe = {"read_gbs": round(flush.numel() * 4 / t_read / 1e9, 1),
                 "copy_gbs": round(2 * copy_src.numel() * 4 / t_copy / 1e9, 1),
                 "note": "torch amax over 1 GiB; torch copy of 256 MiB (read + write bytes)"}
    del copy_src, copy_dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert tq.device_error() == 0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_store = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    t_dec = np.array([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3
    assert tq.device_error() == 0

    # warm cache, reported apart: the same decode back to back with no flush,
    # so the cache is read from L2 / the Infinity Cache where it fits
    wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    tq.decode(q, cache, bt, sl, max_len, out=out)
    for e0, e1 in wev:
        e0.record()
        tq.decode(q, cache, bt, sl, max_len, out=out)
        e1.record()
    torch.cuda.synchronize()
    t_warm = np.array([e0.elapsed_time(e1) for e0, e1 in wev]) * 1e-3

    slot = tq.slot_bytes
    dec_bytes = decode_alg_bytes(inp, slot)
    n_tok = inp.num_tokens
    st_bytes = n_tok * store_alg_bytes_per_token(w, slot)
    dec_gbs = dec_bytes / t_dec.mean() / 1e9
    st_gbs = st_bytes / t_store.mean() / 1e9
    res = {
        "metric": "packed-KV decode attn HBM GB/s (% of peak) + tq_store tokens/s",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((t_store.mean() + t_dec.mean()) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "preset": w.preset, "batch": w.batch,
                   "seq_len": int(inp.seq_lens.max()), "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "cache_bytes": int(n_tok * w.num_kv_heads * slot),
                   "layout": args.layout, "cache_flush": args.flush},
        "decode_us": round(t_dec.mean() * 1e6, 2),
        "decode_us_p10_p90": [round(float(np.percentile(t_dec, 10)) * 1e6, 2),
                              round(float(np.percentile(t_dec, 90)) * 1e6, 2)],
        "decode_pct_of_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
        "decode_pct_of_probe": {"read": round(100 * dec_gbs / hbm_probe["read_gbs"], 1),
                                "copy": round(100 * dec_gbs / hbm_probe["copy_gbs"], 1)},
        "decode_warm_us": round(float(np.median(t_warm)) * 1e6, 2),
        "decode_warm_note": "median of back-to-back decodes with no cache flush (not the metric)",
        "store_tokens_per_s": round(n_tok / t_store.mean(), 1),
        "store_us": round(t_store.mean() * 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic("decode", w.name, args.layout),
                     "kernel": "tq_decode (split kernel + merge kernel)",
                     "alg_bytes_per_launch": dec_bytes},
        "roofline_store": {"bound": "hbm", "achieved": round(st_gbs, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(st_gbs / HBM_PEAK_GBS, 4),
                           "traffic": counted_traffic("store", w.name, args.layout), "kernel": "tq_store",
                           "alg_bytes_per_launch": st_bytes},
        "kernel_sources_sha256": {k: sources_sha256(k) for k in KERNEL_SOURCES},
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 3),
        "hbm_probe": hbm_probe,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, slot)
    tq.close()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
