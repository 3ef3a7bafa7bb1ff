"""Benchmark of the packed KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_131k]

One step = the whole hot path over one batch of the workload: tq_store of
every (token, kv head) of the batch into the paged cache, then one tq_decode
step for every sequence.  The default workload is the long-context one: a
bulk store of 4 x 131072 tokens x 8 kv heads (4-bit keys with norm
correction, 4-bit values, 134-byte slots) through a random slot mapping, then
one decode with 32 query heads.  Inputs (bf16 K/V/q, slot mapping, block
tables) are seeded synthetic data of the workload's shape, resident in HBM
before timing.  Before each kernel a 1 GiB buffer is read (outside the
event-timed intervals) so neither call is served from L2 or the 256 MB
Infinity Cache; reading, unlike writing, leaves no dirty lines to be written
back during the timed kernel.

Printed: one JSON line.  `value` is decode HBM throughput in GB/s: the
algorithmic bytes of one decode (packed cache of every token and kv head,
q, output, block-table entries, seq_lens) divided by the event-timed
duration of tq_decode (all its kernels), averaged over the K timed steps.
The store's tokens/s comes from the same steps.  `hbm_probe` holds the read
rates of the library's streaming-read probes (each load form of the kernels)
and of a device copy, measured in the same session.

`cpu_baseline` times the CPU oracle as it is on the host's cores (one worker
process per core available to this process, at most 16, one BLAS thread
each) over a bounded sample of the same workload.
"""

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from packed_cache_decode_amd.profile_summary import KERNEL_SOURCES, sources_sha256  # noqa: E402

HBM_PEAK_GBS = 8000.0


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


def workload_for(name, head_dim=0):
    """The named workload, or its shapes at another head dim (named <name>_d<dim>)."""
    from packed_cache_decode_amd import synth
    w = synth.WORKLOADS[name]
    if head_dim and head_dim != w.head_dim:
        w = dataclasses.replace(w, head_dim=head_dim, name=f"{w.name}_d{head_dim}")
    return w


def store_alg_bytes_per_token(w, slot):
    return w.num_kv_heads * (2 * w.head_dim * 2 + slot) + 8


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_cores():
    """Worker processes for the oracle baseline: the cores this process may
    run on, at most 16 (one GPU's share of its host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_worker(barrier, results, idx, preset, head_dim, block_size, slot, k_st, v_st,
                   groups):
    """One worker of the oracle baseline.  Untimed: encode the decode groups'
    slots.  Then, after every worker is ready, two timed phases separated by
    the barrier: the fp32-contract store oracle on k_st/v_st, and the float64
    decode oracle on the groups.  Reports wall-clock intervals."""
    import numpy as np

    from oracle import codebook as cb
    from oracle import decode as odec
    from oracle import layout, rotation
    from oracle import store as ost

    lay = layout.slot_layout(preset, head_dim)
    signs = rotation.rotation_signs(99, head_dim)
    c, m = cb.codebook(head_dim, 4 if lay.key_fp8 else lay.key_bits)
    caches = []
    for k, v, q, T in groups:
        slots = ost.encode_slots(k, v, lay, signs, m)
        npg = -(-T // block_size)
        local = np.zeros((npg, block_size, 1, slot), np.uint8)
        t = np.arange(T)
        local[t // block_size, t % block_size] = slots
        caches.append((local, q, T, npg))
    barrier.wait()
    t0 = time.perf_counter()
    if len(k_st):
        ost.encode_slots(k_st, v_st, lay, signs, m)
    t1 = time.perf_counter()
    barrier.wait()
    t2 = time.perf_counter()
    nbytes = 0
    for local, q, T, npg in caches:
        odec.decode_f64(q, local, np.arange(npg)[None], np.array([T]), lay, signs, c, 1)
        nbytes += T * slot + 2 * q.shape[1] * head_dim * 2 + 4 * npg + 4
    t3 = time.perf_counter()
    results.put((idx, t0, t1, t2, t3, nbytes))


def cpu_baseline(inp, slot, cores=None, store_tokens_per_core=2048):
    """Time the CPU oracle (as it is) on the host's cores over a bounded sample
    of the workload: one (sequence, kv head) decode group per worker, and
    store_tokens_per_core tokens (all kv heads) per worker for the store.
    Throughput = the sample's bytes (tokens) / the wall time from the first
    worker's start to the last one's end of each timed phase."""
    import multiprocessing as mp

    w = inp.w
    n = cores or oracle_cores()
    groups = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    n = min(n, len(groups))
    offs = inp.token_offsets()
    G = w.gqa
    ctx = mp.get_context("forkserver")
    barrier = ctx.Barrier(n)
    results = ctx.Queue()
    procs = []
    n_store = 0
    for i in range(n):
        b, g = groups[i]
        T = int(inp.seq_lens[b])
        grp = [(inp.k[offs[b]:offs[b] + T, g:g + 1].copy(), inp.v[offs[b]:offs[b] + T, g:g + 1].copy(),
                inp.q[b:b + 1, g * G:(g + 1) * G].copy(), T)]
        a = min(inp.num_tokens, i * store_tokens_per_core)
        e = min(inp.num_tokens, a + store_tokens_per_core)
        n_store += e - a
        procs.append(ctx.Process(target=_oracle_worker,
                                 args=(barrier, results, i, w.preset, w.head_dim, w.block_size, slot,
                                       inp.k[a:e].copy(), inp.v[a:e].copy(), grp)))
    for p in procs:
        p.start()
    got = [results.get(timeout=900) for _ in procs]
    for p in procs:
        p.join()
    t_store = max(r[2] for r in got) - min(r[1] for r in got)
    t_dec = max(r[4] for r in got) - min(r[3] for r in got)
    dec_bytes = sum(r[5] for r in got)
    return dict(
        value=round(dec_bytes / t_dec / 1e9, 6), unit="GB/s", cores=n, kind="oracle",
        cpu_model=cpu_model(),
        sample=(f"float64 decode oracle on {n} (sequence, kv head) groups of this workload, one per "
                f"worker process ({dec_bytes} algorithmic bytes in {t_dec:.2f} s wall); "
                f"fp32-contract store oracle on {n_store} tokens x {w.num_kv_heads} heads "
                f"({t_store:.2f} s wall); {n} processes, one BLAS thread each"),
        store_tokens_per_s=round(n_store / t_store, 1))


def start_oracle_server():
    """Start the process server the oracle workers fork from, before this
    process initialises the GPU (one BLAS thread per worker)."""
    import multiprocessing as mp
    from multiprocessing import forkserver
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
    os.environ.update(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    mp.get_context("forkserver").set_forkserver_preload(["numpy", "oracle.store", "oracle.decode"])
    forkserver.ensure_running()
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_131k")
    ap.add_argument("--layout", choices=["aos", "soa"], default="aos",
                    help="page layout: slots back to back (default), or the split page "
                         "(data region + fp16 meta region, K norm folded at store time)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-reps", type=int, default=None,
                    help="back-to-back decodes with no flush, reported apart (default: --steps; "
                         "0 leaves them out, so a profile of the run holds cold launches only)")
    ap.add_argument("--head-dim", type=int, default=0, choices=[0, 64, 128, 256],
                    help="run the workload's shapes at another head dim (default: its own); the "
                         "line then names the workload <name>_d<dim>")
    ap.add_argument("--decode-kernel", default="",
                    choices=["", "ring", "page", "staged", "direct", "general"],
                    help="force a decode kernel where it applies (default: chosen by shape)")
    ap.add_argument("--page-heads", type=int, default=0, choices=[0, 1, 2, 4],
                    help="page decode: kv heads per workgroup (default: the whole row, at most 8)")
    ap.add_argument("--ring-waves", type=int, default=0, choices=[0, 8, 16],
                    help="ring decode: wavefronts per workgroup (default: chosen by shape)")
    ap.add_argument("--dynamic-claims", action="store_true",
                    help="ring decode: wavefronts claim slabs from a counter (not reproducible "
                         "bit for bit)")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="how caches are evicted before each timed kernel: read a 1 GiB buffer "
                         "(default; leaves no dirty lines), write it, or not at all")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if not args.no_cpu_baseline:
        start_oracle_server()          # before this process touches the GPU

    import numpy as np
    import torch

    from packed_cache_decode_amd import _lib, synth
    from packed_cache_decode_amd.runtime import PackedKVCache

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workload_for(args.workload, args.head_dim)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    inp = synth.generate(w)
    synth.assert_unique_slots(inp.slot_mapping)      # one store may not write a slot twice

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    k, v, q = up(inp.k), up(inp.v), up(inp.q)
    sm, bt, sl = up(inp.slot_mapping), up(inp.block_table), up(inp.seq_lens)
    tq = PackedKVCache(w.preset, w.head_dim, w.num_kv_heads, w.block_size, rot_seed=2024,
                       device=dev, layout=args.layout)
    tq.set_decode_options(kernel=args.decode_kernel, dynamic_claims=args.dynamic_claims,
                          ring_waves=args.ring_waves, page_heads=args.page_heads)
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
    flush_bytes = flush.numel() * 4
    psink = torch.empty(_lib.tq_probe_sink_words(flush_bytes), dtype=torch.int32, device=dev)
    hbm_probe = {}
    for mode in ("regs", "regs_nt", "lds", "lds_nt"):
        t = probe(lambda: _lib.tq_probe_read(mode, flush, flush_bytes, psink))
        hbm_probe[f"read_{mode}_gbs"] = round(flush_bytes / t / 1e9, 1)
    t_read = probe(lambda: torch.amax(flush, dim=0, out=sink))
    t_copy = probe(lambda: copy_dst.copy_(copy_src))
    hbm_probe["read_torch_amax_gbs"] = round(flush_bytes / t_read / 1e9, 1)
    hbm_probe["copy_gbs"] = round(2 * copy_src.numel() * 4 / t_copy / 1e9, 1)
    hbm_probe["note"] = ("tq_probe_read over 1 GiB with 16-byte loads into registers or LDS, plain "
                         "or non-temporal; torch amax over the same 1 GiB; torch copy of 256 MiB "
                         "(read + write bytes)")
    best_read = max(hbm_probe[f"read_{m}_gbs"] for m in ("regs", "regs_nt", "lds", "lds_nt"))
    del copy_src, copy_dst, psink

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
    warm_reps = args.steps if args.warm_reps is None else args.warm_reps
    t_warm = None
    if warm_reps > 0:
        wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(warm_reps)]
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
                   "layout": args.layout, "cache_flush": args.flush,
                   "decode_options": _lib.tq_get_decode_options(tq.ctx)},
        "decode_us": round(t_dec.mean() * 1e6, 2),
        "decode_us_p10_p90": [round(float(np.percentile(t_dec, 10)) * 1e6, 2),
                              round(float(np.percentile(t_dec, 90)) * 1e6, 2)],
        "decode_pct_of_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
        "decode_pct_of_probe": {"best_read": round(100 * dec_gbs / best_read, 1),
                                "copy": round(100 * dec_gbs / hbm_probe["copy_gbs"], 1)},
        "decode_warm_us": None if t_warm is None else round(float(np.median(t_warm)) * 1e6, 2),
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
