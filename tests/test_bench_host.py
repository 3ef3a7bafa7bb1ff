"""Host-side checks of bench.py (no GPU): its byte accounting and its refusal
of more than one GPU.

The algorithmic bytes are the method's own traffic: the packed slots of every
cached token and kv head, the bf16 query and output, one int32 page id per
page and one int32 length per sequence for a decode; a token's bf16 K and V
in, its packed slots out and its int64 slot index for a store.  The expected
totals below are that count written out by hand for each workload's shape
(slot bytes 134 / 118 / 196 for the 4-bit, 3-bit-key and FP8-key presets of
the first page's preset table).
"""

import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from packed_cache_decode_amd import synth  # noqa: E402


def _uniform(name, T):
    w = synth.WORKLOADS[name]
    return SimpleNamespace(w=w, seq_lens=np.full(w.batch, T, np.int32))


@pytest.mark.parametrize("name,T,slot,want", [
    # 32 x 4096 tokens x 8 heads x 134 B + 2 x 32 x 32 x 128 x 2 B + 4 x 8192 pages + 4 x 32
    ("llama3_8b", 4096, 134, 141_066_368),
    # 16 x 32768 x 8 x 196 + 2 x 16 x 64 x 128 x 2 + 4 x 32768 + 4 x 16
    ("k8v4_32k", 32768, 196, 822_739_008),
    # 4 x 131072 x 8 x 134 + 2 x 4 x 32 x 128 x 2 + 4 x 32768 + 4 x 4
    ("long_131k", 131072, 134, 562_233_360),
])
def test_decode_algorithmic_bytes(name, T, slot, want):
    assert bench.decode_alg_bytes(_uniform(name, T), slot) == want


def test_decode_algorithmic_bytes_ragged():
    # partial last pages count as whole pages of ids; an empty sequence
    # still reads its length
    w = synth.WORKLOADS["k3v4_gqa8"]
    lens = np.array([0, 1, 16, 17] + [1024] * (w.batch - 4), np.int32)
    got = bench.decode_alg_bytes(SimpleNamespace(w=w, seq_lens=lens), 118)
    pages = 0 + 1 + 1 + 2 + 64 * (w.batch - 4)
    want = (int(lens.sum()) * w.num_kv_heads * 118 + 2 * w.batch * w.num_q_heads * w.head_dim * 2
            + 4 * pages + 4 * w.batch)
    assert got == want


def test_workload_at_another_head_dim():
    # --head-dim: the same shapes at d = 64, named apart; 32 x 4096 tokens x
    # 8 heads x 70 B + 2 x 32 x 32 x 64 x 2 B + 4 x 8192 pages + 4 x 32
    w = bench.workload_for("llama3_8b", 64)
    base = synth.WORKLOADS["llama3_8b"]
    assert (w.name, w.head_dim) == ("llama3_8b_d64", 64)
    assert (w.batch, w.num_q_heads, w.num_kv_heads, w.seq_len, w.seed) == (
        base.batch, base.num_q_heads, base.num_kv_heads, base.seq_len, base.seed)
    assert bench.workload_for("llama3_8b", 128) is base
    assert bench.workload_for("llama3_8b") is base
    inp = SimpleNamespace(w=w, seq_lens=np.full(w.batch, 4096, np.int32))
    assert bench.decode_alg_bytes(inp, 70) == 73_695_360


@pytest.mark.parametrize("slot,want", [(134, 5176), (118, 5048), (196, 5672)])
def test_store_algorithmic_bytes_per_token(slot, want):
    # 8 heads x (K and V bf16 in: 2 x 128 x 2 B, plus the slot out) + 8 B slot index
    assert bench.store_alg_bytes_per_token(synth.WORKLOADS["llama3_8b"], slot) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_default_workload_is_the_long_context_store_and_decode():
    import argparse
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="long_131k")' in src
    w = synth.WORKLOADS["long_131k"]
    assert (w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim) == (4, 8, 32, 128)


def test_cpu_baseline_runs_on_several_cores():
    """The oracle baseline on a small workload with two worker processes:
    rates are positive and the core count is the number of workers."""
    bench.start_oracle_server()
    w = synth.scaled_down(synth.WORKLOADS["llama3_8b"], batch=1, seq_len=256, name="bench_small")
    inp = synth.generate(w)
    r = bench.cpu_baseline(inp, 134, cores=2, store_tokens_per_core=64)
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["store_tokens_per_s"] > 0
    assert r["cpu_model"]
