"""Seeded synthetic inputs for the store and the decode.

This module draws inputs only: it holds none of the method's arithmetic
(no rotation, no codebook, no quantisation).  Tests feed the same arrays to
the HIP library and to the CPU oracle; the benchmark uses them as its
workload.  Everything comes from numpy ``Generator(PCG64(seed))``; values are
drawn as float32 and rounded to bfloat16 (nearest even) because the pages'
activations are fp16/bf16.

The pages evaluate on models and datasets that are not available; these
distributions stand in for real activations:
  * K[token, h, c] = z * S[h, c], z ~ N(0, 1), with per-(kv head, channel)
    scales S = exp(0.5 * N(0, 1)) (lognormal(0, 0.5)) and round(1% of H*d)
    outlier (h, c) pairs scaled x20; the tiny case uses S = 1 with 4 outlier
    channels x20.
  * V, q ~ N(0, 1).
  * block tables: a seeded permutation of all pages; sequence b takes the
    next ceil(T_b / block_size) page ids; unused table entries are 0.
  * slot_mapping for the cache fill: token t of sequence b goes to slot
    block_table[b][t // bs] * bs + t % bs.

Two tokens written to one slot in one store race (the library leaves that
undefined; a serving scheduler hands out unique slots), so every mapping
drawn here passes assert_unique_slots, which the benchmark also applies.
"""

from dataclasses import dataclass, field, replace

import numpy as np

PRESET_NAMES = ("turboquant_k8v4", "turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc")


def assert_unique_slots(slot_mapping):
    """Raise ValueError if two tokens of one store map to the same slot
    (negative entries are padding tokens and may repeat)."""
    sm = np.asarray(slot_mapping).reshape(-1)
    live = sm[sm >= 0]
    if live.size:
        u, counts = np.unique(live, return_counts=True)
        if (counts > 1).any():
            dup = u[counts > 1]
            raise ValueError(f"slot_mapping holds {dup.size} duplicate slots (first: {int(dup[0])})")


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 bit patterns, nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    preset: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seed: int
    seq_len: int = 0                   # fixed context length (if lens is None)
    len_range: tuple = None            # (lo, hi) inclusive uniform lengths
    lognormal_sigma: float = 0.5       # 0 -> unit scales
    outlier_pairs: int = -1            # -1 -> round(1% of H*d)
    outlier_channels: int = 0          # tiny case: whole channels
    outlier_factor: float = 20.0
    permute_pages: bool = True
    note: str = ""

    @property
    def gqa(self):
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    "tiny": Workload(
        "tiny", "turboquant_4bit_nc", batch=1, num_q_heads=1, num_kv_heads=1,
        head_dim=128, block_size=16, seed=1001, seq_len=256, lognormal_sigma=0.0,
        outlier_pairs=0, outlier_channels=4, permute_pages=False,
        note="1 sequence x 256 tokens, 1 kv head, 1 q head, 4 outlier channels x20"),
    "llama3_8b": Workload(
        "llama3_8b", "turboquant_4bit_nc", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, seed=1002, seq_len=4096,
        note="Llama-3-8B-shaped decode layer: 32 q heads, 8 kv heads, batch 32 x 4096"),
    "k3v4_gqa8": Workload(
        "k3v4_gqa8", "turboquant_k3v4_nc", batch=64, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, seed=1003, len_range=(1024, 8192),
        note="3-bit K + 4-bit V, GQA 8, batch 64, lengths uniform in [1024, 8192]"),
    "k8v4_32k": Workload(
        "k8v4_32k", "turboquant_k8v4", batch=16, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=16, seed=1004, seq_len=32768,
        note="FP8 K + 4-bit V, GQA 8, batch 16 x 32768"),
    "long_131k": Workload(
        "long_131k", "turboquant_4bit_nc", batch=4, num_q_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, seed=1005, seq_len=131072,
        note="bulk store of 4 x 131072 tokens x 8 kv heads, then one decode step"),
}


def scaled_down(w, batch=None, seq_len=None, len_range=None, name=None, seed=None):
    """The same distributions at a smaller size (for oracle-sized tests)."""
    kw = {}
    if batch is not None:
        kw["batch"] = batch
    if seq_len is not None:
        kw["seq_len"] = seq_len
        kw["len_range"] = None
    if len_range is not None:
        kw["len_range"] = len_range
    if seed is not None:
        kw["seed"] = seed
    kw["name"] = name or (w.name + "_small")
    return replace(w, **kw)


@dataclass
class Inputs:
    w: Workload
    seq_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray       # int32 [B, max_blocks]
    num_blocks: int
    slot_mapping: np.ndarray      # int64 [N]
    k: np.ndarray                 # uint16 bf16 [N, H, d]
    v: np.ndarray                 # uint16 bf16 [N, H, d]
    q: np.ndarray                 # uint16 bf16 [B, Hq, d]
    scales: np.ndarray = field(repr=False, default=None)   # float32 [H, d]

    @property
    def num_tokens(self):
        return int(self.slot_mapping.shape[0])

    def token_offsets(self):
        return np.concatenate([[0], np.cumsum(self.seq_lens.astype(np.int64))])


def _channel_scales(rng, w):
    H, d = w.num_kv_heads, w.head_dim
    if w.lognormal_sigma > 0:
        S = np.exp(w.lognormal_sigma * rng.standard_normal((H, d))).astype(np.float32)
    else:
        S = np.ones((H, d), dtype=np.float32)
    if w.outlier_channels > 0:
        ch = rng.choice(d, size=w.outlier_channels, replace=False)
        S[:, ch] *= np.float32(w.outlier_factor)
    n_pairs = int(round(0.01 * H * d)) if w.outlier_pairs < 0 else w.outlier_pairs
    if n_pairs > 0:
        flat = rng.choice(H * d, size=n_pairs, replace=False)
        S.reshape(-1)[flat] *= np.float32(w.outlier_factor)
    return S


def generate(w, with_kv=True):
    """Draw the inputs of workload ``w`` (deterministic in w.seed)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, H, Hq, d, bs = w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, w.block_size
    if w.len_range is not None:
        lo, hi = w.len_range
        seq_lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        seq_lens = np.full(B, w.seq_len, dtype=np.int32)
    pages_per_seq = -(-seq_lens.astype(np.int64) // bs)
    num_blocks = int(pages_per_seq.sum())
    max_blocks = int(pages_per_seq.max()) if B else 0
    perm = rng.permutation(num_blocks) if w.permute_pages else np.arange(num_blocks)
    block_table = np.zeros((B, max(max_blocks, 1)), dtype=np.int32)
    pos = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        block_table[b, :n] = perm[pos:pos + n]
        pos += n
    slot_parts = []
    for b in range(B):
        t = np.arange(int(seq_lens[b]), dtype=np.int64)
        slot_parts.append(block_table[b, t // bs].astype(np.int64) * bs + t % bs)
    slot_mapping = np.concatenate(slot_parts) if slot_parts else np.zeros(0, np.int64)
    assert_unique_slots(slot_mapping)
    S = _channel_scales(rng, w)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, d), dtype=np.float32))
    N = int(seq_lens.sum())
    k = v = None
    if with_kv:
        k = np.empty((N, H, d), dtype=np.uint16)
        v = np.empty((N, H, d), dtype=np.uint16)
        off = 0
        for b in range(B):
            T = int(seq_lens[b])
            kz = rng.standard_normal((T, H, d), dtype=np.float32)
            kz *= S[None]
            k[off:off + T] = f32_to_bf16_bits(kz)
            del kz
            v[off:off + T] = f32_to_bf16_bits(rng.standard_normal((T, H, d), dtype=np.float32))
            off += T
    return Inputs(w, seq_lens, block_table, num_blocks, slot_mapping, k, v, q, S)
