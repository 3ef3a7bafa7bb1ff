"""A small convenience layer over the C ABI: a context plus its decode
workspace, with torch tensors for device memory and streams.

All computation happens in the HIP library; this only sizes buffers and
passes pointers.
"""

import torch

from . import _lib

PRESET_IDS = _lib.PRESETS


class PackedKVCache:
    """One context (codebook, signs, geometry) on the current device."""

    def __init__(self, preset, head_dim, num_kv_heads, block_size, rot_seed, sign_flip=True,
                 codebook_mode="exact", device="cuda", layout="aos"):
        self.device = torch.device(device)
        self.preset = preset
        self.head_dim = head_dim
        self.num_kv_heads = num_kv_heads
        self.block_size = block_size
        self.layout = layout
        with torch.cuda.device(self.device):
            self.ctx = _lib.tq_codebook_init_layout(preset, head_dim, num_kv_heads, block_size,
                                                    rot_seed, sign_flip, codebook_mode, layout)
        self.slot_bytes = _lib.tq_slot_bytes(self.ctx)
        self._ws = None

    def close(self):
        if self.ctx:
            _lib.tq_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def new_cache(self, num_blocks, fill=0):
        """uint8 [num_blocks, bs, H, slot] (AoS) or [num_blocks, page bytes] (SoA)."""
        if self.layout == "soa":
            shape = (num_blocks, self.block_size * self.num_kv_heads * self.slot_bytes)
        else:
            shape = (num_blocks, self.block_size, self.num_kv_heads, self.slot_bytes)
        return torch.full(shape, fill, dtype=torch.uint8, device=self.device)

    def store(self, k, v, slot_mapping, cache, stream=None):
        """k, v: bf16 [N, H, d] (or [N, stride] with heads packed first);
        slot_mapping: int64 [N]; cache: uint8 [num_blocks, bs, H, slot]."""
        n = slot_mapping.shape[0]
        stride = k.stride(0)
        assert k.stride(0) == v.stride(0) and k.dtype == v.dtype == torch.bfloat16
        _lib.tq_store(self.ctx, k, v, stride, slot_mapping, n, cache, cache.shape[0], stream)

    def workspace(self, batch, num_q_heads, max_seq_len):
        nbytes = _lib.tq_decode_workspace_bytes(self.ctx, batch, num_q_heads, max_seq_len)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws, nbytes

    def decode(self, q, cache, block_table, seq_lens, max_seq_len, out=None, out_fp32=False,
               sm_scale=0.0, stream=None):
        """q: bf16 [B, Hq, d]; block_table: int32 [B, max_blocks]; seq_lens: int32 [B]."""
        B, Hq, d = q.shape
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32 if out_fp32 else torch.bfloat16,
                              device=q.device)
        ws, nbytes = self.workspace(B, Hq, max_seq_len)
        _lib.tq_decode(self.ctx, q, cache, cache.shape[0], block_table, block_table.shape[1],
                       seq_lens, B, Hq, max_seq_len, sm_scale, out, out.dtype == torch.float32,
                       ws, ws.numel(), stream)
        return out

    def dequant(self, cache, block_table_row, seq_len, out_fp32=False, stream=None):
        """K, V [seq_len, H, d] of one sequence, back in the original space."""
        dt = torch.float32 if out_fp32 else torch.bfloat16
        k = torch.empty((seq_len, self.num_kv_heads, self.head_dim), dtype=dt, device=self.device)
        v = torch.empty_like(k)
        _lib.tq_dequant(self.ctx, cache, cache.shape[0], block_table_row, block_table_row.shape[0],
                        seq_len, k, v, out_fp32, stream)
        return k, v

    def decode_continuation(self, q, cache, block_table_row, seq_len, out=None, out_fp32=False,
                            sm_scale=0.0, stream=None):
        """q: bf16 [q_len, Hq, d], the chunk's queries; their tokens are the
        last q_len of the seq_len stored ones.  Causal attention per query."""
        q_len, Hq, d = q.shape
        if out is None:
            out = torch.empty((q_len, Hq, d), dtype=torch.float32 if out_fp32 else torch.bfloat16,
                              device=q.device)
        mb = block_table_row.shape[0]
        nbytes = _lib.tq_continuation_workspace_bytes(self.ctx, q_len, Hq, seq_len, mb)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        _lib.tq_decode_continuation(self.ctx, q, cache, cache.shape[0], block_table_row, mb, seq_len, q_len,
                                    Hq, sm_scale, out, out.dtype == torch.float32, ws, ws.numel(), stream)
        return out

    def set_decode_options(self, kernel="", dynamic_claims=False, ring_waves=0, page_heads=0):
        """Decode plan options of the context (tq_set_decode_options)."""
        _lib.tq_set_decode_options(self.ctx, kernel, dynamic_claims, ring_waves, page_heads)
        self._ws = None

    def device_error(self, clear=True, stream=None):
        """Sticky error bits once the work on ``stream`` (default: torch's
        current stream) has finished."""
        return _lib.tq_get_device_error(self.ctx, clear, stream)
