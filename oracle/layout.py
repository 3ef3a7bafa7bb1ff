"""Presets, slot sizes, slot byte map and paged-cache addressing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* Presets (P1, section "四个预设对应什么"): key bits 8 means FP8 K, 3 or 4
  means Lloyd-Max codes; value bits 3 or 4; norm correction on or off.
* Slot arithmetic (P1, section "从 slot_size 的三项算术开始"):
    key bytes   = d                       (FP8 K)
                = ceil(d * kb / 8) + 2    (codes + fp16 norm)
    value bytes = ceil(d * vb / 8) + 4    (codes + fp16 scale + fp16 zero)
    slot        = key + value, rounded up to even.
  At d = 128 this gives 196 / 134 / 118 / 102 (same page, the table of the
  four presets; P5, section "三、TurboQuant" confirms 64 + 2 and 64 + 4).
* Byte map of one slot (P1, section "一个 slot 的字节图"):
    [K codes | K norm fp16 | V codes | V scale fp16 | V zero fp16]
  FP8 K has no norm.  All fp16 fields are little-endian.
* Cache tensor: uint8 [num_blocks][block_size][num_kv_heads][slot]
  (P1, sections "后端能力声明" and "页内寻址"): the stride between tokens of
  a page is num_kv_heads * slot, between heads slot.  A store slot index s
  lands in page s // block_size, row s % block_size (P1, section "融合
  kernel 的骨架").  A page holds block_size * num_kv_heads * slot bytes
  (16 * 8 * 118 = 15104 in the page's example).
"""

import math
from dataclasses import dataclass

PRESETS = {
    "turboquant_k8v4": dict(key_bits=8, value_bits=4, norm_correction=False),
    "turboquant_4bit_nc": dict(key_bits=4, value_bits=4, norm_correction=True),
    "turboquant_k3v4_nc": dict(key_bits=3, value_bits=4, norm_correction=True),
    "turboquant_3bit_nc": dict(key_bits=3, value_bits=3, norm_correction=True),
}


@dataclass(frozen=True)
class SlotLayout:
    head_dim: int
    key_bits: int
    value_bits: int
    norm_correction: bool

    @property
    def key_fp8(self):
        return self.key_bits == 8

    @property
    def key_code_bytes(self):
        return self.head_dim if self.key_fp8 else math.ceil(self.head_dim * self.key_bits / 8)

    @property
    def key_packed_size(self):
        return self.head_dim if self.key_fp8 else self.key_code_bytes + 2

    @property
    def value_code_bytes(self):
        return math.ceil(self.head_dim * self.value_bits / 8)

    @property
    def value_packed_size(self):
        return self.value_code_bytes + 4

    @property
    def slot_size(self):
        return self.key_packed_size + self.value_packed_size

    @property
    def slot_size_aligned(self):
        s = self.slot_size
        return s + (s % 2)

    # byte offsets inside a slot
    @property
    def off_key_norm(self):
        return None if self.key_fp8 else self.key_code_bytes

    @property
    def off_value(self):
        return self.key_packed_size

    @property
    def off_value_scale(self):
        return self.key_packed_size + self.value_code_bytes

    @property
    def off_value_zero(self):
        return self.off_value_scale + 2


def slot_layout(preset, head_dim):
    p = PRESETS[preset]
    return SlotLayout(head_dim, p["key_bits"], p["value_bits"], p["norm_correction"])


def page_bytes(layout, block_size, num_kv_heads):
    return block_size * num_kv_heads * layout.slot_size_aligned


def cache_shape(layout, num_blocks, block_size, num_kv_heads):
    return (num_blocks, block_size, num_kv_heads, layout.slot_size_aligned)
