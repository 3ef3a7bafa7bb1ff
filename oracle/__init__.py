"""CPU oracle for the TurboQuant packed KV-cache store and paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call, link or execute anything in this package.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, tables or constants with the HIP
path: it computes its own codebook, rotation signs, slot layout and
arithmetic from the pages' description, and receives nothing but the seeded
synthetic inputs.

Sources (cited by page title and section in every module):
  * "vLLM 源码完全拆解(十九):TurboQuant KV Cache 量化——Hadamard 旋转、
    Lloyd-Max 标量量化与分页缓存内核" (pinghaoyang.com.cn) -- called P1 below;
  * "vLLM TurboQuant 介绍：极低比特 KV Cache 量化" (beaiera.top) -- P2;
  * "NVIDIA KV Cache 量化中的 NVFP4 与 TurboQuant" (moonnryan.github.io) -- P5.

Two arithmetic modes:
  * the fp32 *contract* (``store.store_contract``): every rounding is fixed
    (single IEEE binary32 operations, round-to-nearest-even, no fused
    multiply-add, correctly rounded division and square root, a fixed
    reduction tree and butterfly order).  The GPU store must reproduce its
    bytes exactly.
  * float64 (``store.rotate_f64``, ``decode.decode_f64``): the mathematical
    reference used for tie analysis and for decode parity.

Modules:
  fpfmt     -- bf16 / fp16 / OCP E4M3FN encode and decode
  rotation  -- Sylvester Hadamard, SplitMix64 sign flips, FWHT
  codebook  -- Lloyd-Max codebooks for N(0, 1/d)
  layout    -- presets, slot sizes and byte offsets, page bytes
  store     -- the store (quantise + pack + scatter), contract and float64
  decode    -- dequantise-then-softmax paged decode attention, float64
  soa       -- the structure-of-arrays page layout with the folded norm
  haar      -- the Haar (random orthogonal) rotation, alternative to Hadamard
"""

from . import fpfmt, rotation, codebook, layout, store, decode, soa, haar  # noqa: F401,E402
