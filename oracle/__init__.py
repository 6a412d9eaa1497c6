"""Plain, slow CPU oracle for paged-attention decode and its cache operations.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (``paged_kv_cache_426_amd``) never imports it, and this package
imports nothing from the product path: the two share no code, headers, tables
or helpers.

Everything is computed in numpy float64 (exact widening of the stored 16-bit,
8-bit and 32-bit values), one definition at a time, with no blocking or fusion.

Array conventions (the stored element type is carried by the numpy dtype):

* ``float32``  -- IEEE binary32 values;
* ``float16``  -- IEEE binary16 values;
* ``uint16``   -- bfloat16 bit patterns;
* ``uint8``    -- OCP E4M3FN (fp8) codes;
* ``int8``     -- symmetric int8 codes (value = code x the tensor's scale, or
  x the scale of the code's block and head, see ``scaled``).

Sources, cited by page title and section (all four pages are about the KV
cache and PagedAttention):

* "KV-Cache evolution" -- smallfiredragon.com, "现代 AI 的推理加速之谜：从 KV Cache
  到 PagedAttention 的演进";
* "PagedAttention deep dive" -- juejin.cn, "深度解构 LLM 推理优化：从 KV Cache 冗余到
  PagedAttention 内存分页映射";
* "KV-cache sharing article" -- intelliparadigm.com, "KVCache 技术背景与核心挑战";
* "vLLM inference principles" -- krshare.site, "vLLM 推理原理 从 KV Cache 到分页与
  连续批处理".

Parity pins: every function here is checked by ``tests/test_oracle_*.py`` and
``tests/test_closed_forms.py`` against values the pages print, closed forms,
brute force on tiny inputs, library routines on special cases, and invariants.
No function in this package is parity-unpinned.
"""

from .numerics import (
    bf16_bits_to_f64,
    e4m3fn_decode,
    e4m3fn_encode,
    int8_decode,
    int8_encode,
    to_f64,
)
from .attention import (
    paged_decode,
    paged_decode_partials,
    reduce_partials,
    gather_logical_kv,
    balanced_pieces,
    paged_decode_pieces,
    reduce_pieces,
    widen_blocks,
)
from .cache_ops import reshape_and_cache, copy_blocks
from .prefill import paged_prefill, prefill_flops
from .scaled import (
    expand_scales,
    reshape_and_cache_scaled,
    reshape_and_cache_scaled_bulk,
    copy_blocks_scaled,
)
from . import sizes

__all__ = [
    "bf16_bits_to_f64",
    "e4m3fn_decode",
    "e4m3fn_encode",
    "int8_decode",
    "int8_encode",
    "to_f64",
    "paged_decode",
    "paged_decode_partials",
    "reduce_partials",
    "gather_logical_kv",
    "balanced_pieces",
    "paged_decode_pieces",
    "reduce_pieces",
    "widen_blocks",
    "expand_scales",
    "reshape_and_cache_scaled",
    "reshape_and_cache_scaled_bulk",
    "copy_blocks_scaled",
    "paged_prefill",
    "prefill_flops",
    "reshape_and_cache",
    "copy_blocks",
    "sizes",
]
