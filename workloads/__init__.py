"""Seeded synthetic inputs and the host block manager.

Shared by the device path's tests/bench and the oracle's tests; holds no
attention or cache-write arithmetic.
"""

from .blockpool import BlockPool, PoolExhausted, Sequence
from .torch_io import to_device, to_numpy, widen_to_f64
from .configs import (
    BUILDERS,
    ELEM_BYTES,
    Workload,
    build,
    custom,
    llama3_8b_b32,
    long_ctx_fp8_b8,
    mha_b32_ctx4096,
    shared_prefix_cow_b64,
    shared_prefix_lens,
    tiny_fp32_gqa2,
    permute_physical,
    unshare,
    with_scale_tables,
    PrefillWorkload,
    PREFILL_BUILDERS,
    prefill_custom,
    prefill_llama3_8b_b8,
)

__all__ = [
    "BlockPool",
    "PoolExhausted",
    "Sequence",
    "BUILDERS",
    "ELEM_BYTES",
    "Workload",
    "build",
    "custom",
    "llama3_8b_b32",
    "long_ctx_fp8_b8",
    "mha_b32_ctx4096",
    "shared_prefix_cow_b64",
    "shared_prefix_lens",
    "tiny_fp32_gqa2",
    "permute_physical",
    "PrefillWorkload",
    "PREFILL_BUILDERS",
    "prefill_custom",
    "prefill_llama3_8b_b8",
    "unshare",
    "with_scale_tables",
    "to_device",
    "to_numpy",
    "widen_to_f64",
]
