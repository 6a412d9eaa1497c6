"""pa_decode_noalloc: decode with the split partials in the library's fixed
per-device scratch instead of a caller's workspace.

Called through the C ABI (ctypes) with the output preallocated, it must give
bit for bit the output of pa_decode with a workspace (the same kernels run on
the same inputs), and both must meet the oracle's tolerance. Two calls in a
row, the second on a smaller batch, check that the scratch's leftovers from
the first call do not leak into the second. A split whose partials exceed the
scratch is refused before anything is enqueued, and the output is left as it
was."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_426_amd as pa
import workloads as W
from _helpers import assert_close, device_step, oracle_step

pytestmark = pytest.mark.gpu


def _noalloc_c(wl, d, out, P):
    """pa_decode_noalloc straight through the C ABI; returns the status."""
    B, Hq, dd = wl.q.shape
    NB, bs, Hkv, _ = wl.k_cache.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return pa.lib().pa_decode_noalloc(
        p(out), p(d["q"]), p(d["k_cache"]), p(d["v_cache"]), p(d["block_tables"]),
        p(d["context_lens"]), B, Hq, Hkv, dd, bs, NB, wl.max_blocks_per_seq,
        float(wl.scale), pa.dtype_code(d["q"]), pa.dtype_code(d["k_cache"]), float(wl.k_scale),
        float(wl.v_scale), int(P), stream)


def _both(wl, P):
    print(f"[noalloc] {wl.name} B={wl.num_seqs} P={P}", flush=True)
    d, ref_out = device_step(wl, P)          # slot writes, then pa_decode with a workspace
    out = torch.full_like(d["q"], float("nan"))
    assert _noalloc_c(wl, d, out, P) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), f"{wl.name} P={P}: differs from pa_decode"
    _, _, ref = oracle_step(wl)
    assert_close(W.widen_to_f64(out), ref, wl.q_dtype, f"{wl.name} P={P}")
    return out


@pytest.mark.parametrize("P", [-1, 512, -7])
def test_noalloc_matches_decode_then_smaller_call(P):
    big = W.build("llama3_8b_b32")
    small = W.custom([33, 1, 700, 0, 16, 129], 32, 8, 128, q_dtype="bf16", kv_dtype="bf16",
                     seed=77)
    _both(big, P)
    _both(small, P)


def test_noalloc_single_pass_fp8_and_fp32():
    fp8 = W.custom([5, 300, 17, 1000], 32, 8, 128, q_dtype="bf16", kv_dtype="fp8_e4m3fn", seed=3)
    for P in (0, -1, 256):
        _both(fp8, P)
    _both(W.build("tiny_fp32_gqa2"), 16)


def test_noalloc_8_token_blocks():
    """Two calls in a row over 8-token blocks, the second on a smaller batch."""
    big = W.custom([9, 700, 1031, 64, 8], 32, 8, 128, q_dtype="bf16", kv_dtype="bf16", bs=8,
                   seed=41)
    small = W.custom([17, 1, 300], 32, 8, 128, q_dtype="bf16", kv_dtype="bf16", bs=8, seed=42)
    for P in (-1, 32):
        _both(big, P)
        _both(small, P)


def test_noalloc_refuses_partials_beyond_the_scratch():
    """1024 sequences with 512-token partitions of up to 256 of them need
    1024 * 32 * 256 * 130 * 4 bytes of partials, more than the scratch: the
    call returns PA_ERR_SCRATCH_LIMIT and writes nothing."""
    assert pa.decode_noalloc_scratch_bytes() == 16 << 20
    wl = W.custom([1] * 1024, 32, 8, 128, q_dtype="bf16", kv_dtype="bf16", seed=5,
                  mbs=8192)
    need = pa.decode_workspace_size(wl.num_seqs, 32, 128, wl.max_blocks_per_seq, 16, 512)
    assert need > pa.decode_noalloc_scratch_bytes()
    d, _ = device_step(wl, 0)
    out = torch.full_like(d["q"], 7.0)
    torch.cuda.synchronize()
    assert _noalloc_c(wl, d, out, 512) == 6
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    with pytest.raises(pa.PaError, match="scratch"):
        pa.decode_noalloc(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                          d["context_lens"], partition_size=512, out=out)
