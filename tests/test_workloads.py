"""The synthetic workloads have the shapes, lengths and pool sizes they
describe, and the relabelling helpers keep the logical caches."""

import numpy as np
import pytest

import workloads as W
from oracle import gather_logical_kv, to_f64


def test_tiny_fp32_gqa2():
    wl = W.build("tiny_fp32_gqa2")
    assert wl.context_lens.tolist() == [37, 50]
    assert (wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size) == (4, 2, 64, 16)
    assert wl.num_blocks == 16 and wl.info["blocks_used"] == 7
    assert wl.k_cache.dtype == np.float32 and wl.scale == 0.125
    # the new token goes to logical position ctx - 1
    for b, n in enumerate(wl.context_lens):
        blk = wl.block_tables[b, (n - 1) // 16]
        assert wl.new_slots[b] == blk * 16 + (n - 1) % 16
    used = {int(x) for b, n in enumerate(wl.context_lens) for x in wl.block_tables[b, :-(-n // 16)]}
    assert len(used) == 7


def test_llama3_8b_b32_shape():
    wl = W.build("llama3_8b_b32")
    assert wl.num_seqs == 32 and wl.group == 4 and wl.head_dim == 128
    assert wl.context_lens.min() >= 512 and wl.context_lens.max() <= 4096
    needed = sum(-(-int(n) // 16) for n in wl.context_lens)
    assert wl.num_blocks == int(np.ceil(1.1 * needed))
    assert wl.max_blocks_per_seq == 256
    assert wl.kv_bytes_attended() == wl.tokens_attended * 4096


def test_shared_prefix_cow_b64_structure():
    wl = W.shared_prefix_cow_b64(groups=2, samples=4, prompt=64, parent_decoded=8, private=24,
                                 Hq=4, Hkv=1, d=8)
    assert wl.num_seqs == 8
    assert wl.context_lens.tolist() == [96] * 8
    assert len(wl.cow_pairs) == 2 * 3                      # all holders but one copy
    assert len(wl.hist_slots) == 8 * 23 and len(wl.new_slots) == 8
    srcs = set(wl.cow_pairs[:, 0].tolist())
    assert len(srcs) == 2                                  # one shared partial block per group
    # prompt blocks shared by the 4 samples of a group
    for g in range(2):
        rows = wl.block_tables[4 * g: 4 * g + 4, :4]
        assert (rows == rows[0]).all()


def test_shared_prefix_full_size_counts():
    wl = W.shared_prefix_cow_b64()
    assert wl.num_seqs == 64 and len(wl.cow_pairs) == 48
    assert (wl.context_lens == 2184).all()
    assert wl.info["blocks_used"] == 2624 and wl.num_blocks == 2887
    assert len(wl.hist_slots) == 64 * 127


def test_long_ctx_fp8_shape():
    wl = W.long_ctx_fp8_b8()
    assert wl.kv_dtype == "fp8_e4m3fn" and wl.q_dtype == "bf16"
    assert wl.context_lens.min() >= 16384 and wl.context_lens.max() <= 32768
    assert wl.max_blocks_per_seq == 2048 and wl.partition_size == 512
    assert len(wl.hist_slots) == int(wl.context_lens.sum()) - 8
    assert 0 < wl.k_scale < 0.1 and 0 < wl.v_scale < 0.1


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
def test_custom_handles_zero_and_one(kv):
    wl = W.custom([0, 1, 17], 4, 2, 16, kv_dtype=kv, seed=1)
    assert wl.new_slots[0] == -1 and wl.new_slots[1] >= 0
    assert wl.block_tables.shape == (3, 2)


def test_permute_keeps_logical_content():
    wl = W.custom([5, 40, 33], 4, 2, 16, kv_dtype="f16", seed=2)
    wp = W.permute_physical(wl, seed=3)
    for b, n in enumerate(wl.context_lens):
        a = gather_logical_kv(to_f64(wl.k_cache), wl.block_tables[b], int(n))
        c = gather_logical_kv(to_f64(wp.k_cache), wp.block_tables[b], int(n))
        assert np.array_equal(a, c)
    bs = wl.block_size
    for s_old, s_new in zip(wl.new_slots, wp.new_slots):
        assert np.array_equal(wl.k_cache.reshape(-1, 2, 16)[s_old], wp.k_cache.reshape(-1, 2, 16)[s_new])


def test_shared_prefix_lens_of_forked_groups():
    """Groups of forked samples share every whole prompt block: 2048 prompt
    tokens (the 8 tokens the parent decoded sit in a block that three of the
    four samples copied before writing)."""
    wl = W.build("shared_prefix_cow_b64")
    assert wl.prefix_members.shape == (16, 4)
    assert (wl.prefix_lens == 2048).all()


def test_shared_prefix_lens_small_cases():
    bt = np.array([[5, 6, 7, 8],
                   [5, 6, 9, 10],
                   [5, 6, 7, 11],
                   [1, 2, 3, 4]], dtype=np.int32)
    ctx = np.array([60, 64, 33, 64], dtype=np.int32)
    members = np.array([[0, 1, -1], [0, 2, -1], [3, -1, -1], [-1, -1, -1]], dtype=np.int32)
    got = W.shared_prefix_lens(bt, ctx, 16, members)
    # {0, 1}: two common blocks; {0, 2}: three common, but sequence 2 holds
    # only two whole blocks (33 tokens); {3}: all four of its whole blocks;
    # no members: 0
    assert got.tolist() == [32, 32, 64, 0]
