"""Closed-form sizes the pages print, checked against ``oracle.sizes`` and
against the byte sizes of the synthetic workloads' cache tensors."""

import json
import os

import numpy as np
import pytest

from oracle import sizes

KiB = 1024
GiB = 1024 ** 3


@pytest.fixture(scope="module")
def gold(golden_dir):
    with open(os.path.join(golden_dir, "closed_forms.json")) as f:
        return json.load(f)


def test_llama3_bytes_per_token(gold):
    g = gold["llama3_8b_bytes_per_token"]
    p = g["params"]
    v = sizes.kv_bytes_per_token(p["layers"], p["kv_heads"], p["head_dim"], p["elem_bytes"])
    assert v == g["value"] == 131072
    assert v // KiB == g["approx_kib"]


def test_mha_per_layer_and_per_token(gold):
    g1, g2 = gold["mha_bytes_per_token_per_layer"], gold["mha_bytes_per_token"]
    p = g1["params"]
    assert sizes.kv_bytes_per_token_per_layer(p["heads"], p["head_dim"], p["elem_bytes"]) == \
        g1["value_kib"] * KiB
    p = g2["params"]
    assert sizes.kv_bytes_per_token(p["layers"], p["heads"], p["head_dim"], p["elem_bytes"]) == \
        g2["value_kib"] * KiB


def test_mha_batch_bytes_is_64_gib(gold):
    g = gold["mha_batch_bytes"]
    p = g["params"]
    v = sizes.kv_bytes_batch(p["batch"], p["seq_len"], p["layers"], p["heads"], p["head_dim"],
                             p["elem_bytes"])
    assert v == g["exact_value"] == 64 * GiB
    # the page's "about 67 GB" lies between the exact product in GiB (64) and in GB (68.7)
    assert 64 <= g["approx_gb_printed"] <= v / 1e9


def test_m_kv_closed_form(gold):
    g32, g8 = gold["m_kv_one_sequence_h32"], gold["m_kv_one_sequence_h8"]
    p = g32["params"]
    v32 = sizes.kv_bytes_sequence(p["layers"], p["tokens"], p["kv_heads"], p["head_dim"],
                                  p["elem_bytes"])
    assert v32 == g32["value"] == g32["gib"] * GiB
    p = g8["params"]
    v8 = sizes.kv_bytes_sequence(p["layers"], p["tokens"], p["kv_heads"], p["head_dim"],
                                 p["elem_bytes"])
    assert v8 == g8["gib"] * GiB


def test_rtx4090_capacity(gold):
    g = gold["rtx4090_capacity"]
    per_token_kib = sizes.kv_bytes_per_token(32, 8, 128, 2) // KiB          # 128 KiB
    budget_kib = g["kv_budget_gb"] * 1000 * KiB                            # 9000 MB in KiB
    assert sizes.tokens_that_fit(budget_kib, per_token_kib) == g["tokens_fp16"]
    per_token_fp8_kib = sizes.kv_bytes_per_token(32, 8, 128, 1) // KiB
    assert sizes.tokens_that_fit(budget_kib, per_token_fp8_kib) == g["tokens_fp8"]


@pytest.mark.parametrize("n,bs,expect", [(0, 16, 0), (1, 16, 1), (16, 16, 1), (17, 16, 2),
                                         (37, 16, 3), (50, 16, 4), (2056, 16, 129),
                                         (4096, 16, 256), (32768, 16, 2048)])
def test_blocks_needed(n, bs, expect):
    assert sizes.blocks_needed(n, bs) == expect


def test_mha_workload_is_the_m_kv_example():
    """One layer of the MHA-shaped batch (32 sequences x 4096 tokens, 32 KV
    heads, d 128, fp16) holds 32 x M_KV / 32 layers = 2 GiB of K+V, the same
    number as the one-sequence, 32-layer example."""
    per_layer = 32 * sizes.kv_bytes_sequence(1, 4096, 32, 128, 2)
    assert per_layer == sizes.kv_bytes_sequence(32, 4096, 32, 128, 2) == 2 * GiB
    # the workload's two cache tensors have exactly this size
    nb, bs, hkv, d = 32 * 256, 16, 32, 128
    assert 2 * nb * bs * hkv * d * np.dtype(np.float16).itemsize == per_layer
