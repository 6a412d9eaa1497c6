"""The five synthetic workloads at full size, in the launch configuration the
benchmark times, against the oracle: the step's cache writes bit for bit and
the decode output within tolerance, every sequence and head, with the cache
compared over the whole pool."""

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import assert_close, device_step, oracle_step

pytestmark = pytest.mark.gpu


def _oracle(wl):
    print(f"[workload] {wl.name}: oracle", flush=True)
    return oracle_step(wl)


def _run(wl, expect, partition_size=None):
    kc, vc, ref = expect
    print(f"[workload] {wl.name} P={wl.partition_size if partition_size is None else partition_size}",
          flush=True)
    d, out = device_step(wl, partition_size)
    torch.cuda.synchronize()
    gk, gv = W.to_numpy(d["k_cache"]), W.to_numpy(d["v_cache"])
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    assert not np.isnan(ref).any()
    return assert_close(W.widen_to_f64(out), ref, wl.q_dtype, wl.name)


def test_tiny_fp32_gqa2():
    wl = W.build("tiny_fp32_gqa2")
    expect = _oracle(wl)
    for P in (wl.partition_size, 16, 32, -1, -3):
        _run(wl, expect, P)


def test_llama3_8b_b32():
    wl = W.build("llama3_8b_b32")
    expect = _oracle(wl)
    for P in (wl.partition_size, 0, 256, 512):
        _run(wl, expect, P)


def test_mha_b32_ctx4096():
    wl = W.build("mha_b32_ctx4096")
    expect = _oracle(wl)
    for P in (wl.partition_size, 0, 512):
        _run(wl, expect, P)


def test_shared_prefix_cow_b64():
    wl = W.build("shared_prefix_cow_b64")
    assert len(wl.cow_pairs) == 48
    expect = _oracle(wl)
    for P in (wl.partition_size, 0, 256):
        _run(wl, expect, P)


def test_long_ctx_fp8_b8():
    wl = W.build("long_ctx_fp8_b8")
    expect = _oracle(wl)
    for P in (wl.partition_size, -1):
        _run(wl, expect, P)
