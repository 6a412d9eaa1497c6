"""The five synthetic workloads at full size, in the launch configuration the
benchmark times, against the oracle: the step's cache writes bit for bit and
the decode output within tolerance (every output where the oracle finishes
in seconds, sampled sequences otherwise)."""

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import assert_close, device_step, oracle_step

pytestmark = pytest.mark.gpu


def _run(wl, partition_size=None, seqs=None, full_pool=True):
    print(f"[workload] {wl.name} P={wl.partition_size if partition_size is None else partition_size}"
          f" seqs={'all' if seqs is None else list(seqs)}", flush=True)
    kc, vc, ref = oracle_step(wl, seqs=seqs)
    d, out = device_step(wl, partition_size)
    torch.cuda.synchronize()
    gk, gv = W.to_numpy(d["k_cache"]), W.to_numpy(d["v_cache"])
    if full_pool:
        assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    else:
        blocks = np.unique(np.concatenate([
            wl.block_tables[b, : -(-int(wl.context_lens[b]) // wl.block_size)] for b in seqs]))
        assert np.array_equal(gk[blocks], kc[blocks]) and np.array_equal(gv[blocks], vc[blocks])
    return assert_close(W.widen_to_f64(out), ref, wl.q_dtype, wl.name)


def test_llama3_8b_b32():
    wl = W.build("llama3_8b_b32")
    for P in (wl.partition_size, 0, 256, 512):
        _run(wl, P)


def test_mha_b32_ctx4096():
    wl = W.build("mha_b32_ctx4096")
    for P in (wl.partition_size, 0, 512):
        _run(wl, P, seqs=[0, 17, 31])


def test_shared_prefix_cow_b64():
    wl = W.build("shared_prefix_cow_b64")
    assert len(wl.cow_pairs) == 48
    for P in (wl.partition_size, 0, 256):
        _run(wl, P)


def test_long_ctx_fp8_b8():
    wl = W.build("long_ctx_fp8_b8")
    seqs = [int(np.argmin(wl.context_lens)), int(np.argmax(wl.context_lens))]
    for P in (wl.partition_size, -1):
        _run(wl, P, seqs=seqs, full_pool=False)
