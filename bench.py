"""Paged-attention decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--partition-size P] [--layers L] [--no-cpu-baseline]
                    [--block-size BS] [--placement permuted|contiguous]

One step is one pass of the whole decode hot path over one batch of synthetic
input, on one attention layer: the copy-on-write block copies the workload
needs (none for most), the slot write of every sequence's new K/V token, and
paged decode (split-context partials plus the cross-partition merge when the
partition size is non-zero). Steps rotate over L layer caches that share one
block table -- as real decode does layer by layer -- so that consecutive
steps read K/V from HBM rather than from the 256 MB last-level cache.

Inputs are resident in HBM before the timed region starts. Rank 0 prints one
JSON line:

  value      KV tokens attended per second (sum of context lengths / step time)
  gbps       algorithmic HBM GB/s of the step (every attended K/V byte once,
             plus q, out and the block-table entries read)
  roofline   the decode timed alone with HIP events on the stream it is
             launched on -- for a split decode the launch pair (partials
             kernel + merge kernel), with the partials kernel alone beside
             it: algorithmic bytes per call / average call time, against
             8 TB/s
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
             workload, on this host's cores (a reported baseline only)
  prefill    the chunked-prefill batch (8 x 2048-token chunks after 2048-token
             prefixes, Llama-3-8B heads): pa_prefill against the MFMA roofline
  per_config every workload (tiny fp32, Llama-shaped, MHA, shared-prefix CoW,
             long-context fp8, and the same with an int8 cache) at its own
             launch configuration: decode time, KV tokens/s, GB/s and
             fraction of 8 TB/s, the slot write and block copies, and the
             oracle timed on a sample of that workload
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
DEFAULT_WORKLOAD = "llama3_8b_b32"
DTYPE_NAME = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8_e4m3fn": "fp8_e4m3fn",
              "int8": "int8"}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3fn": 1, "int8": 1}
# the decode kernel's sources: the traffic counters of a summary are tied to
# them, or to the files its `sources` field lists
CSRC = os.path.join(ROOT, "paged_kv_cache_426_amd", "csrc")
DECODE_SRCS = ("pa_decode_kernel.h", "pa_device.h")
PROFILES = os.path.join(ROOT, "profiles")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--block-size", type=int, default=None,
                    help="tokens per cache block (Llama-shaped workload only; default 16)")
    ap.add_argument("--placement", choices=("permuted", "contiguous"), default=None,
                    help="physical block order (Llama-shaped workload only; default permuted)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="tokens per split-context partition (0 = single pass); "
                         "default: the workload's own launch configuration")
    ap.add_argument("--layers", type=int, default=4,
                    help="layer caches rotated over (defeats the last-level cache)")
    ap.add_argument("--roofline-launches", type=int, default=400)
    ap.add_argument("--fused-append", action="store_true",
                    help="one decode-with-append launch instead of the slot-write kernel "
                         "followed by decode (measured no faster on these workloads)")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode through pa_decode_shared_prefix (workloads with groups of "
                         "sequences sharing a prefix): shared blocks are read once per group")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the pass over every workload at its own launch configuration")
    ap.add_argument("--cpu-seconds-per-config", type=float, default=4.0,
                    help="wall-clock budget of the CPU oracle sample of each per-config entry")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the CPU oracle sample")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill batch (pa_prefill) and print its JSON object")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (a known byte count for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args(argv)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic byte counts
# ---------------------------------------------------------------------------

def decode_bytes(wl):
    """Algorithmic HBM bytes of one decode: every attended token's K and V row
    of every KV head once, q read once, out written once, and the block-table
    entries of the blocks attended."""
    kv_tok = 2 * wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_dtype]
    q_bytes = wl.q.size * ELEM_BYTES[wl.q_dtype]
    blocks = sum(-(-int(n) // wl.block_size) for n in wl.context_lens)
    tables = blocks * 4
    kv = wl.tokens_attended * kv_tok
    # scale tables (K and V, float32): per attended block and KV head, per
    # attended block, or per KV head
    scales = {0: 0, 1: 8 * wl.num_kv_heads, 2: 8 * blocks,
              3: 8 * blocks * wl.num_kv_heads}[wl.scale_layout]
    return {"kv": kv, "kv_per_token": kv_tok, "q": q_bytes, "out": q_bytes,
            "tables": tables + scales, "ctx_lens": 4 * wl.num_seqs,
            "total": kv + 2 * q_bytes + tables + scales + 4 * wl.num_seqs}


def unique_kv_bytes(wl):
    """K/V bytes of the distinct (block, offset) slots attended: the minimum a
    decode must read when blocks are shared between sequences."""
    import numpy as np

    bs = wl.block_size
    slots = set()
    for b in range(wl.num_seqs):
        n = int(wl.context_lens[b])
        ids = np.asarray(wl.block_tables[b, : -(-n // bs)], dtype=np.int64)
        pos = np.arange(n)
        slots.update((ids[pos // bs] * bs + pos % bs).tolist())
    return len(slots) * 2 * wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_dtype]


def write_bytes(wl):
    """Slot write: read each new token's K/V rows, write them to the cache."""
    if wl.new_slots is None:
        return 0
    n = int((wl.new_slots >= 0).sum())
    row = wl.num_kv_heads * wl.head_dim
    return n * 2 * row * (ELEM_BYTES[wl.q_dtype] + ELEM_BYTES[wl.kv_dtype]) + 8 * len(wl.new_slots)


def append_bytes(wl):
    """Decode with append, beyond the decode's own bytes: each new token's K/V
    rows are read from the inputs and written to the slot, and its cache rows,
    which the decode's count includes, need not be read."""
    if wl.new_slots is None:
        return 0
    n = int((wl.new_slots >= 0).sum())
    row = wl.num_kv_heads * wl.head_dim
    return n * 2 * row * ELEM_BYTES[wl.q_dtype]


def new_token_is_last(wl):
    """Every sequence's new token sits at its last position (what decode with
    append assumes)."""
    import numpy as np

    if wl.new_slots is None:
        return False
    bs = wl.block_size
    for b, n in enumerate(wl.context_lens):
        want = -1 if n <= 0 else int(wl.block_tables[b, (n - 1) // bs]) * bs + (n - 1) % bs
        if int(wl.new_slots[b]) != want:
            return False
    return True


def copy_bytes(wl):
    blk = wl.block_size * wl.num_kv_heads * wl.head_dim * ELEM_BYTES[wl.kv_dtype]
    return len(wl.cow_pairs) * 2 * 2 * blk


# ---------------------------------------------------------------------------
# traffic measured by rocprofv3 counters (committed summary)
# ---------------------------------------------------------------------------

def decode_source_hash(files=DECODE_SRCS):
    """First 16 hex digits of the sha256 of the named csrc files, in order."""
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload, shared):
    return os.path.join(PROFILES, f"pa_decode_{workload}{'_shared_mode' if shared else ''}"
                                  "_traffic.md")


def committed_traffic(workload, partition_size, shared=False):
    """HBM bytes per timed call (the decode: for a split the partials kernel
    and the merge kernel together; for the shared-prefix call its four kernels
    together) from the committed rocprofv3 counter summary of this workload,
    or None when there is none for this workload / partition size / mode, when
    it does not cover the whole call (field `scope`), or when a source it
    names changed since the counters were taken."""
    path = traffic_file(workload, shared)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    try:
        if fields.get("workload") != workload or int(fields["partition_size"]) != partition_size:
            return None
        if partition_size and not shared and fields.get("scope") != "partials+merge":
            return None
        files = tuple(fields["sources"].split()) if "sources" in fields else DECODE_SRCS
        if fields.get("decode_source_sha256") != decode_source_hash(files):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError, OSError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(wl, budget_s):
    """The oracle as it stands (slot write of the new tokens, then decode) on
    whole sequences of the same workload, one sequence at a time, until the
    time budget is spent. Returns KV tokens attended per second."""
    import numpy as np

    import oracle

    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()  # the workload's own arrays stay as built
    blk = {}
    if wl.scale_layout:
        nb, hkv = wl.num_blocks, wl.num_kv_heads
        blk = dict(k_block_scales=oracle.expand_scales(wl.k_scales, wl.scale_layout, nb, hkv),
                   v_block_scales=oracle.expand_scales(wl.v_scales, wl.scale_layout, nb, hkv))
    done_tokens, done_seqs, t_used = 0, 0, 0.0
    order = [int(b) for b in np.random.default_rng(0).permutation(wl.num_seqs)]
    while t_used < budget_s:
        b = order[done_seqs % len(order)]
        t0 = time.perf_counter()
        if wl.new_slots is not None and wl.new_slots[b] >= 0:
            if wl.scale_layout:
                oracle.reshape_and_cache_scaled(wl.new_key[b:b + 1], wl.new_value[b:b + 1], kc,
                                                vc, wl.new_slots[b:b + 1], wl.k_scales,
                                                wl.v_scales, wl.scale_layout)
            else:
                oracle.reshape_and_cache(wl.new_key[b:b + 1], wl.new_value[b:b + 1], kc, vc,
                                         wl.new_slots[b:b + 1], wl.k_scale, wl.v_scale)
        oracle.paged_decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale,
                            wl.k_scale, wl.v_scale, seqs=[b], **blk)
        t_used += time.perf_counter() - t0
        done_tokens += int(wl.context_lens[b])
        done_seqs += 1
    try:  # BLAS threads actually in use, read after the oracle has run
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
    except Exception:  # noqa: BLE001
        info = []
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    return {
        "value": done_tokens / t_used,
        "unit": "KV tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{done_seqs} sequence decodes ({done_seqs / wl.num_seqs:.2f} passes over "
                   f"the {wl.num_seqs} sequences) of {wl.name} "
                   f"({done_tokens} KV tokens attended, slot write + float64 decode), "
                   f"{t_used:.1f} s wall-clock; python loop with numpy BLAS on "
                   f"{threads} thread(s), {len(os.sched_getaffinity(0))} host cores visible"),
    }


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def avg_launch_s(fn, n, stream, warm=10):
    """Average duration of fn(i) over n back-to-back launches: HIP events on
    the stream the work runs on, around all n, divided by n (the time between
    launches is included)."""
    import torch

    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n / 1e3


def bracketed_median_s(fn, n, stream):
    """Median of n launches each bracketed by its own pair of events (higher
    than avg_launch_s by the events' own cost)."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return ms[len(ms) // 2] / 1e3


class Prepared:
    """A workload's device inputs: the cache state after the step's history
    writes (fp8 fill, private tokens) in L layer caches sharing one block
    table, plus the step's own inputs."""

    def __init__(self, wl, dev, layers):
        import torch

        import paged_kv_cache_426_amd as pa
        import workloads as W

        t = lambda a: W.to_device(a, dev)  # noqa: E731
        self.wl = wl
        self.dev = dev
        self.q = t(wl.q)
        self.bt = t(wl.block_tables)
        self.cl = t(wl.context_lens)
        self.cow = t(wl.cow_pairs)
        self.new_k = t(wl.new_key) if wl.new_key is not None else None
        self.new_v = t(wl.new_value) if wl.new_value is not None else None
        self.new_s = t(wl.new_slots) if wl.new_slots is not None else None
        k0, v0 = t(wl.k_cache), t(wl.v_cache)
        # scale tables of an 8-bit cache (shared by the layer copies: the
        # writes below use every block's scales, never change them)
        self.ks = t(wl.k_scales) if wl.scale_layout else None
        self.vs = t(wl.v_scales) if wl.scale_layout else None
        if wl.hist_slots is not None and len(wl.hist_slots):
            if wl.scale_layout:
                pa.copy_blocks_scaled(k0, v0, self.ks, self.vs, wl.scale_layout, self.cow)
                pa.reshape_and_cache_scaled(t(wl.hist_key), t(wl.hist_value), k0, v0,
                                            t(wl.hist_slots), self.ks, self.vs, wl.scale_layout)
            else:
                pa.copy_blocks(k0, v0, self.cow)
                pa.reshape_and_cache(t(wl.hist_key), t(wl.hist_value), k0, v0,
                                     t(wl.hist_slots), wl.k_scale, wl.v_scale)
        self.layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(layers - 1)]
        self.out = torch.empty_like(self.q)
        self.gm = self.pl = self.ws_sp = None
        if wl.prefix_members is not None:
            self.gm = t(wl.prefix_members)
            self.pl = t(wl.prefix_lens)
            self.ws_sp = torch.empty(pa.decode_shared_prefix_workspace_size(
                wl.num_seqs, self.gm.shape[0], self.gm.shape[1], wl.num_q_heads, wl.head_dim,
                wl.max_blocks_per_seq, self.q.dtype), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def workspace(self, P):
        import torch

        import paged_kv_cache_426_amd as pa

        wl = self.wl
        if not P:
            return None
        return torch.empty(pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                                    wl.max_blocks_per_seq, wl.block_size, P),
                           dtype=torch.uint8, device=self.dev)

    def decode_fn(self, P, ws):
        """pa_decode (for a split: the partials kernel and the merge kernel)."""
        import paged_kv_cache_426_amd as pa

        wl = self.wl

        def fn(i):
            kc, vc = self.layers[i % len(self.layers)]
            if wl.scale_layout:
                pa.decode_scaled(self.q, kc, vc, self.bt, self.cl, self.ks, self.vs,
                                 wl.scale_layout, scale=wl.scale, partition_size=P,
                                 out=self.out, workspace=ws)
            else:
                pa.decode(self.q, kc, vc, self.bt, self.cl, scale=wl.scale, k_scale=wl.k_scale,
                          v_scale=wl.v_scale, partition_size=P, out=self.out, workspace=ws)
        return fn

    def write_fn(self):
        """The slot write of the step's new tokens."""
        import paged_kv_cache_426_amd as pa

        wl = self.wl

        def fn(i):
            kc, vc = self.layers[i % len(self.layers)]
            if wl.scale_layout:
                pa.reshape_and_cache_scaled(self.new_k, self.new_v, kc, vc, self.new_s, self.ks,
                                            self.vs, wl.scale_layout)
            else:
                pa.reshape_and_cache(self.new_k, self.new_v, kc, vc, self.new_s, wl.k_scale,
                                     wl.v_scale)
        return fn

    def shared_fn(self):
        import paged_kv_cache_426_amd as pa

        wl = self.wl

        def fn(i):
            kc, vc = self.layers[i % len(self.layers)]
            pa.decode_shared_prefix(self.q, kc, vc, self.bt, self.cl, self.gm, self.pl,
                                    scale=wl.scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                                    out=self.out, workspace=self.ws_sp)
        return fn

    def partials_fn(self, P):
        """The partials kernel alone (no merge), for a split P != 0."""
        import torch

        import paged_kv_cache_426_amd as pa

        wl = self.wl
        B, Hq, d = wl.num_seqs, wl.num_q_heads, wl.head_dim
        if P > 0:
            NP = pa.num_partitions(wl.max_blocks_per_seq, wl.block_size, P)
            lead, arg = (B, Hq, NP), P
        else:
            S = pa.decode_balanced_splits(Hq, wl.num_kv_heads, d, self.q.dtype,
                                          self.layers[0][0].dtype) if P == -1 else -P
            lead, arg = (Hq, S + B), -S
        f32 = dict(dtype=torch.float32, device=self.dev)
        tmp = torch.empty(lead + (d,), **f32)
        mx = torch.empty(lead, **f32)
        sm = torch.empty(lead, **f32)

        def fn(i):
            kc, vc = self.layers[i % len(self.layers)]
            pa.decode_partials(self.q, kc, vc, self.bt, self.cl, arg, scale=wl.scale,
                               k_scale=wl.k_scale, v_scale=wl.v_scale, tmp_out=tmp,
                               max_logits=mx, exp_sums=sm)
        return fn, arg


def measure_config(wl, dev, args, stream, cpu_seconds):
    """One workload at its own launch configuration: the decode launch pair
    (partials + merge; a single-pass decode is one launch), the partials
    kernel alone, the shared-prefix call where the workload has prefix
    groups, the slot write and the block copies; each against its
    algorithmic bytes, with the oracle timed on a sample beside it."""
    import torch

    layers = 2 if wl.kv_bytes_attended() > (1 << 30) else args.layers
    prep = Prepared(wl, dev, layers)
    P = wl.partition_size
    n = max(20, args.roofline_launches // 2)
    ws = prep.workspace(P)
    db = decode_bytes(wl)
    alg = db["kv"] + db["q"] + db["out"] + db["tables"] + db["ctx_lens"]
    tokens = wl.tokens_attended
    pair_s = avg_launch_s(prep.decode_fn(P, ws), n, stream)
    e = {
        "workload": wl.name,
        "batch": wl.num_seqs,
        "heads": f"{wl.num_q_heads}/{wl.num_kv_heads}/{wl.head_dim}",
        "dtypes": f"{wl.q_dtype}/{wl.kv_dtype}",
        "partition_size": P,
        "tokens_attended": tokens,
        "algorithmic_bytes": alg,
        "decode_us": pair_s * 1e6,
        "decode_launches": "partials + merge" if P else "single pass",
        "kv_tokens_per_s": tokens / pair_s,
        "gbps": alg / pair_s / 1e9,
        "frac": alg / pair_s / 1e9 / HBM_PEAK_GBPS,
        "traffic": committed_traffic(wl.name, P),
    }
    if P and not wl.scale_layout:  # (no partials entry point for scale tables)
        fn, arg = prep.partials_fn(P)
        ps = avg_launch_s(fn, n, stream)
        e["partials_only_us"] = ps * 1e6
        e["partials_only_frac"] = alg / ps / 1e9 / HBM_PEAK_GBPS
    if "distinct_blocks" in wl.info:
        ub = unique_kv_bytes(wl)
        ualg = ub + db["q"] + db["out"] + db["tables"] + db["ctx_lens"]
        e["unique_kv_bytes"] = ub
        e["frac_of_unique_bytes"] = ualg / pair_s / 1e9 / HBM_PEAK_GBPS
        if prep.gm is not None:
            ss = avg_launch_s(prep.shared_fn(), n, stream)
            e["shared_prefix"] = {
                "us": ss * 1e6, "kv_tokens_per_s": tokens / ss,
                "gbps_unique": ualg / ss / 1e9, "frac": ualg / ss / 1e9 / HBM_PEAK_GBPS,
                "effective_gbps_logical": alg / ss / 1e9,
                "traffic": committed_traffic(wl.name, P, shared=True),
                "launches": "prep + prefix pass + suffix pass + merge"}
    # a1: the slot write of the step's new tokens; a2: the copy-on-write copies
    import paged_kv_cache_426_amd as pa
    if prep.new_s is not None:
        wt = avg_launch_s(prep.write_fn(), 200, stream)
        e["slot_write"] = {"us": wt * 1e6, "tokens": int((wl.new_slots >= 0).sum()),
                           "bytes": write_bytes(wl), "gbps": write_bytes(wl) / wt / 1e9}
    if len(wl.cow_pairs) and not wl.scale_layout:
        def cfn(i):
            kc, vc = prep.layers[i % len(prep.layers)]
            pa.copy_blocks(kc, vc, prep.cow)
        ct = avg_launch_s(cfn, 200, stream)
        e["block_copy"] = {"us": ct * 1e6, "pairs": int(len(wl.cow_pairs)),
                           "bytes": copy_bytes(wl), "gbps": copy_bytes(wl) / ct / 1e9,
                           "note": "the copied blocks fit the last-level cache across repeats"}
    del prep, ws
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        e["cpu_baseline"] = cpu_baseline(wl, cpu_seconds)
        e["gpu_over_cpu"] = e["kv_tokens_per_s"] / e["cpu_baseline"]["value"]
    return e


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / f16 MFMA, published peak


def prefill_flops(pw):
    """Causal attention work of a prefill batch: per query head and attended
    (query, key) pair, 2 d flops for q.k and 2 d for p.v; query i of a chunk
    of C after n - C cached tokens attends n - C + i + 1 keys."""
    wl = pw.cache
    pairs = 0
    for n, c in zip(wl.context_lens, pw.chunk_lens):
        n, c = int(n), int(c)
        pairs += c * (n - c) + c * (c + 1) // 2
    return 4 * wl.head_dim * wl.num_q_heads * pairs


def cpu_baseline_prefill(pw, budget_s):
    """The prefill oracle as it stands on seeded sampled query rows of the
    same batch, until the time budget is spent. Returns query tokens/s."""
    import numpy as np

    import oracle

    wl = pw.cache
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    if wl.hist_slots is not None and len(wl.hist_slots):
        oracle.reshape_and_cache(wl.hist_key, wl.hist_value, kc, vc, wl.hist_slots,
                                 wl.k_scale, wl.v_scale)
    oracle.reshape_and_cache(wl.new_key, wl.new_value, kc, vc, wl.new_slots, wl.k_scale,
                             wl.v_scale)
    order = [int(r) for r in np.random.default_rng(0).permutation(pw.num_query_tokens)]
    done, t_used = 0, 0.0
    while t_used < budget_s and done < len(order):
        rows = order[done:done + 16]
        t0 = time.perf_counter()
        oracle.paged_prefill(pw.q, kc, vc, wl.block_tables, wl.context_lens, pw.query_start,
                             wl.scale, wl.k_scale, wl.v_scale, rows=rows)
        t_used += time.perf_counter() - t0
        done += len(rows)
    return {"value": done / t_used, "unit": "query tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} seeded random query rows of {pw.name} (all {wl.num_q_heads} "
                      f"heads each, float64 numpy), {t_used:.1f} s wall-clock"}


def measure_prefill(name, dev, args, stream, cpu_seconds):
    """The prefill batch: pa_prefill timed alone, against the MFMA roofline
    (causal flops / time, dense bf16 peak)."""
    import torch

    import paged_kv_cache_426_amd as pa
    import workloads as W

    pw = W.PREFILL_BUILDERS[name]()
    wl = pw.cache
    layers = []
    for _ in range(2):
        prep = Prepared(wl, dev, 1)
        kc, vc = prep.layers[0]
        pa.reshape_and_cache(prep.new_k, prep.new_v, kc, vc, prep.new_s, wl.k_scale, wl.v_scale)
        layers.append((kc, vc))
    q = W.to_device(pw.q, dev)
    qs = torch.as_tensor(pw.query_start, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    bt, cl = prep.bt, prep.cl
    torch.cuda.synchronize()

    def fn(i):
        kc, vc = layers[i % 2]
        pa.prefill(q, kc, vc, bt, cl, qs, max_query_len=pw.max_query_len, scale=wl.scale,
                   k_scale=wl.k_scale, v_scale=wl.v_scale, out=out)
    t = avg_launch_s(fn, 50, stream)
    flops = prefill_flops(pw)
    e = {
        "workload": name,
        "batch": wl.num_seqs,
        "heads": f"{wl.num_q_heads}/{wl.num_kv_heads}/{wl.head_dim}",
        "dtypes": f"{wl.q_dtype}/{wl.kv_dtype}",
        "context_lens": sorted(set(int(x) for x in wl.context_lens)),
        "chunk_lens": sorted(set(int(x) for x in pw.chunk_lens)),
        "query_tokens": pw.num_query_tokens,
        "prefill_us": t * 1e6,
        "query_tokens_per_s": pw.num_query_tokens / t,
        "roofline": {"bound": "mfma", "achieved": flops / t / 1e12,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "flops_per_launch": flops,
                     "kernel": "prefill_kernel (one launch)"},
    }
    del layers, q, out, prep
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        e["cpu_baseline"] = cpu_baseline_prefill(pw, cpu_seconds)
    return e


PER_CONFIG = ("tiny_fp32_gqa2", "llama3_8b_b32", "mha_b32_ctx4096", "shared_prefix_cow_b64",
              "long_ctx_fp8_b8", "long_ctx_int8_b8",
              "long_ctx_fp8_b8_scales3", "long_ctx_int8_b8_scales3")


def build_config(name):
    """A workload by name; a `_scales<L>` suffix: the same workload with scale
    tables of layout L (an 8-bit cache) instead of per-tensor scales."""
    import workloads as W

    m = re.match(r"(.*)_scales(\d)$", name)
    if m:
        return W.with_scale_tables(W.build(m.group(1)), int(m.group(2)))
    return W.build(name)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: paged decode here runs on a single MI355X "
              f"with no sharding or collectives (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_426_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.prefill_only:
        e = measure_prefill("prefill_llama3_8b_b8", dev, args, stream, 0.0)
        log(f"prefill_llama3_8b_b8: {e['prefill_us']:.1f} us, "
            f"{e['roofline']['achieved']:.0f} TFLOP/s = {e['roofline']['frac'] * 100:.1f} % of "
            f"{MFMA_BF16_PEAK_TFLOPS:.0f}")
        print(json.dumps({"prefill": e}), flush=True)
        return 0

    t0 = time.perf_counter()
    kw = {} if args.partition_size is None else {"partition_size": args.partition_size}
    if args.block_size is not None:
        kw["block_size"] = args.block_size
    if args.placement is not None:
        kw["placement"] = args.placement
    wl = W.build(args.workload, **kw)
    P = wl.partition_size
    log(f"workload {wl.name}: B={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"d={wl.head_dim} kv={wl.kv_dtype} P={P} tokens={wl.tokens_attended} "
        f"pool={wl.num_blocks} blocks (built in {time.perf_counter() - t0:.1f} s)")
    prep = Prepared(wl, dev, args.layers)
    q, bt, cl, layers, out = prep.q, prep.bt, prep.cl, prep.layers, prep.out
    new_k, new_v, new_s, cow = prep.new_k, prep.new_v, prep.new_s, prep.cow
    ws = prep.workspace(P)
    has_cow = len(wl.cow_pairs) > 0

    # With --fused-append the slot write rides in the decode launch
    # (decode_append), which needs every new token at its sequence's last
    # position.
    fused = new_s is not None and args.fused_append and new_token_is_last(wl)
    shared = args.shared_prefix
    if shared and prep.gm is None:
        print(f"--shared-prefix: workload {wl.name} has no prefix groups", file=sys.stderr)
        return 2

    shared_call = prep.shared_fn() if shared else None

    def step(i):
        kc, vc = layers[i % len(layers)]
        if has_cow:
            pa.copy_blocks(kc, vc, cow)
        if fused:
            pa.decode_append(q, new_k, new_v, kc, vc, bt, cl, scale=wl.scale,
                             k_scale=wl.k_scale, v_scale=wl.v_scale, partition_size=P,
                             out=out, workspace=ws)
            return
        if new_s is not None:
            pa.reshape_and_cache(new_k, new_v, kc, vc, new_s, wl.k_scale, wl.v_scale)
        if shared:
            shared_call(i)
            return
        pa.decode(q, kc, vc, bt, cl, scale=wl.scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                  partition_size=P, out=out, workspace=ws)

    # --- whole-step throughput ---------------------------------------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    w0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    log(f"{args.steps} steps: {ms_per_step * 1e3:.2f} us/step on events, "
        f"{wall / args.steps * 1e6:.2f} us/step wall-clock")

    # --- the dominant work alone, on its stream ------------------------------
    # The decode as one launch pair: for a split, the partials kernel and the
    # merge kernel (pa_decode enqueues both); the partials kernel alone is
    # reported beside it.
    n_launch = args.roofline_launches
    if shared:
        kernel = prep.shared_fn()
    else:
        kernel = prep.decode_fn(P, ws)
    kern_avg_s = avg_launch_s(kernel, n_launch, stream)
    kern_med_s = bracketed_median_s(kernel, n_launch, stream)
    part_avg_s = None
    if P and not shared:
        pfn, split_arg = prep.partials_fn(P)
        part_avg_s = avg_launch_s(pfn, n_launch, stream)
        if P < 0:
            log(f"balanced split: {-split_arg} shares")
    log(f"decode: {kern_avg_s * 1e6:.2f} us per call" +
        (f" (partials alone {part_avg_s * 1e6:.2f} us)" if part_avg_s else ""))

    # --- optional copy calibration for counter scaling ----------------------
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: one 1 GiB device-to-device copy (1 GiB read + 1 GiB written)")
        del src, dst

    # --- bytes and the JSON line ---------------------------------------------
    db = decode_bytes(wl)
    kernel_alg = db["kv"] + db["q"] + db["out"] + db["tables"] + db["ctx_lens"]
    step_alg = db["total"] + (append_bytes(wl) if fused else write_bytes(wl)) + copy_bytes(wl)
    if shared:
        # every distinct K/V row once: shared blocks are read once per group
        ub = unique_kv_bytes(wl)
        kernel_alg = ub + db["q"] + db["out"] + db["tables"] + db["ctx_lens"]
        step_alg += ub - db["kv"]
    tokens = wl.tokens_attended
    step_s = ms_per_step / 1e3
    achieved = kernel_alg / kern_avg_s / 1e9
    if shared:
        kname = ("shared-prefix decode: prep, prefix-pass and suffix-pass decode kernels and "
                 "merge, timed together, against the distinct K/V bytes")
    elif P:
        kname = ("decode launch pair: decode_kernel (split partials) + the merge kernel "
                 "(reduce_fixed_kernel for fixed partitions, reduce_kernel for the balanced split)")
    else:
        kname = "decode_kernel (single pass)"
    roof = {
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBPS,
        "traffic": committed_traffic(wl.name, P, shared),
        "kernel": kname + ("; the step runs its variant with the slot write fused"
                           if fused else ""),
        "kernel_avg_us": kern_avg_s * 1e6,
        "kernel_timing": f"HIP events around {n_launch} back-to-back calls",
        "kernel_bracketed_median_us": kern_med_s * 1e6,
        "algorithmic_bytes_per_launch": kernel_alg,
        "bytes_per_unit": db["kv_per_token"],
        "units_per_launch": (unique_kv_bytes(wl) // db["kv_per_token"]) if shared else tokens,
    }
    if part_avg_s:
        roof["partials_only_us"] = part_avg_s * 1e6
        roof["partials_only_frac"] = kernel_alg / part_avg_s / 1e9 / HBM_PEAK_GBPS
    result = {
        "metric": "paged decode: KV tokens attended/s and achieved HBM GB/s (% of peak), 1 GPU",
        "value": tokens / step_s,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[wl.kv_dtype] if wl.kv_dtype == wl.q_dtype
        else f"{wl.q_dtype}/{wl.kv_dtype}",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": wl.num_seqs,
            "context_tokens_total": tokens,
            "context_len_min": int(wl.context_lens.min()),
            "context_len_max": int(wl.context_lens.max()),
            "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim,
            "block_size": wl.block_size,
            "placement": args.placement or "permuted",
            "num_blocks": wl.num_blocks,
            "q_dtype": wl.q_dtype,
            "kv_dtype": wl.kv_dtype,
            "partition_size": P,
            "layers_rotated": args.layers,
            "step": ("copy_blocks + " if has_cow else "") +
                    ("decode_append (new tokens' slot writes in the decode launch)" if fused
                     else "reshape_and_cache(new tokens) + decode") +
                    (" shared-prefix (prep + prefix pass + suffix pass + merge)" if shared
                     else " (partials + merge)" if P else " (single pass)"),
        },
        "gbps": step_alg / step_s / 1e9,
        "hbm_frac": step_alg / step_s / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_alg,
        "roofline": roof,
    }
    if "distinct_blocks" in wl.info:
        ub = unique_kv_bytes(wl)
        result["unique_kv_bytes"] = ub
        result["unique_kv_gbps_kernel"] = ub / kern_avg_s / 1e9
        result["shared_ratio"] = wl.info.get("shared_ratio")
    del prep, ws, layers, out, q
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None

    # --- every workload at its own launch configuration ----------------------
    if not args.no_per_config and args.block_size is None and args.placement is None \
            and args.partition_size is None:
        per = []
        for name in PER_CONFIG:
            t1 = time.perf_counter()
            w = wl if name == wl.name else build_config(name)
            e = measure_config(w, dev, args, stream,
                               0.0 if args.no_cpu_baseline else args.cpu_seconds_per_config)
            log(f"per-config {name}: decode {e['decode_us']:.2f} us, {e['frac'] * 100:.1f} % of "
                f"8 TB/s ({time.perf_counter() - t1:.1f} s)")
            per.append(e)
        result["per_config"] = per
        t1 = time.perf_counter()
        e = measure_prefill("prefill_llama3_8b_b8", dev, args, stream,
                            0.0 if args.no_cpu_baseline else args.cpu_seconds_per_config)
        log(f"prefill_llama3_8b_b8: {e['prefill_us']:.1f} us, "
            f"{e['roofline']['achieved']:.0f} TFLOP/s = {e['roofline']['frac'] * 100:.1f} % of "
            f"{MFMA_BF16_PEAK_TFLOPS:.0f} ({time.perf_counter() - t1:.1f} s)")
        result["prefill"] = e
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
