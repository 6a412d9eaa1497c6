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
  roofline   the dominant kernel (the decode kernel) timed alone with HIP
             events on the stream it is launched on: algorithmic bytes per
             launch / average launch time, against 8 TB/s
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
             workload, on this host's cores (a reported baseline only)
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the CPU oracle sample")
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
    tables = sum(-(-int(n) // wl.block_size) for n in wl.context_lens) * 4
    kv = wl.tokens_attended * kv_tok
    return {"kv": kv, "kv_per_token": kv_tok, "q": q_bytes, "out": q_bytes, "tables": tables,
            "ctx_lens": 4 * wl.num_seqs,
            "total": kv + 2 * q_bytes + tables + 4 * wl.num_seqs}


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
    """HBM bytes per timed launch (the decode kernel; for the shared-prefix call
    its four kernels together) from the committed rocprofv3 counter summary of
    this workload, or None when there is none for this workload / partition
    size / mode or a source it names changed since the counters were taken."""
    path = traffic_file(workload, shared)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    try:
        if fields.get("workload") != workload or int(fields["partition_size"]) != partition_size:
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

    kc, vc = wl.k_cache, wl.v_cache
    done_tokens, done_seqs, t_used = 0, 0, 0.0
    order = [int(b) for b in np.random.default_rng(0).permutation(wl.num_seqs)]
    while t_used < budget_s:
        b = order[done_seqs % len(order)]
        t0 = time.perf_counter()
        if wl.new_slots is not None and wl.new_slots[b] >= 0:
            oracle.reshape_and_cache(wl.new_key[b:b + 1], wl.new_value[b:b + 1], kc, vc,
                                     wl.new_slots[b:b + 1], wl.k_scale, wl.v_scale)
        oracle.paged_decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale,
                            wl.k_scale, wl.v_scale, seqs=[b])
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

def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: paged decode here runs on a single MI355X "
              f"with no sharding or collectives (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_426_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

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

    # device inputs; the step's history writes (fp8 fill, private tokens) are
    # applied once, before timing, to every layer cache
    t = lambda a: W.to_device(a, dev)  # noqa: E731
    q = t(wl.q)
    bt = t(wl.block_tables)
    cl = t(wl.context_lens)
    cow = t(wl.cow_pairs)
    new_k = t(wl.new_key) if wl.new_key is not None else None
    new_v = t(wl.new_value) if wl.new_value is not None else None
    new_s = t(wl.new_slots) if wl.new_slots is not None else None
    k0, v0 = t(wl.k_cache), t(wl.v_cache)
    if wl.hist_slots is not None and len(wl.hist_slots):
        pa.copy_blocks(k0, v0, cow)
        pa.reshape_and_cache(t(wl.hist_key), t(wl.hist_value), k0, v0, t(wl.hist_slots),
                             wl.k_scale, wl.v_scale)
    layers = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(args.layers - 1)]
    out = torch.empty_like(q)
    MBS = wl.max_blocks_per_seq
    NP = pa.num_partitions(MBS, wl.block_size, P) if P > 0 else 0
    ws = None
    if P:
        ws = torch.empty(pa.decode_workspace_size(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                                  MBS, wl.block_size, P),
                         dtype=torch.uint8, device=dev)
    has_cow = len(wl.cow_pairs) > 0
    torch.cuda.synchronize()

    # With --fused-append the slot write rides in the decode launch
    # (decode_append), which needs every new token at its sequence's last
    # position.
    fused = new_s is not None and args.fused_append and new_token_is_last(wl)
    shared = args.shared_prefix
    if shared:
        if wl.prefix_members is None:
            print(f"--shared-prefix: workload {wl.name} has no prefix groups", file=sys.stderr)
            return 2
        gm = t(wl.prefix_members)
        pl = t(wl.prefix_lens)
        ws_sp = torch.empty(pa.decode_shared_prefix_workspace_size(
            wl.num_seqs, gm.shape[0], gm.shape[1], wl.num_q_heads, wl.head_dim, wl.max_blocks_per_seq,
            q.dtype), dtype=torch.uint8, device=dev)

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
            pa.decode_shared_prefix(q, kc, vc, bt, cl, gm, pl, scale=wl.scale,
                                    k_scale=wl.k_scale, v_scale=wl.v_scale, out=out,
                                    workspace=ws_sp)
            return
        pa.decode(q, kc, vc, bt, cl, scale=wl.scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                  partition_size=P, out=out, workspace=ws)

    # --- whole-step throughput ---------------------------------------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
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

    # --- the dominant kernel alone, on its stream ----------------------------
    # Its average launch duration is the elapsed time of HIP events recorded
    # around n back-to-back launches, divided by n (the time between launches
    # is included). Events bracketing each launch are recorded as well: their
    # median is reported beside it, and is higher by the events' own cost.
    n_launch = args.roofline_launches
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]
    if P > 0:
        nbh = wl.num_seqs * wl.num_q_heads * NP
        flat = ws.view(torch.float32)
        tmp_out = flat[: nbh * wl.head_dim].view(wl.num_seqs, wl.num_q_heads, NP, wl.head_dim)
        max_logits = flat[nbh * wl.head_dim: nbh * (wl.head_dim + 1)].view(
            wl.num_seqs, wl.num_q_heads, NP)
        exp_sums = flat[nbh * (wl.head_dim + 1): nbh * (wl.head_dim + 2)].view(
            wl.num_seqs, wl.num_q_heads, NP)
        split_arg = P
    elif P < 0:
        # the balanced split's partial kernel alone, with the share count the
        # automatic choice resolves to
        S = pa.decode_balanced_splits(wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                      q.dtype, layers[0][0].dtype) if P == -1 else -P
        npc = S + wl.num_seqs
        tmp_out = torch.empty((wl.num_q_heads, npc, wl.head_dim), dtype=torch.float32, device=dev)
        max_logits = torch.empty((wl.num_q_heads, npc), dtype=torch.float32, device=dev)
        exp_sums = torch.empty((wl.num_q_heads, npc), dtype=torch.float32, device=dev)
        split_arg = -S
        log(f"balanced split: {S} shares")
    if shared:
        def kernel(i):
            kc, vc = layers[i % len(layers)]
            pa.decode_shared_prefix(q, kc, vc, bt, cl, gm, pl, scale=wl.scale,
                                    k_scale=wl.k_scale, v_scale=wl.v_scale, out=out,
                                    workspace=ws_sp)
    elif P:
        def kernel(i):
            kc, vc = layers[i % len(layers)]
            pa.decode_partials(q, kc, vc, bt, cl, split_arg, scale=wl.scale, k_scale=wl.k_scale,
                               v_scale=wl.v_scale, tmp_out=tmp_out, max_logits=max_logits,
                               exp_sums=exp_sums)
    else:
        def kernel(i):
            kc, vc = layers[i % len(layers)]
            pa.decode(q, kc, vc, bt, cl, scale=wl.scale, k_scale=wl.k_scale,
                      v_scale=wl.v_scale, partition_size=0, out=out)
    for i in range(10):
        kernel(i)
    torch.cuda.synchronize()
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for i in range(n_launch):
        kernel(i)
    r1.record(stream)
    torch.cuda.synchronize()
    kern_avg_s = r0.elapsed_time(r1) / n_launch / 1e3
    for i in range(n_launch):
        starts[i].record(stream)
        kernel(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_med_s = sorted(kern_ms)[len(kern_ms) // 2] / 1e3

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
    kernel_alg = db["kv"] + db["q"] + db["tables"] + db["ctx_lens"]
    if not P:
        kernel_alg += db["out"]
    step_alg = db["total"] + (append_bytes(wl) if fused else write_bytes(wl)) + copy_bytes(wl)
    if shared:
        # every distinct K/V row once: shared blocks are read once per group
        ub = unique_kv_bytes(wl)
        kernel_alg = ub + db["q"] + db["out"] + db["tables"] + db["ctx_lens"]
        step_alg += ub - db["kv"]
    tokens = wl.tokens_attended
    step_s = ms_per_step / 1e3
    achieved = kernel_alg / kern_avg_s / 1e9
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
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": committed_traffic(wl.name, P, shared),
            "kernel": ("shared-prefix decode: prep, prefix-pass and suffix-pass decode kernels "
                       "and merge, timed together, against the distinct K/V bytes" if shared
                       else "decode_kernel" + (" (split partials)" if P else " (single pass)") +
                       ("; the step runs its variant with the slot write fused"
                        if fused else "")),
            "kernel_avg_us": kern_avg_s * 1e6,
            "kernel_timing": f"HIP events around {n_launch} back-to-back launches",
            "kernel_bracketed_median_us": kern_med_s * 1e6,
            "algorithmic_bytes_per_launch": kernel_alg,
            "bytes_per_unit": db["kv_per_token"],
            "units_per_launch": (unique_kv_bytes(wl) // db["kv_per_token"]) if shared else tokens,
        },
    }
    if "distinct_blocks" in wl.info:
        ub = unique_kv_bytes(wl)
        result["unique_kv_bytes"] = ub
        result["unique_kv_gbps_kernel"] = ub / kern_avg_s / 1e9
        result["shared_ratio"] = wl.info.get("shared_ratio")

    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
