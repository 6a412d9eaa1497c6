"""Oracle for paged prefill and chunked prefill: many new query tokens per
sequence attend causally over the sequence's paged K/V, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

What is computed (restated from the pages, with the readings taken):

* Generation has two phases: prefill processes the input tokens and builds
  their K/V state; decode then extends the cache one token at a time
  ("vLLM inference principles", section on the two phases of one
  generation). Prefill tends to be compute-bound, decode memory-bound
  (same section; "PagedAttention deep dive", section 1, on the asymmetry of
  the two phases). A long input may be cut into chunks that are scheduled
  together with decode work (chunked prefill, same section of "vLLM
  inference principles").
* Attention is softmax(Q K^T / sqrt(d_k)) V ("KV-Cache evolution", section
  1); with grouped-query attention query head h reads KV head h // (Hq/Hkv)
  ("KV-Cache evolution", section 3A).
* The cache is paged: token j of sequence b sits in physical block
  block_tables[b][j // bs] at row j % bs ("PagedAttention deep dive",
  section 2.1; "vLLM inference principles", block-table figure).

Readings taken where the pages are silent:

* The model is autoregressive, so a token attends to itself and to earlier
  tokens only (causal mask); that is what makes the cache of the earlier
  tokens the model's state.
* A chunk is the last C tokens of its sequence's context: with n =
  context_lens[b] tokens in the cache (the chunk's own K/V already written,
  as prefill builds them before attending) and C query tokens, query row i
  of the chunk sits at position n - C + i and attends over cache tokens
  0 .. n - C + i. C = n is a whole prompt's prefill; C = 1 is a decode step.
* Query rows of all sequences are stacked: rows query_start[b] ..
  query_start[b + 1] - 1 belong to sequence b (query_start[0] = 0).
"""

import numpy as np

from .attention import gather_logical_kv
from .numerics import to_f64


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                  k_scale=1.0, v_scale=1.0, rows=None):
    """Causal attention of each chunk's query rows: float64 [T, Hq, d].

    q [T, Hq, d]; k_cache, v_cache [num_blocks, block_size, Hkv, d];
    block_tables [B, max_blocks_per_seq]; context_lens [B];
    query_start [B + 1], non-decreasing, query_start[B] = T, and
    query_start[b + 1] - query_start[b] <= context_lens[b].
    ``scale`` is taken as the float32 value the caller passes, widened.
    ``rows`` restricts the work to those query rows (the others stay NaN), so
    that full-size workloads can be checked on samples.
    """
    q64 = to_f64(q)
    T, Hq, d = q64.shape
    Hkv = k_cache.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    bs = k_cache.shape[1]
    scale64 = float(np.float32(scale))
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    qs = np.asarray(query_start, dtype=np.int64)
    assert qs[0] == 0 and qs[-1] == T and (np.diff(qs) >= 0).all()
    out = np.zeros((T, Hq, d)) if rows is None else np.full((T, Hq, d), np.nan)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(len(context_lens)):
        n = int(context_lens[b])
        C = int(qs[b + 1] - qs[b])
        assert C <= n
        if C == 0 or (wanted is not None and not wanted & set(range(int(qs[b]), int(qs[b + 1])))):
            continue
        nblk = -(-n // bs)
        ids = np.asarray(block_tables[b][:nblk], dtype=np.int64)
        K = gather_logical_kv(to_f64(k_cache[ids]), np.arange(nblk), n) * ks
        V = gather_logical_kv(to_f64(v_cache[ids]), np.arange(nblk), n) * vs
        for i in range(C):
            pos = n - C + i
            row = int(qs[b]) + i
            if wanted is not None and row not in wanted:
                continue
            for h in range(Hq):
                g = h // group
                s = (K[: pos + 1, g, :] @ q64[row, h]) * scale64
                p = np.exp(s - s.max())
                out[row, h] = (p @ V[: pos + 1, g, :]) / p.sum()
    return out


def prefill_flops(context_lens, query_start, num_q_heads, head_dim):
    """Multiply-add work of the causal attention, counted as flops: per query
    head and attended (query, key) pair, 2 d for q . k and 2 d for p v."""
    qs = np.asarray(query_start, dtype=np.int64)
    pairs = 0
    for b, n in enumerate(context_lens):
        C = int(qs[b + 1] - qs[b])
        n = int(n)
        # query i attends n - C + i + 1 keys
        pairs += C * (n - C) + C * (C + 1) // 2
    return 4 * head_dim * num_q_heads * pairs
