"""Oracle for paged-attention decode: gather through the block table, then
dense attention in float64.

What is computed (restated from the pages):

* Attention of a query row against a set of keys and values is
  softmax(q . K^T / sqrt(d_k)) V ("KV-Cache evolution", §1).
* In decode, each sequence contributes one new query token that attends over
  all of the sequence's cached tokens ("KV-Cache evolution", §1; "vLLM
  inference principles", section on the two phases of generation).
* With grouped-query attention, query heads are split into groups and each
  group shares one K/V head ("KV-Cache evolution", §3A; "PagedAttention deep
  dive", §1.1). Reading taken: contiguous groups, query head h uses KV head
  h // (Hq / Hkv).
* The cache is cut into fixed-size physical blocks; a per-sequence block table
  maps logical block j (tokens j*bs .. j*bs+bs-1 in sequence order) to a
  physical block id; the physical blocks need not be contiguous or ordered
  ("PagedAttention deep dive", §2.1; "vLLM inference principles", block-table
  figure, where logical blocks 0, 1, 2 of sequence A live in physical blocks
  2, 5, 1 and the last one may be only partly filled).

Paging changes only where K/V live, so the exact result is dense attention
over the K/V rows gathered in logical order; that is what ``paged_decode``
writes out.

Layouts: q [B, Hq, d]; k_cache, v_cache [num_blocks, block_size, Hkv, d];
block_tables [B, max_blocks_per_seq] int; context_lens [B] int.
"""

import math

import numpy as np

from .numerics import to_f64


def gather_logical_kv(cache_f64: np.ndarray, block_table_row: np.ndarray, n: int) -> np.ndarray:
    """Rows 0..n-1 of one sequence, in logical order: [n, Hkv, d].

    Logical token j lives in physical block block_table_row[j // bs] at offset
    j % bs. Only the first ceil(n / bs) table entries are read (the number of
    blocks a length-n sequence occupies, "KV-cache sharing article" §5.1).
    """
    bs = cache_f64.shape[1]
    nblk = -(-n // bs)
    ids = np.asarray(block_table_row[:nblk], dtype=np.int64)
    rows = cache_f64[ids]  # [nblk, bs, Hkv, d]
    return rows.reshape(nblk * bs, *cache_f64.shape[2:])[:n]


def widen_blocks(cache, ids, block_scales=None) -> np.ndarray:
    """Physical blocks ``ids`` of a cache as float64 [len(ids), bs, Hkv, d]:
    the stored values widened exactly and, when a scale table
    ``block_scales`` [num_blocks, Hkv] is given (an 8-bit cache with a scale
    per block and head, see ``oracle.scaled``), each row multiplied by the
    scale of its own physical block and KV head."""
    x = to_f64(cache[ids])
    if block_scales is not None:
        x = x * np.asarray(block_scales, dtype=np.float64)[ids][:, None, :, None]
    return x


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                 k_scale=1.0, v_scale=1.0, seqs=None, heads=None,
                 k_block_scales=None, v_block_scales=None):
    """Decode attention for every (sequence, query head): float64 [B, Hq, d].

    ``scale`` is the softmax scale (normally 1/sqrt(d)), taken as the float32
    value the caller passes and widened exactly. ``k_scale`` / ``v_scale``
    multiply the widened cache values (per-tensor dequantisation of an 8-bit
    cache; 1.0 otherwise). A sequence with context length 0 attends over
    nothing; its output is defined as zeros.

    ``seqs`` / ``heads`` restrict the work to a subset (the rest of the output
    stays NaN) so that full-size workloads can be checked on samples.
    ``k_block_scales`` / ``v_block_scales`` ([num_blocks, Hkv], see
    ``widen_blocks``) give each block and head its own dequantisation scale.
    """
    q64 = to_f64(q)
    B, Hq, d = q64.shape
    Hkv = k_cache.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    scale64 = float(np.float32(scale))
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    seqs = range(B) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    for b in seqs:
        n = int(context_lens[b])
        if n == 0:
            out[b, list(heads)] = 0.0
            continue
        nblk = -(-n // k_cache.shape[1])
        ids = np.asarray(block_tables[b][:nblk], dtype=np.int64)
        # widen only the blocks this sequence uses
        K = gather_logical_kv(widen_blocks(k_cache, ids, k_block_scales), np.arange(nblk), n) * ks
        V = gather_logical_kv(widen_blocks(v_cache, ids, v_block_scales), np.arange(nblk), n) * vs
        for h in heads:
            g = h // group
            s = (K[:, g, :] @ q64[b, h]) * scale64
            p = np.exp(s - s.max())
            out[b, h] = (p @ V[:, g, :]) / p.sum()
    return out


def paged_decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale,
                          partition_size, k_scale=1.0, v_scale=1.0):
    """Split-context step: per-partition softmax statistics and outputs.

    Partition p of sequence b covers logical tokens [p*P, min((p+1)*P, n)).
    For each (b, h, p) it returns

        m   = max_j s_j,
        l   = sum_j exp(s_j - m),
        o~  = sum_j exp(s_j - m) v_j / l,

    with s_j = scale * q . k_j. Entries for partitions past ceil(n / P) are NaN.
    Shapes: m, l [B, Hq, NP]; o~ [B, Hq, NP, d], NP = ceil(max_tokens / P)
    with max_tokens = max_blocks_per_seq * block_size.
    """
    q64 = to_f64(q)
    B, Hq, d = q64.shape
    bs = k_cache.shape[1]
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    P = int(partition_size)
    NP = -(-(block_tables.shape[1] * bs) // P)
    scale64 = float(np.float32(scale))
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    m = np.full((B, Hq, NP), np.nan)
    l = np.full((B, Hq, NP), np.nan)
    o = np.full((B, Hq, NP, d), np.nan)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        nblk = -(-n // bs)
        ids = np.asarray(block_tables[b][:nblk], dtype=np.int64)
        K = gather_logical_kv(to_f64(k_cache[ids]), np.arange(nblk), n) * ks
        V = gather_logical_kv(to_f64(v_cache[ids]), np.arange(nblk), n) * vs
        for p in range(-(-n // P)):
            lo, hi = p * P, min((p + 1) * P, n)
            for h in range(Hq):
                g = h // group
                s = (K[lo:hi, g, :] @ q64[b, h]) * scale64
                mp = s.max()
                e = np.exp(s - mp)
                m[b, h, p] = mp
                l[b, h, p] = e.sum()
                o[b, h, p] = (e @ V[lo:hi, g, :]) / e.sum()
    return m, l, o


def reduce_partials(m, l, o, context_lens, partition_size):
    """Merge per-partition results into the decode output: float64 [B, Hq, d].

    With M = max_p m_p and w_p = l_p * exp(m_p - M), the output is
    sum_p w_p o~_p / sum_p w_p. Only the first ceil(n / P) partitions of a
    sequence are read; a sequence with n = 0 gives zeros.
    """
    B, Hq, NP, d = o.shape
    out = np.zeros((B, Hq, d))
    P = int(partition_size)
    for b in range(B):
        n = int(context_lens[b])
        npart = -(-n // P)
        if npart == 0:
            continue
        for h in range(Hq):
            mp = m[b, h, :npart]
            M = mp.max()
            w = l[b, h, :npart] * np.exp(mp - M)
            out[b, h] = (w @ o[b, h, :npart]) / w.sum()
    return out


def balanced_pieces(context_lens, block_size, num_splits):
    """The pieces of the balanced split, as the library's header defines it.

    The blocks of all sequences are taken end to end in sequence order
    (ceil(n_b / bs) blocks for sequence b, T in all); with S' = min(S, T),
    share s holds blocks [floor(s T / S'), floor((s+1) T / S')). A piece is
    the intersection of a share with one sequence. Returns a list of
    (s, b, first_block, end_block), block indices local to sequence b, in
    (share, sequence) order. The split is the library's own work division
    (the pages do not describe one); merging the pieces gives the dense
    result whatever the split.
    """
    nblk = [-(-max(int(n), 0) // block_size) for n in context_lens]
    T = sum(nblk)
    if T == 0:
        return []
    S = min(int(num_splits), T)
    starts = np.concatenate([[0], np.cumsum(nblk)])
    pieces = []
    for s in range(S):
        lo, hi = s * T // S, (s + 1) * T // S
        for b in range(len(nblk)):
            a, z = max(lo, int(starts[b])), min(hi, int(starts[b + 1]))
            if a < z:
                pieces.append((s, b, a - int(starts[b]), z - int(starts[b])))
    return pieces


def paged_decode_pieces(q, k_cache, v_cache, block_tables, context_lens, scale, pieces,
                        k_scale=1.0, v_scale=1.0, unit=None, k_block_scales=None,
                        v_block_scales=None):
    """(m, l, o~) of each piece (s, b, first_block, end_block) for every query
    head: the softmax statistics of the piece's own tokens
    [first_block * u, min(end_block * u, n)), as in paged_decode_partials,
    where u = unit, the number of tokens the piece bounds count in (the
    cache's block size unless given; the library's balanced split counts
    16-token sub-blocks whatever the block size). Block scales as in
    ``paged_decode``.
    Shapes: m, l [len(pieces), Hq]; o~ [len(pieces), Hq, d]."""
    q64 = to_f64(q)
    B, Hq, d = q64.shape
    bs = k_cache.shape[1]
    group = Hq // k_cache.shape[2]
    scale64 = float(np.float32(scale))
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    m = np.zeros((len(pieces), Hq))
    l = np.zeros((len(pieces), Hq))
    o = np.zeros((len(pieces), Hq, d))
    for i, (_, b, fb, eb) in enumerate(pieces):
        n = int(context_lens[b])
        nblk = -(-n // bs)
        ids = np.asarray(block_tables[b][:nblk], dtype=np.int64)
        K = gather_logical_kv(widen_blocks(k_cache, ids, k_block_scales), np.arange(nblk), n) * ks
        V = gather_logical_kv(widen_blocks(v_cache, ids, v_block_scales), np.arange(nblk), n) * vs
        u = bs if unit is None else int(unit)
        lo, hi = fb * u, min(eb * u, n)
        for h in range(Hq):
            g = h // group
            sc = (K[lo:hi, g, :] @ q64[b, h]) * scale64
            mp = sc.max()
            e = np.exp(sc - mp)
            m[i, h] = mp
            l[i, h] = e.sum()
            o[i, h] = (e @ V[lo:hi, g, :]) / e.sum()
    return m, l, o


def reduce_pieces(m, l, o, pieces, num_seqs):
    """Merge pieces per sequence exactly as reduce_partials merges partitions:
    float64 [B, Hq, d]; a sequence with no piece gives zeros."""
    Hq, d = o.shape[1:]
    out = np.zeros((num_seqs, Hq, d))
    for b in range(num_seqs):
        idx = [i for i, pc in enumerate(pieces) if pc[1] == b]
        if not idx:
            continue
        for h in range(Hq):
            mp = m[idx, h]
            M = mp.max()
            w = l[idx, h] * np.exp(mp - M)
            out[b, h] = (w @ o[idx, h]) / w.sum()
    return out


def default_scale(head_dim: int) -> float:
    """The softmax scale 1/sqrt(d_k) of the attention formula, as float32."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))
