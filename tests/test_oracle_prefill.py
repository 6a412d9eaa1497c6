"""Pins for the prefill oracle (``oracle.prefill``): causal attention of each
chunk's query rows over the sequence's paged K/V.

Each check can catch a plausible slip (a causal bound off by one, the chunk
placed at position 0 instead of at the end of the context, a wrong GQA head,
a transposed operand, the gather through the block table):

* brute force in plain Python over the contiguous, pre-scatter K/V;
* the last row of every chunk equals the decode oracle over the whole
  context, and a one-token chunk is a decode step;
* a whole prompt (chunk = context) equals torch's fp64 scaled-dot-product
  attention with its causal flag; a chunk after a cached prefix equals it
  with the explicit mask (key j visible to row i iff j <= n - C + i);
* causality: changing K/V after a row's position leaves that row bitwise
  unchanged; splitting a prompt into chunks gives bitwise the same rows;
* the flop count against a brute-force count of attended pairs;
* planted mistakes in a copy of the oracle fail these checks.
"""

import math

import numpy as np
import pytest
import torch

from oracle import paged_decode, paged_prefill, prefill_flops
from oracle import prefill as prefill_mod


def _case(rng, ctx, chunks, Hq, Hkv, d, bs, spare=3):
    """Random paged K/V for sequences of ctx tokens, queries for the last
    chunks[b] tokens of each; returns (q, K list, V list, caches, table,
    context_lens, query_start)."""
    nblk = [-(-n // bs) for n in ctx]
    nb = sum(nblk) + spare
    perm = rng.permutation(nb)
    kc = rng.standard_normal((nb, bs, Hkv, d))
    vc = rng.standard_normal((nb, bs, Hkv, d))
    table = np.zeros((len(ctx), max(max(nblk), 1)), np.int32)
    K, V, pos = [], [], 0
    for b, n in enumerate(ctx):
        ids = perm[pos:pos + nblk[b]]
        pos += nblk[b]
        table[b, :nblk[b]] = ids
        Kb = rng.standard_normal((n, Hkv, d))
        Vb = rng.standard_normal((n, Hkv, d))
        for j in range(n):
            kc[ids[j // bs], j % bs] = Kb[j]
            vc[ids[j // bs], j % bs] = Vb[j]
        K.append(Kb)
        V.append(Vb)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), Hq, d))
    return q, K, V, kc, vc, table, np.asarray(ctx, np.int32), qs


def _brute(q, K, V, ctx, qs, scale, group):
    T, Hq, d = q.shape
    out = np.zeros((T, Hq, d))
    for b, n in enumerate(ctx):
        C = int(qs[b + 1] - qs[b])
        for i in range(C):
            row = int(qs[b]) + i
            last = n - C + i
            for h in range(Hq):
                g = h // group
                s = [scale * sum(q[row, h, e] * K[b][j, g, e] for e in range(d))
                     for j in range(last + 1)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                for e in range(d):
                    out[row, h, e] = sum(w[j] * V[b][j, g, e] for j in range(last + 1)) / tot
    return out


@pytest.mark.parametrize("ctx,chunks,Hq,Hkv,d,bs", [
    ([5, 9], [5, 3], 2, 1, 4, 4),        # a whole prompt and a chunk after a prefix
    ([17, 3, 8], [1, 3, 6], 4, 2, 3, 4),  # a decode-like chunk, tiny blocks
    ([33], [10], 3, 3, 5, 16),            # MHA, one block boundary inside the chunk
])
def test_against_brute_force(ctx, chunks, Hq, Hkv, d, bs):
    rng = np.random.default_rng(sum(ctx) + d)
    q, K, V, kc, vc, table, cl, qs = _case(rng, ctx, chunks, Hq, Hkv, d, bs)
    got = paged_prefill(q, kc, vc, table, cl, qs, 0.37)
    want = _brute(q, K, V, ctx, qs, float(np.float32(0.37)), Hq // Hkv)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_last_row_is_decode_and_one_token_chunk_is_decode():
    rng = np.random.default_rng(3)
    ctx, chunks = [40, 17, 64, 1], [12, 17, 1, 1]
    q, K, V, kc, vc, table, cl, qs = _case(rng, ctx, chunks, 8, 2, 16, 16)
    out = paged_prefill(q, kc, vc, table, cl, qs, 0.25)
    last_rows = q[qs[1:] - 1]                          # [B, Hq, d]: each chunk's last query
    dec = paged_decode(last_rows, kc, vc, table, cl, 0.25)
    np.testing.assert_allclose(out[qs[1:] - 1], dec, rtol=0, atol=1e-12)


def _sdpa(q, K, V, n, C, scale, group):
    """torch fp64 attention with repeated KV heads; rows are the C chunk
    tokens at positions n - C .. n - 1."""
    qt = torch.from_numpy(q).permute(1, 0, 2)                  # [Hq, C, d]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(group, 0).contiguous()
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(group, 0).contiguous()
    if C == n:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                             scale=scale)
    else:
        i = torch.arange(C)[:, None]
        j = torch.arange(n)[None, :]
        mask = j <= (n - C + i)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                             scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("n,C,Hq,Hkv", [(48, 48, 4, 1), (70, 70, 8, 2), (96, 31, 4, 4),
                                        (50, 1, 6, 3)])
def test_against_torch_sdpa(n, C, Hq, Hkv):
    rng = np.random.default_rng(n * C)
    q, K, V, kc, vc, table, cl, qs = _case(rng, [n], [C], Hq, Hkv, 32, 16)
    got = paged_prefill(q, kc, vc, table, cl, qs, 0.125)
    want = _sdpa(q, K[0], V[0], n, C, 0.125, Hq // Hkv)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_causality_and_chunking_are_exact():
    rng = np.random.default_rng(11)
    n = 45
    q, K, V, kc, vc, table, cl, qs = _case(rng, [n], [n], 4, 2, 8, 8)
    whole = paged_prefill(q, kc, vc, table, cl, qs, 0.3)
    # changing K/V after position 20 leaves rows 0..20 bitwise unchanged
    kc2, vc2 = kc.copy(), vc.copy()
    for j in range(21, n):
        blk, off = table[0, j // 8], j % 8
        kc2[blk, off] += 5.0
        vc2[blk, off] -= 3.0
    moved = paged_prefill(q, kc2, vc2, table, cl, qs, 0.3)
    assert np.array_equal(moved[:21], whole[:21])
    assert not np.allclose(moved[21:], whole[21:])
    # the same prompt in three chunks (contexts 10, 30, 45) gives the same rows
    parts = []
    for lo, hi in [(0, 10), (10, 30), (30, 45)]:
        parts.append(paged_prefill(q[lo:hi], kc, vc, table, np.array([hi], np.int32),
                                   np.array([0, hi - lo], np.int32), 0.3))
    assert np.array_equal(np.concatenate(parts), whole)


def test_flops_count():
    ctx, chunks = [40, 17, 64, 5], [12, 17, 1, 0]
    qs = np.concatenate([[0], np.cumsum(chunks)])
    pairs = sum(n - c + i + 1 for n, c in zip(ctx, chunks) for i in range(c))
    assert prefill_flops(ctx, qs, 32, 128) == 4 * 128 * 32 * pairs


def test_planted_mistakes_are_caught(monkeypatch):
    """Each slip, planted in the oracle on the CPU, fails a check above."""
    rng = np.random.default_rng(5)
    q, K, V, kc, vc, table, cl, qs = _case(rng, [20], [7], 4, 2, 4, 4)
    want = _brute(q, K, V, [20], qs, float(np.float32(0.5)), 2)
    real = paged_prefill(q, kc, vc, table, cl, qs, 0.5)
    np.testing.assert_allclose(real, want, rtol=0, atol=1e-12)
    src = open(prefill_mod.__file__).read()
    slips = [("pos = n - C + i", "pos = i"),                       # chunk placed at position 0
             ("s = (K[: pos + 1, g, :]", "s = (K[: pos, g, :]"),  # causal bound off by one
             ("g = h // group", "g = h % Hkv")]                    # wrong GQA head
    for old, new in slips:
        assert old in src
        ns = {}
        exec(compile(src.replace(old, new, 1).replace("from .attention", "from oracle.attention")
                     .replace("from .numerics", "from oracle.numerics"), "mut", "exec"), ns)
        with np.errstate(all="ignore"):
            try:
                bad = ns["paged_prefill"](q, kc, vc, table, cl, qs, 0.5)
            except Exception:
                continue
        assert not np.allclose(bad, want, atol=1e-9), f"slip not caught: {new}"


def test_sampled_rows_match_full():
    rng = np.random.default_rng(13)
    q, K, V, kc, vc, table, cl, qs = _case(rng, [30, 12], [20, 5], 4, 2, 8, 8)
    full = paged_prefill(q, kc, vc, table, cl, qs, 0.2)
    part = paged_prefill(q, kc, vc, table, cl, qs, 0.2, rows=[3, 21])
    assert np.array_equal(part[[3, 21]], full[[3, 21]])
    keep = np.ones(len(q), bool)
    keep[[3, 21]] = False
    assert np.isnan(part[keep]).all()
