"""Pins for the oracle's decode attention (``oracle.attention``).

Independent checks, each able to catch a plausible slip in the oracle:

* brute force in plain Python (math.exp, explicit sums) over the contiguous,
  pre-scatter K/V of tiny cases -- catches gather, index, scale and
  normalisation mistakes;
* torch's scaled_dot_product_attention in float64 with the KV heads repeated
  per group -- catches a wrong GQA head mapping or a transposed operand;
* special cases with closed forms (one token, zero query, equal keys, one
  dominant logit) and context length 0;
* the pages' block-table example (logical blocks -> physical 2, 5, 1);
* invariances: physical relabelling and aliased-vs-private blocks give
  bitwise-equal results;
* the split-context identity: merging per-partition results equals dense
  attention;
* fp8 caches: attention over the decoded, scaled values.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import (balanced_pieces, e4m3fn_decode, e4m3fn_encode, paged_decode,
                    paged_decode_partials, paged_decode_pieces, reduce_partials, reduce_pieces,
                    to_f64)


def _scatter(logical_k, logical_v, physical_ids, bs, num_blocks, rng):
    """Place each sequence's logical rows into blocks of a pool.
    logical_k[b]: [n_b, Hkv, d] float64; physical_ids[b]: list of block ids."""
    Hkv, d = logical_k[0].shape[1:]
    kc = rng.standard_normal((num_blocks, bs, Hkv, d))
    vc = rng.standard_normal((num_blocks, bs, Hkv, d))
    mbs = max(len(p) for p in physical_ids)
    table = np.zeros((len(logical_k), mbs), np.int32)
    for b, (K, V, ids) in enumerate(zip(logical_k, logical_v, physical_ids)):
        for j, blk in enumerate(ids):
            rows = slice(j * bs, min((j + 1) * bs, len(K)))
            n = rows.stop - rows.start
            kc[blk, :n] = K[rows]
            vc[blk, :n] = V[rows]
            table[b, j] = blk
    return kc, vc, table


def _brute_force(q, K, V, scale, group):
    """Plain-Python decode attention over contiguous K/V of one sequence."""
    Hq, d = q.shape
    out = np.zeros((Hq, d))
    for h in range(Hq):
        g = h // group
        s = [scale * sum(q[h, i] * K[j, g, i] for i in range(d)) for j in range(len(K))]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = sum(e)
        for i in range(d):
            out[h, i] = sum(e[j] * V[j, g, i] for j in range(len(K))) / tot
    return out


def _random_case(rng, ctx, Hq, Hkv, d, bs, spare=3):
    nblk = [-(-n // bs) for n in ctx]
    nb = sum(nblk) + spare
    perm = rng.permutation(nb)
    ids, pos = [], 0
    for k in nblk:
        ids.append([int(x) for x in perm[pos:pos + k]])
        pos += k
    K = [rng.standard_normal((n, Hkv, d)) for n in ctx]
    V = [rng.standard_normal((n, Hkv, d)) for n in ctx]
    q = rng.standard_normal((len(ctx), Hq, d))
    kc, vc, table = _scatter(K, V, ids, bs, nb, rng)
    return q, K, V, kc, vc, table, np.asarray(ctx, np.int32)


@pytest.mark.parametrize("ctx,Hq,Hkv,d,bs", [
    ([1, 5, 16, 17], 2, 1, 8, 4),
    ([37, 50], 4, 2, 16, 16),
    ([9, 3], 6, 2, 4, 2),
    ([33], 3, 3, 5, 8),
])
def test_against_brute_force(ctx, Hq, Hkv, d, bs):
    rng = np.random.default_rng(sum(ctx) + Hq)
    q, K, V, kc, vc, table, cl = _random_case(rng, ctx, Hq, Hkv, d, bs)
    scale = 1.0 / math.sqrt(d)
    out = paged_decode(q, kc, vc, table, cl, scale)
    for b in range(len(ctx)):
        ref = _brute_force(q[b], K[b], V[b], float(np.float32(scale)), Hq // Hkv)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_planted_mistakes_are_caught():
    """The brute-force pin is sensitive to the slips it is meant to catch:
    a wrong GQA mapping (h % Hkv), a dropped scale, and an off-by-one gather
    all move the result far outside its 1e-12 tolerance."""
    rng = np.random.default_rng(5)
    q, K, V, kc, vc, table, cl = _random_case(rng, [21], 4, 2, 8, 4)
    ref = _brute_force(q[0], K[0], V[0], 0.25, 2)
    good = paged_decode(q, kc, vc, table, cl, 0.25)[0]
    assert np.abs(good - ref).max() < 1e-12
    wrong_map = np.stack([_brute_force(q[0][h:h + 1], K[0][:, [h % 2]], V[0][:, [h % 2]], 0.25, 1)[0]
                          for h in range(4)])
    assert np.abs(wrong_map - ref).max() > 1e-3
    no_scale = paged_decode(q, kc, vc, table, cl, 1.0)[0]
    assert np.abs(no_scale - ref).max() > 1e-3
    shorter = paged_decode(q, kc, vc, table, cl - 1, 0.25)[0]
    assert np.abs(shorter - ref).max() > 1e-3


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_against_torch_sdpa(group):
    rng = np.random.default_rng(group)
    Hkv, d, bs = 2, 32, 16
    ctx = [1, 15, 16, 17, 100]
    q, K, V, kc, vc, table, cl = _random_case(rng, ctx, Hkv * group, Hkv, d, bs)
    out = paged_decode(q, kc, vc, table, cl, 1.0 / math.sqrt(d))
    for b, n in enumerate(ctx):
        qt = torch.from_numpy(q[b]).unsqueeze(1)                                   # [Hq, 1, d]
        kt = torch.from_numpy(K[b]).permute(1, 0, 2).repeat_interleave(group, 0)  # [Hq, n, d]
        vt = torch.from_numpy(V[b]).permute(1, 0, 2).repeat_interleave(group, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.contiguous(), vt.contiguous(), scale=float(np.float32(1.0 / math.sqrt(d))))
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(7)
    Hkv, d, bs = 2, 8, 4
    # one token: the output is that token's V row, exactly
    q, K, V, kc, vc, table, cl = _random_case(rng, [1], 4, Hkv, d, bs)
    out = paged_decode(q, kc, vc, table, cl, 0.3)
    for h in range(4):
        assert np.array_equal(out[0, h], V[0][0, h // 2])
    # zero query: uniform weights, the mean of V
    q, K, V, kc, vc, table, cl = _random_case(rng, [13], 2, Hkv, d, bs)
    out = paged_decode(np.zeros_like(q), kc, vc, table, cl, 0.3)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], V[0][:, h].mean(0), rtol=0, atol=1e-14)
    # all keys equal: also the mean of V
    K0 = [np.repeat(K[0][:1], 13, axis=0)]
    kc2, vc2, table2 = _scatter(K0, V, [list(table[0, :4])], bs, kc.shape[0], rng)
    out = paged_decode(q, kc2, vc2, table2, cl, 0.3)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], V[0][:, h].mean(0), rtol=0, atol=1e-14)
    # one dominant logit: that token's V row
    Kd = [np.zeros((13, Hkv, d))]
    Kd[0][6] = 1.0
    qd = np.full((1, 2, d), 1000.0)
    kc3, vc3, table3 = _scatter(Kd, V, [list(table[0, :4])], bs, kc.shape[0], rng)
    out = paged_decode(qd, kc3, vc3, table3, cl, 1.0)
    for h in range(2):
        assert np.array_equal(out[0, h], V[0][6, h])


def test_zero_context_gives_zeros():
    rng = np.random.default_rng(8)
    q, K, V, kc, vc, table, cl = _random_case(rng, [5, 7], 2, 1, 4, 4)
    cl = np.asarray([0, 7], np.int32)
    out = paged_decode(q, kc, vc, table, cl, 0.5)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.isfinite(out[1]).all()


def test_block_table_example_from_the_pages(golden_dir):
    """Sequence A's logical blocks 0, 1, 2 are physical blocks 2, 5, 1, the
    last one partly filled: gathering through that table equals attention over
    the contiguous sequence."""
    with open(os.path.join(golden_dir, "block_table_example.json")) as f:
        ids = json.load(f)["logical_to_physical"]
    rng = np.random.default_rng(9)
    bs, n, Hkv, d = 4, 10, 1, 6                 # 10 tokens: blocks of 4, 4, 2
    K = [rng.standard_normal((n, Hkv, d))]
    V = [rng.standard_normal((n, Hkv, d))]
    q = rng.standard_normal((1, 2, d))
    kc, vc, table = _scatter(K, V, [ids], bs, 6, rng)
    assert table[0].tolist() == [2, 5, 1]
    out = paged_decode(q, kc, vc, table, np.asarray([n], np.int32), 0.4)
    ref = _brute_force(q[0], K[0], V[0], float(np.float32(0.4)), 2)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)
    # the unused tail of physical block 1 never enters the result
    kc[1, 2:] = np.nan
    vc[1, 2:] = np.nan
    assert np.array_equal(paged_decode(q, kc, vc, table, np.asarray([n], np.int32), 0.4), out)


def test_permutation_invariance_bitwise():
    wl = W.custom([37, 50, 3, 16], 8, 2, 32, q_dtype="bf16", kv_dtype="bf16", seed=3,
                  extra_blocks=5)
    a = paged_decode(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.scale)
    wp = W.permute_physical(wl, seed=4)
    assert not np.array_equal(wp.block_tables, wl.block_tables)
    b = paged_decode(wp.q, wp.k_cache, wp.v_cache, wp.block_tables, wp.context_lens, wp.scale)
    assert np.array_equal(a, b)


def test_aliased_equals_private_bitwise():
    """Forked sequences share prompt blocks; giving each a private copy of
    every shared block does not change any output bit."""
    pool = W.BlockPool(40, 4, order=np.random.default_rng(1).permutation(40))
    parent = pool.new_sequence()
    for _ in range(10):
        pool.append_slot(parent)
    kids = [pool.fork(parent) for _ in range(2)]
    seqs = [parent] + kids
    rng = np.random.default_rng(2)
    kc = rng.standard_normal((40, 4, 1, 8))
    vc = rng.standard_normal((40, 4, 1, 8))
    table = np.zeros((3, 3), np.int32)
    for i, s in enumerate(seqs):
        table[i, : len(s.block_table)] = s.block_table
    cl = np.full(3, 10, np.int32)
    q = rng.standard_normal((3, 2, 8))
    wl = W.Workload("t", 3, 2, 1, 8, 4, 40, "f32", "f32", q, kc, vc, table, cl, 0.35)
    assert pool.shared_blocks() == 3
    a = paged_decode(q, kc, vc, table, cl, 0.35)
    wu = W.unshare(wl)
    assert wu.num_blocks == 40 + 6
    assert len(set(wu.block_tables[:, :3].ravel().tolist())) == 9
    b = paged_decode(q, wu.k_cache, wu.v_cache, wu.block_tables, cl, 0.35)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("P", [4, 8, 16, 48, 512])
def test_split_context_identity(P):
    rng = np.random.default_rng(P)
    q, K, V, kc, vc, table, cl = _random_case(rng, [1, 47, 48, 49, 200], 4, 2, 16, 4)
    dense = paged_decode(q, kc, vc, table, cl, 0.2)
    m, l, o = paged_decode_partials(q, kc, vc, table, cl, 0.2, P)
    merged = reduce_partials(m, l, o, cl, P)
    np.testing.assert_allclose(merged, dense, rtol=0, atol=1e-12)
    # a partition that covers the whole context is the dense result itself
    for b, n in enumerate(cl):
        if n <= P:
            np.testing.assert_allclose(o[b, :, 0], dense[b], rtol=0, atol=1e-13)
            assert np.isnan(m[b, :, 1:]).all()


def test_split_partials_brute_force():
    """Each partition's (m, l, o~) is the softmax statistics of its own slice."""
    rng = np.random.default_rng(21)
    q, K, V, kc, vc, table, cl = _random_case(rng, [23], 2, 1, 4, 4)
    P = 8
    m, l, o = paged_decode_partials(q, kc, vc, table, cl, 0.5, P)
    for p in range(3):
        lo, hi = p * P, min((p + 1) * P, 23)
        for h in range(2):
            s = [0.5 * float(np.dot(q[0, h], K[0][j, 0])) for j in range(lo, hi)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            assert m[0, h, p] == pytest.approx(mx, abs=1e-13)
            assert l[0, h, p] == pytest.approx(sum(e), abs=1e-12)
            ref = sum(ei * V[0][lo + j, 0] for j, ei in enumerate(e)) / sum(e)
            np.testing.assert_allclose(o[0, h, p], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("ctx,S", [([1, 47, 0, 48, 49, 200], 3), ([1, 47, 0, 48, 49, 200], 7),
                                   ([5], 4), ([0, 0], 3), ([16, 1, 2], 64), ([200, 17], 2)])
def test_balanced_pieces_tile_every_sequence(ctx, S):
    """Brute force over blocks: every block of every sequence lies in exactly
    one piece, pieces of a share are consecutive, and shares differ in size
    by at most one block."""
    bs = 4
    pieces = balanced_pieces(ctx, bs, S)
    owner = {}
    for s, b, fb, eb in pieces:
        assert 0 <= fb < eb <= -(-ctx[b] // bs)
        for j in range(fb, eb):
            assert (b, j) not in owner
            owner[(b, j)] = s
    every = [(b, j) for b, n in enumerate(ctx) for j in range(-(-n // bs))]
    assert sorted(owner) == sorted(every)
    # logical order of the concatenation is non-decreasing in share
    shares = [owner[k] for k in every]
    assert shares == sorted(shares)
    sizes = np.bincount(shares) if shares else np.zeros(0, int)
    if len(every):
        assert len(sizes) == min(S, len(every)) and sizes.max() - sizes.min() <= 1


@pytest.mark.parametrize("S", [2, 3, 5, 64])
def test_balanced_split_identity(S):
    """Merging the balanced pieces gives dense attention (float64), and each
    piece's statistics are those of its own token slice (brute force)."""
    rng = np.random.default_rng(S)
    ctx = [1, 47, 0, 48, 49, 200]
    q, K, V, kc, vc, table, cl = _random_case(rng, ctx, 4, 2, 16, 4)
    dense = paged_decode(q, kc, vc, table, cl, 0.2)
    pieces = balanced_pieces(cl, 4, S)
    m, l, o = paged_decode_pieces(q, kc, vc, table, cl, 0.2, pieces)
    np.testing.assert_allclose(reduce_pieces(m, l, o, pieces, len(ctx)), dense, rtol=0,
                               atol=1e-12)
    for i, (s, b, fb, eb) in enumerate(pieces):
        lo, hi = fb * 4, min(eb * 4, ctx[b])
        for h in range(4):
            sc = [float(np.float32(0.2)) * float(np.dot(q[b, h], K[b][j, h // 2]))
                  for j in range(lo, hi)]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            assert m[i, h] == pytest.approx(mx, abs=1e-12)
            assert l[i, h] == pytest.approx(sum(e), abs=1e-12)


def test_fp8_cache_is_attention_over_dequantised_values():
    rng = np.random.default_rng(31)
    ctx, Hkv, d, bs = [19, 40], 2, 16, 16
    q, K, V, kc, vc, table, cl = _random_case(rng, ctx, 4, Hkv, d, bs)
    kcode = e4m3fn_encode((kc * 20).astype(np.float32))
    vcode = e4m3fn_encode((vc * 20).astype(np.float32))
    ks, vs = 0.05, 0.05
    out = paged_decode(q, kcode, vcode, table, cl, 0.25, k_scale=ks, v_scale=vs)
    for b, n in enumerate(ctx):
        nblk = -(-n // bs)
        Kd = e4m3fn_decode(kcode[table[b, :nblk]]).reshape(-1, Hkv, d)[:n] * float(np.float32(ks))
        Vd = e4m3fn_decode(vcode[table[b, :nblk]]).reshape(-1, Hkv, d)[:n] * float(np.float32(vs))
        ref = _brute_force(q[b], Kd, Vd, 0.25, 2)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_sampled_subset_matches_full():
    wl = W.custom([20, 33, 7], 4, 2, 16, q_dtype="f16", kv_dtype="f16", seed=5)
    full = paged_decode(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.scale)
    part = paged_decode(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.scale,
                        seqs=[1], heads=[0, 3])
    assert np.array_equal(part[1, [0, 3]], full[1, [0, 3]])
    assert np.isnan(part[0]).all()
    assert to_f64(wl.q).shape == (3, 4, 16)


@pytest.mark.parametrize("bs", [32, 64, 256])
def test_pieces_in_16_token_units_on_large_blocks(bs):
    """``paged_decode_pieces(unit=16)`` on a cache of bs-token blocks: the
    bounds of each piece count 16-token sub-blocks, whatever the block size.
    Checked by brute force over each piece's own token slice, and against the
    same pieces on the cache's 16-token view (a block of bs tokens is bs/16
    consecutive 16-token blocks); a piece list read in bs-token units (the
    plausible slip) gives different statistics."""
    rng = np.random.default_rng(bs)
    ctx = [1, 47, 0, 200, 129, 64]
    q, K, V, kc, vc, table, cl = _random_case(rng, ctx, 4, 2, 8, bs)
    pieces = balanced_pieces(ctx, 16, 5)
    m, l, o = paged_decode_pieces(q, kc, vc, table, cl, 0.3, pieces, unit=16)
    sc32 = float(np.float32(0.3))
    for i, (s, b, fb, eb) in enumerate(pieces):
        lo, hi = 16 * fb, min(16 * eb, ctx[b])
        assert lo < hi
        for h in range(4):
            sc = [sc32 * float(np.dot(q[b, h], K[b][j, h // 2])) for j in range(lo, hi)]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            assert m[i, h] == pytest.approx(mx, abs=1e-12)
            assert l[i, h] == pytest.approx(sum(e), abs=1e-12)
            ref = sum(ei * V[b][lo + j, h // 2] for j, ei in enumerate(e)) / sum(e)
            np.testing.assert_allclose(o[i, h], ref, rtol=0, atol=1e-12)
    # the 16-token view of the same pool and tables
    k = bs // 16
    kc16 = kc.reshape(kc.shape[0] * k, 16, *kc.shape[2:])
    vc16 = vc.reshape(vc.shape[0] * k, 16, *vc.shape[2:])
    t16 = (table.astype(np.int64)[:, :, None] * k + np.arange(k)).reshape(len(ctx), -1)
    m2, l2, o2 = paged_decode_pieces(q, kc16, vc16, t16, cl, 0.3, pieces)
    assert np.array_equal(m, m2) and np.array_equal(l, l2) and np.array_equal(o, o2)
    np.testing.assert_allclose(reduce_pieces(m, l, o, pieces, len(ctx)),
                               paged_decode(q, kc, vc, table, cl, 0.3), rtol=0, atol=1e-12)
    # bounds read in bs-token units instead select other tokens (or none)
    try:
        m3, _, _ = paged_decode_pieces(q, kc, vc, table, cl, 0.3, pieces)
    except ValueError:  # an empty slice
        return
    assert not np.allclose(m3, m)
