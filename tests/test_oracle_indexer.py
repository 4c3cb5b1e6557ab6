"""Pins for the oracle's indexer (scores, block maxima, pool, Reindex).

Pins: exact integer arithmetic for the fp8 dot products, special cases that
reduce to numpy's dot or to a flat argsort over all candidates, brute force on
tiny inputs, and invariants the pages fix (pool size 8 * P, Reindex output
inside the pool, the window never selected, causality, ties to the lower
position).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats


def _fp8(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _int_dots(q_codes, k_codes):
    """Dot products as exact integers in units of 2^-18 (fp8 values are
    multiples of 2^-9)."""
    qi = np.rint(formats.e4m3_decode(q_codes) * 512).astype(np.int64)
    ki = np.rint(formats.e4m3_decode(k_codes) * 512).astype(np.int64)
    assert np.array_equal(qi / 512.0, formats.e4m3_decode(q_codes))
    return ki @ qi.T                                   # [c, H] exact int64


def test_scores_single_head_is_relu_dot():
    rng = np.random.default_rng(1)
    q = _fp8(rng, (1, 128))
    k = _fp8(rng, (999, 128), 3.0)
    s = oracle.index_scores(q, np.ones(1, np.float32), k)
    ref = np.maximum(_int_dots(q, k)[:, 0], 0) * 2.0 ** -18
    assert np.array_equal(s, ref)                      # exact, not approximate
    ref2 = np.maximum(formats.e4m3_decode(k) @ formats.e4m3_decode(q[0]), 0)
    assert np.allclose(s, ref2, rtol=0, atol=0)


def test_scores_weighted_heads():
    rng = np.random.default_rng(2)
    H = 8
    q = _fp8(rng, (H, 64))
    k = _fp8(rng, (300, 64))
    w = rng.uniform(0, 1, H).astype(np.float32)
    s = oracle.index_scores(q, w, k)
    dots = _int_dots(q, k) * 2.0 ** -18
    # one-hot weights select one head's ReLU(dot)
    for h in range(H):
        e = np.zeros(H, np.float32)
        e[h] = 1
        assert np.array_equal(oracle.index_scores(q, e, k), np.maximum(dots[:, h], 0))
    # linear in w; heads with a negative dot contribute nothing
    w2 = rng.uniform(0, 1, H).astype(np.float32)
    lin = oracle.index_scores(q, w, k) + oracle.index_scores(q, w2, k)
    both = oracle.index_scores(q, w.astype(np.float64) + w2, k)
    assert np.allclose(lin, both, rtol=1e-13, atol=0)
    neg = dots < 0
    flip = q.copy()
    # negating a head's query flips its dot sign: s(q) + s(-q) = sum w |dot|
    flip ^= 0x80
    tot = oracle.index_scores(q, w, k) + oracle.index_scores(flip, w, k)
    assert np.allclose(tot, np.abs(dots) @ w.astype(np.float64), rtol=1e-13)
    assert neg.any() and (~neg).any()


def test_block_scores_brute_force_and_partial_block():
    rng = np.random.default_rng(3)
    for c in [1, 7, 8, 9, 63, 64, 65, 100]:
        s = rng.standard_normal(c)
        b = oracle.block_scores(s)
        assert len(b) == -(-c // 8)
        for j in range(len(b)):
            seg = s[8 * j: min(8 * j + 8, c)]
            assert b[j] == max(seg.tolist())
    assert len(oracle.block_scores(np.zeros(0))) == 0


def test_pool_brute_force_tiny():
    rng = np.random.default_rng(4)
    for nb, P in [(10, 3), (10, 10), (10, 20), (50, 7), (1, 1)]:
        b = rng.integers(0, 5, nb).astype(np.float64)      # many ties
        pool = oracle.select_pool(b, P)
        want = sorted(sorted(range(nb), key=lambda j: (-b[j], j))[:min(P, nb)])
        assert pool.tolist() == want
        # selection property: nothing outside beats anything inside
        out = np.setdiff1d(np.arange(nb), pool)
        if len(out) and len(pool):
            assert b[out].max() <= b[pool].min()


def test_pool_contains_global_top_positions():
    """Every position whose global rank (score desc, position asc) is <= P
    lies in a pool block (each pool-excluded block has P blocks above it)."""
    rng = np.random.default_rng(5)
    q, k = _fp8(rng, (4, 64)), _fp8(rng, (2000, 64))
    w = rng.uniform(0, 1, 4).astype(np.float32)
    for P in [1, 5, 30]:
        pool, b, s = oracle.index_full(q, w, k, n=2000 + 128, W=128, P=P)
        assert len(pool) == P
        top = oracle.rank_order(s)[:P]
        assert set((top // 8).tolist()) <= set(pool.tolist())


def test_reindex_equals_flat_topk_when_pool_covers():
    rng = np.random.default_rng(6)
    H, d, n, W = 8, 128, 3000, 128
    q, k = _fp8(rng, (H, d)), _fp8(rng, (n, d))
    w = rng.uniform(0, 1, H).astype(np.float32)
    c = n - W
    s_all = oracle.index_scores(q, w, k[:c])
    flat = np.sort(np.argsort(-s_all, kind="stable")[:40])
    # P >= K with the same query: the hierarchical result equals the flat one
    pool, _, _ = oracle.index_full(q, w, k, n, W, P=40)
    keep, _, _ = oracle.reindex(q, w, k, pool, c, K=40)
    assert keep.tolist() == flat.tolist()
    # the pool holding every block also gives the flat Top-K
    allb = np.arange(-(-c // 8))
    keep2, _, R = oracle.reindex(q, w, k, allb, c, K=40)
    assert keep2.tolist() == flat.tolist() and len(R) == c


def test_reindex_scores_only_pool():
    rng = np.random.default_rng(7)
    H, d, n, W, P, K = 8, 64, 4096, 128, 16, 32
    q, k = _fp8(rng, (H, d)), _fp8(rng, (n, d))
    w = rng.uniform(0, 1, H).astype(np.float32)
    pool, _, _ = oracle.index_full(q, w, k, n, W, P)
    # adversarial fresh query whose best positions lie outside the pool
    outside = np.setdiff1d(np.arange((n - W) // 8), pool)[:4] * 8
    q2 = q.copy()
    k2 = k.copy()
    k2[outside] = _fp8(rng, (1, d), 50.0)[0]
    q2[:] = k2[outside[0]]
    keep, s, R = oracle.reindex(q2, w, k2, pool, n - W, K)
    assert len(keep) == K
    assert set(keep.tolist()) <= set(R.tolist())
    assert not set(keep.tolist()) & set(outside.tolist())
    assert len(R) == 8 * P


def test_ties_lower_position_wins():
    rng = np.random.default_rng(8)
    H, d = 4, 64
    q = _fp8(rng, (H, d))
    w = np.ones(H, np.float32)
    k = _fp8(rng, (512, d))
    k[[40, 41, 300, 301, 302]] = k[40]                 # five equal scores
    k[40][:] = k[40]
    s = oracle.index_scores(q, w, k)
    s_ord = oracle.rank_order(s)
    dup = [40, 41, 300, 301, 302]
    pos = [int(np.where(s_ord == p)[0][0]) for p in dup]
    assert pos == sorted(pos)                           # equal scores: ascending positions
    keep, _, _ = oracle.reindex(q, w, k, np.arange(64), 512, K=int(pos[0]) + 2)
    assert 40 in keep and 41 in keep and 300 not in keep


def test_window_and_future_never_selected_and_causal():
    rng = np.random.default_rng(9)
    H, d, n, W = 8, 64, 1000, 128
    q, k = _fp8(rng, (H, d)), _fp8(rng, (n + 50, d))
    w = rng.uniform(0, 1, H).astype(np.float32)
    pool, b, s = oracle.index_full(q, w, k, n, W, P=200)  # P > nb: all blocks
    c = n - W
    assert len(b) == -(-c // 8) and len(pool) == len(b)
    keep, _, _ = oracle.reindex(q, w, k, pool, c, K=5000)
    assert keep.max() < c and len(keep) == c
    # perturbing rows >= c (window and future) changes nothing
    k2 = k.copy()
    k2[c:] = _fp8(rng, (len(k) - c, d), 9.0)
    pool2, b2, _ = oracle.index_full(q, w, k2, n, W, P=20)
    pool1, b1, _ = oracle.index_full(q, w, k, n, W, P=20)
    assert np.array_equal(pool1, pool2) and np.array_equal(b1, b2)
    assert np.array_equal(oracle.reindex(q, w, k, pool1, c, 37)[0],
                          oracle.reindex(q, w, k2, pool1, c, 37)[0])


@pytest.mark.parametrize("n", [0, 1, 128, 129, 130, 137])
def test_degenerate_short_contexts(n):
    rng = np.random.default_rng(10)
    q, k = _fp8(rng, (8, 64)), _fp8(rng, (max(n, 1), 64))
    w = np.ones(8, np.float32)
    pool, b, s = oracle.index_full(q, w, k, n, 128, P=4)
    c = max(0, n - 128)
    assert len(s) == c and len(b) == -(-c // 8) and len(pool) == min(4, len(b))
    keep, _, _ = oracle.reindex(q, w, k, pool, c, K=16)
    assert len(keep) == min(16, c)
