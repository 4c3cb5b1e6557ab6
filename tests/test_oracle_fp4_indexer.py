"""Pins of the oracle's FP4 indexer variant (FP4 indexer query and key rows,
[newsaint] section 4: DeepSeek-V4 trained the indexer's query and key with
FP4 QAT).  The row codec is the main-KV codec at width d_i; these tests fix it
at width 128 by closed forms and check the scores and selections that consume
FP4 rows against exact arithmetic and brute force."""
from fractions import Fraction

import numpy as np
import pytest

import oracle

D = 128
LEVELS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]      # the page's E2M1 list


def bf16_bits(x):
    """float64 values exactly representable in bf16 -> uint16 bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def pow2_e4m3_code(k):
    """E4M3FN byte of 2^k for a normal exponent: biased exponent k + 7, mantissa 0."""
    assert -6 <= k <= 8
    return (k + 7) << 3


def test_fp4_rows_closed_form_width_128():
    # group g holds level[i % 8] * 2^(g-4) with alternating signs, so its amax
    # is 6 * 2^(g-4): the scale is exactly 2^(g-4) and every ratio is a level
    x = np.zeros((2, D))
    codes_expect = np.zeros((2, D), dtype=np.uint8)
    for r in range(2):
        for g in range(D // 16):
            s = 2.0 ** (g - 4)
            for i in range(16):
                m = (i + 3 * r) % 8 if i != 5 else 7          # every group reaches level 6
                neg = (i + r) % 2 == 1 and m != 0
                x[r, 16 * g + i] = (-1.0 if neg else 1.0) * LEVELS[m] * s
                codes_expect[r, 16 * g + i] = (8 if neg else 0) | m
    codes, scales = oracle.encode_fp4(bf16_bits(x))
    assert codes.shape == (2, 64) and scales.shape == (2, 8)
    assert np.array_equal(scales, np.array([[pow2_e4m3_code(g - 4) for g in range(8)]] * 2))
    # two codes per byte, the even channel in the low nibble
    assert np.array_equal(codes, codes_expect[:, 0::2] | (codes_expect[:, 1::2] << 4))
    assert np.array_equal(oracle.decode_fp4(codes, scales), x)


def test_fp4_rows_one_hot_decode():
    # a single nonzero nibble decodes to one channel: byte b's high nibble is
    # channel 2b + 1, and channel ch uses scale byte ch // 16
    for ch, mag, neg in [(0, 7, False), (1, 3, True), (37, 1, False), (127, 4, True)]:
        codes = np.zeros((1, 64), dtype=np.uint8)
        nib = (8 if neg else 0) | mag
        codes[0, ch // 2] = nib << (4 * (ch % 2))
        scales = np.full((1, 8), pow2_e4m3_code(0), dtype=np.uint8)    # 1.0
        scales[0, ch // 16] = pow2_e4m3_code(-2)                       # 0.25
        v = oracle.decode_fp4(codes, scales)[0]
        expect = np.zeros(D)
        expect[ch] = (-1.0 if neg else 1.0) * LEVELS[mag] * 0.25
        assert np.array_equal(v, expect)


def test_fp4_scores_closed_form():
    # keys: every channel +1.0 (code 0x2, scale 1.0); query head 0: every
    # channel +0.5 x 2.0 = 1.0; head 1: -1.0; head 2: +0.5 x 1.0 on channels
    # 0..63 and 0 elsewhere.  Dots: 128, -128, 32.
    k = (np.full((3, 64), 0x22, np.uint8), np.full((3, 8), pow2_e4m3_code(0), np.uint8))
    qc = np.zeros((3, 64), np.uint8)
    qs = np.zeros((3, 8), np.uint8)
    qc[0], qs[0] = 0x11, pow2_e4m3_code(1)
    qc[1], qs[1] = 0xAA, pow2_e4m3_code(0)
    qc[2, :32], qs[2] = 0x11, pow2_e4m3_code(0)
    w = np.array([0.25, 0.5, 2.0], np.float32)
    s = oracle.index_scores((qc, qs), w, k)
    assert np.array_equal(s, np.full(3, 0.25 * 128 + 0.5 * 0 + 2.0 * 32))


def _fp4_rows(rng, n, scale=1.0):
    x = (rng.standard_normal((n, D)) * scale).astype(np.float32)
    return oracle.encode_fp4((x.view(np.uint32) >> 16).astype(np.uint16))


def test_fp4_scores_exact_rational():
    # the float64 score equals the exact rational sum (weights chosen exactly
    # representable, so the weighted head sum is exact as well)
    rng = np.random.default_rng(11)
    q = _fp4_rows(rng, 4, 3.0)
    k = _fp4_rows(rng, 6, 0.01)
    w = np.array([0.125, 0.75, 1.5, 0.0625], np.float32)
    s = oracle.index_scores(q, w, k)
    qv, kv = oracle.decode_rows(q), oracle.decode_rows(k)
    for p in range(6):
        tot = Fraction(0)
        for h in range(4):
            dot = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv[h], kv[p])), Fraction(0))
            tot += Fraction(float(w[h])) * max(dot, Fraction(0))
        assert Fraction(float(s[p])) == tot


def test_fp4_pool_and_reindex_brute_force():
    rng = np.random.default_rng(5)
    n, W, P, K = 700, 128, 9, 40
    c = n - W
    keys = _fp4_rows(rng, n)
    q = _fp4_rows(rng, 4)
    w = rng.random(4).astype(np.float32)
    pool, b, s = oracle.index_full(q, w, keys, n, W, P)
    # brute force: every candidate's score from its own single-row call
    s1 = np.array([oracle.index_scores(q, w, oracle.take_rows(keys, [p]))[0] for p in range(c)])
    assert np.array_equal(s, s1)
    blocks = sorted(range(-(-c // 8)), key=lambda j: (-max(s1[8 * j: min(8 * j + 8, c)]), j))
    assert np.array_equal(pool, np.sort(blocks[:P]))
    keep, sp, R = oracle.reindex(q, w, keys, pool, c, K)
    R1 = [p for j in pool for p in range(8 * j, min(8 * j + 8, c))]
    assert np.array_equal(R, R1)
    best = sorted(R1, key=lambda p: (-s1[p], p))[:K]
    assert np.array_equal(keep, np.sort(best))
    # the pool covering every block gives the flat Top-K over all candidates
    allp = np.arange(-(-c // 8))
    keep_all, _, _ = oracle.reindex(q, w, keys, allp, c, K)
    assert np.array_equal(keep_all, np.sort(sorted(range(c), key=lambda p: (-s1[p], p))[:K]))


def test_fp4_ties_and_causality():
    rng = np.random.default_rng(8)
    n, W, P, K = 300, 128, 4, 16
    c = n - W
    codes, scales = _fp4_rows(rng, n)
    # duplicate the best row into a later position: equal scores, lower wins
    q = _fp4_rows(rng, 2)
    w = np.ones(2, np.float32)
    s = oracle.index_scores(q, w, (codes[:c], scales[:c]))
    best = int(np.argmax(s))
    dup = c - 1 if best != c - 1 else 0
    codes[dup], scales[dup] = codes[best], scales[best]
    keep, _, _ = oracle.reindex(q, w, (codes, scales), np.arange(-(-c // 8)), c, 1)
    assert keep.tolist() == [min(best, dup)]
    # rows at or past c (window and future) never change the outputs
    pool, b, _ = oracle.index_full(q, w, (codes, scales), n, W, P)
    c2, s2 = codes.copy(), scales.copy()
    c2[c:] = 0x77
    s2[c:] = 0x7E
    pool2, b2, _ = oracle.index_full(q, w, (c2, s2), n, W, P)
    assert np.array_equal(pool, pool2) and np.array_equal(b, b2)
    keep1, _, _ = oracle.reindex(q, w, (codes, scales), pool, c, K)
    keep2, _, _ = oracle.reindex(q, w, (c2, s2), pool, c, K)
    assert np.array_equal(keep1, keep2) and keep1.max() < c


@pytest.mark.parametrize("width", [16, 64, 128, 512])
def test_fp4_row_codec_error_bound_any_width(width):
    # |x - decode(encode(x))| <= the group's scale, and each group's largest
    # element encodes to magnitude 6 for normal-range scales
    rng = np.random.default_rng(width)
    x = rng.standard_normal((64, width)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = oracle.bf16_to_f64(bits)
    codes, scales = oracle.encode_fp4(bits)
    err = np.abs(oracle.decode_fp4(codes, scales) - xv).reshape(64, width // 16, 16).max(axis=-1)
    assert np.all(err <= oracle.e4m3_decode(scales))
    nib = np.empty((64, width), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = codes & 0xF, codes >> 4
    arg = np.abs(xv).reshape(64, width // 16, 16).argmax(axis=-1)
    top = np.take_along_axis((nib & 7).reshape(64, width // 16, 16), arg[..., None], axis=-1)
    assert np.all(top == 7)
