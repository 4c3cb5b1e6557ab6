"""Pins of the oracle's group-32 main-KV codec variant ([akhunji], "Microscopic
FP4 (E2M1) Cache Compression": E2M1 values with block-level FP8 scaling over
blocks of 32 elements): closed forms, its relation to the group-16 codec, and
the codec invariants at group 32."""
import numpy as np

import oracle

LEVELS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]      # the page's E2M1 list


def bf16_bits(x):
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def test_group32_closed_form():
    # group g (32 channels) holds E2M1 levels times 2^e(g), e(g) = -6 + g % 15
    # (normal E4M3 scales up to 2^8), mixed signs and one level-6 value: the
    # scale is 2^e(g) exactly and the codes are the level indices
    x = np.zeros((1, 512))
    nib = np.zeros(512, dtype=np.uint8)
    for g in range(16):
        s = 2.0 ** (-6 + g % 15)
        for i in range(32):
            m = 7 if i == 9 else (i * 3) % 8
            neg = i % 3 == 1 and m != 0
            x[0, 32 * g + i] = (-1.0 if neg else 1.0) * LEVELS[m] * s
            nib[32 * g + i] = (8 if neg else 0) | m
    codes, scales = oracle.encode_kv(bf16_bits(x), group=32)
    assert codes.shape == (1, 256) and scales.shape == (1, 16)
    assert scales[0].tolist() == [(-6 + g % 15 + 7) << 3 for g in range(16)]
    assert np.array_equal(codes[0], nib[0::2] | (nib[1::2] << 4))
    assert np.array_equal(oracle.decode_kv(codes, scales), x)


def test_group32_equals_group16_when_halves_share_amax():
    # if both 16-channel halves of every 32-group have the same amax, the
    # group-32 scales are the group-16 scales taken once per pair, and the
    # codes are identical
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 512)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    v = oracle.bf16_to_f64(xb).reshape(50, 16, 2, 16)
    amax = np.abs(v).max(axis=(2, 3))
    # put the 32-group's amax (with its sign) into channel 0 of both halves
    for half in range(2):
        v[:, :, half, 0] = amax
    xb = bf16_bits(v.reshape(50, 512))
    c16, s16 = oracle.encode_kv(xb)
    c32, s32 = oracle.encode_kv(xb, group=32)
    assert np.array_equal(s16[:, 0::2], s32) and np.array_equal(s16[:, 1::2], s32)
    assert np.array_equal(c16, c32)


def test_group32_decode_is_group16_decode_with_repeated_scales():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (20, 256), dtype=np.uint8)
    s32 = rng.integers(0, 0x7F, (20, 16), dtype=np.uint8)
    assert np.array_equal(oracle.decode_kv(codes, s32), oracle.decode_kv(codes, np.repeat(s32, 2, axis=1)))


def test_group32_invariants():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((200, 512)).astype(np.float32) * rng.uniform(0.01, 50, (200, 1)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = oracle.bf16_to_f64(xb)
    codes, scales = oracle.encode_kv(xb, group=32)
    s = oracle.e4m3_decode(scales)
    err = np.abs(oracle.decode_kv(codes, scales) - xv).reshape(200, 16, 32).max(axis=-1)
    assert np.all(err <= s)
    nib = np.empty((200, 512), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = codes & 0xF, codes >> 4
    arg = np.abs(xv).reshape(200, 16, 32).argmax(axis=-1)
    top = np.take_along_axis((nib & 7).reshape(200, 16, 32), arg[..., None], axis=-1)
    assert np.all(top == 7)
    # the scale rule per 32-group: E4M3 RNE of min(amax / 6, 448)
    amax = np.abs(xv).reshape(200, 16, 32).max(axis=-1)
    assert np.array_equal(scales, oracle.e4m3_encode_rne(np.minimum(amax / 6.0, 448.0)))
