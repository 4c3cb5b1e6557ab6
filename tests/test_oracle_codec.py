"""Pins for the oracle's FP4 codec and number formats (CPU only).

Each pin comes from outside the oracle: values printed on the pages (golden
fixtures), torch's own float8_e4m3fn cast (a library routine), an independent
brute-force nearest-level search, or invariants of the format.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_constants():
    out = {}
    for line in open(os.path.join(GOLDEN, "format_constants.txt"), encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (t.strip() for t in line.split("="))
            out[k] = int(v)
    return out


def _bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = formats.bf16_to_f64(b)
    return b[np.isfinite(v)], v[np.isfinite(v)]


def test_e2m1_levels_match_page():
    lev = [float(l) for l in open(os.path.join(GOLDEN, "e2m1_levels.txt"))
           if l.strip() and not l.startswith("#")]
    assert list(formats.E2M1_LEVELS) == lev


def test_format_constants():
    c = _golden_constants()
    assert oracle.GROUP == c["fp4_group_channels"]
    assert oracle.BYTES_CODES == c["fp4_code_bytes"] == c["latent_dim"] // 2
    assert oracle.BYTES_SCALES == c["fp4_scale_bytes"] == c["latent_dim"] // c["fp4_group_channels"]
    assert formats.e4m3_decode(0x7E) == c["e4m3_max"]
    assert c["pool_blocks"] * c["indexer_block"] == c["pool_positions"]
    codes, scales = oracle.encode_kv(np.zeros((3, 512), np.uint16))
    assert codes.shape == (3, 256) and scales.shape == (3, 32)


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_encode_matches_torch_rne():
    b, v = _all_finite_bf16()
    m = (v >= 0) & (v <= 448) & ~np.signbit(v)
    v = v[m]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.e4m3_encode_rne(v)
    assert np.array_equal(ref, got)
    # midpoints between consecutive E4M3 values: ties go to the even code
    pos = formats.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    got = formats.e4m3_encode_rne(mids)
    ref = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    assert np.all(got % 2 == 0)


def test_scale_rule_all_bf16_amax():
    """Scale byte = RNE_E4M3(min(amax / 6, 448)) for every finite bf16 amax;
    torch casts fl32(amax / 6) (correctly rounded division) -- the same value
    for every bf16 amax -- so it pins the oracle's float64 rule."""
    b, v = _all_finite_bf16()
    keep = v > 0
    b, v = b[keep], v[keep]
    n = len(b)
    rows = -(-n // 32)
    lat = np.zeros(rows * 512, np.uint16)
    lat[np.arange(n) * 16] = b                     # one element per group
    _, sc = oracle.encode_kv(lat.reshape(rows, 512))
    got = sc.reshape(-1)[:n]
    t = np.minimum((v.astype(np.float32) / np.float32(6)).astype(np.float32), np.float32(448))
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # the tie amax = 6.375 -> 1.0625, exactly between 1.0 and 1.125 -> 1.0
    _, sc = oracle.encode_kv(np.pad(_bf16_bits([6.375]), (0, 511))[None, :])
    assert formats.e4m3_decode(sc[0, 0]) == 1.0


def _brute_code(x: np.ndarray, s: float) -> np.ndarray:
    """Nearest E2M1 level to |x| / s by distances in x-space (exact here),
    ties to the even code; an independent search, no division."""
    ax = np.abs(x)
    lv = formats.E2M1_LEVELS * s                    # exact products
    d = np.abs(ax[:, None] - lv[None, :])            # exact for |x| >= 2^-20 s
    best = d.min(1, keepdims=True)
    tie = (d == best)
    code = np.where(tie.sum(1) > 1, np.argmax(tie & (np.arange(8) % 2 == 0), 1), np.argmax(tie, 1))
    code = np.where(ax < s * 2.0 ** -20, 0, code)
    sign = (np.signbit(x)).astype(np.uint8) << 3
    return (sign | code).astype(np.uint8)


def _unpack(codes):
    nib = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    return nib


@pytest.mark.parametrize("part", range(4))
def test_fp4_brute_force_all_scales_all_bf16(part):
    """Every positive finite E4M3 scale s x every finite bf16 x with |x| <= 6s:
    group [6s, x, ...] has scale byte s and x's code is the nearest level."""
    b, v = _all_finite_bf16()
    scales = np.arange(1, 0x7F)[part::4]
    for sc in scales:
        s = float(formats.e4m3_decode(sc))
        m = np.abs(v) <= 6 * s
        xb, xv = b[m], v[m]
        n = len(xb)
        per = 15
        ng = -(-n // per)
        grp = np.zeros((ng, 16), np.uint16)
        grp[:, 0] = _bf16_bits([6 * s])[0]
        flat = np.zeros(ng * per, np.uint16)
        flat[:n] = xb
        grp[:, 1:] = flat.reshape(ng, per)
        rows = -(-ng // 32)
        lat = np.zeros((rows * 32, 16), np.uint16)
        lat[:ng] = grp
        codes, scl = oracle.encode_kv(lat.reshape(rows, 512))
        assert np.all(scl.reshape(-1)[:ng] == sc)
        nib = _unpack(codes).reshape(-1, 16)[:ng, 1:].reshape(-1)[:n]
        assert np.array_equal(nib, _brute_code(xv, s)), f"scale code {sc:#x}"


def test_fp4_known_tie_and_layout():
    # s = 0.029296875 (E4M3 0x17 ... exact), x = 0.03662109375: x / s = 1.25
    s = 0.029296875
    assert formats.e4m3_decode(formats.e4m3_encode_rne(s)) == s
    x = 0.03662109375
    assert x / s == 1.25
    lat = np.zeros((1, 512), np.uint16)
    lat[0, :3] = _bf16_bits([6 * s, x, -x])
    codes, sc = oracle.encode_kv(lat)
    assert formats.e4m3_decode(sc[0, 0]) == s
    assert codes[0, 0] == (7 | (2 << 4))           # ch0 low nibble: 6.0; ch1: 1.0 (even tie)
    assert codes[0, 1] & 0xF == 0x8 | 2             # ch2: -1.0
    # ties at 0.25 / 0.75 / 1.75 / 2.5 / 3.5 / 5 go to the even code
    ratios = [0.25, 0.75, 1.75, 2.5, 3.5, 5.0]
    expect = [0, 2, 4, 4, 6, 6]
    got = formats.e2m1_encode_rne(np.array(ratios))
    assert list(got) == expect


def test_fp4_invariants_gaussian():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((256, 512)).astype(np.float32)
    bits = _bf16_bits(x)
    codes, sc = oracle.encode_kv(bits)
    xv = formats.bf16_to_f64(bits)
    deq = oracle.decode_kv(codes, sc)
    s = np.repeat(formats.e4m3_decode(sc), 16, axis=1)
    # |x - deq| <= s (largest half-gap of the E2M1 grid is 1 level unit)
    assert np.all(np.abs(xv - deq) <= s)
    # the group maximum encodes to magnitude 6 for normal-range scales
    g = np.abs(xv).reshape(256, 32, 16)
    nib = _unpack(codes).reshape(256, 32, 16)
    at = np.argmax(g, axis=2)
    assert np.all(np.take_along_axis(nib & 7, at[..., None], 2) == 7)
    # decode(encode(level * s)) is exact
    re_codes, re_sc = oracle.encode_kv(_bf16_bits(deq.astype(np.float32)))
    assert np.array_equal(oracle.decode_kv(re_codes, re_sc), deq)


def test_fp4_degenerate_groups():
    lat = np.zeros((1, 512), np.uint16)
    lat[0, 16:18] = _bf16_bits([-1e-6, 1e-6])      # amax/6 < 2^-10 -> scale 0
    lat[0, 32] = _bf16_bits([-1.0])[0]
    lat[0, 33] = _bf16_bits([-0.01])[0]            # rounds to magnitude 0, keeps sign
    lat[0, 48] = _bf16_bits([1e4])[0]              # scale clamps at 448; 1e4/448 > 6
    lat[0, 49] = _bf16_bits([-3000.0])[0]
    codes, sc = oracle.encode_kv(lat)
    nib = _unpack(codes)[0]
    assert sc[0, 0] == 0 and np.all(nib[:16] == 0)  # all-zero group
    assert sc[0, 1] == 0 and np.all(nib[16:32] == 0)
    assert nib[32] == 0x8 | 7 and nib[33] == 0x8
    assert formats.e4m3_decode(sc[0, 3]) == 448 and nib[48] == 7 and nib[49] == 0x8 | 7
