"""Pins for the oracle's attention: dense attention when the selection covers
every position (torch's scaled_dot_product_attention in float64 on the CPU),
closed forms (one entry, equal logits) and the log-sum-exp merge."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import formats


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def _case(rng, H=16, n=300, W=128):
    lat = _bf16(rng.standard_normal((n, 512)))
    rp = _bf16(rng.standard_normal((n, 64)))
    codes, sc = oracle.encode_kv(lat)
    ql = _bf16(rng.standard_normal((H, 512)) / 24)
    qr = _bf16(rng.standard_normal((H, 64)) / 24)
    return lat, rp, codes, sc, ql, qr


def test_full_coverage_equals_dense_sdpa():
    rng = np.random.default_rng(11)
    H, n, W = 16, 300, 128
    lat, rp, codes, sc, ql, qr = _case(rng, H, n, W)
    c = n - W
    sel = np.arange(c)                                    # every candidate selected
    swa = np.concatenate([lat[c:n], rp[c:n]], axis=1)
    keys = oracle.gather_entries(codes[sel], sc[sel], rp[sel], swa)
    out, lse = oracle.attend(ql, qr, 0.7, keys)
    # dense reference: all n positions, FP4 values for [0,c), bf16 for [c,n)
    kd = np.concatenate([np.concatenate([oracle.decode_kv(codes[:c], sc[:c]),
                                         formats.bf16_to_f64(rp[:c])], 1),
                         formats.bf16_to_f64(swa)], 0)
    q = np.concatenate([formats.bf16_to_f64(ql), formats.bf16_to_f64(qr)], 1)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :],
        torch.from_numpy(kd)[None, None].expand(1, H, n, 576),
        torch.from_numpy(kd[:, :512])[None, None].expand(1, H, n, 512),
        scale=0.7)[0, :, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)
    lse_ref = torch.logsumexp(torch.from_numpy(0.7 * q @ kd.T), dim=1).numpy()
    assert np.allclose(lse, lse_ref, rtol=1e-13)


def test_one_entry_and_equal_logits():
    rng = np.random.default_rng(12)
    lat, rp, codes, sc, ql, qr = _case(rng, 4, 40)
    keys = oracle.gather_entries(codes[:1], sc[:1], rp[:1], np.zeros((0, 576), np.uint16))
    out, lse = oracle.attend(ql, qr, 1.0, keys)
    assert np.array_equal(out, np.broadcast_to(keys[0, :512], out.shape))
    q = np.concatenate([formats.bf16_to_f64(ql), formats.bf16_to_f64(qr)], 1)
    assert np.allclose(lse, q @ keys[0], rtol=1e-14)
    # zero query: every logit equal -> plain mean of the values, lse = log E
    z = np.zeros_like(ql)
    keys = oracle.gather_entries(codes[:30], sc[:30], rp[:30],
                                 np.concatenate([lat[30:40], rp[30:40]], 1))
    out, lse = oracle.attend(z, np.zeros_like(qr), 1.0, keys)
    assert np.allclose(out, keys[:, :512].mean(0)[None], rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, np.log(40.0))


def test_lse_merge_of_halves_equals_whole():
    rng = np.random.default_rng(13)
    lat, rp, codes, sc, ql, qr = _case(rng, 8, 200)
    keys = oracle.gather_entries(codes[:150], sc[:150], rp[:150],
                                 np.concatenate([lat[150:200], rp[150:200]], 1))
    o, l = oracle.attend(ql, qr, 1.3, keys)
    o1, l1 = oracle.attend(ql, qr, 1.3, keys[:77])
    o2, l2 = oracle.attend(ql, qr, 1.3, keys[77:])
    m = np.maximum(l1, l2)
    a1, a2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (a1[:, None] * o1 + a2[:, None] * o2) / (a1 + a2)[:, None]
    assert np.allclose(merged, o, rtol=1e-12, atol=1e-15)
    assert np.allclose(m + np.log(a1 + a2), l, rtol=1e-14)


def test_empty_context():
    ql = np.zeros((4, 512), np.uint16)
    out, lse = oracle.attend(ql, np.zeros((4, 64), np.uint16), 1.0,
                             oracle.gather_entries(np.zeros((0, 256), np.uint8), np.zeros((0, 32), np.uint8),
                                                   np.zeros((0, 64), np.uint16), np.zeros((0, 576), np.uint16)))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
