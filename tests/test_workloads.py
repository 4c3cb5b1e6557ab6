"""The seeded input generator: published SplitMix64 values, determinism,
chunk independence, and the distributions the workloads ask for."""
import math

import numpy as np
import torch

import workloads as wl


def test_mix64_matches_python_definition():
    seed = 0x1234567890ABCDEF
    got = wl._bits(seed, 0, 5, "cpu").tolist()
    for i, g in enumerate(got):
        z = (seed + (i + 1) * 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
        assert (g & ((1 << 64) - 1)) == wl.mix64_reference(z)
    # SplitMix64 seeded with 0: first outputs of the published generator
    first = [wl.mix64_reference((k * 0x9E3779B97F4A7C15) & ((1 << 64) - 1)) for k in (1, 2)]
    assert first == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4]


def test_chunk_independent_and_deterministic():
    w = wl.workload(1)
    a = wl.idx_keys(w, 1000, 64)
    b = torch.cat([wl.idx_keys(w, 1000, 20), wl.idx_keys(w, 1020, 44)])
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert torch.equal(wl.latent(w, 5, 3).view(torch.int16), wl.latent(w, 5, 3).view(torch.int16))
    # different streams differ
    assert not torch.equal(wl.latent(w, 5, 3).view(torch.int16), wl.rope(w, 5, 3)[:, :64].repeat(1, 8).view(torch.int16))


def test_distributions():
    w = wl.workload(1)
    x = wl.latent(w, 0, 2048).float()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1) < 0.01
    k = wl.idx_keys(w, 0, 4096).float()
    assert abs(k.std().item() - 1) < 0.02
    q = wl.q_latent(w, 0, 0, 2).float()
    assert abs(q.std().item() - 1 / 24) < 0.002
    u = wl.idx_weight(w, 0, 0, 64)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean().item() - 0.5) < 0.1
    assert x.abs().max().item() < 5.0


def test_layouts():
    for w in wl.WORKLOADS:
        lay = wl.layout(w)
        assert len(lay.q_visible) == w.n_q
        lo, hi = w.ctx
        assert all(lo <= c <= hi for c in lay.ctx)
        assert lay.rows == sum(lay.seq_rows)
        for q in range(w.n_q):
            s = q // w.tokens_per_seq
            n = lay.q_visible[q]
            assert n <= lay.ctx[s] + w.tokens_per_seq - 1
            c = max(0, n - w.dims.swa)
            # the query's window starts at swa row q_swa_base and stays in its sequence
            first = lay.q_swa_base[q] - lay.swa_seq_base[s] + lay.swa_lo[s]
            assert first == c
    lay3 = wl.layout(wl.workload(3))
    assert len(set(lay3.ctx)) > 1
