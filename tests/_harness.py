"""Shared set-up for the GPU parity tests and the benchmark's checks.

GPU side: caches and queries generated on the device by `workloads` and run
through the HIP library.  Oracle side: the same seeded inputs regenerated on
the CPU for one sampled query at a time and run through `oracle`.  Nothing
produced by the HIP library is ever handed to the oracle; oracle outputs may be
fed to the library (e.g. an oracle pool into Reindex) to test one stage alone.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402
import oracle  # noqa: E402

SEL_BAND = 1e-5      # index sets may differ only within this relative score gap
SCORE_TOL = 1e-3     # indexer scores
ATTN_TOL = 2e-3      # attention: max|d| / max|ref| per (query, head) row


def have_gpu() -> bool:
    return torch.cuda.is_available()


def lib():
    """The HIP binding; with a GPU present, a missing library is an error, not a skip."""
    if not have_gpu():
        pytest.skip("no GPU")
    import compressed_sparse_attention_decode_amd as csa2
    csa2.lib()
    return csa2


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().astype(np.uint16)


def GpuCase(w: wl.Workload, device="cuda", **kw):
    """Caches, window rows and query batch of a workload on the GPU (the
    benchmark's device state)."""
    lib()
    from bench import DeviceState
    return DeviceState(w, device=device, **kw)


class OracleQuery:
    """The oracle's view of one query of a workload (all inputs regenerated on
    the CPU from the seeded generator)."""

    def __init__(self, w: wl.Workload, lay: wl.Layout, qi: int, keys=None):
        self.w, self.lay, self.qi = w, lay, qi
        d = w.dims
        self.n = lay.q_visible[qi]
        self.base = lay.q_seq_base[qi]
        self.c = oracle.candidates(self.n, d.swa)
        seq = qi // w.tokens_per_seq
        if keys is None:
            rows = max(lay.seq_rows[seq], 1)
            if w.idx_fp4:
                keys = oracle.encode_fp4(u16(wl.idx_keys_bf16(w, self.base, rows)))
            else:
                keys = u8(wl.idx_keys(w, self.base, rows))
        assert oracle.n_rows(keys) >= self.c
        self.keys = keys

    def iq(self, layer):
        wt = wl.idx_weight(self.w, layer, self.qi, 1)[0].numpy()
        if self.w.idx_fp4:
            return oracle.encode_fp4(u16(wl.idx_query_bf16(self.w, layer, self.qi, 1)[0])), wt
        return u8(wl.idx_query(self.w, layer, self.qi, 1)[0]), wt

    def full(self, layer=0):
        q, wt = self.iq(layer)
        return oracle.index_full(q, wt, self.keys, self.n, self.w.dims.swa, self.w.dims.pool_blocks)

    def reindex(self, layer, pool):
        q, wt = self.iq(layer)
        return oracle.reindex(q, wt, self.keys, pool, self.c, self.w.dims.topk)

    def scores_at(self, layer, pos):
        q, wt = self.iq(layer)
        pos = np.asarray(pos, dtype=np.int64)
        return oracle.index_scores(q, wt, oracle.take_rows(self.keys, pos)) if len(pos) else np.zeros(0)

    def attention(self, layer, keep, scale=1.0):
        w = self.w
        rows = self.base + np.asarray(keep, dtype=np.int64)
        lat = u16(wl.latent_at(w, rows)) if len(rows) else np.zeros((0, 512), np.uint16)
        rp = u16(wl.rope_at(w, rows)) if len(rows) else np.zeros((0, 64), np.uint16)
        grp = w.dims.kv_group
        codes, scales = oracle.encode_kv(lat, grp) if len(rows) else (np.zeros((0, 256), np.uint8),
                                                                      np.zeros((0, 512 // grp), np.uint8))
        win = self.base + np.arange(self.c, self.n, dtype=np.int64)
        swa = np.concatenate([u16(wl.latent_at(w, win)), u16(wl.rope_at(w, win))], axis=1) \
            if len(win) else np.zeros((0, 576), np.uint16)
        keys = oracle.gather_entries(codes, scales, rp, swa)
        ql = u16(wl.q_latent(w, layer, self.qi, 1)[0])
        qr = u16(wl.q_rope(w, layer, self.qi, 1)[0])
        return oracle.attend(ql, qr, scale, keys)


def check_set(got, ref, scores_of, label=""):
    """Index sets: equal size; each element of the symmetric difference has an
    oracle score within SEL_BAND (relative) of the oracle's k-th score.
    `scores_of(idx_array)` returns oracle scores; ref is ordered by rank
    through `kth`."""
    got = np.asarray(got, dtype=np.int64)
    ref = np.asarray(ref, dtype=np.int64)
    assert len(got) == len(ref), f"{label}: size {len(got)} != {len(ref)}"
    assert np.all(np.diff(got) > 0), f"{label}: output not strictly ascending"
    diff = np.setxor1d(got, ref)
    if len(diff) == 0:
        return 0
    ref_scores = scores_of(ref)
    kth = ref_scores.min()
    d_scores = scores_of(diff)
    gap = np.abs(d_scores - kth)
    bad = gap > SEL_BAND * max(abs(kth), 1e-30)
    assert not bad.any(), (f"{label}: {bad.sum()} of {len(diff)} differing indices outside the tie band; "
                           f"k-th score {kth!r}, worst {d_scores[bad][:5]!r}")
    return len(diff)


def check_attention(out, lse, ref_out, ref_lse, label=""):
    out = np.asarray(out, dtype=np.float64)
    err = np.abs(out - ref_out).max(axis=-1)
    den = np.abs(ref_out).max(axis=-1)
    rel = err / np.maximum(den, 1e-30)
    assert np.all(rel <= ATTN_TOL), f"{label}: attention rel err {rel.max():.3e} > {ATTN_TOL}"
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse), fin), f"{label}: lse finiteness differs"
        assert np.allclose(lse[fin], ref_lse[fin], rtol=1e-4, atol=1e-4), f"{label}: lse mismatch"
    return float(rel.max()) if rel.size else 0.0


def with_oracle_rows(tk: torch.Tensor, tc: torch.Tensor, rows: dict):
    """Copies of the library's topk_pos / topk_count inputs in which the
    queries in `rows` (query -> oracle Top-K, ascending) carry the oracle's
    own kept positions, so that the library's attention can be compared with
    the oracle's on the same set (oracle outputs feed the library, never the
    other way round)."""
    tk2, tc2 = tk.clone(), tc.clone()
    for qi, keep in rows.items():
        tk2[qi].fill_(-1)
        if len(keep):
            tk2[qi, :len(keep)] = torch.as_tensor(np.asarray(keep, dtype=np.int32), device=tk.device)
        tc2[qi] = len(keep)
    return tk2, tc2


def with_oracle_pool(pool: torch.Tensor, cnt: torch.Tensor, rows: dict):
    """Copies of the library's pool_blocks / pool_count in which the queries
    in `rows` (query -> oracle pool, ascending block ids) carry the oracle's
    own pool.  When the library's pool differs from the oracle's inside the
    selection band, a later layer's Reindex on the two pools can differ by
    more than the band (its query is not the one that ranked the blocks), so
    its Top-K is compared with the oracle's by running the library's Reindex
    on the oracle's pool (oracle outputs feed the library, never the other
    way round)."""
    p2, c2 = pool.clone(), cnt.clone()
    for qi, rp in rows.items():
        p2[qi].fill_(-1)
        if len(rp):
            p2[qi, :len(rp)] = torch.as_tensor(np.asarray(rp, dtype=np.int32), device=pool.device)
        c2[qi] = len(rp)
    return p2, c2
