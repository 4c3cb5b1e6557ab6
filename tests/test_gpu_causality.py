"""Causality on the GPU: rows a query may not use never change its results.

A query with n visible positions selects only among positions [0, c),
c = max(0, n - W), and attends to its kept positions (FP4 main KV) plus the
window [c, n) read from the separate bf16 window rows ("DeepSeek-V4.1-Flash
梗概" §3.2, heterogeneous KV: the indexer and Top-K serve only the sparse
branch).  So neither the indexer keys nor the FP4 main-KV rows at positions
>= c, nor any row past the sequence, may change a pool, a Top-K set or an
attention output.

Each case copies the caches into planes where every sequence is followed by
a gap of extra rows, then runs the Full index, Reindex and attention twice:
with zeros in the gaps, and with huge values (fp8 448, FP4 code 6 at scale
448, bf16 32768) in the gaps and in every row at positions >= c.  The two
runs must agree bit for bit, and the first must agree bit for bit with the
same calls on the unshifted caches.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests._harness import GpuCase, lib
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu

GAP = 320                      # rows after each sequence
CAUSAL_CASES = ["ragged_b3", "fp4_ragged_b3", "kvg32_ragged_b3", "edge_short", "ragged_g4", "h24_ragged"]


def _relocate(t: torch.Tensor, lay: wl.Layout, fill: torch.Tensor):
    """t's rows with GAP rows after every sequence (filled with `fill`), and
    the new first row of each sequence."""
    n_seq = len(lay.seq_rows)
    rows = t.shape[0] + n_seq * GAP
    out = fill.expand((rows,) + tuple(t.shape[1:])).clone()
    new_base = []
    for s in range(n_seq):
        b, r = lay.seq_base[s], lay.seq_rows[s]
        nb = b + s * GAP
        out[nb:nb + r] = t[b:b + r]
        new_base.append(nb)
    return out, new_base


def _garble(t: torch.Tensor, lay: wl.Layout, new_base, c_max, fill: torch.Tensor):
    """Overwrite, in relocated planes, each sequence's rows at positions >= its
    tokens' largest c (the window and beyond) with `fill`."""
    for s in range(len(lay.seq_rows)):
        lo, hi = new_base[s] + c_max[s], new_base[s] + lay.seq_rows[s]
        if hi > lo:
            t[lo:hi] = fill.expand((hi - lo,) + tuple(t.shape[1:]))
    return t


def _run(g, dims, batch, planes):
    csa2 = g.csa2
    idx_k, codes, scales, kv_rope, swa_kv = planes
    q, w = g.iq(0)
    pool, cnt = csa2.index_full(dims, batch, q, w, idx_k)
    tk, tc = csa2.index_reindex(dims, batch, q, w, idx_k, pool, cnt)
    ql, qr = g.mq(0)
    out, lse = csa2.attend(dims, batch, ql, qr, 1.0, codes, scales, kv_rope, tk, tc, swa_kv, g.swa_base)
    torch.cuda.synchronize()
    res = {"pool_count": cnt.cpu(), "topk_count": tc.cpu(), "topk_pos": tk.cpu(),
           "out": out.cpu().view(torch.int32), "lse": lse.cpu().view(torch.int32)}
    pb = pool.cpu()
    res["pool"] = [pb[i, :int(cnt[i])] for i in range(pb.shape[0])]
    return res


def _same(a, b, label):
    for k in a:
        if k == "pool":
            for i, (x, y) in enumerate(zip(a[k], b[k])):
                assert torch.equal(x, y), f"{label}: pool of query {i} changed"
        else:
            assert torch.equal(a[k], b[k]), f"{label}: {k} changed"


@pytest.mark.parametrize("name", CAUSAL_CASES)
def test_rows_past_the_candidates_change_nothing(name):
    csa2 = lib()
    w = CASES[name]
    g = GpuCase(w)
    lay = g.lay
    dims = g.dims
    g_tok = w.tokens_per_seq
    # per sequence: the largest c of its tokens (rows at positions >= it are
    # used by no token's sparse branch)
    c_max = [max(max(0, lay.q_visible[s * g_tok + j] - dims.swa) for j in range(g_tok))
             for s in range(len(lay.seq_rows))]
    base = _run(g, dims, g.batch, g.planes[0])

    idx_k, codes, scales, kv_rope, swa_kv = g.planes[0]
    dev = codes.device
    zero8 = torch.zeros(1, dtype=torch.uint8, device=dev)
    big_fp8 = torch.tensor([0x7E], dtype=torch.uint8, device=dev)        # e4m3 448
    big_code = torch.tensor([0x77], dtype=torch.uint8, device=dev)       # two E2M1 6.0
    big_bf16 = torch.tensor([0x4700], dtype=torch.int16, device=dev)     # bf16 32768

    def planes(gap_fill: bool):
        def reloc(t, big):
            t8 = t.view(torch.uint8) if t.dtype != torch.int16 else t
            fill = big if gap_fill else torch.zeros_like(big)
            out, nb = _relocate(t8, lay, fill)
            if gap_fill:
                out = _garble(out, lay, nb, c_max, big)
            return out, nb
        if isinstance(idx_k, tuple):
            (kc, nb), (ks, _) = reloc(idx_k[0], big_code), reloc(idx_k[1], big_fp8)
            ik = (kc, ks)
        else:
            k8, nb = reloc(idx_k, big_fp8)
            ik = k8.view(torch.float8_e4m3fn)
        c2, _ = reloc(codes, big_code)
        s2, _ = reloc(scales, big_fp8)
        r2, _ = reloc(kv_rope.view(torch.int16), big_bf16)
        return (ik, c2, s2, r2.view(torch.bfloat16), swa_kv), nb

    p0, nb = planes(False)
    p1, _ = planes(True)
    seq_of = [qi // g_tok for qi in range(w.n_q)]
    shift = torch.tensor([nb[s] - lay.seq_base[s] for s in seq_of], dtype=torch.int64, device=dev)
    batch = csa2.Batch(g.batch.seq_base + shift, g.batch.n_visible, g.batch.max_visible, g.batch.tokens_per_seq)
    shifted = _run(g, dims, batch, p0)
    _same(base, shifted, f"{name}: relocated caches")
    garbled = _run(g, dims, batch, p1)
    _same(base, garbled, f"{name}: rows at positions >= c and past the sequence overwritten")
    # the garbage is reachable: a query that could see those rows would change
    assert any(int(x) > 0 for x in base["topk_count"]) or name == "edge_short"
