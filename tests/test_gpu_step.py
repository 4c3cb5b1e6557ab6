"""csa2_decode_step: one call per layer in each mode of the pages' mode table
(Full, Reindex, Reuse), against the separate stage calls (the same kernels, so
bit for bit), and the same call captured into a HIP graph and replayed.

The stage calls themselves are checked against the oracle in
test_gpu_parity.py; here the step's outputs are also checked against the
oracle: every query's Full layer, and a Reuse layer (a fresh main query over
the oracle's own Top-K of the Reindex layer)."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests._harness import GpuCase, OracleQuery, check_attention, check_set, lib, with_oracle_pool, with_oracle_rows
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu

STEP_CASES = ["ragged_b3", "edge_short", "fp4_ragged_b3", "kvg32_ragged_b3", "ragged_g4"]


def _buffers(g):
    w, dev = g.w, "cuda"
    n_q, d = w.n_q, w.dims
    return dict(pool_blocks=torch.full((n_q, d.pool_blocks), 7, dtype=torch.int32, device=dev),
                pool_count=torch.full((n_q,), 7, dtype=torch.int32, device=dev),
                topk_pos=torch.full((n_q, d.topk), 7, dtype=torch.int32, device=dev),
                topk_count=torch.full((n_q,), 7, dtype=torch.int32, device=dev),
                out=torch.full((n_q, d.n_heads, 512), 7.0, dtype=torch.float32, device=dev),
                lse=torch.full((n_q, d.n_heads), 7.0, dtype=torch.float32, device=dev))


def _step(g, mode, layer, bufs, ws, prepare=False):
    csa2 = g.csa2
    q, wt = g.iq(layer)
    ql, qr = g.mq(layer)
    idx_k, codes, scales, kv_rope, swa_kv = g.planes[0]
    return csa2.decode_step(g.dims, g.batch, mode, q, wt, idx_k, bufs["pool_blocks"], bufs["pool_count"],
                            bufs["topk_pos"], bufs["topk_count"], ql, qr, 1.0, codes, scales, kv_rope, swa_kv,
                            g.swa_base, bufs["out"], bufs["lse"], ws=ws, prepare=prepare)


def _same(a, b, label):
    a, b = a.cpu(), b.cpu()
    if a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    assert torch.equal(a, b), label


@pytest.mark.parametrize("name", STEP_CASES)
def test_step_modes_match_stage_calls(name):
    lib()
    w = CASES[name]
    g = GpuCase(w)
    csa2 = g.csa2
    ws = torch.zeros(csa2.workspace_step(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    bufs = _buffers(g)
    # Full layer
    _step(g, csa2.LAYER_FULL, 0, bufs, ws)
    pool, cnt, _ = g.full(0)
    tk, tc, _ = g.reindex(0, pool, cnt)
    out, lse = g.attend(0, tk, tc)
    torch.cuda.synchronize()
    n_q = w.n_q
    for qi in range(n_q):
        k = int(cnt[qi])
        _same(bufs["pool_blocks"][qi, :k], pool[qi, :k], f"{name} q{qi} pool")
    _same(bufs["pool_count"], cnt, f"{name} pool count")
    _same(bufs["topk_pos"], tk, f"{name} topk")
    _same(bufs["topk_count"], tc, f"{name} topk count")
    _same(bufs["out"], out, f"{name} out")
    _same(bufs["lse"], lse, f"{name} lse")
    # every query's Full layer against the oracle: pool and Top-K within the
    # selection band; attention on the step's own output when the Top-K is
    # the oracle's, else the same attention call on the oracle's set
    lay = wl.layout(w)
    oqs, rpools, keep1, other = {}, {}, {}, {}
    for qi in range(n_q):
        oq = oqs[qi] = OracleQuery(w, lay, qi)
        rpool, rb, _ = oq.full(0)
        rpools[qi] = rpool
        check_set(bufs["pool_blocks"][qi, :int(cnt[qi])].cpu().numpy(), rpool, lambda j: rb[j], f"{name} q{qi} step pool")
        keep, _, _ = oq.reindex(0, rpool)
        got = bufs["topk_pos"][qi, :int(tc[qi])].cpu().numpy()
        if not np.array_equal(bufs["pool_blocks"][qi, :int(cnt[qi])].cpu().numpy(), rpool):
            # pools that differ inside the band: the Top-K of the library's
            # Reindex (this layer's query) on the oracle's pool
            p2, c2 = with_oracle_pool(pool, cnt, {qi: rpool})
            tk_o, tc_o, _ = g.reindex(0, p2, c2)
            torch.cuda.synchronize()
            got = tk_o[qi, :int(tc_o[qi])].cpu().numpy()
        check_set(got, keep, lambda p, oq=oq: oq.scores_at(0, p), f"{name} q{qi} step topk")
        ro, rl = oq.attention(0, keep)
        if np.array_equal(got, keep):
            check_attention(bufs["out"][qi].cpu().numpy(), bufs["lse"][qi].cpu().numpy(), ro, rl, f"{name} q{qi} step")
        else:
            other[qi] = (keep, ro, rl)
        keep1[qi] = oq.reindex(1, rpool)[0]
    if other:
        tk2, tc2 = with_oracle_rows(tk, tc, {qi: v[0] for qi, v in other.items()})
        out_o, lse_o = g.attend(0, tk2, tc2)
        torch.cuda.synchronize()
        for qi, (_, ro, rl) in other.items():
            check_attention(out_o[qi].cpu().numpy(), lse_o[qi].cpu().numpy(), ro, rl, f"{name} q{qi} oracle-set")
    # Reindex layer (fresh indexer and main queries) on the Full layer's pool
    _step(g, csa2.LAYER_REINDEX, 1, bufs, ws)
    tk1, tc1, _ = g.reindex(1, pool, cnt)
    out1, lse1 = g.attend(1, tk1, tc1)
    torch.cuda.synchronize()
    _same(bufs["topk_pos"], tk1, f"{name} reindex topk")
    _same(bufs["out"], out1, f"{name} reindex out")
    _same(bufs["lse"], lse1, f"{name} reindex lse")
    # Reuse layer: only a new main query over the inherited Top-K
    bufs["out"].fill_(3.0)
    ql, qr = g.mq(2)
    idx_k, codes, scales, kv_rope, swa_kv = g.planes[0]
    csa2.decode_step(g.dims, g.batch, csa2.LAYER_REUSE, None, None, None, bufs["pool_blocks"], bufs["pool_count"],
                     bufs["topk_pos"], bufs["topk_count"], ql, qr, 1.0, codes, scales, kv_rope, swa_kv,
                     g.swa_base, bufs["out"], bufs["lse"], ws=ws)
    out2, lse2 = g.attend(2, tk1, tc1)
    torch.cuda.synchronize()
    _same(bufs["out"], out2, f"{name} reuse out")
    _same(bufs["lse"], lse2, f"{name} reuse lse")
    # a Reuse layer against the oracle: a fresh main query (layer 2) over an
    # inherited Top-K, here the oracle's Top-K of the Reindex layer (layer 1)
    tk_o, tc_o = with_oracle_rows(tk1, tc1, keep1)
    bufs["out"].fill_(3.0)
    csa2.decode_step(g.dims, g.batch, csa2.LAYER_REUSE, None, None, None, bufs["pool_blocks"], bufs["pool_count"],
                     tk_o, tc_o, ql, qr, 1.0, codes, scales, kv_rope, swa_kv, g.swa_base, bufs["out"], bufs["lse"],
                     ws=ws)
    torch.cuda.synchronize()
    for qi in range(n_q):
        ro, rl = oqs[qi].attention(2, keep1[qi])
        check_attention(bufs["out"][qi].cpu().numpy(), bufs["lse"][qi].cpu().numpy(), ro, rl, f"{name} q{qi} reuse")
    # the step leaves the Reindex completion counters in its workspace at
    # zero: a second Reindex layer on the same workspace selects the same set
    # (with a counter left nonzero no workgroup would see itself last)
    _step(g, csa2.LAYER_REINDEX, 1, bufs, ws)
    torch.cuda.synchronize()
    _same(bufs["topk_pos"], tk1, f"{name} reindex again topk")
    _same(bufs["topk_count"], tc1, f"{name} reindex again count")


@pytest.mark.parametrize("name", ["ragged_b3", "fp4_ragged_b3"])
def test_step_graph_replays(name):
    """A Full layer captured into a HIP graph: every replay (with eager work
    and a synchronisation between replays, outputs overwritten before each)
    reproduces the eager outputs bit for bit."""
    lib()
    w = CASES[name]
    g = GpuCase(w)
    csa2 = g.csa2
    ws = torch.zeros(csa2.workspace_step(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    eager = _buffers(g)
    _step(g, csa2.LAYER_FULL, 0, eager, ws)
    torch.cuda.synchronize()
    bufs = _buffers(g)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the binding's host path on the capture stream
        _step(g, csa2.LAYER_FULL, 0, bufs, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(g, csa2.LAYER_FULL, 0, bufs, ws)
    for rep in range(4):
        for t in bufs.values():
            t.fill_(5)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key in eager:
            if key == "pool_blocks":
                for qi in range(w.n_q):
                    k = int(eager["pool_count"][qi])
                    _same(bufs[key][qi, :k], eager[key][qi, :k], f"{name} replay {rep} pool q{qi}")
            else:
                _same(bufs[key], eager[key], f"{name} replay {rep} {key}")
    del graph
