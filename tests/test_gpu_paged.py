"""GPU parity of the paged caches (csa2_pages): the same rows scattered into
pages in a shuffled physical order give the contiguous path's outputs bit
for bit (Reindex Top-K sets and scores, attention outputs and LSE), the
contiguous path being the one checked against the oracle elsewhere; one
query per case is also checked against the oracle directly.
csa2_page_rows + csa2_encode_kv append fresh entries into their pages
with the contiguous encoder's bytes."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests._harness import GpuCase, OracleQuery, check_attention, check_set, with_oracle_pool, with_oracle_rows
from tests.test_gpu_parity import BIG, small

pytestmark = pytest.mark.gpu

CASES = {
    "ragged_b3_p64": (small(201, BIG, [20005, 9003, 4099]), 64),
    "fp4_ragged_b3_p256": (small(202, BIG, [20005, 9003, 4099], fp4=True), 256),
    "edge_short_p16": (small(203, wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=4, topk=16),
                             [0, 1, 100, 128, 129, 136, 137, 160]), 16),
    "g4_p128": (small(204, BIG, [6001, 12345], g=4), 128),
    # a long query (the group-key selection) beside a short one
    "long_p64": (small(206, wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=2048, topk=512),
                       [300000, 5000]), 64),
    "kvg32_p32": (small(205, wl.Dims(n_heads=32, idx_heads=8, idx_dim=64, pool_blocks=64, topk=128, kv_group=32),
                        [7777, 3000]), 32),
}


class Paged:
    """Every per-position plane of a case with each sequence's rows in pages
    of `ps` positions at shuffled physical pages (with unused pages between
    them), the page table, and a batch whose seq_base holds table offsets."""

    def __init__(self, g, ps: int, seed: int):
        csa2, lay, w = g.csa2, g.lay, g.w
        rng = np.random.default_rng(seed)
        npg = [-(-r // ps) for r in lay.seq_rows]
        total = sum(npg) + 7                      # a few pages no sequence uses
        perm = rng.permutation(total).astype(np.int32)
        table, off, k = [], [], 0
        for n in npg:
            off.append(len(table))
            table.extend(perm[k:k + n])
            k += n
        table.append(0)                           # a table of at least one entry
        self.ps, self.rows = ps, total * ps
        self.table = torch.tensor(np.asarray(table, np.int32), device=g.dev)
        # physical row of every logical row of the flat layout
        src, dst = [], []
        for s, r in enumerate(lay.seq_rows):
            p = np.arange(r, dtype=np.int64)
            phys = np.asarray(table, np.int64)[off[s] + p // ps] * ps + p % ps
            src.append(lay.seq_base[s] + p)
            dst.append(phys)
        src = torch.tensor(np.concatenate(src), device=g.dev)
        dst = torch.tensor(np.concatenate(dst), device=g.dev)

        def scatter(t):
            out = torch.zeros((self.rows,) + tuple(t.shape[1:]), dtype=t.dtype, device=g.dev)
            if len(src):
                out.view(torch.uint8).view(self.rows, -1)[dst] = t.view(torch.uint8).view(t.shape[0], -1)[src]
            return out

        idx_k, codes, scales, kv_rope, _ = g.planes[0]
        self.idx_k = tuple(scatter(x) for x in idx_k) if isinstance(idx_k, tuple) else scatter(idx_k)
        self.codes, self.scales, self.kv_rope = scatter(codes), scatter(scales), scatter(kv_rope)
        q_off = [off[qi // w.tokens_per_seq] for qi in range(w.n_q)]
        self.batch = csa2.Batch(torch.tensor(q_off, dtype=torch.int64, device=g.dev), g.batch.n_visible,
                                g.batch.max_visible, g.batch.tokens_per_seq)
        self.pages = csa2.Pages(self.table, ps, self.rows)
        self.seq_off = off


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    w, ps = CASES[request.param]
    g = GpuCase(w)
    return request.param, g, Paged(g, ps, seed=ps + len(request.param))


def test_paged_reindex_and_attention_match_contiguous(case):
    name, g, pg = case
    csa2, w = g.csa2, g.w
    pool, cnt, _ = g.full(0)
    q, wt = g.iq(0)
    ts = torch.empty(w.n_q, w.dims.topk, dtype=torch.float32, device="cuda")
    tk, tc = csa2.index_reindex(g.dims, g.batch, q, wt, g.planes[0][0], pool, cnt, topk_scores=ts)
    ts2 = torch.empty_like(ts)
    tk2, tc2 = csa2.index_reindex(g.dims, pg.batch, q, wt, pg.idx_k, pool, cnt, topk_scores=ts2, pages=pg.pages)
    ql, qr = g.mq(0)
    _, codes, scales, kv_rope, swa_kv = g.planes[0]
    out, lse = csa2.attend(g.dims, g.batch, ql, qr, 1.0, codes, scales, kv_rope, tk, tc, swa_kv, g.swa_base)
    out2, lse2 = csa2.attend(g.dims, pg.batch, ql, qr, 1.0, pg.codes, pg.scales, pg.kv_rope, tk, tc, swa_kv,
                             g.swa_base, pages=pg.pages)
    torch.cuda.synchronize()
    assert torch.equal(tc2, tc), f"{name}: paged Top-K counts differ"
    for qi in range(w.n_q):
        k = int(tc[qi])
        assert torch.equal(tk2[qi, :k], tk[qi, :k]), f"{name} q{qi}: paged Top-K differs"
        assert torch.equal(ts2[qi, :k].view(torch.int32), ts[qi, :k].view(torch.int32)), \
            f"{name} q{qi}: paged Top-K scores differ"
    assert torch.equal(out2.view(torch.int32), out.view(torch.int32)), f"{name}: paged attention output differs"
    assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32)), f"{name}: paged LSE differs"

    # the oracle, on the query with the longest context
    qi = int(np.argmax(g.lay.q_visible))
    oq = OracleQuery(w, g.lay, qi)
    rpool, rb, _ = oq.full(0)
    check_set(pool.cpu().numpy()[qi, :int(cnt[qi])], rpool, lambda j: rb[j], f"{name} pool")
    keep, _, _ = oq.reindex(0, rpool)
    got = tk2.cpu().numpy()[qi, :int(tc2[qi])]
    same_pool = np.array_equal(pool.cpu().numpy()[qi, :int(cnt[qi])], rpool)
    if not same_pool:
        # pools that differ inside the band: the paged Reindex on the oracle's pool
        p3, c3 = with_oracle_pool(pool, cnt, {qi: rpool})
        tk2, tc2 = csa2.index_reindex(g.dims, pg.batch, q, wt, pg.idx_k, p3, c3, pages=pg.pages)
        torch.cuda.synchronize()
        got = tk2.cpu().numpy()[qi, :int(tc2[qi])]
    check_set(got, keep, lambda x: oq.scores_at(0, x), f"{name} paged topk")
    ref_o, ref_l = oq.attention(0, keep)
    if not same_pool or not np.array_equal(got, keep):
        # the paged attention on the oracle's own Top-K
        tk3, tc3 = with_oracle_rows(tk2, tc2, {qi: keep})
        out2, lse2 = csa2.attend(g.dims, pg.batch, ql, qr, 1.0, pg.codes, pg.scales, pg.kv_rope, tk3, tc3, swa_kv,
                                 g.swa_base, pages=pg.pages)
        torch.cuda.synchronize()
    check_attention(out2.cpu().numpy()[qi], lse2.cpu().numpy()[qi], ref_o, ref_l, f"{name} paged attention")


def test_page_rows_append_into_pages(case):
    """Fresh entries encoded at the rows csa2_page_rows gives land in their
    pages byte for byte as the contiguous encoder writes them."""
    name, g, pg = case
    csa2, lay = g.csa2, g.lay
    rng = np.random.default_rng(7)
    seqs = [s for s, r in enumerate(lay.seq_rows) if r > 0]
    if not seqs:
        pytest.skip("no rows")
    n = 300
    s_of = rng.choice(seqs, n)
    pos = np.array([rng.integers(0, lay.seq_rows[s]) for s in s_of], np.int32)
    # one entry per (sequence, position): the writes must not overlap
    _, keep = np.unique(s_of.astype(np.int64) * (1 << 32) + pos, return_index=True)
    s_of, pos = s_of[keep], pos[keep]
    table_off = torch.tensor([pg.seq_off[s] for s in s_of], dtype=torch.int64, device="cuda")
    pos_t = torch.tensor(pos, device="cuda")
    rows = csa2.page_rows(pg.pages, table_off, pos_t)
    table = pg.table.cpu().numpy().astype(np.int64)
    want = table[np.array([pg.seq_off[s] for s in s_of]) + pos // pg.ps] * pg.ps + pos % pg.ps
    assert np.array_equal(rows.cpu().numpy(), want), f"{name}: page rows differ"
    m = len(pos)
    lat = wl.fresh_latent(g.w, 0, 0, m, "cuda")
    rope = wl.fresh_rope(g.w, 0, 0, m, "cuda")
    grp = g.w.dims.kv_group
    codes = pg.codes.clone()
    scales = pg.scales.clone()
    kv_rope = pg.kv_rope.clone()
    csa2.encode_kv(lat, rope, codes, scales, kv_rope, dst_row=rows, group=grp)
    ref = (torch.zeros(m, 256, dtype=torch.uint8, device="cuda"),
           torch.zeros(m, 512 // grp, dtype=torch.uint8, device="cuda"),
           torch.zeros(m, 64, dtype=torch.bfloat16, device="cuda"))
    csa2.encode_kv(lat, rope, *ref, group=grp)
    torch.cuda.synchronize()
    assert torch.equal(codes[rows], ref[0]), f"{name}: appended codes differ"
    assert torch.equal(scales[rows], ref[1]), f"{name}: appended scales differ"
    assert torch.equal(kv_rope[rows].view(torch.int16), ref[2].view(torch.int16)), f"{name}: appended rope differs"
    untouched = torch.ones(pg.rows, dtype=torch.bool, device="cuda")
    untouched[rows] = False
    assert torch.equal(codes[untouched], pg.codes[untouched]), f"{name}: rows outside the appended ones changed"


def test_paged_full_index_matches_contiguous(case):
    """csa2_index_full_paged: the scan reads each tile's keys through the
    page table; block scores and pool equal the contiguous call's bit for
    bit (twice in a row on one workspace)."""
    name, g, pg = case
    csa2, w = g.csa2, g.w
    q, wt = g.iq(0)
    ld = csa2.block_scores_ld(g.dims, g.batch)
    bs = torch.full((w.n_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    bs2 = torch.full_like(bs, float("nan"))
    pool, cnt = csa2.index_full(g.dims, g.batch, q, wt, g.planes[0][0], block_scores=bs)
    ws = torch.zeros(csa2.workspace_full(g.dims, pg.batch) + 256, dtype=torch.uint8, device="cuda")
    outs = [csa2.index_full(g.dims, pg.batch, q, wt, pg.idx_k, block_scores=bs2, ws=ws, pages=pg.pages)
            for _ in range(2)]
    torch.cuda.synchronize()
    for qi in range(w.n_q):
        k = max(0, -(-(g.lay.q_visible[qi] - w.dims.swa) // 8))
        assert torch.equal(bs2[qi, :k].view(torch.int32), bs[qi, :k].view(torch.int32)), \
            f"{name} q{qi}: paged block scores differ"
    for p2, c2 in outs:
        assert torch.equal(c2, cnt), f"{name}: paged pool counts differ"
        for qi in range(w.n_q):
            k = int(cnt[qi])
            assert torch.equal(p2[qi, :k], pool[qi, :k]), f"{name} q{qi}: paged pool differs"


def test_paged_decode_step_matches_contiguous(case):
    """csa2_decode_step_paged (Full layer: paged scan, Reindex and attention)
    writes the contiguous step's pool, Top-K, outputs and LSE bit for bit."""
    name, g, pg = case
    csa2, w, d = g.csa2, g.w, g.w.dims
    n_q = w.n_q
    q, wt = g.iq(0)
    ql, qr = g.mq(0)
    _, codes, scales, kv_rope, swa_kv = g.planes[0]

    def bufs():
        return dict(pool_blocks=torch.empty(n_q, d.pool_blocks, dtype=torch.int32, device="cuda"),
                    pool_count=torch.empty(n_q, dtype=torch.int32, device="cuda"),
                    topk_pos=torch.empty(n_q, d.topk, dtype=torch.int32, device="cuda"),
                    topk_count=torch.empty(n_q, dtype=torch.int32, device="cuda"),
                    out=torch.empty(n_q, d.n_heads, 512, dtype=torch.float32, device="cuda"),
                    lse=torch.empty(n_q, d.n_heads, dtype=torch.float32, device="cuda"))

    a, b = bufs(), bufs()
    csa2.decode_step(g.dims, g.batch, csa2.LAYER_FULL, q, wt, g.planes[0][0], a["pool_blocks"], a["pool_count"],
                     a["topk_pos"], a["topk_count"], ql, qr, 1.0, codes, scales, kv_rope, swa_kv, g.swa_base,
                     a["out"], a["lse"])
    csa2.decode_step(g.dims, pg.batch, csa2.LAYER_FULL, q, wt, pg.idx_k, b["pool_blocks"], b["pool_count"],
                     b["topk_pos"], b["topk_count"], ql, qr, 1.0, pg.codes, pg.scales, pg.kv_rope, swa_kv,
                     g.swa_base, b["out"], b["lse"], pages=pg.pages)
    torch.cuda.synchronize()
    assert torch.equal(b["pool_count"], a["pool_count"]) and torch.equal(b["topk_count"], a["topk_count"])
    for qi in range(n_q):
        k = int(a["pool_count"][qi])
        assert torch.equal(b["pool_blocks"][qi, :k], a["pool_blocks"][qi, :k]), f"{name} q{qi}: step pool differs"
        k = int(a["topk_count"][qi])
        assert torch.equal(b["topk_pos"][qi, :k], a["topk_pos"][qi, :k]), f"{name} q{qi}: step Top-K differs"
    assert torch.equal(b["out"].view(torch.int32), a["out"].view(torch.int32)), f"{name}: step output differs"
    assert torch.equal(b["lse"].view(torch.int32), a["lse"].view(torch.int32)), f"{name}: step LSE differs"


def test_paged_reindex_step_matches_contiguous(case):
    """csa2_decode_step_paged in Reindex mode (the Reindex keys scored
    through the page table, the Top-K selected inside the attention kernel)
    writes the contiguous Reindex step's Top-K, outputs and LSE bit for bit,
    on the pool of a contiguous Full step."""
    name, g, pg = case
    csa2, w, d = g.csa2, g.w, g.w.dims
    n_q = w.n_q
    q, wt = g.iq(0)
    ql, qr = g.mq(0)
    _, codes, scales, kv_rope, swa_kv = g.planes[0]

    def bufs():
        return dict(topk_pos=torch.empty(n_q, d.topk, dtype=torch.int32, device="cuda"),
                    topk_count=torch.empty(n_q, dtype=torch.int32, device="cuda"),
                    out=torch.empty(n_q, d.n_heads, 512, dtype=torch.float32, device="cuda"),
                    lse=torch.empty(n_q, d.n_heads, dtype=torch.float32, device="cuda"))

    pool = torch.empty(n_q, d.pool_blocks, dtype=torch.int32, device="cuda")
    cnt = torch.empty(n_q, dtype=torch.int32, device="cuda")
    f = bufs()
    csa2.decode_step(g.dims, g.batch, csa2.LAYER_FULL, q, wt, g.planes[0][0], pool, cnt, f["topk_pos"],
                     f["topk_count"], ql, qr, 1.0, codes, scales, kv_rope, swa_kv, g.swa_base, f["out"], f["lse"])
    q1, w1 = g.iq(1)
    ql1, qr1 = g.mq(1)
    a, b = bufs(), bufs()
    csa2.decode_step(g.dims, g.batch, csa2.LAYER_REINDEX, q1, w1, g.planes[0][0], pool, cnt, a["topk_pos"],
                     a["topk_count"], ql1, qr1, 1.0, codes, scales, kv_rope, swa_kv, g.swa_base, a["out"], a["lse"])
    csa2.decode_step(g.dims, pg.batch, csa2.LAYER_REINDEX, q1, w1, pg.idx_k, pool, cnt, b["topk_pos"],
                     b["topk_count"], ql1, qr1, 1.0, pg.codes, pg.scales, pg.kv_rope, swa_kv, g.swa_base,
                     b["out"], b["lse"], pages=pg.pages)
    torch.cuda.synchronize()
    assert torch.equal(b["topk_count"], a["topk_count"]), f"{name}: Reindex Top-K counts differ"
    for qi in range(n_q):
        k = int(a["topk_count"][qi])
        assert torch.equal(b["topk_pos"][qi, :k], a["topk_pos"][qi, :k]), f"{name} q{qi}: Reindex Top-K differs"
    assert torch.equal(b["out"].view(torch.int32), a["out"].view(torch.int32)), f"{name}: Reindex output differs"
    assert torch.equal(b["lse"].view(torch.int32), a["lse"].view(torch.int32)), f"{name}: Reindex LSE differs"


def test_paged_step_graph_replays(case):
    """csa2_decode_step_paged (Full layer) captured into a HIP graph: every
    replay, with eager work and a synchronisation between replays and the
    outputs overwritten before each, reproduces the eager outputs bit for
    bit (the paged calls enqueue no memset and allocate nothing)."""
    name, g, pg = case
    csa2, w, d = g.csa2, g.w, g.w.dims
    n_q = w.n_q
    q, wt = g.iq(0)
    ql, qr = g.mq(0)
    swa_kv = g.planes[0][4]
    ws = torch.zeros(csa2.workspace_step(g.dims, pg.batch) + 256, dtype=torch.uint8, device="cuda")

    def bufs():
        return dict(pool_blocks=torch.full((n_q, d.pool_blocks), 7, dtype=torch.int32, device="cuda"),
                    pool_count=torch.full((n_q,), 7, dtype=torch.int32, device="cuda"),
                    topk_pos=torch.full((n_q, d.topk), 7, dtype=torch.int32, device="cuda"),
                    topk_count=torch.full((n_q,), 7, dtype=torch.int32, device="cuda"),
                    out=torch.full((n_q, d.n_heads, 512), 7.0, dtype=torch.float32, device="cuda"),
                    lse=torch.full((n_q, d.n_heads), 7.0, dtype=torch.float32, device="cuda"))

    def step(b):
        csa2.decode_step(g.dims, pg.batch, csa2.LAYER_FULL, q, wt, pg.idx_k, b["pool_blocks"], b["pool_count"],
                         b["topk_pos"], b["topk_count"], ql, qr, 1.0, pg.codes, pg.scales, pg.kv_rope, swa_kv,
                         g.swa_base, b["out"], b["lse"], ws=ws, pages=pg.pages)

    eager = bufs()
    step(eager)
    torch.cuda.synchronize()
    b = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the binding's host path on the capture stream
        step(b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(b)
    for rep in range(4):
        for t in b.values():
            t.fill_(5)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key in eager:
            if key in ("pool_blocks", "topk_pos"):
                cnt = eager["pool_count" if key == "pool_blocks" else "topk_count"]
                for qi in range(n_q):
                    k = int(cnt[qi])
                    assert torch.equal(b[key][qi, :k], eager[key][qi, :k]), f"{name} replay {rep} {key} q{qi}"
            else:
                x, y = b[key], eager[key]
                if x.dtype == torch.float32:
                    x, y = x.view(torch.int32), y.view(torch.int32)
                assert torch.equal(x, y), f"{name} replay {rep} {key}"
    del graph
