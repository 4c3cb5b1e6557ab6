"""GPU parity: the HIP library against the oracle on the same seeded inputs.

Bars: FP4 bytes bit-exact; index sets equal except within a 1e-5 relative
score band around the k-th score (ties to the lower index); indexer scores
within 1e-3 relative; attention within 2e-3 of max|ref| per (query, head).
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._harness import (GpuCase, OracleQuery, check_attention, check_set, lib, u8, u16,
                            SCORE_TOL, with_oracle_rows)

pytestmark = pytest.mark.gpu

BIG = wl.Dims(n_heads=64, idx_heads=64, idx_dim=128, pool_blocks=256, topk=512)


def small(idx, dims, ctx_list, g=1, name="small", fp4=False):
    ns = len(ctx_list)
    return wl.Workload(idx, name, dims, n_seq=ns, ctx=(0, 0), tokens_per_seq=g, ctx_list=tuple(ctx_list),
                       idx_fp4=fp4)


# several scan tiles (2048 positions) with ragged tails, several queries
CASES = {
    "tiny_c0": wl.workload(0),
    "ragged_b3": small(101, BIG, [20005, 9000 + 3, 4099]),
    "ragged_g4": small(102, BIG, [6001, 12345], g=4),
    "d64_h8": small(103, wl.Dims(n_heads=16, idx_heads=8, idx_dim=64, pool_blocks=64, topk=128), [7777, 300]),
    "h_odd": small(104, wl.Dims(n_heads=32, idx_heads=40, idx_dim=128, pool_blocks=100, topk=300, swa=64), [5000, 2001]),
    "edge_short": small(105, wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=4, topk=16),
                        [0, 1, 100, 128, 129, 136, 137, 160]),
    "w0_h128": small(106, wl.Dims(n_heads=128, idx_heads=1, idx_dim=128, pool_blocks=32, topk=64, swa=0), [3000]),
    # head counts that are multiples of 8 but not of 16 (padded head blocks)
    "h24_ragged": small(108, wl.Dims(n_heads=24, idx_heads=64, idx_dim=128, pool_blocks=200, topk=400),
                        [12000, 5003]),
    "h8_d64": small(109, wl.Dims(n_heads=8, idx_heads=8, idx_dim=64, pool_blocks=16, topk=64), [700, 129, 2050]),
    "max_pk": small(107, wl.Dims(n_heads=64, idx_heads=64, idx_dim=128, pool_blocks=2048, topk=2048, swa=1024),
                    [40000, 17000]),
    # FP4 indexer rows (codes + one E4M3 scale per 16 channels, d_i = 128)
    "fp4_ragged_b3": small(121, BIG, [20005, 9003, 4099], fp4=True),
    "fp4_ragged_g4": small(122, BIG, [6001, 12345], g=4, fp4=True),
    "fp4_h_odd": small(123, wl.Dims(n_heads=32, idx_heads=40, idx_dim=128, pool_blocks=100, topk=300, swa=64),
                       [5000, 2001], fp4=True),
    "fp4_edge_short": small(124, wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=4, topk=16),
                            [0, 1, 100, 128, 129, 136, 137, 160], fp4=True),
    "fp4_w0_h1": small(125, wl.Dims(n_heads=16, idx_heads=1, idx_dim=128, pool_blocks=32, topk=64, swa=0),
                       [3000], fp4=True),
    # 16 query tokens of one sequence (a chunk scored against one key stream)
    "chunk_g16": small(141, BIG, [9000], g=16),
    # two and four sequences whose scan tiles (2048 positions) split evenly
    # over their XCDs: each XCD takes contiguous runs of one sequence's tiles
    "xcd_runs_b2": small(151, BIG, [65536 + 128, 30000]),
    "xcd_runs_b4": small(152, BIG, [32768 + 128, 20000, 5001, 32768 + 100]),
    # the group-32 main-KV codec (one E4M3 scale per 32 latent channels)
    "kvg32_ragged_b3": small(131, dataclasses.replace(BIG, kv_group=32), [20005, 9003, 4099]),
    "kvg32_edge_short": small(132, wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=4, topk=16,
                                           kv_group=32), [0, 1, 100, 128, 129, 136, 137, 160]),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    w = CASES[request.param]
    return request.param, GpuCase(w), wl.layout(w)


def _oq(w, lay, keys_cache, qi):
    s = lay.q_seq_base[qi]
    oq = OracleQuery(w, lay, qi, keys_cache.get(s))
    keys_cache.setdefault(s, oq.keys)
    return oq


@pytest.mark.parametrize("group", [16, 32])
def test_encode_bit_exact_generated(group):
    csa2 = lib()
    w = wl.workload(4)
    n = 4096 + 37
    lat, rp = wl.fresh_latent(w, 0, 0, n, "cuda"), wl.fresh_rope(w, 0, 0, n, "cuda")
    rows = 3 * n
    perm = torch.randperm(rows, generator=torch.Generator().manual_seed(5))[:n].to("cuda")
    codes = torch.zeros(rows, 256, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(rows, 512 // group, dtype=torch.uint8, device="cuda")
    kr = torch.zeros(rows, 64, dtype=torch.bfloat16, device="cuda")
    csa2.encode_kv(lat, rp, codes, scales, kr, dst_row=perm, group=group)
    torch.cuda.synchronize()
    rc, rs = oracle.encode_kv(u16(wl.fresh_latent(w, 0, 0, n)), group)
    p = perm.cpu().numpy()
    assert np.array_equal(u8(codes)[p], rc)
    assert np.array_equal(u8(scales)[p], rs)
    assert np.array_equal(u16(kr)[p], u16(wl.fresh_rope(w, 0, 0, n)))
    untouched = np.setdiff1d(np.arange(rows), p)
    assert not u8(codes)[untouched].any()


def _exhaustive_groups():
    """Groups [6s, x1..x15] for every positive finite E4M3 scale s and every
    finite bf16 x with |x| <= 6s, plus degenerate groups."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_to_f64(b)
    fin = np.isfinite(v)
    b, v = b[fin], v[fin]
    groups = []
    for sc in range(1, 0x7F):
        s = float(oracle.e4m3_decode(sc))
        xb = b[np.abs(v) <= 6 * s]
        ng = -(-len(xb) // 15)
        flat = np.zeros(ng * 15, np.uint16)
        flat[:len(xb)] = xb
        g = np.zeros((ng, 16), np.uint16)
        g[:, 0] = (np.array([6 * s], np.float32).view(np.uint32) >> 16).astype(np.uint16)
        g[:, 1:] = flat.reshape(ng, 15)
        groups.append(g)
    def bf(x):
        return (np.array(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    deg = np.zeros((6, 16), np.uint16)
    deg[1, :2] = bf([-1e-6, 1e-6])                       # scale rounds to 0
    deg[2, :2] = bf([-1.0, -0.01])                       # -0 code for small negatives
    deg[3, :2] = bf([1e4, -3000.0])                      # scale clamps at 448, saturates
    deg[4, :3] = bf([6.375, 1.0625, -0.03125])           # scale tie 1.0625 -> 1.0
    deg[5, :] = bf(np.linspace(-2688, 2688, 16))
    groups.append(deg)
    allg = np.concatenate(groups)
    rows = -(-len(allg) // 32)
    out = np.zeros((rows * 32, 16), np.uint16)
    out[:len(allg)] = allg
    return out.reshape(rows, 512)


@pytest.mark.parametrize("group", [16, 32])
def test_encode_exhaustive_scales_and_values(group):
    csa2 = lib()
    lat = _exhaustive_groups()
    n = lat.shape[0]
    rc, rs = oracle.encode_kv(lat, group)
    t = torch.from_numpy(lat.astype(np.int16)).view(torch.bfloat16).to("cuda")
    rp = torch.zeros(n, 64, dtype=torch.bfloat16, device="cuda")
    codes = torch.empty(n, 256, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n, 512 // group, dtype=torch.uint8, device="cuda")
    kr = torch.empty(n, 64, dtype=torch.bfloat16, device="cuda")
    csa2.encode_kv(t, rp, codes, scales, kr, group=group)
    torch.cuda.synchronize()
    assert np.array_equal(u8(scales), rs)
    bad = np.argwhere(u8(codes) != rc)
    assert len(bad) == 0, f"{len(bad)} code bytes differ, first rows {bad[:5]}"


@pytest.mark.parametrize("width,n", [(128, 4096 + 37), (16, 1000), (512, 777), (1024, 300)])
def test_encode_fp4_rows_bit_exact(width, n):
    """csa2_encode_fp4 against the oracle's row codec, scattered rows."""
    csa2 = lib()
    w = wl.workload(6)
    src = wl.idx_keys_bf16(w, 0, n * width // 128 + 1, "cuda").view(-1)[:n * width].view(n, width).contiguous()
    rows = 2 * n
    perm = torch.randperm(rows, generator=torch.Generator().manual_seed(width))[:n].to("cuda")
    codes = torch.zeros(rows, width // 2, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(rows, width // 16, dtype=torch.uint8, device="cuda")
    csa2.encode_fp4(src, codes, scales, dst_row=perm)
    torch.cuda.synchronize()
    rc, rs = oracle.encode_fp4(u16(src))
    p = perm.cpu().numpy()
    assert np.array_equal(u8(codes)[p], rc)
    assert np.array_equal(u8(scales)[p], rs)
    untouched = np.setdiff1d(np.arange(rows), p)
    assert not u8(codes)[untouched].any() and not u8(scales)[untouched].any()


def test_encode_fp4_exhaustive_groups_width_128():
    """Every (E4M3 scale, bf16 value) group of the main-KV exhaustive test,
    as 128-wide rows."""
    csa2 = lib()
    rows = _exhaustive_groups().reshape(-1, 128)
    n = rows.shape[0]
    rc, rs = oracle.encode_fp4(rows)
    t = torch.from_numpy(rows.astype(np.int16)).view(torch.bfloat16).to("cuda")
    codes = torch.empty(n, 64, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n, 8, dtype=torch.uint8, device="cuda")
    csa2.encode_fp4(t, codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(u8(scales), rs)
    assert np.array_equal(u8(codes), rc)


def test_full_index(case):
    name, g, lay = case
    w = g.w
    pool, cnt, bs = g.full(0, block_scores=True)
    torch.cuda.synchronize()
    pool, cnt, bs = pool.cpu().numpy(), cnt.cpu().numpy(), bs.cpu().numpy()
    kc = {}
    for qi in range(w.n_q):
        oq = _oq(w, lay, kc, qi)
        rpool, rb, _ = oq.full(0)
        nb = len(rb)
        assert cnt[qi] == len(rpool), f"{name} q{qi}: pool count {cnt[qi]} != {len(rpool)}"
        assert np.all(pool[qi, cnt[qi]:] == -1)
        if nb:
            got_b = bs[qi, :nb].astype(np.float64)
            tol = SCORE_TOL * np.maximum(np.abs(rb), 1e-3 * np.abs(rb).max())
            assert np.all(np.abs(got_b - rb) <= tol), f"{name} q{qi}: block scores off by {np.abs(got_b - rb).max()}"
        check_set(pool[qi, :cnt[qi]], rpool, lambda j: rb[j], f"{name} q{qi} pool")


def test_reindex_on_oracle_pool(case):
    name, g, lay = case
    w = g.w
    kc = {}
    P = w.dims.pool_blocks
    pools = np.full((w.n_q, P), -1, np.int32)
    cnts = np.zeros(w.n_q, np.int32)
    oqs = []
    for qi in range(w.n_q):
        oq = _oq(w, lay, kc, qi)
        rpool, _, _ = oq.full(0)
        pools[qi, :len(rpool)] = rpool
        cnts[qi] = len(rpool)
        oqs.append((oq, rpool))
    layer = 1 if w.reindex_layers > 1 else 0
    tk, tc, ts = g.reindex(layer, torch.from_numpy(pools).cuda(), torch.from_numpy(cnts).cuda(), scores=True)
    torch.cuda.synchronize()
    tk, tc, ts = tk.cpu().numpy(), tc.cpu().numpy(), ts.cpu().numpy()
    for qi, (oq, rpool) in enumerate(oqs):
        keep, s, R = oq.reindex(layer, rpool)
        assert tc[qi] == len(keep), f"{name} q{qi}: topk count {tc[qi]} != {len(keep)}"
        got = tk[qi, :tc[qi]]
        assert np.all(tk[qi, tc[qi]:] == -1)
        assert set(got.tolist()) <= set(R.tolist()), f"{name} q{qi}: selection outside the pool"
        check_set(got, keep, lambda p: oq.scores_at(layer, p), f"{name} q{qi} topk")
        if tc[qi]:
            ref = oq.scores_at(layer, got)
            assert np.allclose(ts[qi, :tc[qi]], ref, rtol=SCORE_TOL, atol=1e-6 * np.abs(ref).max())


def test_attention_on_oracle_topk(case):
    name, g, lay = case
    w = g.w
    K = w.dims.topk
    kc = {}
    tks = np.full((w.n_q, K), -1, np.int32)
    tcs = np.zeros(w.n_q, np.int32)
    refs = []
    layer = 1 if w.reindex_layers > 1 else 0
    for qi in range(w.n_q):
        oq = _oq(w, lay, kc, qi)
        rpool, _, _ = oq.full(0)
        keep, _, _ = oq.reindex(layer, rpool)
        tks[qi, :len(keep)] = keep
        tcs[qi] = len(keep)
        refs.append(oq.attention(layer, keep))
    out, lse = g.attend(layer, torch.from_numpy(tks).cuda(), torch.from_numpy(tcs).cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for qi in range(w.n_q):
        check_attention(out[qi], lse[qi], refs[qi][0], refs[qi][1], f"{name} q{qi}")


def test_full_topk_from_scan_keys_matches_reindex(case):
    """A Full layer's Top-K selected from the scan's own position scores
    (csa2_index_scan_keys + csa2_index_topk_keys) is csa2_index_reindex with
    the same query, bit for bit: the same positions, counts and scores; and
    the scan's block scores are unchanged by keeping the position scores."""
    name, g, lay = case
    csa2, w = g.csa2, g.w
    q, wt = g.iq(0)
    idx_k = g.planes[0][0]
    ld = csa2.block_scores_ld(g.dims, g.batch)
    bs = torch.full((w.n_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    pk = torch.full((w.n_q, csa2.pos_keys_ld(g.dims, g.batch)), -1, dtype=torch.int32, device="cuda")
    pws = torch.empty(csa2.workspace_pool(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    csa2.index_scan(g.dims, g.batch, q, wt, idx_k, bs, pool_ws=pws, pos_keys=pk)
    pool, cnt = csa2.index_pool(g.dims, g.batch, bs, ws=pws, from_scan=True)
    ts = torch.empty(w.n_q, w.dims.topk, dtype=torch.float32, device="cuda")
    tk, tc = csa2.index_topk_keys(g.dims, g.batch, pool, cnt, bs, pk, topk_scores=ts)
    ts2 = torch.empty_like(ts)
    tk2, tc2 = csa2.index_reindex(g.dims, g.batch, q, wt, idx_k, pool, cnt, topk_scores=ts2)
    bs2 = torch.full_like(bs, float("nan"))
    csa2.index_scan(g.dims, g.batch, q, wt, idx_k, bs2)
    torch.cuda.synchronize()
    assert torch.equal(tc, tc2), f"{name}: Top-K counts differ from Reindex"
    for qi in range(w.n_q):
        k = int(tc[qi])
        assert torch.equal(tk[qi, :k], tk2[qi, :k]), f"{name} q{qi}: Top-K differs from Reindex"
        assert torch.equal(ts[qi, :k].view(torch.int32), ts2[qi, :k].view(torch.int32)), \
            f"{name} q{qi}: Top-K scores differ from Reindex"
        assert bool((tk[qi, k:] == -1).all())
        nb = -(-max(0, lay.q_visible[qi] - w.dims.swa) // 8)
        assert torch.equal(bs[qi, :nb].view(torch.int32), bs2[qi, :nb].view(torch.int32)), \
            f"{name} q{qi}: block scores differ with position keys kept"


@pytest.mark.parametrize("tile", ["2048", "128"])
def test_scan_tile_independent(case, tile, monkeypatch):
    """The scan's tile (2048 positions, halved down to 128 for launches of
    few workgroups; forced here with CSA2_SCAN_TILE) changes neither the block
    scores, the position keys, nor the pool selected after the scan from its
    key ranges: each position's score is the same contraction whatever tile
    holds it."""
    name, g, lay = case
    csa2, w = g.csa2, g.w
    q, wt = g.iq(0)
    idx_k = g.planes[0][0]

    def run():
        bs = torch.zeros(w.n_q, csa2.block_scores_ld(g.dims, g.batch), dtype=torch.float32, device="cuda")
        pk = torch.zeros(w.n_q, csa2.pos_keys_ld(g.dims, g.batch), dtype=torch.int32, device="cuda")
        pws = torch.zeros(csa2.workspace_pool(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
        csa2.index_scan(g.dims, g.batch, q, wt, idx_k, bs, pool_ws=pws, pos_keys=pk)
        pool, cnt = csa2.index_pool(g.dims, g.batch, bs, ws=pws, from_scan=True)
        torch.cuda.synchronize()
        return bs.cpu(), pk.cpu(), pool.cpu(), cnt.cpu()

    bs, pk, pool, cnt = run()
    monkeypatch.setenv("CSA2_SCAN_TILE", tile)
    bs2, pk2, pool2, cnt2 = run()
    assert torch.equal(cnt, cnt2), f"{name}: pool counts differ with tile {tile}"
    for qi in range(w.n_q):
        c = max(0, lay.q_visible[qi] - w.dims.swa)
        nb = -(-c // 8)
        assert torch.equal(bs[qi, :nb].view(torch.int32), bs2[qi, :nb].view(torch.int32)), \
            f"{name} q{qi}: block scores differ with tile {tile}"
        assert torch.equal(pk[qi, :c], pk2[qi, :c]), f"{name} q{qi}: position keys differ with tile {tile}"
        k = int(cnt[qi])
        assert torch.equal(pool[qi, :k], pool2[qi, :k]), f"{name} q{qi}: pool differs with tile {tile}"


@pytest.mark.parametrize("small", ["1", "0"])
def test_pool_topk_matches_separate_calls(case, small, monkeypatch):
    """csa2_index_pool_topk (the pool and the Full layer's Top-K in one call:
    one kernel for small pools, the chunked kernels then the Top-K kernel
    otherwise, here forced with CSA2_POOL_SMALL=0) writes the same pool and
    the same Top-K as csa2_index_pool followed by csa2_index_topk_keys."""
    name, g, lay = case
    monkeypatch.setenv("CSA2_POOL_SMALL", small)
    csa2, w = g.csa2, g.w
    q, wt = g.iq(0)
    idx_k = g.planes[0][0]
    ld = csa2.block_scores_ld(g.dims, g.batch)
    bs = torch.empty(w.n_q, ld, dtype=torch.float32, device="cuda")
    pk = torch.empty(w.n_q, csa2.pos_keys_ld(g.dims, g.batch), dtype=torch.int32, device="cuda")
    pws = torch.zeros(csa2.workspace_pool(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    csa2.index_scan(g.dims, g.batch, q, wt, idx_k, bs, pool_ws=pws, pos_keys=pk)
    pool, cnt = csa2.index_pool(g.dims, g.batch, bs, ws=pws, from_scan=True)
    tk, tc = csa2.index_topk_keys(g.dims, g.batch, pool, cnt, bs, pk)
    fill = lambda shape: torch.full(shape, 7, dtype=torch.int32, device="cuda")
    pool2, cnt2 = fill((w.n_q, w.dims.pool_blocks)), fill((w.n_q,))
    tk2, tc2 = fill((w.n_q, w.dims.topk)), fill((w.n_q,))
    csa2.index_pool_topk(g.dims, g.batch, bs, pk, pool2, cnt2, tk2, tc2, ws=pws, from_scan=True)
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2), f"{name}: pool counts differ"
    assert torch.equal(tc, tc2), f"{name}: Top-K counts differ"
    assert torch.equal(tk, tk2), f"{name}: Top-K differs"
    for qi in range(w.n_q):
        k = int(cnt[qi])
        assert torch.equal(pool[qi, :k], pool2[qi, :k]), f"{name} q{qi}: pool differs"


@pytest.mark.parametrize("small,splits", [("1", ""), ("0", ""), ("1", "1"), ("1", "3"), ("0", "2")])
def test_pool_topk_attend_matches_separate_calls(case, small, splits, monkeypatch):
    """csa2_pool_topk_attend (the Full layer's Top-K, and for small pools the
    pool too, selected inside the attention kernel by every workgroup with
    kept-entry tiles; with CSA2_POOL_SMALL=0 the chunked pool kernels run
    first and the attention selects the Top-K of their pool, or for K above
    1024 the Top-K kernel does) writes the same pool, Top-K, output and
    log-sum-exp, bit for bit, as csa2_index_pool_topk followed by
    csa2_attend.  CSA2_ATTEND_SPLITS forces splits of several tiles, so that
    window and kept-entry tiles share a workgroup (as at large batch)."""
    name, g, lay = case
    monkeypatch.setenv("CSA2_POOL_SMALL", small)
    if splits:
        monkeypatch.setenv("CSA2_ATTEND_SPLITS", splits)
    csa2, w = g.csa2, g.w
    q, wt = g.iq(0)
    idx_k, codes, scales, kv_rope, swa_kv = g.planes[0]
    ld = csa2.block_scores_ld(g.dims, g.batch)
    bs = torch.empty(w.n_q, ld, dtype=torch.float32, device="cuda")
    pk = torch.empty(w.n_q, csa2.pos_keys_ld(g.dims, g.batch), dtype=torch.int32, device="cuda")
    pws = torch.zeros(csa2.workspace_pool(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    csa2.index_scan(g.dims, g.batch, q, wt, idx_k, bs, pool_ws=pws, pos_keys=pk)
    pool, cnt, tk, tc = csa2.index_pool_topk(g.dims, g.batch, bs, pk, ws=pws, from_scan=True)
    ql, qr = g.mq(0)
    out, lse = csa2.attend(g.dims, g.batch, ql, qr, 1.0, codes, scales, kv_rope, tk, tc, swa_kv, g.swa_base)
    fill = lambda shape, dt=torch.int32: torch.full(shape, 7, dtype=dt, device="cuda")
    pool2, cnt2 = fill((w.n_q, w.dims.pool_blocks)), fill((w.n_q,))
    tk2, tc2 = fill((w.n_q, w.dims.topk)), fill((w.n_q,))
    out2 = fill((w.n_q, w.dims.n_heads, 512), torch.float32)
    lse2 = fill((w.n_q, w.dims.n_heads), torch.float32)
    csa2.pool_topk_attend(g.dims, g.batch, bs, pk, ql, qr, 1.0, codes, scales, kv_rope, swa_kv, g.swa_base,
                          pool2, cnt2, tk2, tc2, out2, lse2, pool_ws=pws, from_scan=True)
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2), f"{name}: pool counts differ"
    for qi in range(w.n_q):
        k = int(cnt[qi])
        assert torch.equal(pool[qi, :k], pool2[qi, :k]), f"{name} q{qi}: pool differs"
        assert bool((pool2[qi, k:] == -1).all()), f"{name} q{qi}: pool tail"
    assert torch.equal(tc, tc2), f"{name}: Top-K counts differ"
    assert torch.equal(tk, tk2), f"{name}: Top-K differs"
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32)), f"{name}: attention output differs"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), f"{name}: log-sum-exp differs"


@pytest.mark.parametrize("splits", ["", "1", "3"])
def test_reindex_attend_matches_separate_calls(case, splits, monkeypatch):
    """csa2_reindex_attend (the Reindex kernel writes its order keys only and
    every attention workgroup with kept-entry tiles selects the Top-K from
    them) writes the same Top-K, output and log-sum-exp, bit for bit, as
    csa2_index_reindex followed by csa2_attend; also with splits of several
    tiles forced (CSA2_ATTEND_SPLITS)."""
    name, g, lay = case
    if splits:
        monkeypatch.setenv("CSA2_ATTEND_SPLITS", splits)
    csa2, w = g.csa2, g.w
    pool, cnt, _ = g.full(0)
    layer = 1
    tk, tc, _ = g.reindex(layer, pool, cnt)
    out, lse = g.attend(layer, tk, tc)
    q, wt = g.iq(layer)
    ql, qr = g.mq(layer)
    idx_k, codes, scales, kv_rope, swa_kv = g.planes[0]
    fill = lambda shape, dt=torch.int32: torch.full(shape, 7, dtype=dt, device="cuda")
    tk2, tc2 = fill((w.n_q, w.dims.topk)), fill((w.n_q,))
    out2 = fill((w.n_q, w.dims.n_heads, 512), torch.float32)
    lse2 = fill((w.n_q, w.dims.n_heads), torch.float32)
    csa2.reindex_attend(g.dims, g.batch, q, wt, idx_k, pool, cnt, ql, qr, 1.0, codes, scales, kv_rope, swa_kv,
                        g.swa_base, tk2, tc2, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(tc, tc2), f"{name}: Top-K counts differ"
    assert torch.equal(tk, tk2), f"{name}: Top-K differs"
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32)), f"{name}: attention output differs"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), f"{name}: log-sum-exp differs"


def test_pipeline_end_to_end_and_deterministic(case):
    name, g, lay = case
    w = g.w
    runs = []
    for _ in range(2):
        pool, cnt, _ = g.full(0)
        layer = 1 if w.reindex_layers > 1 else 0
        tk, tc, _ = g.reindex(layer, pool, cnt)
        out, lse = g.attend(layer, tk, tc)
        torch.cuda.synchronize()
        runs.append([t.cpu().clone() for t in (pool, cnt, tk, tc, out, lse)])
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                           b.view(torch.uint8) if b.dtype == torch.float32 else b), f"{name}: run-to-run difference"
    tk_t, tc_t = runs[0][2].cuda(), runs[0][3].cuda()
    pool, cnt, tk, tc, out, lse = [t.numpy() for t in runs[0]]
    kc = {}
    other = {}
    for qi in range(w.n_q):
        oq = _oq(w, lay, kc, qi)
        rpool, rb, _ = oq.full(0)
        check_set(pool[qi, :cnt[qi]], rpool, lambda j: rb[j], f"{name} q{qi} pool")
        keep, _, _ = oq.reindex(layer, rpool)
        check_set(tk[qi, :tc[qi]], keep, lambda p: oq.scores_at(layer, p), f"{name} q{qi} topk")
        ro, rl = oq.attention(layer, keep)
        if np.array_equal(tk[qi, :tc[qi]], keep):
            check_attention(out[qi], lse[qi], ro, rl, f"{name} q{qi}")
        else:
            other[qi] = (keep, ro, rl)
    if other:
        # attention on the oracle's own Top-K where the sets differ in the band
        tk2, tc2 = with_oracle_rows(tk_t, tc_t, {qi: v[0] for qi, v in other.items()})
        o2, l2 = g.attend(layer, tk2, tc2)
        torch.cuda.synchronize()
        for qi, (_, ro, rl) in other.items():
            check_attention(o2[qi].cpu().numpy(), l2[qi].cpu().numpy(), ro, rl, f"{name} q{qi} oracle-set")


def test_ties_lower_position_wins():
    """Duplicated keys give equal scores: the lower positions must be kept."""
    csa2 = lib()
    dims = wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=4, topk=20)
    w = small(110, dims, [3000])
    g = GpuCase(w)
    lay = wl.layout(w)
    oq = OracleQuery(w, lay, 0)
    # copy the best block's keys over several other blocks (all < c)
    pool0, b0, s0 = oq.full(0)
    best = int(np.argmax(b0))
    src = oq.keys[best * 8:(best + 1) * 8].copy()
    for j in [3, 40, 41, 200, 301]:
        oq.keys[j * 8:(j + 1) * 8] = src
        g.idx_k[j * 8:(j + 1) * 8] = torch.from_numpy(src).view(torch.float8_e4m3fn).cuda()
    rpool, rb, _ = oq.full(0)
    pool, cnt, _ = g.full(0)
    tk, tc, _ = g.reindex(0, pool, cnt)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy()[0, :cnt.item()], rpool)
    keep, _, _ = oq.reindex(0, rpool)
    assert np.array_equal(tk.cpu().numpy()[0, :tc.item()], keep)


def _set_key_rows(oq, g, rows, row):
    """Overwrite key rows of a one-sequence case in the oracle's and the
    GPU's copy alike."""
    oq.keys[rows] = row
    g.idx_k[rows] = torch.from_numpy(np.ascontiguousarray(row)).view(torch.float8_e4m3fn).cuda()


@pytest.fixture(params=["default", "chunked"])
def pool_path(request):
    """The pool selection as chosen (one workgroup per query for these
    sizes), or the chunked kernels forced."""
    if request.param == "chunked":
        os.environ["CSA2_POOL_SMALL"] = "0"
    yield request.param
    os.environ.pop("CSA2_POOL_SMALL", None)


@pytest.mark.parametrize("pool_blocks,ctx", [(256, 20000), (2048, 40000)])
def test_all_scores_equal(pool_blocks, ctx, pool_path):
    """Every position holds the same key, so every score ties: the pool is the
    lowest blocks and the Top-K the lowest positions.  This drives the equal-
    run paths of both selections (a pool crossing bin that overflows its
    chunk candidate slots, and a Top-K run of equal keys longer than the
    exact-rank cap)."""
    dims = wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=pool_blocks, topk=512)
    w = small(111, dims, [ctx])
    g = GpuCase(w)
    oq = OracleQuery(w, wl.layout(w), 0)
    _set_key_rows(oq, g, slice(None), oq.keys[5].copy())
    rpool, _, _ = oq.full(0)
    assert np.array_equal(rpool, np.arange(len(rpool)))
    pool, cnt, _ = g.full(0)
    tk, tc, _ = g.reindex(0, pool, cnt)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy()[0, :cnt.item()], rpool)
    keep, _, _ = oq.reindex(0, rpool)
    assert np.array_equal(tk.cpu().numpy()[0, :tc.item()], keep)


def test_outlier_score_narrows_the_range(pool_path):
    """One position whose key follows the sign of the weighted query gets a
    score far above the rest, and its neighbour (an all-zero key) scores 0.
    The key range then spans both, so the first histogram crowds the
    ordinary scores into a few bins and the selections must narrow the
    crossing bin with further digits (on this input: 538 keys in the Top-K
    crossing bin, against an exact-rank cap of 128)."""
    dims = wl.Dims(n_heads=16, idx_heads=64, idx_dim=128, pool_blocks=2048, topk=512)
    w = small(112, dims, [40000])
    g = GpuCase(w)
    oq = OracleQuery(w, wl.layout(w), 0)
    q, wt = oq.iq(0)
    qs = (wt[:, None] * oracle.e4m3_decode(q)).sum(0)
    _set_key_rows(oq, g, 777, np.where(qs >= 0, 0x7E, 0xFE).astype(np.uint8))     # +-448
    _set_key_rows(oq, g, 776, np.zeros(128, np.uint8))
    rpool, rb, _ = oq.full(0)
    assert rb[777 // 8] > 100 * np.median(rb)
    pool, cnt, _ = g.full(0)
    tk, tc, _ = g.reindex(0, pool, cnt)
    torch.cuda.synchronize()
    got_pool = pool.cpu().numpy()[0, :cnt.item()]
    check_set(got_pool, rpool, lambda j: rb[j], "outlier pool")
    if np.array_equal(got_pool, rpool):
        keep, _, _ = oq.reindex(0, rpool)
        check_set(tk.cpu().numpy()[0, :tc.item()], keep, lambda p: oq.scores_at(0, p), "outlier topk")


def _full_topk(g):
    """csa2_index_scan keeping the position keys, then csa2_index_pool_topk:
    the pool and a Full layer's Top-K of query 0."""
    csa2, w = g.csa2, g.w
    q, wt = g.iq(0)
    bs = torch.empty(w.n_q, csa2.block_scores_ld(g.dims, g.batch), dtype=torch.float32, device="cuda")
    pk = torch.empty(w.n_q, csa2.pos_keys_ld(g.dims, g.batch), dtype=torch.int32, device="cuda")
    pws = torch.zeros(csa2.workspace_pool(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    csa2.index_scan(g.dims, g.batch, q, wt, g.planes[0][0], bs, pool_ws=pws, pos_keys=pk)
    pool, cnt, tk, tc = csa2.index_pool_topk(g.dims, g.batch, bs, pk, ws=pws, from_scan=True)
    # the selection inside the attention kernel: the same pool and Top-K
    idx_k, codes, scales, kv_rope, swa_kv = g.planes[0]
    ql, qr = g.mq(0)
    pool2, cnt2, tk2, tc2, _, _ = csa2.pool_topk_attend(g.dims, g.batch, bs, pk, ql, qr, 1.0, codes, scales,
                                                         kv_rope, swa_kv, g.swa_base, pool_ws=pws, from_scan=True)
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2) and torch.equal(tc, tc2) and torch.equal(tk, tk2)
    assert torch.equal(pool[0, :cnt.item()], pool2[0, :cnt.item()])
    torch.cuda.synchronize()
    return pool.cpu().numpy()[0, :cnt.item()], tk.cpu().numpy()[0, :tc.item()]


@pytest.mark.parametrize("pool_blocks,topk", [(256, 512), (2048, 512), (2048, 1024)])
def test_pool_topk_all_scores_equal(pool_blocks, topk, pool_path):
    """Every score ties: the first histogram's crossing bin holds every block,
    so the Full layer's Top-K candidates are the whole pool.  With a pool
    larger than the positions step takes (2048 blocks against 1024 or 2048
    slots) the exact second block selection runs; the Top-K is then the
    lowest K positions of the lowest blocks, as the oracle's."""
    dims = wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=pool_blocks, topk=topk)
    w = small(113, dims, [40000])
    g = GpuCase(w)
    oq = OracleQuery(w, wl.layout(w), 0)
    _set_key_rows(oq, g, slice(None), oq.keys[5].copy())
    rpool, _, _ = oq.full(0)
    keep, _, _ = oq.reindex(0, rpool)
    assert np.array_equal(keep, np.arange(topk))
    pool, tk = _full_topk(g)
    assert np.array_equal(pool, rpool)
    assert np.array_equal(tk, keep)


def test_pool_topk_outlier(pool_path):
    """One far outlier stretches the block-score range, so the first
    histogram's bins are coarse: the Full layer's Top-K candidates (the
    pool's blocks from the K-th best block's bin up) are a strict superset of
    the K best blocks (513 for K = 512 on this input)."""
    dims = wl.Dims(n_heads=16, idx_heads=64, idx_dim=128, pool_blocks=2048, topk=512)
    w = small(112, dims, [40000])
    g = GpuCase(w)
    oq = OracleQuery(w, wl.layout(w), 0)
    q, wt = oq.iq(0)
    qs = (wt[:, None] * oracle.e4m3_decode(q)).sum(0)
    _set_key_rows(oq, g, 777, np.where(qs >= 0, 0x7E, 0xFE).astype(np.uint8))
    _set_key_rows(oq, g, 776, np.zeros(128, np.uint8))
    rpool, rb, _ = oq.full(0)
    pool, tk = _full_topk(g)
    check_set(pool, rpool, lambda j: rb[j], "outlier pool")
    if np.array_equal(pool, rpool):
        keep, _, _ = oq.reindex(0, rpool)
        check_set(tk, keep, lambda p: oq.scores_at(0, p), "outlier full topk")


def test_pool_paths_agree(case):
    """csa2_index_full (scan-prepared pool workspace), csa2_index_scan +
    csa2_index_pool (the pool's own key-range pass), repeated pool calls on
    one scan-prepared workspace, and the chunked pool kernels forced where
    the one-workgroup selection would run (with a marking workgroup per
    chunk, and with one per query) give the same pool bit for bit."""
    name, g, lay = case
    w = g.w
    csa2 = g.csa2
    q, wt = g.iq(0)
    ref_pool, ref_cnt, _ = g.full(0)
    bs = csa2.index_scan(g.dims, g.batch, q, wt, g.idx_k)
    p1, c1 = csa2.index_pool(g.dims, g.batch, bs)
    ws = torch.empty(csa2.workspace_pool(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    bs2 = csa2.index_scan(g.dims, g.batch, q, wt, g.idx_k, pool_ws=ws)
    outs = [csa2.index_pool(g.dims, g.batch, bs2, ws=ws, from_scan=True) for _ in range(3)]
    # the chunked kernels also where the one-workgroup selection would run,
    # and with one marking workgroup per query taking all of its chunks (the
    # layout large batches use)
    os.environ["CSA2_POOL_SMALL"] = "0"
    try:
        outs.append(csa2.index_pool(g.dims, g.batch, bs2, ws=ws, from_scan=True))
        outs.append(csa2.index_pool(g.dims, g.batch, bs))
        os.environ["CSA2_POOL_MARK_WGS"] = "1"
        outs.append(csa2.index_pool(g.dims, g.batch, bs2, ws=ws, from_scan=True))
        outs.append(csa2.index_pool(g.dims, g.batch, bs))
    finally:
        del os.environ["CSA2_POOL_SMALL"]
        os.environ.pop("CSA2_POOL_MARK_WGS", None)
    torch.cuda.synchronize()
    nb = csa2.n_blocks(g.dims, g.batch)
    for qi in range(w.n_q):     # rows are written up to each query's own block count
        k = max(0, -(-(lay.q_visible[qi] - w.dims.swa) // 8))
        assert torch.equal(bs[qi, :k].view(torch.int32), bs2[qi, :k].view(torch.int32))
    assert nb >= 0
    for p, c in [(p1, c1)] + outs:
        assert torch.equal(c, ref_cnt), f"{name}: pool counts differ between paths"
        for qi in range(w.n_q):
            k = int(ref_cnt[qi])
            assert torch.equal(p[qi, :k], ref_pool[qi, :k]), f"{name} q{qi}: pools differ between paths"


def test_reindex_workgroup_sizes_agree(case):
    """Reindex scored by 32-, 64-, 128- and 256-block workgroups (the library
    picks by batch size) selects the same Top-K with bit-identical scores:
    the per-position arithmetic does not depend on how the pool is split."""
    name, g, lay = case
    csa2 = g.csa2
    pool, cnt, _ = g.full(0)
    q, wt = g.iq(0)
    idx_k = g.planes[0][0]
    outs = []
    for bpw in ("64", "128", "32", "256"):
        os.environ["CSA2_REINDEX_BLOCKS"] = bpw
        try:
            ts = torch.empty(g.w.n_q, g.w.dims.topk, dtype=torch.float32, device="cuda")
            tk, tc = csa2.index_reindex(g.dims, g.batch, q, wt, idx_k, pool, cnt, topk_scores=ts)
            outs.append((tk, tc, ts))
        finally:
            del os.environ["CSA2_REINDEX_BLOCKS"]
    torch.cuda.synchronize()
    tk0, tc0, ts0 = outs[0]
    for tk1, tc1, ts1 in outs[1:]:
        assert torch.equal(tc0, tc1), f"{name}: Top-K counts differ between workgroup sizes"
        for qi in range(g.w.n_q):
            k = int(tc0[qi])
            assert torch.equal(tk0[qi, :k], tk1[qi, :k]), f"{name} q{qi}: Top-K differs between workgroup sizes"
            assert torch.equal(ts0[qi, :k].view(torch.int32), ts1[qi, :k].view(torch.int32)), \
                f"{name} q{qi}: Top-K scores differ between workgroup sizes"


def test_reindex_workspace_reuse(case):
    """Repeated Reindex calls on one workspace agree bit for bit (with and
    without the score output), and leave its per-query completion counters
    at zero, as the next call needs."""
    name, g, lay = case
    csa2 = g.csa2
    pool, cnt, _ = g.full(0)
    q, wt = g.iq(0)
    idx_k = g.planes[0][0]
    ws = torch.zeros(csa2.workspace_reindex(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    ts = torch.empty(g.w.n_q, g.w.dims.topk, dtype=torch.float32, device="cuda")
    outs = [csa2.index_reindex(g.dims, g.batch, q, wt, idx_k, pool, cnt, ws=ws,
                               topk_scores=ts if i == 1 else None) for i in range(3)]
    torch.cuda.synchronize()
    for tk, tc in outs[1:]:
        assert torch.equal(tc, outs[0][1]), f"{name}: topk counts differ between calls"
        assert torch.equal(tk, outs[0][0]), f"{name}: topk differs between calls"
    off = (-ws.data_ptr()) % 256
    assert int(ws[off:off + 4 * g.w.n_q].count_nonzero()) == 0, f"{name}: counters not left at zero"
