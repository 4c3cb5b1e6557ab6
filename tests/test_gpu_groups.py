"""The in-kernel selection of long queries from the Full scan's group keys.

csa2_pool_topk_attend after a scan that prepared the pool workspace selects,
for a query of more than 16,384 blocks, the pool and the Full layer's Top-K
inside the attention launch from the scan's group keys (the largest block key
of every 16 blocks; "DeepSeek-V4.1-Flash 梗概" §3.1-§3.2: the pool is the P
best blocks, the Top-K the K best positions of the pool).  Its pool, Top-K,
attention output and log-sum-exp must equal, bit for bit, those of the
chunked pool kernels, the Top-K kernel and csa2_attend (themselves checked
against the oracle in test_gpu_parity.py), and those of the fused call with
the group path switched off (CSA2_POOL_GROUPS=0).  The batches mix a query on
the fast path (enough groups for the pool's bound), one just past the
one-workgroup limit (fewer groups than the pool: the pool streams every block
score), and a short one (the register selection in the same launch).  With
every score equal the candidates overflow and the exact streaming selection
decides both; the pool and Top-K are then the lowest blocks and positions, as
the oracle's.
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
from tests._harness import GpuCase, OracleQuery  # noqa: E402

pytestmark = pytest.mark.gpu


def _long(idx, dims, ctx_list):
    return wl.Workload(idx, "long", dims, n_seq=len(ctx_list), ctx=(0, 0), ctx_list=tuple(ctx_list))


LONG = {
    # 600,000: 74,984 blocks, 4,687 groups (the pool's bound and the Top-K's);
    # 140,000: 17,484 blocks, 1,093 groups (< P: the pool streams); 5,000: small
    "mixed_k512": _long(201, wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=2048, topk=512),
                        [600000, 140000, 5000]),
    # K = 1024 (four candidate groups per thread); 131,300: 16,397 blocks, one past the limit
    "mixed_k1024": _long(202, wl.Dims(n_heads=32, idx_heads=16, idx_dim=128, pool_blocks=2048, topk=1024),
                         [400000, 131300]),
    # a small pool and Top-K, the largest context the group keys take (131,072 blocks)
    "p256_max": _long(203, wl.Dims(n_heads=16, idx_heads=8, idx_dim=64, pool_blocks=256, topk=128),
                      [131072 * 8 + 128]),
    # K > P: the Top-K is taken from exactly the pool, so the chunked pool
    # kernels run (no group path), and the short query selects its exact pool
    "k_above_p": _long(205, wl.Dims(n_heads=16, idx_heads=8, idx_dim=64, pool_blocks=64, topk=128),
                       [200000, 3000]),
}


@pytest.fixture(scope="module", params=list(LONG))
def long_case(request):
    return request.param, GpuCase(LONG[request.param])


def _scan(g):
    csa2, w = g.csa2, g.w
    q, wt = g.iq(0)
    bs = torch.empty(w.n_q, csa2.block_scores_ld(g.dims, g.batch), dtype=torch.float32, device="cuda")
    pk = torch.empty(w.n_q, csa2.pos_keys_ld(g.dims, g.batch), dtype=torch.int32, device="cuda")
    pws = torch.zeros(csa2.workspace_pool(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
    csa2.index_scan(g.dims, g.batch, q, wt, g.planes[0][0], bs, pool_ws=pws, pos_keys=pk)
    return bs, pk, pws


def _fused(g, bs, pk, pws):
    csa2, w = g.csa2, g.w
    _, codes, scales, kv_rope, swa_kv = g.planes[0]
    ql, qr = g.mq(0)
    fill = lambda shape, dt=torch.int32: torch.full(shape, 7, dtype=dt, device="cuda")
    r = (fill((w.n_q, w.dims.pool_blocks)), fill((w.n_q,)), fill((w.n_q, w.dims.topk)), fill((w.n_q,)),
         fill((w.n_q, w.dims.n_heads, 512), torch.float32), fill((w.n_q, w.dims.n_heads), torch.float32))
    csa2.pool_topk_attend(g.dims, g.batch, bs, pk, ql, qr, 1.0, codes, scales, kv_rope, swa_kv, g.swa_base, *r,
                          pool_ws=pws, from_scan=True)
    return r


def _same(name, ref, got):
    pool, cnt, tk, tc, out, lse = ref
    pool2, cnt2, tk2, tc2, out2, lse2 = got
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2), f"{name}: pool counts differ"
    for qi in range(cnt.shape[0]):
        k = int(cnt[qi])
        assert torch.equal(pool[qi, :k], pool2[qi, :k]), f"{name} q{qi}: pool differs"
        assert bool((pool2[qi, k:] == -1).all()), f"{name} q{qi}: pool tail"
    assert torch.equal(tc, tc2), f"{name}: Top-K counts differ"
    assert torch.equal(tk, tk2), f"{name}: Top-K differs"
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32)), f"{name}: attention output differs"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), f"{name}: log-sum-exp differs"


@pytest.mark.parametrize("splits", ["", "3"])
def test_groups_match_chunked(long_case, splits, monkeypatch):
    """The group-key selection against the chunked kernels and csa2_attend,
    and against the fused call with the chunked pool; also with splits of
    several tiles forced (CSA2_ATTEND_SPLITS), so that the selecting
    workgroups hold window tiles too."""
    name, g = long_case
    if splits:
        monkeypatch.setenv("CSA2_ATTEND_SPLITS", splits)
    csa2 = g.csa2
    bs, pk, pws = _scan(g)
    _, codes, scales, kv_rope, swa_kv = g.planes[0]
    ql, qr = g.mq(0)
    pool, cnt, tk, tc = csa2.index_pool_topk(g.dims, g.batch, bs, pk, ws=pws, from_scan=True)
    out, lse = csa2.attend(g.dims, g.batch, ql, qr, 1.0, codes, scales, kv_rope, tk, tc, swa_kv, g.swa_base)
    ref = (pool, cnt, tk, tc, out, lse)
    _same(name + " groups", ref, _fused(g, bs, pk, pws))
    monkeypatch.setenv("CSA2_POOL_GROUPS", "0")
    _same(name + " chunked fused", ref, _fused(g, bs, pk, pws))
    monkeypatch.delenv("CSA2_POOL_GROUPS")
    # a second group call on the same prepared workspace
    _same(name + " groups again", ref, _fused(g, bs, pk, pws))


def test_groups_all_scores_equal():
    """Every key row equal, so every score ties: each candidate set overflows
    and the exact streaming selection decides the pool (2,048 of 37,484
    blocks) and the Top-K's blocks; the pool is the lowest blocks and the
    Top-K the lowest positions, as the oracle's."""
    dims = wl.Dims(n_heads=16, idx_heads=16, idx_dim=128, pool_blocks=2048, topk=512)
    w = _long(204, dims, [300000])
    g = GpuCase(w)
    oq = OracleQuery(w, wl.layout(w), 0)
    row = oq.keys[5].copy()
    oq.keys[:] = row
    g.idx_k[:] = torch.from_numpy(np.ascontiguousarray(row)).view(torch.float8_e4m3fn).cuda()
    rpool, _, _ = oq.full(0)
    keep, _, _ = oq.reindex(0, rpool)
    assert np.array_equal(rpool, np.arange(dims.pool_blocks))
    assert np.array_equal(keep, np.arange(dims.topk))
    bs, pk, pws = _scan(g)
    pool, cnt, tk, tc, _, _ = _fused(g, bs, pk, pws)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy()[0, :cnt.item()], rpool)
    assert np.array_equal(tk.cpu().numpy()[0, :tc.item()], keep)
