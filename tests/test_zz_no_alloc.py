"""csa2_decode_step_noalloc: the layer step without a workspace argument (its
scratch is the library's own per-GPU array) against csa2_decode_step with a
caller workspace: the same kernels, so every output must match bit for bit.
Two calls in a row, the second on a smaller batch, so that whatever the
first left in the shared array cannot leak into the second."""
import pytest
import torch

import workloads as wl
from tests._harness import GpuCase, lib
from tests.test_gpu_parity import BIG, small

pytestmark = pytest.mark.gpu

FIRST = small(161, BIG, [20005, 9003, 4099])                                  # three queries, several tiles
SECOND = small(162, wl.Dims(n_heads=24, idx_heads=16, idx_dim=128, pool_blocks=64, topk=128), [5003])


def _bufs(w):
    n_q, d = w.n_q, w.dims
    return dict(pool_blocks=torch.full((n_q, d.pool_blocks), 7, dtype=torch.int32, device="cuda"),
                pool_count=torch.full((n_q,), 7, dtype=torch.int32, device="cuda"),
                topk_pos=torch.full((n_q, d.topk), 7, dtype=torch.int32, device="cuda"),
                topk_count=torch.full((n_q,), 7, dtype=torch.int32, device="cuda"),
                out=torch.full((n_q, d.n_heads, 512), 7.0, dtype=torch.float32, device="cuda"),
                lse=torch.full((n_q, d.n_heads), 7.0, dtype=torch.float32, device="cuda"))


def _call(g, fn, mode, layer, bufs, **kw):
    q, wt = g.iq(layer) if mode != g.csa2.LAYER_REUSE else (None, None)
    ql, qr = g.mq(layer)
    idx_k, codes, scales, kv_rope, swa_kv = g.planes[0]
    fn(g.dims, g.batch, mode, q, wt, idx_k if q is not None else None, bufs["pool_blocks"], bufs["pool_count"],
       bufs["topk_pos"], bufs["topk_count"], ql, qr, 1.0, codes, scales, kv_rope, swa_kv, g.swa_base, bufs["out"],
       bufs["lse"], **kw)


def _same(a, b, w, label):
    for k in a:
        x, y = a[k].cpu(), b[k].cpu()
        if k == "pool_blocks":
            for qi in range(w.n_q):
                n = int(a["pool_count"][qi])
                assert torch.equal(x[qi, :n], y[qi, :n]), f"{label}: pool of query {qi}"
            continue
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"{label}: {k}"


def test_noalloc_step_matches_workspace_step():
    csa2 = lib()
    for w in (FIRST, SECOND):
        g = GpuCase(w)
        ws = torch.zeros(csa2.workspace_step(g.dims, g.batch) + 256, dtype=torch.uint8, device="cuda")
        ref, got = _bufs(w), _bufs(w)
        for mode, layer in ((csa2.LAYER_FULL, 0), (csa2.LAYER_REINDEX, 1), (csa2.LAYER_REUSE, 2)):
            _call(g, csa2.decode_step, mode, layer, ref, ws=ws)
            _call(g, csa2.decode_step_noalloc, mode, layer, got)
            torch.cuda.synchronize()
            _same(ref, got, w, f"{w.name} mode {mode}")
