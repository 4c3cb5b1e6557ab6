#!/usr/bin/env python3
"""Benchmark of the CSA2 decode path on one MI355X.

One step = one pass of the whole decode-side path over the workload's batch:
Full-mode scan + Top-P pool, Reindex (Top-K), and the sparse FP4 + window
attention (plus, for the speculative-verify workload, the FP4 encode of the
freshly appended entries; for the decoder-cluster workload, five Reindex +
attention layers after one Full scan).  Inputs are resident in HBM; each step
reads a different replica of the caches so that the 256 MB Infinity Cache
cannot serve repeated reads.

Prints ONE JSON line: queries/s of the primary workload (default: batch 8 at
128K context), a roofline object for the dominant kernel (the Full scan,
HBM-bound: algorithmic key bytes / scan-kernel time from HIP events), the
1M-context workload as a secondary measurement, and the CPU oracle timed on
this host's cores on a bounded sample (a reported baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16 / bf16 matrix, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 matrix, published
SCAN_SOURCES = ["compressed_sparse_attention_decode_amd/csrc/scan.hip",
                "compressed_sparse_attention_decode_amd/csrc/common.h",
                "compressed_sparse_attention_decode_amd/csrc/scan_args.h"]


# ---------------------------------------------------------------- device state
class DeviceState:
    """Caches, window rows and queries of a workload on the GPU, with
    `replicas` copies of every cache plane."""

    def __init__(self, w: wl.Workload, device="cuda", replicas: int = 1, chunk_rows: int = 1 << 18,
                 encode: bool = True):
        import compressed_sparse_attention_decode_amd as csa2
        csa2.lib()
        self.csa2, self.w, self.dev = csa2, w, device
        self.lay = lay = wl.layout(w)
        d = w.dims
        self.dims = csa2.Dims(n_heads=d.n_heads, idx_heads=d.idx_heads, idx_dim=d.idx_dim,
                              pool_blocks=d.pool_blocks, topk=d.topk, swa=d.swa, kv_group=d.kv_group)
        rows = max(lay.rows, 1)
        if w.idx_fp4:
            # FP4 indexer rows: (codes, scales) planes encoded on the device
            idx_k = (torch.empty(rows, d.idx_dim // 2, dtype=torch.uint8, device=device),
                     torch.empty(rows, d.idx_dim // 16, dtype=torch.uint8, device=device))
        else:
            idx_k = torch.empty(rows, d.idx_dim, dtype=torch.float8_e4m3fn, device=device)
        codes = torch.empty(rows, 256, dtype=torch.uint8, device=device)
        scales = torch.empty(rows, 512 // d.kv_group, dtype=torch.uint8, device=device)
        kv_rope = torch.empty(rows, 64, dtype=torch.bfloat16, device=device)
        for r0 in range(0, lay.rows, chunk_rows):
            n = min(chunk_rows, lay.rows - r0)
            if w.idx_fp4:
                csa2.encode_fp4(wl.idx_keys_bf16(w, r0, n, device), idx_k[0][r0:r0 + n], idx_k[1][r0:r0 + n])
            else:
                idx_k[r0:r0 + n] = wl.idx_keys(w, r0, n, device)
            if encode:
                csa2.encode_kv(wl.latent(w, r0, n, device), wl.rope(w, r0, n, device),
                               codes[r0:r0 + n], scales[r0:r0 + n], kv_rope[r0:r0 + n], group=d.kv_group)
        parts = [wl.swa_rows(w, lay, s, device) for s in range(len(lay.ctx))]
        parts = [p for p in parts if p.shape[0]]
        swa_kv = torch.cat(parts) if parts else torch.zeros(1, 576, dtype=torch.bfloat16, device=device)
        self.planes = [(idx_k, codes, scales, kv_rope, swa_kv)]
        for _ in range(replicas - 1):
            self.planes.append(tuple(tuple(x.clone() for x in t) if isinstance(t, tuple) else t.clone()
                                     for t in self.planes[0]))
        self.idx_k, self.codes, self.scales, self.kv_rope, self.swa_kv = self.planes[0]
        self.batch = csa2.Batch(
            seq_base=torch.tensor(lay.q_seq_base, dtype=torch.int64, device=device),
            n_visible=torch.tensor(lay.q_visible, dtype=torch.int32, device=device),
            max_visible=max(lay.q_visible) if lay.q_visible else 0,
            tokens_per_seq=w.tokens_per_seq)
        self.swa_base = torch.tensor(lay.q_swa_base, dtype=torch.int64, device=device)
        self._q = {}
        self.pages = None
        if w.page_size:
            self._page(w.page_size)
        torch.cuda.synchronize()

    def _page(self, ps: int):
        """Moves every per-position plane into pages of `ps` positions at a
        seeded shuffled physical order (with a few unused pages), and points
        the batch's seq_base at each sequence's page-table row."""
        csa2, lay, w, dev = self.csa2, self.lay, self.w, self.dev
        rng = np.random.default_rng(w.key)
        npg = [-(-r // ps) for r in lay.seq_rows]
        total = sum(npg) + 7
        perm = rng.permutation(total).astype(np.int64)
        off, k, table = [], 0, []
        for n in npg:
            off.append(k)                    # the sequence's first entry in the table
            table.append(perm[k:k + n])
            k += n
        table = np.concatenate(table + [np.zeros(1, np.int64)])
        rows = total * ps
        src = np.concatenate([lay.seq_base[s] + np.arange(r, dtype=np.int64) for s, r in enumerate(lay.seq_rows)])
        dst = np.concatenate([table[off[s] + np.arange(r) // ps] * ps + np.arange(r) % ps
                              for s, r in enumerate(lay.seq_rows)])
        src_t, dst_t = torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev)

        def scatter(t):
            out = torch.zeros((rows,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
            out.view(torch.uint8).view(rows, -1)[dst_t] = t.view(torch.uint8).view(t.shape[0], -1)[src_t]
            return out

        paged = []
        for idx_k, codes, scales, kv_rope, swa_kv in self.planes:
            pk = tuple(scatter(x) for x in idx_k) if isinstance(idx_k, tuple) else scatter(idx_k)
            paged.append((pk, scatter(codes), scatter(scales), scatter(kv_rope), swa_kv))
        self.planes = paged
        self.idx_k, self.codes, self.scales, self.kv_rope, self.swa_kv = self.planes[0]
        self.table = torch.from_numpy(table.astype(np.int32)).to(dev)
        self.pages = csa2.Pages(self.table, ps, rows)
        q_off = [off[qi // w.tokens_per_seq] for qi in range(w.n_q)]
        self.batch = csa2.Batch(torch.tensor(q_off, dtype=torch.int64, device=dev), self.batch.n_visible,
                                self.batch.max_visible, self.batch.tokens_per_seq)

    # queries are generated once per layer and kept resident
    def iq(self, layer: int):
        k = ("i", layer)
        if k not in self._q:
            n, d = self.w.n_q, self.w.dims
            if self.w.idx_fp4:
                qb = wl.idx_query_bf16(self.w, layer, 0, n, self.dev)
                qc = torch.empty(n, d.idx_heads, d.idx_dim // 2, dtype=torch.uint8, device=self.dev)
                qs = torch.empty(n, d.idx_heads, d.idx_dim // 16, dtype=torch.uint8, device=self.dev)
                self.csa2.encode_fp4(qb.view(-1, d.idx_dim), qc.view(-1, d.idx_dim // 2), qs.view(-1, d.idx_dim // 16))
                q = (qc, qs)
            else:
                q = wl.idx_query(self.w, layer, 0, n, self.dev)
            self._q[k] = (q, wl.idx_weight(self.w, layer, 0, n, self.dev))
        return self._q[k]

    def mq(self, layer: int):
        k = ("m", layer)
        if k not in self._q:
            n = self.w.n_q
            self._q[k] = (wl.q_latent(self.w, layer, 0, n, self.dev), wl.q_rope(self.w, layer, 0, n, self.dev))
        return self._q[k]

    def full(self, layer=0, block_scores=False, r=0):
        q, w = self.iq(layer)
        bs = None
        if block_scores:
            nb = self.csa2.block_scores_ld(self.dims, self.batch)
            bs = torch.full((self.w.n_q, nb), float("nan"), dtype=torch.float32, device=self.dev)
        pool, cnt = self.csa2.index_full(self.dims, self.batch, q, w, self.planes[r][0], block_scores=bs,
                                          pages=self.pages)
        return pool, cnt, bs

    def reindex(self, layer, pool, cnt, scores=False, r=0):
        q, w = self.iq(layer)
        ts = torch.empty(self.w.n_q, self.w.dims.topk, dtype=torch.float32, device=self.dev) if scores else None
        tk, tc = self.csa2.index_reindex(self.dims, self.batch, q, w, self.planes[r][0], pool, cnt, topk_scores=ts,
                                         pages=self.pages)
        return tk, tc, ts

    def attend(self, layer, tk, tc, r=0):
        ql, qr = self.mq(layer)
        _, codes, scales, kv_rope, swa_kv = self.planes[r]
        return self.csa2.attend(self.dims, self.batch, ql, qr, 1.0, codes, scales, kv_rope,
                                tk, tc, swa_kv, self.swa_base, pages=self.pages)


# ---------------------------------------------------------------- one step
class Step:
    """Preallocated buffers and the launch sequence of one decode step."""

    def __init__(self, st: DeviceState):
        self.st = st
        w, csa2, dev = st.w, st.csa2, st.dev
        n_q = w.n_q
        self.layers = list(range(1, w.reindex_layers + 1)) if w.fresh_q_per_layer else [0]
        self.bs = torch.empty(n_q, csa2.block_scores_ld(st.dims, st.batch), dtype=torch.float32, device=dev)
        self.pool = torch.empty(n_q, w.dims.pool_blocks, dtype=torch.int32, device=dev)
        self.pcnt = torch.empty(n_q, dtype=torch.int32, device=dev)
        self.tk = torch.empty(len(self.layers), n_q, w.dims.topk, dtype=torch.int32, device=dev)
        self.tc = torch.empty(len(self.layers), n_q, dtype=torch.int32, device=dev)
        self.out = torch.empty(len(self.layers), n_q, w.dims.n_heads, 512, dtype=torch.float32, device=dev)
        self.lse = torch.empty(len(self.layers), n_q, w.dims.n_heads, dtype=torch.float32, device=dev)
        self.ws_p = torch.empty(csa2.workspace_pool(st.dims, st.batch) + 256, dtype=torch.uint8, device=dev)
        self.ws_r = torch.zeros(csa2.workspace_reindex(st.dims, st.batch) + 256, dtype=torch.uint8, device=dev)
        self.ws_a = torch.zeros(csa2.workspace_attend(st.dims, st.batch) + 256, dtype=torch.uint8, device=dev)
        # a Full layer's Top-K comes from the scan's own scores (same query):
        # the scan keeps every position's score as an order key
        self.full_topk = not w.fresh_q_per_layer
        self.pk = torch.empty(n_q, csa2.pos_keys_ld(st.dims, st.batch), dtype=torch.int32, device=dev) \
            if self.full_topk else None
        # the pool and the Top-K are selected inside the attention kernel
        self.fused = self.full_topk
        for layer in [0] + self.layers:
            st.iq(layer)
            st.mq(layer)
        if w.fresh_encode:
            n = w.fresh_encode
            self.enc_lat = wl.fresh_latent(w, 0, 0, n, dev)
            self.enc_rope = wl.fresh_rope(w, 0, 0, n, dev)
            self.enc_planes = (torch.empty(n, 256, dtype=torch.uint8, device=dev),
                               torch.empty(n, 512 // w.dims.kv_group, dtype=torch.uint8, device=dev),
                               torch.empty(n, 64, dtype=torch.bfloat16, device=dev))
        torch.cuda.synchronize()

        # launches of one step per replica, arguments marshalled once
        self.calls = []
        for r in range(len(st.planes)):
            idx_k, codes, scales, kv_rope, swa_kv = st.planes[r]
            seq = []
            if w.fresh_encode:
                seq.append(("encode", csa2.encode_kv(self.enc_lat, self.enc_rope, *self.enc_planes, prepare=True,
                                                     group=w.dims.kv_group)))
            q0, w0 = st.iq(0)
            # the stages of a Full layer (csa2_decode_step's chain), issued
            # separately to time each
            seq.append(("scan", csa2.index_scan(st.dims, st.batch, q0, w0, idx_k, self.bs, pool_ws=self.ws_p,
                                                prepare=True, pages=st.pages, pos_keys=self.pk)))
            if self.fused:
                # the pool, the Full layer's Top-K and the attention, both
                # selected inside the attention kernel: csa2_decode_step's
                # Full chain
                ql, qr = st.mq(0)
                seq.append(("pool_topk_attend", csa2.pool_topk_attend(
                    st.dims, st.batch, self.bs, self.pk, ql, qr, 1.0, codes, scales, kv_rope, swa_kv, st.swa_base,
                    self.pool, self.pcnt, self.tk[0], self.tc[0], out=self.out[0], lse=self.lse[0], ws=self.ws_a,
                    pool_ws=self.ws_p, from_scan=True, prepare=True, pages=st.pages)))
            else:
                seq.append(("pool", csa2.index_pool(st.dims, st.batch, self.bs, self.pool, self.pcnt, ws=self.ws_p,
                                                    from_scan=True, prepare=True)))
            for i, layer in enumerate(self.layers if not self.full_topk else []):
                q, wt = st.iq(layer)
                ql, qr = st.mq(layer)
                # the Reindex keys, the Top-K selected inside the attention
                # kernel: csa2_decode_step's Reindex chain
                seq.append(("reindex_attend", csa2.reindex_attend(
                    st.dims, st.batch, q, wt, idx_k, self.pool, self.pcnt, ql, qr, 1.0, codes, scales, kv_rope,
                    swa_kv, st.swa_base, self.tk[i], self.tc[i], out=self.out[i], lse=self.lse[i],
                    reindex_ws=self.ws_r, ws=self.ws_a, prepare=True, pages=st.pages)))
            self.calls.append(seq)

    def run(self, r: int):
        """One step on replica r."""
        for _, call in self.calls[r]:
            call()


# ---------------------------------------------------------------- accounting
def key_bytes(w: wl.Workload) -> int:
    """Bytes of one indexer key: d_i fp8 bytes, or d_i / 2 FP4 code bytes
    plus d_i / 16 scale bytes."""
    d = w.dims.idx_dim
    return d // 2 + d // 16 if w.idx_fp4 else d


def scan_bytes(w: wl.Workload) -> int:
    """Algorithmic bytes of one scan launch: one key per candidate position,
    summed over the batch's sequences (tokens of one sequence share one key
    stream)."""
    lay = wl.layout(w)
    g = w.tokens_per_seq
    tot = 0
    for s in range(len(lay.ctx)):
        n_max = lay.q_visible[s * g + g - 1]
        tot += max(0, n_max - w.dims.swa) * key_bytes(w)
    return tot


def scan_flops(w: wl.Workload) -> int:
    """Algorithmic flops of one scan launch: 2 * H_i * d_i per candidate
    position of every query (tokens of one sequence share the keys, not the
    dot products)."""
    lay = wl.layout(w)
    d = w.dims
    return sum(2 * d.idx_heads * d.idx_dim * max(0, n - d.swa) for n in lay.q_visible)


def step_bytes(w: wl.Workload) -> int:
    """Algorithmic HBM bytes of one step (scan + Reindex + attention + encode)."""
    d = w.dims
    lay = wl.layout(w)
    b = scan_bytes(w)
    n_layers = w.reindex_layers if w.fresh_q_per_layer else 1
    for qi in range(w.n_q):
        n = lay.q_visible[qi]
        c = max(0, n - d.swa)
        nb = -(-c // 8)
        pool = min(d.pool_blocks, nb)
        kk = min(d.topk, 8 * pool)
        win = n - c
        reidx = 8 * pool * key_bytes(w)
        entry = 256 + 512 // d.kv_group + 128            # FP4 codes + scales + bf16 rope
        att = kk * entry + win * 1152 + d.n_heads * (1152 + 2048)
        b += n_layers * (reidx + att)
    b += w.fresh_encode * (1152 + 256 + 512 // d.kv_group + 128)
    return b


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per scan launch measured with rocprofv3 counters, if the
    record matches the current scan source (profiles/scan_traffic.txt)."""
    path = os.path.join(ROOT, "profiles", "scan_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = source_sha(SCAN_SOURCES)
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and not line.startswith("#") and f[0] == workload and f[1] == sha:
            return int(f[2]) + int(f[3])
    return None


# ---------------------------------------------------------------- GPU timing
def _spin_rate() -> float:
    """Seconds per torch.cuda._sleep cycle."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / 1_000_000


def _timed(launch, n: int, spin_s_per_cycle: float, issue_s: float) -> float:
    """GPU milliseconds of n back-to-back launch(i) calls.  A bounded spin
    (at most 2 s) holds the GPU while the host queues every launch, so the
    events bracket GPU time, not the Python issue rate."""
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(min(4.0 * issue_s, 2.0) / spin_s_per_cycle))
    t0.record()
    for i in range(n):
        launch(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


WARM_S = 0.3   # seconds of steps before each workload's timing


def measure(w: wl.Workload, steps: int, warmup: int, replicas: int):
    per_step = scan_bytes(w)
    if replicas <= 0:
        replicas = max(1, min(8, math.ceil(1.0e9 / max(per_step, 1))))
    st = DeviceState(w, replicas=replicas)
    step = Step(st)
    # steady state: the GPU idles while the host builds inputs or runs the
    # oracle between workloads, and a few warm-up steps do not bring it back
    # to speed, so steps run for WARM_S of wall time first, then the warm-up
    t_warm = time.perf_counter() + WARM_S
    i = 0
    while time.perf_counter() < t_warm:
        step.run(i % replicas)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        step.run(i % replicas)
    torch.cuda.synchronize()
    rate = _spin_rate()
    t0 = time.perf_counter()
    for i in range(min(steps, 10)):
        step.run(i % replicas)
    issue_s = (time.perf_counter() - t0) / min(steps, 10) * steps
    torch.cuda.synchronize()

    # whole steps: no event inside a step (recording one drains the queue)
    wall0 = time.perf_counter()
    total_ms = _timed(lambda i: step.run(i % replicas), steps, rate, issue_s)
    wall = time.perf_counter() - wall0
    ms = total_ms / steps

    # per stage: the stage's launches of `steps` steps back to back (every
    # stage reads inputs the previous stages left and rewrites the same
    # outputs, so repeating it is the same work), one event pair per stage
    stages = {}
    names = []
    for name, _ in step.calls[0]:
        if name not in names:
            names.append(name)
    for name in names:
        per_r = [[c for n, c in step.calls[r] if n == name] for r in range(replicas)]
        k = len(per_r[0])

        def launch(i, per_r=per_r):
            for c in per_r[i % replicas]:
                c()
        # the faster of two passes: a host stall longer than the spin (the
        # GPU then waits for launches) inflates one pass, never both alike
        stages[name] = min(_timed(launch, steps, rate, issue_s) for _ in range(2)) / (steps * k) * 1e3
    scan_us = stages["scan"]
    achieved = per_step / (scan_us * 1e-6) / 1e9
    res = {
        "value": w.n_q / (ms * 1e-3),
        "ms_per_step": ms,
        "wall_s": wall,
        "stages_us": {k: round(v, 2) for k, v in stages.items()},
        "replicas": replicas,
        "scan": {"bytes_per_launch": per_step, "avg_us": round(scan_us, 3),
                 "achieved_gbs": round(achieved, 1), "frac": round(achieved / HBM_PEAK_GBS, 4),
                 "mfma_tflops": round(scan_flops(w) / (scan_us * 1e-6) / 1e12, 1),
                 "mfma_frac": round(scan_flops(w) / (scan_us * 1e-6) / 1e12 / scan_peak_tflops(w), 4)},
        "step_bytes": step_bytes(w),
    }
    res["step_gbs"] = round(res["step_bytes"] / (ms * 1e-3) / 1e9, 1)
    # the same step as one csa2_decode_step call (Full layer), and that call
    # captured into one HIP graph per replica and replayed
    if w.reindex_layers == 1 and not w.fresh_encode:
        csa2 = st.csa2
        ws_g = torch.zeros(csa2.workspace_step(st.dims, st.batch) + 256, dtype=torch.uint8, device=st.dev)
        q0, w0 = st.iq(0)
        ql, qr = st.mq(0)

        def layer(r):
            idx_k, codes, scales, kv_rope, swa_kv = st.planes[r]
            csa2.decode_step(st.dims, st.batch, csa2.LAYER_FULL, q0, w0, idx_k, step.pool, step.pcnt, step.tk[0],
                             step.tc[0], ql, qr, 1.0, codes, scales, kv_rope, swa_kv, st.swa_base, step.out[0],
                             step.lse[0], ws=ws_g, pages=st.pages)
        for i in range(warmup):
            layer(i % replicas)
        torch.cuda.synchronize()
        call_ms = _timed(lambda i: layer(i % replicas), steps, rate, issue_s)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for r in range(replicas):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                layer(r)
            graphs.append(gr)
        for i in range(warmup):
            graphs[i % replicas].replay()
        torch.cuda.synchronize()
        graph_ms = _timed(lambda i: graphs[i % replicas].replay(), steps, rate, issue_s)
        del graphs
        # ten consecutive layer calls (rotating replicas) in one graph, as a
        # model step would capture its layers: the graph launch's fixed cost
        # spread over ten layers
        G = 10
        graphs = []
        for r in range(replicas):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for j in range(G):
                    layer((r + j) % replicas)
            graphs.append(gr)
        for i in range(max(1, warmup // G)):
            graphs[i % replicas].replay()
        torch.cuda.synchronize()
        n10 = max(1, steps // G)
        graph10_ms = _timed(lambda i: graphs[i % replicas].replay(), n10, rate, issue_s)
        del graphs
        res["layer_step_us"] = {"stage_calls": round(ms * 1e3, 2), "decode_step": round(call_ms / steps * 1e3, 2),
                                "graph_replay": round(graph_ms / steps * 1e3, 2),
                                "graph_replay_10_layers": round(graph10_ms / (n10 * G) * 1e3, 2)}
    # spread of the step time: 20 short blocks of 5 steps, one event pair each
    import numpy as np
    blocks = []
    for b in range(20):
        blocks.append(_timed(lambda i, b=b: step.run((5 * b + i) % replicas), 5, rate, issue_s * 5 / steps) / 5 * 1e3)
    p10, p50, p90 = np.percentile(blocks, [10, 50, 90])
    res["step_us_spread"] = {"p10": round(float(p10), 2), "median": round(float(p50), 2),
                             "p90": round(float(p90), 2), "blocks": 20, "steps_per_block": 5}
    return st, step, res


# ---------------------------------------------------------------- CPU oracle
def _oracle_query(w, oq, layers, keys, qi, gpu=None):
    """The oracle's calls for one query of a step (Full scan + pool, then
    Reindex + attention per layer, and its share of the step's fresh-entry
    encode).  Returns (timed seconds, parity record updates).  Inputs the
    GPU side also holds resident (keys, queries, encoded cache rows, window
    rows) are prepared untimed.  With `gpu` (pool, count, topk, topk count,
    out, lse as numpy arrays, and a callable running the GPU attention of a
    layer on given Top-K rows) the query's GPU results are checked against
    the oracle's: pool and Top-K within the selection band, attention on the
    GPU's own set when it is the oracle's, else the GPU attention recomputed
    on the oracle's set."""
    import numpy as np
    import oracle
    from tests._harness import check_attention, check_set, u16
    timed = 0.0
    par = {"pool_exact": 0, "topk_exact": 0, "topk_on_oracle_pool": 0, "attention_checked": 0,
           "attention_on_oracle_set": 0, "max_attn_rel": 0.0}
    qs = {layer: oq.iq(layer) for layer in [0] + list(layers)}
    t0 = time.perf_counter()
    rpool, rb, _ = oracle.index_full(qs[0][0], qs[0][1], keys, oq.n, w.dims.swa, w.dims.pool_blocks)
    timed += time.perf_counter() - t0
    same_pool = True
    if gpu is not None:
        pool, pcnt = gpu["pool"], gpu["pcnt"]
        check_set(pool[qi, :pcnt[qi]], rpool, lambda j: rb[j], f"q{qi} pool")
        same_pool = bool(np.array_equal(pool[qi, :pcnt[qi]], rpool))
        par["pool_exact"] += int(same_pool)
    for i, layer in enumerate(layers):
        t0 = time.perf_counter()
        keep, _, _ = oracle.reindex(qs[layer][0], qs[layer][1], keys, rpool, oq.c, w.dims.topk)
        timed += time.perf_counter() - t0
        rows = oq.base + keep
        lat = np.asarray(wl.latent_at(w, rows).view(torch.int16).numpy(), dtype=np.uint16)
        rp = np.asarray(wl.rope_at(w, rows).view(torch.int16).numpy(), dtype=np.uint16)
        codes, scales = oracle.encode_kv(lat, w.dims.kv_group)      # the cache is encoded ahead of time
        win = oq.base + np.arange(oq.c, oq.n)
        swa = np.concatenate([wl.latent_at(w, win).view(torch.int16).numpy(),
                              wl.rope_at(w, win).view(torch.int16).numpy()], axis=1).astype(np.uint16)
        ql = u16(wl.q_latent(w, layer, qi, 1)[0])
        qr = u16(wl.q_rope(w, layer, qi, 1)[0])
        t0 = time.perf_counter()
        ro, rl = oracle.attend(ql, qr, 1.0, oracle.gather_entries(codes, scales, rp, swa))
        timed += time.perf_counter() - t0
        if gpu is not None:
            got = gpu["tk"][i, qi, :gpu["tc"][i, qi]]
            if not same_pool:
                # pools that differ inside the band can give later layers'
                # Reindex sets that differ by more: check this layer's Top-K on
                # the oracle's pool instead
                got = gpu["reindex_on"](layer, qi, rpool)
                par["topk_on_oracle_pool"] += 1
            check_set(got, keep, lambda p: oq.scores_at(layer, p), f"q{qi} layer {layer} topk")
            if same_pool and np.array_equal(got, keep):
                par["topk_exact"] += 1
                o, l = gpu["out"][i, qi], gpu["lse"][i, qi]
            else:
                o, l = gpu["attend_on"](i, layer, qi, keep)
                par["attention_on_oracle_set"] += 1
            e = check_attention(o, l, ro, rl, f"q{qi} layer {layer} attention")
            par["attention_checked"] += 1
            par["max_attn_rel"] = max(par["max_attn_rel"], e)
    if w.fresh_encode:
        # this query's share of the step's fresh-entry encode
        share = max(1, w.fresh_encode // w.n_q)
        e0 = (qi * share) % max(1, w.fresh_encode - share + 1)
        lat = np.asarray(wl.fresh_latent(w, 0, e0, share).view(torch.int16).numpy(), dtype=np.uint16)
        t0 = time.perf_counter()
        oracle.encode_kv(lat, w.dims.kv_group)
        timed += time.perf_counter() - t0
    return timed, par


def cpu_baseline(w: wl.Workload, st: DeviceState, step: Step, seconds: float, one_thread: bool = False):
    """The oracle on this host's cores over queries of the same step, cycling
    over them until `seconds` of oracle time (at least one query); the first
    pass also checks those queries' GPU results (last timed step) against it.
    Returns (cpu_baseline record, parity record)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from tests._harness import OracleQuery, with_oracle_pool, with_oracle_rows

    cores = len(os.sched_getaffinity(0))
    lay = st.lay
    gpu = {"pool": step.pool.cpu().numpy(), "pcnt": step.pcnt.cpu().numpy(), "tk": step.tk.cpu().numpy(),
           "tc": step.tc.cpu().numpy(), "out": step.out.cpu().numpy(), "lse": step.lse.cpu().numpy()}

    def attend_on(i, layer, qi, keep):
        tk2, tc2 = with_oracle_rows(step.tk[i], step.tc[i], {qi: keep})
        o, l = st.attend(layer, tk2, tc2)
        torch.cuda.synchronize()
        return o[qi].cpu().numpy(), l[qi].cpu().numpy()
    gpu["attend_on"] = attend_on

    def reindex_on(layer, qi, rpool):
        # the library's Reindex (this layer's query) on the oracle's pool for query qi
        p2, c2 = with_oracle_pool(step.pool, step.pcnt, {qi: rpool})
        tk, tc, _ = st.reindex(layer, p2, c2)
        torch.cuda.synchronize()
        return tk[qi, :int(tc[qi])].cpu().numpy()
    gpu["reindex_on"] = reindex_on

    timed, done, checked = 0.0, 0, 0
    parity = {"queries": 0, "pool_exact": 0, "topk_exact": 0, "topk_on_oracle_pool": 0, "attention_checked": 0,
              "attention_on_oracle_set": 0, "max_attn_rel": 0.0}
    order = list(range(w.n_q))
    first_pass = True           # later passes over the same queries only add timing
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        keys_cache = {}
        while timed < seconds or done == 0:
            if not order:
                order, first_pass = list(range(w.n_q)), False
            qi = order.pop(0)
            seq = qi // w.tokens_per_seq
            oq = OracleQuery(w, lay, qi, keys_cache.get(seq))
            keys_cache = {seq: oq.keys}
            t, par = _oracle_query(w, oq, step.layers, oq.keys, qi, gpu if first_pass else None)
            timed += t
            done += 1
            if first_pass:
                parity["queries"] += 1
                for k in ("pool_exact", "topk_exact", "topk_on_oracle_pool", "attention_checked",
                          "attention_on_oracle_set"):
                    parity[k] += par[k]
                parity["max_attn_rel"] = max(parity["max_attn_rel"], par["max_attn_rel"])
    parity["max_attn_rel"] = float(f"{parity['max_attn_rel']:.3e}")
    unit = "query-tokens/s" if w.tokens_per_seq > 1 else "queries/s"
    res = {"value": done / timed, "unit": unit, "cores": int(threads), "kind": "oracle",
           "sample": f"{done} query passes over the {w.n_q} queries of one {w.name} step (Full scan + "
                     f"pool, {len(step.layers)} Reindex + attention each"
                     + (", its share of the fresh-entry encode" if w.fresh_encode else "")
                     + f"), float64 NumPy, {cores} host cores available", "seconds": round(timed, 2),
           "host": _host_info(threads)}
    if one_thread:
        # the same oracle calls for query 0 on one thread
        with threadpool_limits(limits=1):
            oq = OracleQuery(w, lay, 0, keys_cache.get(0))
            t1, _ = _oracle_query(w, oq, step.layers, oq.keys, 0)
        res["one_thread"] = {"value": 1.0 / t1, "unit": unit,
                             "sample": "query 0, the same timed oracle calls, 1 BLAS thread"}
    return res, parity


def _host_info(threads: int) -> dict:
    """The host the CPU baseline ran on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": int(threads)}


# ---------------------------------------------------------------- read ceiling
def read_ceiling(steps: int) -> dict:
    """This GPU's plain streaming-read rate (csa2_stream_read: nontemporal
    16-byte loads into registers, one contiguous chunk per workgroup), at the
    1M-context scan's size over 8 rotating buffers (so the 256 MB Infinity
    Cache cannot serve repeats) and over one 1 GiB buffer."""
    import compressed_sparse_attention_decode_amd as csa2
    rate = _spin_rate()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {"kernel": "k_stream_read (csa2_stream_read)"}
    small = scan_bytes(wl.workload("decode_b1_ctx1m"))
    for label, nbytes, nbuf in (("scan_size", small, 8), ("1GiB", 1 << 30, 1)):
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(nbuf)]
        calls = [csa2.stream_read(b, sink, prepare=True) for b in bufs]
        for c in calls:
            c()
        n = max(steps, 16)
        ms = _timed(lambda k: calls[k % nbuf](), n, rate, 1e-3) / n
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[label] = {"bytes": nbytes, "avg_us": round(ms * 1e3, 3), "achieved_gbs": round(gbs, 1),
                      "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del bufs, calls
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- records
def scan_peak_tflops(w: wl.Workload) -> float:
    """The scan's matrix-core peak: fp8 rows run the fp8 MFMA (5 PFLOP/s
    dense), FP4 rows the f16 one on exactly converted values (2.5)."""
    return F16_PEAK_TFLOPS if w.idx_fp4 else FP8_PEAK_TFLOPS


def scan_mfma_dtype(w: wl.Workload) -> str:
    return ("f16 (FP4 rows converted exactly)" if w.idx_fp4
            else "fp8 e4m3 (v_mfma_scale_f32_16x16x128_f8f6f4, unit scales)")


def _is_mfma_bound(w: wl.Workload) -> bool:
    """Tokens of one sequence share each key: the scan does g * 2 H_i d_i
    flops per key of key_bytes bytes, bound by the matrix cores once that
    exceeds their ridge, peak / 8 TB/s (fp8 rows: 625 flops per byte; FP4
    rows on the f16 MFMA: 2.5 PFLOP/s over 72 bytes per key)."""
    per_byte = w.tokens_per_seq * 2 * w.dims.idx_heads * w.dims.idx_dim / key_bytes(w)
    return per_byte > scan_peak_tflops(w) * 1e12 / (HBM_PEAK_GBS * 1e9)


def record(w: wl.Workload, res: dict) -> dict:
    """One workload's figures: throughput, stage times, the step's roofline
    (algorithmic bytes of the whole step over its time) and the scan's
    (HBM-bound, or bound by the f16 matrix cores where tokens share keys)."""
    unit = "query-tokens/s" if w.tokens_per_seq > 1 else "queries/s"
    sc = res["scan"]
    if _is_mfma_bound(w):
        scan_rl = {"bound": "mfma", "achieved": sc["mfma_tflops"], "peak": scan_peak_tflops(w), "unit": "TFLOP/s",
                   "frac": sc["mfma_frac"], "dtype": scan_mfma_dtype(w),
                   "flops_per_launch": scan_flops(w), "avg_us": sc["avg_us"],
                   "hbm_gbs": sc["achieved_gbs"], "hbm_frac": sc["frac"]}
    else:
        scan_rl = {"bound": "hbm", "achieved": sc["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": sc["frac"], "bytes_per_launch": sc["bytes_per_launch"], "avg_us": sc["avg_us"],
                   "traffic": measured_traffic(w.name), "mfma_frac": sc["mfma_frac"],
                   "mfma_dtype": scan_mfma_dtype(w)}
    step_gbs = res["step_bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
    ceiling = w.n_q / (res["step_bytes"] / (HBM_PEAK_GBS * 1e9))
    return {"workload": w.name, "metric": "decode " + unit, "value": round(res["value"], 2), "unit": unit,
            "ms_per_step": round(res["ms_per_step"], 5),
            "indexer_rows": "fp4 (E2M1 + E4M3 per 16)" if w.idx_fp4 else "fp8 e4m3",
            "kv_scale_group": w.dims.kv_group, "page_size": w.page_size or None,
            "batch": w.n_seq, "tokens_per_seq": w.tokens_per_seq, "ctx": list(w.ctx_list or w.ctx),
            "reindex_layers": w.reindex_layers, "fresh_encode": w.fresh_encode,
            "stages_us": res["stages_us"], "step_us_spread": res["step_us_spread"],
            "layer_step_us": res.get("layer_step_us"), "replicas": res["replicas"],
            "step_roofline": {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(step_gbs / HBM_PEAK_GBS, 4), "step_bytes": res["step_bytes"],
                              "ceiling_value": round(ceiling, 1)},
            "scan_roofline": scan_rl}


# ---------------------------------------------------------------- main
CONFIGS = "decode_b1_ctx4k_small,cluster_b32_ctx32k-256k_full1_reindex5,specverify_b64x4_ctx16k-512k_encode64k"
VARIANTS = ("decode_b8_ctx128k_fp4idx,decode_b1_ctx1m_fp4idx,decode_b8_ctx128k_kvg32,chunk_b1x64_ctx128k,"
            "decode_b8_ctx128k_paged64,decode_b1_ctx1m_paged64")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_b8_ctx128k")
    ap.add_argument("--secondary", default="decode_b1_ctx1m", help="second workload ('' to skip)")
    ap.add_argument("--configs", default=CONFIGS, help="the other configurations, each with its oracle figure and "
                                                       "parity ('' to skip)")
    ap.add_argument("--variants", default=VARIANTS,
                    help="comma-separated further workloads reported under 'variants' ('' to skip)")
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas (0: enough for >= 1 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget of the headline "
                                                                    "workload (0 skips every oracle leg)")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0,
                    help="oracle sample budget of the secondary workload and of each configuration")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain fp32 copy of MIB MiB four times (calibrates the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the decode path runs "
              "data-parallel over sequences with no exchange, so N GPUs would run N independent copies; "
              "this build reports the single-GPU figure.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (the HIP library has no CPU path)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 18
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"read_bytes": 4 * n, "write_bytes": 4 * n, "launches": 4}}))
        return

    ceiling = read_ceiling(args.steps)
    print(f"[bench] streaming read: {ceiling['scan_size']['avg_us']} us per {ceiling['scan_size']['bytes']} B "
          f"({ceiling['scan_size']['frac_of_peak']} of 8 TB/s), 1 GiB at {ceiling['1GiB']['frac_of_peak']}",
          file=sys.stderr, flush=True)

    def run(name, cpu_s, one_thread=False, parity_only=False):
        w2 = wl.workload(name)
        st2, step2, res2 = measure(w2, args.steps, args.warmup, args.replicas)
        rec = record(w2, res2)
        print(f"[bench] {w2.name}: {res2['value']:.1f} {rec['unit']}, {res2['ms_per_step'] * 1e3:.1f} us/step, "
              f"scan {res2['scan']['avg_us']} us = {res2['scan']['achieved_gbs']} GB/s", file=sys.stderr, flush=True)
        if args.cpu_seconds > 0:
            cpu, rec["parity"] = cpu_baseline(w2, st2, step2, 0.0 if parity_only else cpu_s, one_thread)
            if not parity_only:
                rec["cpu_baseline"] = cpu
                print(f"[bench] {w2.name} oracle: {cpu['value']:.3f} {cpu['unit']} on {cpu['cores']} threads",
                      file=sys.stderr, flush=True)
            print(f"[bench] {w2.name} parity {rec['parity']}", file=sys.stderr, flush=True)
        del st2, step2
        torch.cuda.empty_cache()
        return w2, res2, rec

    w, res, prim = run(args.workload, args.cpu_seconds, one_thread=True)
    secondary = run(args.secondary, args.config_cpu_seconds)[2] if args.secondary else None
    configs = [run(n, args.config_cpu_seconds, one_thread=(n == "decode_b1_ctx4k_small"))[2]
               for n in args.configs.split(",") if n]
    variants = [run(n, 0.0, parity_only=True)[2] for n in args.variants.split(",") if n]

    d = w.dims
    line = {
        "metric": "decode queries/s at 128K and 1M ctx; indexer-scan HBM GB/s vs peak",
        "value": round(res["value"], 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+f16",
        "dtype_detail": ("indexer: e4m3 keys and queries on the fp8 MFMA (exact products, the instruction's own "
                         "accumulation), fp32 ReLU-weighted head sums; attention: E2M1 x E4M3 KV and bf16 window "
                         "converted exactly to f16 for the MFMAs, fp32 accumulate and softmax, f16 P"),
        "data": "synthetic (seeded N(0,1) fp8 keys and queries, bf16 latents FP4-encoded, U(0,1) weights)",
        "config": {"workload": w.name, "batch": w.n_seq, "tokens_per_seq": w.tokens_per_seq,
                   "ctx": list(w.ctx), "heads": d.n_heads, "idx_heads": d.idx_heads, "idx_dim": d.idx_dim,
                   "pool_blocks": d.pool_blocks, "topk": d.topk, "swa": d.swa,
                   "reindex_layers": w.reindex_layers, "replicas": res["replicas"]},
        "roofline": {"bound": "hbm", "achieved": res["scan"]["achieved_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": res["scan"]["frac"], "traffic": measured_traffic(w.name),
                     "kernel": "k_scan (Full-mode indexer scan)",
                     "bytes_per_launch": res["scan"]["bytes_per_launch"], "avg_us": res["scan"]["avg_us"],
                     "frac_of_read_ceiling": round(res["scan"]["achieved_gbs"] /
                                                   ceiling["scan_size"]["achieved_gbs"], 4)},
        "read_ceiling": ceiling,
        "stages_us": res["stages_us"],
        "step_us_spread": res["step_us_spread"],
        "layer_step_us": res.get("layer_step_us"),
        "step_bytes": res["step_bytes"],
        "step_gbs": res["step_gbs"],
        "step_roofline": prim["step_roofline"],
        "cpu_baseline": prim.get("cpu_baseline"),
        "parity": prim.get("parity"),
        "secondary": secondary,
        "configs": configs,
        "variants": variants,
    }
    if secondary is not None:
        secondary["scan_roofline"]["frac_of_read_ceiling"] = round(
            secondary["scan_roofline"]["achieved"] / ceiling["scan_size"]["achieved_gbs"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
