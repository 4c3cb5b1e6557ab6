"""GPU parity at the full workload sizes, in the benchmark's launch configuration.

One decode step of each full-size workload runs through `bench.Step`, the same
prepared launches that bench.py times:
- the Full scan with the scan-prepared pool workspace, then the pool select;
- Reindex and attention for each layer (five fresh-Q layers in the cluster
  workload);
- the 65,536-entry FP4 encode of the speculative-verify workload.

Sampled queries are then checked one by one against the oracle: pool and
Top-K sets (equal up to the 1e-5 tie band), and attention within 2e-3 of
max|ref| per head. Sampled encoded rows must be bit-exact.

Downstream stages of a query are compared only when its upstream set equals
the oracle's exactly; the GPU's own outputs are never fed to the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._harness import (OracleQuery, check_attention, check_set, lib, u8, u16, with_oracle_pool,
                            with_oracle_rows)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# sampled queries per workload: first and last sequences, and for the
# speculative-verify workload all four tokens of one sequence
SAMPLES = {
    "decode_b8_ctx128k": [0, 7],
    "decode_b1_ctx1m": [0],
    "cluster_b32_ctx32k-256k_full1_reindex5": [0, 19, 31],
    "specverify_b64x4_ctx16k-512k_encode64k": [0, 1, 2, 3, 254],
    "decode_b8_ctx128k_fp4idx": [0, 7],
    "decode_b1_ctx1m_fp4idx": [0],
    "decode_b8_ctx128k_kvg32": [0, 7],
    "chunk_b1x64_ctx128k": [0, 31, 63],
    # every per-position plane in shuffled pages of 64 positions (paged calls)
    "decode_b8_ctx128k_paged64": [0, 7],
    "decode_b1_ctx1m_paged64": [0],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_step(name):
    lib()
    from bench import DeviceState, Step
    w = wl.workload(name)
    st = DeviceState(w, replicas=1)
    step = Step(st)
    step.run(0)
    torch.cuda.synchronize()
    pool, pcnt = step.pool.cpu().numpy(), step.pcnt.cpu().numpy()
    tk, tc = step.tk.cpu().numpy(), step.tc.cpu().numpy()
    out, lse = step.out.cpu().numpy(), step.lse.cpu().numpy()
    lay = st.lay
    checked_attn = 0
    keys = {}
    for qi in SAMPLES[name]:
        seq = qi // w.tokens_per_seq
        oq = OracleQuery(w, lay, qi, keys.get(seq))
        keys = {seq: oq.keys}
        rpool, rb, _ = oq.full(0)
        got_pool = pool[qi, :pcnt[qi]]
        check_set(got_pool, rpool, lambda j: rb[j], f"{name} q{qi} pool")
        assert np.all(pool[qi, pcnt[qi]:] == -1)
        same_pool = np.array_equal(got_pool, rpool)
        for i, layer in enumerate(step.layers):
            keep, _, _ = oq.reindex(layer, rpool)
            got = tk[i, qi, :tc[i, qi]]
            if not same_pool:
                # the pools differ inside the band: this layer's Top-K from the
                # library's Reindex (this layer's query) on the oracle's pool
                p2, c2 = with_oracle_pool(step.pool, step.pcnt, {qi: rpool})
                tk_o, tc_o, _ = st.reindex(layer, p2, c2)
                torch.cuda.synchronize()
                got = tk_o[qi, :int(tc_o[qi])].cpu().numpy()
            check_set(got, keep, lambda p: oq.scores_at(layer, p), f"{name} q{qi} layer {layer} topk")
            ro, rl = oq.attention(layer, keep)
            if same_pool and np.array_equal(got, keep):
                o_q, l_q = out[i, qi], lse[i, qi]
            else:
                # the same attention call on the oracle's own Top-K
                tk2, tc2 = with_oracle_rows(step.tk[i], step.tc[i], {qi: keep})
                o2, l2 = st.attend(layer, tk2, tc2)
                o_q, l_q = o2[qi].cpu().numpy(), l2[qi].cpu().numpy()
            check_attention(o_q, l_q, ro, rl, f"{name} q{qi} layer {layer}")
            checked_attn += 1
    assert checked_attn > 0, f"{name}: no sampled query reached the attention check"

    if w.fresh_encode:
        # the step's fresh entries: sampled rows bit-exact against the oracle's encoder
        codes, scales, rope = (t.cpu() for t in step.enc_planes)
        n = w.fresh_encode
        for e0 in (0, n // 2 - 128, n - 256):
            rows = slice(e0, e0 + 256)
            ref_c, ref_s = oracle.encode_kv(u16(wl.fresh_latent(w, 0, e0, 256)), w.dims.kv_group)
            assert np.array_equal(u8(codes[rows]), ref_c), f"{name}: encoded codes differ at rows {e0}+"
            assert np.array_equal(u8(scales[rows]), ref_s), f"{name}: encoded scales differ at rows {e0}+"
            assert np.array_equal(u16(rope[rows]), u16(wl.fresh_rope(w, 0, e0, 256))), f"{name}: rope copy"
    del step, st
    torch.cuda.empty_cache()
