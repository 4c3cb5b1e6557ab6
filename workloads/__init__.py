"""Seeded synthetic inputs for the CSA2 decode path.

This module is shared by the oracle-side tests and the GPU path. It holds the
workload shapes and a counter-based random generator, and nothing of the
method's own arithmetic: no encoding, scoring, selection or attention.

Generator
---------
Every tensor is a function of (workload key, stream name, flat element index).
The uniform source is SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used in counter mode: element i
of a stream with seed z0 is mix64(z0 + (i + 1) * gamma).  Because it is
integer-only, the same code gives bit-identical values in torch on the CPU and
on the GPU, and any row range can be regenerated without generating the rows
before it.

Gaussian values come from inverse-transform sampling: the top 20 bits of the
64-bit output index a table of the 2^20 mid-point quantiles of N(0,1), computed
once on the CPU in float64 and stored already rounded to the element type
(bf16 or fp8 e4m3fn).  The table lookup is exact on every device, so the GPU
and the CPU produce the same bytes.  Tails are truncated at about +-4.9 sigma.

Uniform U(0,1) floats use the top 24 bits (exact in float32).  Context lengths
U{lo..hi} use the 53 high bits modulo the range width.
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Dict, List, Optional, Tuple

import torch

__all__ = [
    "Dims", "Workload", "WORKLOADS", "workload", "Layout", "layout",
    "idx_keys", "latent", "rope", "idx_query", "idx_weight", "q_latent",
    "q_rope", "fresh_latent", "fresh_rope", "swa_rows", "mix64_reference",
    "latent_at", "rope_at", "idx_keys_bf16", "idx_query_bf16",
]

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB


def _s64(u: int) -> int:
    """Unsigned 64-bit constant as the signed int64 torch stores."""
    u &= _MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def mix64_reference(z: int) -> int:
    """SplitMix64 finaliser on Python ints (the published definition)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _C1) & _MASK64
    z = ((z ^ (z >> 27)) * _C2) & _MASK64
    return z ^ (z >> 31)


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    # logical right shift on int64 (torch's >> is arithmetic)
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _s64(_C1)
    z = (z ^ _srl(z, 27)) * _s64(_C2)
    return z ^ _srl(z, 31)


def _stream_seed(key: int, name: str) -> int:
    return mix64_reference((key << 32) ^ zlib.crc32(name.encode()))


def _bits(seed: int, start: int, count: int, device) -> torch.Tensor:
    i = torch.arange(start + 1, start + 1 + count, dtype=torch.int64, device=device)
    return _mix64(i * _s64(_GAMMA) + _s64(seed))


# ---------------------------------------------------------------- tables
_TABLE_BITS = 20
_tables: Dict[Tuple[str, str], torch.Tensor] = {}


def _table(kind: str, device) -> torch.Tensor:
    dev = str(torch.device(device))
    k = (kind, dev)
    if k not in _tables:
        if ("quantile", "cpu") not in _tables:
            u = (torch.arange(1 << _TABLE_BITS, dtype=torch.float64) + 0.5) / (1 << _TABLE_BITS)
            _tables[("quantile", "cpu")] = torch.special.ndtri(u)
        qn = _tables[("quantile", "cpu")]
        if kind == "bf16":
            t = qn.to(torch.float32).to(torch.bfloat16)
        elif kind == "bf16/24":  # N(0,1)/sqrt(576)
            t = (qn / 24.0).to(torch.float32).to(torch.bfloat16)
        elif kind == "e4m3":
            t = qn.to(torch.float32).to(torch.float8_e4m3fn)
        else:
            raise KeyError(kind)
        _tables[(kind, "cpu")] = t
        _tables[k] = t.to(device)
    return _tables[k]


def _normal(kind: str, seed: int, start: int, count: int, device) -> torch.Tensor:
    idx = _srl(_bits(seed, start, count, device), 64 - _TABLE_BITS)
    return _table(kind, device)[idx]


def _normal_at(kind: str, seed: int, idx: torch.Tensor) -> torch.Tensor:
    """Values at arbitrary flat element indices (int64 tensor)."""
    z = _mix64((idx + 1) * _s64(_GAMMA) + _s64(seed))
    return _table(kind, idx.device)[_srl(z, 64 - _TABLE_BITS)]


def _uniform01(seed: int, start: int, count: int, device) -> torch.Tensor:
    v = _srl(_bits(seed, start, count, device), 40)
    return v.to(torch.float32) * (1.0 / (1 << 24))


def _uniform_int(seed: int, lo: int, hi: int, count: int) -> List[int]:
    v = _srl(_bits(seed, 0, count, "cpu"), 11)
    return [lo + int(x) % (hi - lo + 1) for x in v.tolist()]


# ---------------------------------------------------------------- shapes
@dataclasses.dataclass(frozen=True)
class Dims:
    n_heads: int          # H, main attention heads
    idx_heads: int        # H_i, indexer heads
    idx_dim: int          # d_i, indexer key/query width
    pool_blocks: int      # P, candidate blocks kept by the Full indexer
    topk: int             # K, positions kept by Reindex
    swa: int = 128        # W, sliding-window rows
    d_latent: int = 512
    d_rope: int = 64
    block: int = 8
    kv_group: int = 16    # channels per main-KV FP4 scale (32: the group-32 codec variant)


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    dims: Dims
    n_seq: int
    ctx: Tuple[int, int]          # fixed (lo == hi) or uniform U{lo..hi}
    tokens_per_seq: int = 1       # consecutive causal query tokens per sequence
    reindex_layers: int = 1       # Reindex+Attend layers after the Full scan
    fresh_q_per_layer: bool = False  # True: every Reindex layer draws new Q
    fresh_encode: int = 0         # entries encoded by each step
    ctx_list: Optional[Tuple[int, ...]] = None   # explicit contexts (tests)
    idx_fp4: bool = False         # indexer rows in FP4 (from idx_keys_bf16 / idx_query_bf16)
    page_size: int = 0            # > 0: per-position planes in pages of this many positions, shuffled

    @property
    def key(self) -> int:
        return 0xC5A20000 + self.index

    @property
    def n_q(self) -> int:
        return self.n_seq * self.tokens_per_seq


_BIG = Dims(n_heads=64, idx_heads=64, idx_dim=128, pool_blocks=2048, topk=512)

WORKLOADS: List[Workload] = [
    Workload(0, "decode_b1_ctx4k_small",
             Dims(n_heads=16, idx_heads=8, idx_dim=64, pool_blocks=64, topk=128),
             n_seq=1, ctx=(4096, 4096)),
    Workload(1, "decode_b8_ctx128k", _BIG, n_seq=8, ctx=(131072, 131072)),
    Workload(2, "decode_b1_ctx1m", _BIG, n_seq=1, ctx=(1048576, 1048576)),
    Workload(3, "cluster_b32_ctx32k-256k_full1_reindex5", _BIG, n_seq=32,
             ctx=(32768, 262144), reindex_layers=5, fresh_q_per_layer=True),
    Workload(4, "specverify_b64x4_ctx16k-512k_encode64k", _BIG, n_seq=64,
             ctx=(16384, 524288), tokens_per_seq=4, fresh_encode=65536),
    # the FP4 indexer variant of the two decode workloads
    Workload(5, "decode_b8_ctx128k_fp4idx", _BIG, n_seq=8, ctx=(131072, 131072), idx_fp4=True),
    Workload(6, "decode_b1_ctx1m_fp4idx", _BIG, n_seq=1, ctx=(1048576, 1048576), idx_fp4=True),
    # the group-32 main-KV codec variant of the batch-8 decode workload
    Workload(7, "decode_b8_ctx128k_kvg32", dataclasses.replace(_BIG, kv_group=32), n_seq=8,
             ctx=(131072, 131072)),
    # many query tokens against one cache (a 64-token chunk at 128K context)
    Workload(8, "chunk_b1x64_ctx128k", _BIG, n_seq=1, ctx=(131072, 131072), tokens_per_seq=64),
    # the decode workloads over paged caches (pages of 64 positions in a shuffled physical order)
    Workload(9, "decode_b8_ctx128k_paged64", _BIG, n_seq=8, ctx=(131072, 131072), page_size=64),
    Workload(10, "decode_b1_ctx1m_paged64", _BIG, n_seq=1, ctx=(1048576, 1048576), page_size=64),
    Workload(11, "decode_b8_ctx128k_paged256", _BIG, n_seq=8, ctx=(131072, 131072), page_size=256),
    Workload(12, "decode_b1_ctx1m_paged256", _BIG, n_seq=1, ctx=(1048576, 1048576), page_size=256),
]


def workload(k) -> Workload:
    if isinstance(k, int):
        return WORKLOADS[k]
    for w in WORKLOADS:
        if w.name == k:
            return w
    raise KeyError(k)


@dataclasses.dataclass
class Layout:
    """Row layout of the flat caches for one workload (host-side integers).

    Sequence s owns cache rows [seq_base[s], seq_base[s] + seq_rows[s]);
    query token j of sequence s sees positions [0, ctx[s] + j).  The
    sliding-window buffer holds, per sequence, positions
    [swa_lo[s], ctx[s] + tokens_per_seq - 1) at rows starting swa_seq_base[s].
    """
    ctx: List[int]
    seq_base: List[int]
    seq_rows: List[int]
    rows: int
    q_seq_base: List[int]
    q_visible: List[int]
    swa_lo: List[int]
    swa_seq_base: List[int]
    swa_rows: int
    q_swa_base: List[int]


def layout(w: Workload, n_seq: Optional[int] = None) -> Layout:
    """Row layout; `n_seq` keeps only the first sequences (same values)."""
    ns = w.n_seq if n_seq is None else n_seq
    lo, hi = w.ctx
    if w.ctx_list is not None:
        ctx = list(w.ctx_list)
    elif lo == hi:
        ctx = [lo] * w.n_seq
    else:
        ctx = _uniform_int(_stream_seed(w.key, "ctx"), lo, hi, w.n_seq)
    ctx = ctx[:ns]
    g, W = w.tokens_per_seq, w.dims.swa
    seq_rows = [c + g - 1 for c in ctx]
    seq_base, acc = [], 0
    for r in seq_rows:
        seq_base.append(acc)
        acc += r
    swa_lo = [max(0, c - W) for c in ctx]
    swa_seq_base, sacc = [], 0
    for c, l in zip(ctx, swa_lo):
        swa_seq_base.append(sacc)
        sacc += c + g - 1 - l
    q_seq_base, q_visible, q_swa = [], [], []
    for s in range(ns):
        for j in range(g):
            n = ctx[s] + j
            q_seq_base.append(seq_base[s])
            q_visible.append(n)
            q_swa.append(swa_seq_base[s] + max(0, n - W) - swa_lo[s])
    return Layout(ctx, seq_base, seq_rows, acc, q_seq_base, q_visible,
                  swa_lo, swa_seq_base, sacc, q_swa)


# ---------------------------------------------------------------- tensors
def idx_keys(w: Workload, row0: int, nrows: int, device="cpu") -> torch.Tensor:
    """Indexer keys, fp8 e4m3fn [nrows, d_i], N(0,1) rounded to e4m3fn."""
    d = w.dims.idx_dim
    s = _stream_seed(w.key, "idx_k")
    return _normal("e4m3", s, row0 * d, nrows * d, device).view(nrows, d)


def idx_keys_bf16(w: Workload, row0: int, nrows: int, device="cpu") -> torch.Tensor:
    """Indexer keys before FP4 encoding (FP4 indexer variant), bf16
    [nrows, d_i], N(0,1)."""
    d = w.dims.idx_dim
    s = _stream_seed(w.key, "idx_k_bf16")
    return _normal("bf16", s, row0 * d, nrows * d, device).view(nrows, d)


def idx_query_bf16(w: Workload, layer: int, q0: int, nq: int, device="cpu") -> torch.Tensor:
    """Indexer query before FP4 encoding (FP4 indexer variant), bf16
    [nq, H_i, d_i], N(0,1)."""
    hi, d = w.dims.idx_heads, w.dims.idx_dim
    s = _stream_seed(w.key, f"idx_q_bf16/{layer}")
    return _normal("bf16", s, q0 * hi * d, nq * hi * d, device).view(nq, hi, d)


def latent(w: Workload, row0: int, nrows: int, device="cpu") -> torch.Tensor:
    """Main-KV latent before encoding, bf16 [nrows, 512], N(0,1)."""
    d = w.dims.d_latent
    s = _stream_seed(w.key, "lat")
    return _normal("bf16", s, row0 * d, nrows * d, device).view(nrows, d)


def rope(w: Workload, row0: int, nrows: int, device="cpu") -> torch.Tensor:
    """Main-KV RoPE key, bf16 [nrows, 64], N(0,1)."""
    d = w.dims.d_rope
    s = _stream_seed(w.key, "rope")
    return _normal("bf16", s, row0 * d, nrows * d, device).view(nrows, d)


def _rows_at(rows, width: int, device) -> torch.Tensor:
    r = torch.as_tensor(rows, dtype=torch.int64, device=device).reshape(-1, 1)
    return r * width + torch.arange(width, dtype=torch.int64, device=device)


def latent_at(w: Workload, rows, device="cpu") -> torch.Tensor:
    """latent() at arbitrary cache rows (int64 sequence) -> bf16 [len, 512]."""
    return _normal_at("bf16", _stream_seed(w.key, "lat"), _rows_at(rows, w.dims.d_latent, device))


def rope_at(w: Workload, rows, device="cpu") -> torch.Tensor:
    return _normal_at("bf16", _stream_seed(w.key, "rope"), _rows_at(rows, w.dims.d_rope, device))


def idx_query(w: Workload, layer: int, q0: int, nq: int, device="cpu") -> torch.Tensor:
    """Indexer query for `layer`, fp8 e4m3fn [nq, H_i, d_i], N(0,1)."""
    hi, d = w.dims.idx_heads, w.dims.idx_dim
    s = _stream_seed(w.key, f"idx_q/{layer}")
    return _normal("e4m3", s, q0 * hi * d, nq * hi * d, device).view(nq, hi, d)


def idx_weight(w: Workload, layer: int, q0: int, nq: int, device="cpu") -> torch.Tensor:
    """Per-head indexer weights for `layer`, f32 [nq, H_i], U(0,1)."""
    hi = w.dims.idx_heads
    s = _stream_seed(w.key, f"idx_w/{layer}")
    return _uniform01(s, q0 * hi, nq * hi, device).view(nq, hi)


def q_latent(w: Workload, layer: int, q0: int, nq: int, device="cpu") -> torch.Tensor:
    """Main query latent part, bf16 [nq, H, 512], N(0,1)/sqrt(576)."""
    h, d = w.dims.n_heads, w.dims.d_latent
    s = _stream_seed(w.key, f"q_lat/{layer}")
    return _normal("bf16/24", s, q0 * h * d, nq * h * d, device).view(nq, h, d)


def q_rope(w: Workload, layer: int, q0: int, nq: int, device="cpu") -> torch.Tensor:
    """Main query RoPE part, bf16 [nq, H, 64], N(0,1)/sqrt(576)."""
    h, d = w.dims.n_heads, w.dims.d_rope
    s = _stream_seed(w.key, f"q_rope/{layer}")
    return _normal("bf16/24", s, q0 * h * d, nq * h * d, device).view(nq, h, d)


def fresh_latent(w: Workload, step: int, e0: int, n: int, device="cpu") -> torch.Tensor:
    """Freshly appended latent entries of `step`, bf16 [n, 512], N(0,1)."""
    d = w.dims.d_latent
    s = _stream_seed(w.key, f"enc_src/{step}")
    return _normal("bf16", s, e0 * d, n * d, device).view(n, d)


def fresh_rope(w: Workload, step: int, e0: int, n: int, device="cpu") -> torch.Tensor:
    d = w.dims.d_rope
    s = _stream_seed(w.key, f"enc_rope/{step}")
    return _normal("bf16", s, e0 * d, n * d, device).view(n, d)


def swa_rows(w: Workload, lay: Layout, seq: int, device="cpu") -> torch.Tensor:
    """Window rows of one sequence: bf16 [rows, 576] = latent || rope of the
    positions [swa_lo, ctx + tokens_per_seq - 1), the values before encoding."""
    p0 = lay.swa_lo[seq]
    n = lay.ctx[seq] + w.tokens_per_seq - 1 - p0
    r0 = lay.seq_base[seq] + p0
    return torch.cat([latent(w, r0, n, device), rope(w, r0, n, device)], dim=1)
