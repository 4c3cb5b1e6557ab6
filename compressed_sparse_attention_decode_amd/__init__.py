"""CSA2 decode path on AMD MI355X (gfx950): Python binding of libcsa2.so.

Argument marshalling only: every step of the path runs in the library's HIP
kernels (see include/csa2.h for the contracts).  torch supplies device memory
and the current HIP stream.  There is no CPU fallback: if the library is not
built, or the device is not gfx950, every call raises.

    encode_kv      FP4 main-KV encode (E2M1 + one E4M3 scale per 16 channels)
    encode_fp4     the same codec for rows of any width (FP4 indexer rows)
    index_full     Full-mode indexer: scores, block-of-8 maxima, Top-P pool
    index_reindex  Reindex inside the pool: Top-K positions
    attend         sparse FP4 + sliding-window attention, one softmax

The indexer calls take their query and key rows either as float8_e4m3fn
tensors or, for the FP4 indexer variant, as (codes, scales) uint8 pairs
written by encode_fp4 at width d_i.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

__all__ = ["Dims", "Batch", "Csa2Error", "lib", "lib_path", "encode_kv", "encode_fp4", "index_full",
           "index_scan", "index_pool", "n_blocks", "block_scores_ld", "workspace_pool",
           "index_reindex", "attend", "workspace_full", "workspace_reindex",
           "workspace_attend", "abi_version", "Call", "decode_step", "workspace_step", "Pages", "page_rows",
           "LAYER_FULL", "LAYER_REINDEX", "LAYER_REUSE", "stream_read", "decode_step_noalloc", "index_topk_keys", "pos_keys_ld"]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libcsa2.so")


class Csa2Error(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_heads", "d_latent", "d_rope", "idx_heads", "idx_dim", "block",
                 "pool_blocks", "topk", "swa", "kv_group")]


class _Queries(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("tokens_per_seq", ctypes.c_int32),
                ("max_visible", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("seq_base", ctypes.c_void_p), ("n_visible", ctypes.c_void_p)]


_lib = None


class _Pages(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rows", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    """Load libcsa2.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise Csa2Error(f"{lib_path} is not built; run __graft_entry__.build() "
                            "or python -m compressed_sparse_attention_decode_amd._build")
        L = ctypes.CDLL(lib_path)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        PD, PQ, PP = ctypes.POINTER(_Dims), ctypes.POINTER(_Queries), ctypes.POINTER(_Pages)
        sig = {
            "csa2_abi_version": (I32, []),
            "csa2_status_string": (ctypes.c_char_p, [I32]),
            "csa2_last_error": (ctypes.c_char_p, []),
            "csa2_encode_kv": (I32, [I64, P, P, P, P, P, P, P]),
            "csa2_encode_kv_grouped": (I32, [I64, I32, P, P, P, P, P, P, P]),
            "csa2_encode_fp4": (I32, [I64, I32, P, P, P, P, P]),
            "csa2_index_scan": (I32, [PD, PQ, P, P, P, P, I64, P, SZ, P]),
            "csa2_index_scan_fp4": (I32, [PD, PQ, P, P, P, P, P, P, I64, P, SZ, P]),
            "csa2_index_pool_workspace_size": (I32, [PD, PQ, ctypes.POINTER(SZ)]),
            "csa2_index_pool": (I32, [PD, PQ, P, I64, P, P, P, SZ, I32, P]),
            "csa2_index_full_workspace_size": (I32, [PD, PQ, ctypes.POINTER(SZ)]),
            "csa2_index_full": (I32, [PD, PQ, P, P, P, P, P, P, I64, P, SZ, P]),
            "csa2_index_full_fp4": (I32, [PD, PQ, P, P, P, P, P, P, P, P, I64, P, SZ, P]),
            "csa2_index_reindex_workspace_size": (I32, [PD, PQ, ctypes.POINTER(SZ)]),
            "csa2_index_reindex": (I32, [PD, PQ, P, P, P, P, P, P, P, P, P, SZ, P]),
            "csa2_index_reindex_fp4": (I32, [PD, PQ, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
            "csa2_attend_workspace_size": (I32, [PD, PQ, ctypes.POINTER(SZ)]),
            "csa2_attend": (I32, [PD, PQ, P, P, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, SZ, P]),
            "csa2_index_reindex_paged": (I32, [PD, PQ, PP, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
            "csa2_attend_paged": (I32, [PD, PQ, PP, P, P, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, SZ, P]),
            "csa2_page_rows": (I32, [PP, I64, P, P, P, P]),
            "csa2_index_full_paged": (I32, [PD, PQ, PP, P, P, P, P, P, P, P, P, I64, P, SZ, P]),
            "csa2_index_scan_paged": (I32, [PD, PQ, PP, P, P, P, P, P, P, I64, P, SZ, P]),
            "csa2_decode_step_paged": (I32, [PD, PQ, PP, I32, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float,
                                             P, P, P, P, P, P, P, P, SZ, P]),
            "csa2_decode_step_workspace_size": (I32, [PD, PQ, ctypes.POINTER(SZ)]),
            "csa2_decode_step": (I32, [PD, PQ, I32, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float,
                                       P, P, P, P, P, P, P, P, SZ, P]),
            "csa2_stream_read": (I32, [P, I64, P, P]),
            "csa2_index_scan_keys": (I32, [PD, PQ, PP, P, P, P, P, P, P, I64, P, I64, P, SZ, P]),
            "csa2_index_topk_keys": (I32, [PD, PQ, P, P, P, I64, P, I64, P, P, P, P]),
            "csa2_index_pool_topk": (I32, [PD, PQ, P, I64, P, I64, P, P, P, P, P, SZ, I32, P]),
            "csa2_pool_topk_attend": (I32, [PD, PQ, P, I64, P, I64, P, P, P, P, P, P, ctypes.c_float, P, P, P,
                                            P, P, P, P, P, SZ, I32, P, SZ, P]),
            "csa2_reindex_attend": (I32, [PD, PQ, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P,
                                          P, P, P, SZ, P, SZ, P]),
            "csa2_pool_topk_attend_paged": (I32, [PD, PQ, PP, P, I64, P, I64, P, P, P, P, P, P, ctypes.c_float, P,
                                                  P, P, P, P, P, P, P, SZ, I32, P, SZ, P]),
            "csa2_reindex_attend_paged": (I32, [PD, PQ, PP, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P,
                                                P, P, P, P, P, P, SZ, P, SZ, P]),
            "csa2_decode_step_noalloc": (I32, [PD, PQ, I32, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float,
                                               P, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().csa2_abi_version()


class Call:
    """A library call with its arguments marshalled once: calling it re-issues
    the same launch on the same stream (for serving loops and benchmarks that
    reuse buffers).  Keeps the ctypes structs it points to alive."""

    def __init__(self, fn, args, keep=()):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            _check(st)


def _issue(fn, args, keep, prepare: bool):
    if prepare:
        return Call(fn, args, keep)
    _check(fn(*args))
    return None


def _check(st: int):
    if st != 0:
        L = lib()
        raise Csa2Error(f"{L.csa2_status_string(st).decode()}: {L.csa2_last_error().decode()}")


@dataclasses.dataclass(frozen=True)
class Dims:
    n_heads: int
    idx_heads: int
    idx_dim: int
    pool_blocks: int
    topk: int
    swa: int = 128
    d_latent: int = 512
    d_rope: int = 64
    block: int = 8
    kv_group: int = 16        # channels per main-KV FP4 scale (16, or 32 for the group-32 codec)

    def c(self) -> _Dims:
        return _Dims(self.n_heads, self.d_latent, self.d_rope, self.idx_heads, self.idx_dim,
                     self.block, self.pool_blocks, self.topk, self.swa, self.kv_group)


@dataclasses.dataclass
class Batch:
    """Decode queries: device int64 seq_base [n_q], int32 n_visible [n_q]."""
    seq_base: torch.Tensor
    n_visible: torch.Tensor
    max_visible: int
    tokens_per_seq: int = 1

    @property
    def n_q(self) -> int:
        return self.n_visible.numel()

    def c(self) -> _Queries:
        if self.seq_base.dtype != torch.int64 or self.n_visible.dtype != torch.int32:
            raise TypeError("seq_base must be int64 and n_visible int32")
        _dev(self.seq_base, self.n_visible)
        return _Queries(self.n_q, self.tokens_per_seq, self.max_visible, 0,
                        self.seq_base.data_ptr(), self.n_visible.data_ptr())


@dataclasses.dataclass
class Pages:
    """Paged per-position planes (csa2_pages): device int32 `table` of
    physical page ids; position p of a query's sequence is row
    table[seq_base + p // page_size] * page_size + p % page_size, where the
    Batch's seq_base then holds each query's offset in `table`.  `rows` is
    the row count of every plane the call reads."""
    table: torch.Tensor
    page_size: int
    rows: int

    def c(self) -> _Pages:
        if self.table.dtype != torch.int32 or not self.table.is_contiguous():
            raise TypeError("the page table must be contiguous int32")
        _dev(self.table)
        return _Pages(self.table.data_ptr(), self.page_size, 0, self.rows)


def _check_page_rows(pages: Pages, *planes: torch.Tensor):
    rows = min(t.shape[0] for t in planes)
    if pages.rows > rows:
        raise ValueError(f"pages.rows ({pages.rows}) exceeds the planes' {rows} rows")


def page_rows(pages: Pages, table_off: torch.Tensor, pos: torch.Tensor,
              dst_row: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows of (table offset, position) pairs in paged planes
    (csa2_page_rows), e.g. as encode_kv's dst_row to append into pages."""
    _dev(table_off, pos, dst_row)
    if table_off.dtype != torch.int64 or pos.dtype != torch.int32 or table_off.shape != pos.shape:
        raise TypeError("table_off must be int64 and pos int32, of one shape")
    n = pos.numel()
    if dst_row is None:
        dst_row = torch.empty(n, dtype=torch.int64, device=pos.device)
    pg = pages.c()
    _check(lib().csa2_page_rows(ctypes.byref(pg), n, table_off.data_ptr(), pos.data_ptr(), dst_row.data_ptr(),
                                _stream(pos.device)))
    return dst_row


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError("CSA2 tensors must live on the GPU")
        if not t.is_contiguous():
            raise TypeError("CSA2 tensors must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ws_size(fn, dims: Dims, b: Batch) -> int:
    n = ctypes.c_size_t(0)
    d, q = dims.c(), b.c()
    _check(fn(ctypes.byref(d), ctypes.byref(q), ctypes.byref(n)))
    return n.value


def workspace_full(dims: Dims, b: Batch) -> int:
    return _ws_size(lib().csa2_index_full_workspace_size, dims, b)


def workspace_pool(dims: Dims, b: Batch) -> int:
    return _ws_size(lib().csa2_index_pool_workspace_size, dims, b)


def workspace_reindex(dims: Dims, b: Batch) -> int:
    return _ws_size(lib().csa2_index_reindex_workspace_size, dims, b)


def workspace_attend(dims: Dims, b: Batch) -> int:
    return _ws_size(lib().csa2_attend_workspace_size, dims, b)


def workspace_step(dims: Dims, b: Batch) -> int:
    return _ws_size(lib().csa2_decode_step_workspace_size, dims, b)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() * ws.element_size() < nbytes:
        # zero-filled: the Reindex and attention workspaces start with counters that must
        # read zero on first use (each call leaves them so)
        ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    return ws


def _ws_ptr(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    off = (-p) % 256
    return p + off, ws.numel() * ws.element_size() - off


def encode_kv(latent: torch.Tensor, rope: torch.Tensor, kv_codes: torch.Tensor,
              kv_scales: torch.Tensor, kv_rope: torch.Tensor,
              dst_row: Optional[torch.Tensor] = None, prepare: bool = False, group: int = 16):
    """Encode bf16 latent [n, 512] (+ rope [n, 64]) into the FP4 cache planes
    kv_codes uint8 [rows, 256], kv_scales uint8 [rows, 512/group], kv_rope
    bf16 [rows, 64] at rows dst_row (int64 [n]) or 0..n-1."""
    _dev(latent, rope, kv_codes, kv_scales, kv_rope, dst_row)
    if latent.dtype != torch.bfloat16 or rope.dtype != torch.bfloat16 or kv_rope.dtype != torch.bfloat16:
        raise TypeError("latent, rope and kv_rope must be bfloat16")
    n = latent.shape[0]
    if latent.shape != (n, 512) or rope.shape != (n, 64):
        raise ValueError("latent must be [n, 512] and rope [n, 64]")
    rows = kv_codes.shape[0]
    if group not in (16, 32):
        raise ValueError("group must be 16 or 32")
    if kv_codes.shape != (rows, 256) or kv_scales.shape != (rows, 512 // group) or kv_rope.shape != (rows, 64):
        raise ValueError("cache planes must be [rows, 256] / [rows, 512/group] / [rows, 64]")
    if dst_row is None and n > rows:
        raise ValueError("more entries than cache rows")
    if dst_row is not None and (dst_row.dtype != torch.int64 or dst_row.shape != (n,)):
        raise ValueError("dst_row must be int64 [n]")
    args = (n, group, latent.data_ptr(), rope.data_ptr(), _ptr(dst_row), kv_codes.data_ptr(),
            kv_scales.data_ptr(), kv_rope.data_ptr(), _stream(latent.device))
    return _issue(lib().csa2_encode_kv_grouped, args, (), prepare)


def encode_fp4(src: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
               dst_row: Optional[torch.Tensor] = None, prepare: bool = False):
    """Encode bf16 rows [n, width] into FP4 planes codes uint8 [rows, width/2]
    and scales uint8 [rows, width/16] at rows dst_row (int64 [n]) or 0..n-1."""
    _dev(src, codes, scales, dst_row)
    if src.dtype != torch.bfloat16 or src.dim() != 2:
        raise TypeError("src must be bfloat16 [n, width]")
    n, width = src.shape
    rows = codes.shape[0]
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or codes.shape != (rows, width // 2) \
            or scales.shape != (rows, width // 16):
        raise ValueError("codes / scales must be uint8 [rows, width/2] / [rows, width/16]")
    if dst_row is None and n > rows:
        raise ValueError("more rows than the planes hold")
    if dst_row is not None and (dst_row.dtype != torch.int64 or dst_row.shape != (n,)):
        raise ValueError("dst_row must be int64 [n]")
    args = (n, width, src.data_ptr(), _ptr(dst_row), codes.data_ptr(), scales.data_ptr(), _stream(src.device))
    return _issue(lib().csa2_encode_fp4, args, (), prepare)


def _rows_dev(x) -> torch.device:
    return x[0].device if isinstance(x, tuple) else x.device


def _check_idx(dims: Dims, b: Batch, idx_q, idx_w, idx_k):
    """Validates the indexer rows; returns (fp4, [q ptr(s)], [k ptr(s)]).
    fp8: float8_e4m3fn tensors; FP4: (codes, scales) uint8 pairs."""
    n_q, hi, d = b.n_q, dims.idx_heads, dims.idx_dim
    if idx_w.dtype != torch.float32 or idx_w.shape != (n_q, hi):
        raise ValueError("idx_w must be float32 [n_q, H_i]")
    _dev(idx_w)
    if isinstance(idx_q, tuple) != isinstance(idx_k, tuple):
        raise TypeError("idx_q and idx_k must both be fp8 tensors or both FP4 (codes, scales) pairs")
    if isinstance(idx_q, tuple):
        (qc, qs), (kc, ks) = idx_q, idx_k
        _dev(qc, qs, kc, ks)
        if any(t.dtype != torch.uint8 for t in (qc, qs, kc, ks)):
            raise TypeError("FP4 codes and scales must be uint8")
        if qc.shape != (n_q, hi, d // 2) or qs.shape != (n_q, hi, d // 16):
            raise ValueError("FP4 query must be [n_q, H_i, d_i/2] codes and [n_q, H_i, d_i/16] scales")
        if kc.dim() != 2 or kc.shape[1] != d // 2 or ks.shape != (kc.shape[0], d // 16):
            raise ValueError("FP4 keys must be [rows, d_i/2] codes and [rows, d_i/16] scales")
        return True, [qc.data_ptr(), qs.data_ptr()], [kc.data_ptr(), ks.data_ptr()]
    _dev(idx_q, idx_k)
    if idx_q.dtype != torch.float8_e4m3fn or idx_k.dtype != torch.float8_e4m3fn:
        raise TypeError("idx_q and idx_k must be float8_e4m3fn")
    if idx_q.shape != (n_q, hi, d):
        raise ValueError("idx_q / idx_w shape mismatch")
    if idx_k.dim() != 2 or idx_k.shape[1] != d:
        raise ValueError("idx_k must be [rows, d_i]")
    return False, [idx_q.data_ptr()], [idx_k.data_ptr()]


def index_full(dims: Dims, b: Batch, idx_q, idx_w: torch.Tensor, idx_k,
               pool_blocks: Optional[torch.Tensor] = None, pool_count: Optional[torch.Tensor] = None,
               block_scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
               pages: Optional[Pages] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Full-mode indexer. idx_q fp8 [n_q, H_i, d_i] (or an FP4 pair),
    idx_w f32 [n_q, H_i], idx_k fp8 [rows, d_i] (or an FP4 pair).  Returns
    (pool_blocks int32 [n_q, P], pool_count).  With `pages` the keys are
    paged (csa2_index_full_paged)."""
    dev = _rows_dev(idx_k)
    _dev(pool_blocks, pool_count, block_scores)
    n_q = b.n_q
    fp4, qp, kp = _check_idx(dims, b, idx_q, idx_w, idx_k)
    if pool_blocks is None:
        pool_blocks = torch.empty(n_q, dims.pool_blocks, dtype=torch.int32, device=dev)
    if pool_count is None:
        pool_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    ld = 0
    if block_scores is not None:
        if block_scores.dtype != torch.float32 or block_scores.dim() != 2 or block_scores.shape[0] != n_q:
            raise ValueError("block_scores must be float32 [n_q, ld]")
        ld = block_scores.shape[1]
    ws = _workspace(workspace_full(dims, b), dev, ws)
    wp, wn = _ws_ptr(ws)
    d, q = dims.c(), b.c()
    if pages is not None:
        _check_page_rows(pages, idx_k[0] if fp4 else idx_k)
        pg = pages.c()
        qs, ks = (qp[1], kp[1]) if fp4 else (None, None)
        _check(lib().csa2_index_full_paged(ctypes.byref(d), ctypes.byref(q), ctypes.byref(pg), qp[0], qs,
                                           idx_w.data_ptr(), kp[0], ks, pool_blocks.data_ptr(),
                                           pool_count.data_ptr(), _ptr(block_scores), ld, wp, wn, _stream(dev)))
        return pool_blocks, pool_count
    fn = lib().csa2_index_full_fp4 if fp4 else lib().csa2_index_full
    _check(fn(ctypes.byref(d), ctypes.byref(q), *qp, idx_w.data_ptr(), *kp, pool_blocks.data_ptr(),
              pool_count.data_ptr(), _ptr(block_scores), ld, wp, wn, _stream(dev)))
    return pool_blocks, pool_count


def n_blocks(dims: Dims, b: Batch) -> int:
    """Most candidate blocks of any query: ceil((max_visible - W) / 8)."""
    return max(0, -(-(b.max_visible - dims.swa) // 8))


def block_scores_ld(dims: Dims, b: Batch) -> int:
    """Row stride of a block-score array: n_blocks rounded up to a multiple of 4 (at least 4)."""
    return max(4, (n_blocks(dims, b) + 3) // 4 * 4)


POOL_WS_FROM_SCAN = 1


def pos_keys_ld(dims: Dims, b: Batch) -> int:
    """Row stride of a position-key array: 8 n_blocks rounded up to 32 (at least 32)."""
    return max(32, (8 * n_blocks(dims, b) + 31) // 32 * 32)


def index_scan(dims: Dims, b: Batch, idx_q, idx_w: torch.Tensor, idx_k,
               block_scores: Optional[torch.Tensor] = None, pool_ws: Optional[torch.Tensor] = None,
               prepare: bool = False, pages: Optional[Pages] = None, pos_keys: Optional[torch.Tensor] = None):
    """Full-mode scan: block scores float32 [n_q, ld] (b_j for j < nb).  With
    `pool_ws` (a pool-select workspace) the scan also prepares it for an
    index_pool(..., ws=pool_ws, from_scan=True) call on these scores.  With
    `pages` the keys are paged (csa2_index_scan_paged).  With `pos_keys`
    (int32 [n_q, ld], ld from pos_keys_ld) it also keeps every candidate
    position's score as an order key (csa2_index_scan_keys)."""
    dev = _rows_dev(idx_k)
    _dev(block_scores, pool_ws, pos_keys)
    fp4, qp, kp = _check_idx(dims, b, idx_q, idx_w, idx_k)
    if block_scores is None:
        block_scores = torch.empty(b.n_q, block_scores_ld(dims, b), dtype=torch.float32, device=dev)
    if block_scores.dtype != torch.float32 or block_scores.dim() != 2 or block_scores.shape[0] != b.n_q:
        raise ValueError("block_scores must be float32 [n_q, ld]")
    wp, wn = _ws_ptr(pool_ws)
    d, q = dims.c(), b.c()
    if pos_keys is not None:
        if pos_keys.dtype != torch.int32 or pos_keys.dim() != 2 or pos_keys.shape[0] != b.n_q:
            raise ValueError("pos_keys must be int32 [n_q, ld]")
        pg = pages.c() if pages is not None else None
        if pages is not None:
            _check_page_rows(pages, *(idx_k if fp4 else (idx_k,)))
        qs, ks = (qp[1], kp[1]) if fp4 else (None, None)
        args = (ctypes.byref(d), ctypes.byref(q), ctypes.byref(pg) if pg is not None else None, qp[0], qs,
                idx_w.data_ptr(), kp[0], ks, block_scores.data_ptr(), block_scores.shape[1], pos_keys.data_ptr(),
                pos_keys.shape[1], wp, wn, _stream(dev))
        keep = (d, q, pg, pool_ws) + ((pages.table,) if pages is not None else ())
        call = _issue(lib().csa2_index_scan_keys, args, keep, prepare)
        return call if prepare else block_scores
    args = (ctypes.byref(d), ctypes.byref(q), *qp, idx_w.data_ptr(), *kp, block_scores.data_ptr(),
            block_scores.shape[1], wp, wn, _stream(dev))
    if pages is not None:
        _check_page_rows(pages, *(idx_k if fp4 else (idx_k,)))
        pg = pages.c()
        qs, ks = (qp[1], kp[1]) if fp4 else (None, None)
        args = (ctypes.byref(d), ctypes.byref(q), ctypes.byref(pg), qp[0], qs, idx_w.data_ptr(), kp[0], ks,
                block_scores.data_ptr(), block_scores.shape[1], wp, wn, _stream(dev))
        call = _issue(lib().csa2_index_scan_paged, args, (d, q, pg, pool_ws, pages.table), prepare)
        return call if prepare else block_scores
    fn = lib().csa2_index_scan_fp4 if fp4 else lib().csa2_index_scan
    call = _issue(fn, args, (d, q, pool_ws), prepare)
    return call if prepare else block_scores


def index_pool(dims: Dims, b: Batch, block_scores: torch.Tensor,
               pool_blocks: Optional[torch.Tensor] = None, pool_count: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, from_scan: bool = False, prepare: bool = False):
    """Top-P block pool from index_scan's block scores.  `from_scan`: `ws` was
    passed to the index_scan call that wrote these scores."""
    if from_scan and ws is None:
        raise ValueError("from_scan needs the workspace that index_scan prepared")
    dev = block_scores.device
    _dev(block_scores, pool_blocks, pool_count, ws)
    if block_scores.dtype != torch.float32 or block_scores.dim() != 2 or block_scores.shape[0] != b.n_q:
        raise ValueError("block_scores must be float32 [n_q, ld]")
    if pool_blocks is None:
        pool_blocks = torch.empty(b.n_q, dims.pool_blocks, dtype=torch.int32, device=dev)
    if pool_count is None:
        pool_count = torch.empty(b.n_q, dtype=torch.int32, device=dev)
    ws = _workspace(workspace_pool(dims, b), dev, ws)
    wp, wn = _ws_ptr(ws)
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), block_scores.data_ptr(), block_scores.shape[1],
            pool_blocks.data_ptr(), pool_count.data_ptr(), wp, wn,
            POOL_WS_FROM_SCAN if from_scan else 0, _stream(dev))
    call = _issue(lib().csa2_index_pool, args, (d, q, ws), prepare)
    return call if prepare else (pool_blocks, pool_count)


def index_pool_topk(dims: Dims, b: Batch, block_scores: torch.Tensor, pos_keys: torch.Tensor,
                    pool_blocks: Optional[torch.Tensor] = None, pool_count: Optional[torch.Tensor] = None,
                    topk_pos: Optional[torch.Tensor] = None, topk_count: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, from_scan: bool = False, prepare: bool = False):
    """index_pool then index_topk_keys in one call (csa2_index_pool_topk; one
    kernel for pools of up to 16,384 blocks).  Returns (pool_blocks,
    pool_count, topk_pos, topk_count)."""
    if from_scan and ws is None:
        raise ValueError("from_scan needs the workspace that index_scan prepared")
    dev = block_scores.device
    _dev(block_scores, pos_keys, pool_blocks, pool_count, topk_pos, topk_count, ws)
    n_q = b.n_q
    if block_scores.dtype != torch.float32 or block_scores.dim() != 2 or block_scores.shape[0] != n_q:
        raise ValueError("block_scores must be float32 [n_q, ld]")
    if pos_keys.dim() != 2 or pos_keys.shape[0] != n_q or pos_keys.element_size() != 4:
        raise ValueError("pos_keys must be 32-bit [n_q, ld]")
    if pool_blocks is None:
        pool_blocks = torch.empty(n_q, dims.pool_blocks, dtype=torch.int32, device=dev)
    if pool_count is None:
        pool_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    if topk_pos is None:
        topk_pos = torch.empty(n_q, dims.topk, dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    ws = _workspace(workspace_pool(dims, b), dev, ws)
    wp, wn = _ws_ptr(ws)
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), block_scores.data_ptr(), block_scores.shape[1], pos_keys.data_ptr(),
            pos_keys.shape[1], pool_blocks.data_ptr(), pool_count.data_ptr(), topk_pos.data_ptr(),
            topk_count.data_ptr(), wp, wn, POOL_WS_FROM_SCAN if from_scan else 0, _stream(dev))
    call = _issue(lib().csa2_index_pool_topk, args, (d, q, ws), prepare)
    return call if prepare else (pool_blocks, pool_count, topk_pos, topk_count)


def index_reindex(dims: Dims, b: Batch, idx_q, idx_w: torch.Tensor, idx_k,
                  pool_blocks: torch.Tensor, pool_count: torch.Tensor,
                  topk_pos: Optional[torch.Tensor] = None, topk_count: Optional[torch.Tensor] = None,
                  topk_scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  prepare: bool = False, pages: Optional[Pages] = None):
    """Reindex inside the pool. Returns (topk_pos int32 [n_q, K], topk_count).
    With `pages` the keys are paged (csa2_index_reindex_paged)."""
    dev = _rows_dev(idx_k)
    _dev(pool_blocks, pool_count, topk_pos, topk_count, topk_scores)
    n_q = b.n_q
    fp4, qp, kp = _check_idx(dims, b, idx_q, idx_w, idx_k)
    if pool_blocks.shape != (n_q, dims.pool_blocks) or pool_count.shape != (n_q,):
        raise ValueError("pool shape mismatch")
    if topk_pos is None:
        topk_pos = torch.empty(n_q, dims.topk, dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    if topk_scores is not None and topk_scores.shape != (n_q, dims.topk):
        raise ValueError("topk_scores must be float32 [n_q, K]")
    ws = _workspace(workspace_reindex(dims, b), dev, ws)
    wp, wn = _ws_ptr(ws)
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), *qp, idx_w.data_ptr(), *kp, pool_blocks.data_ptr(),
            pool_count.data_ptr(), topk_pos.data_ptr(), topk_count.data_ptr(), _ptr(topk_scores), wp, wn,
            _stream(dev))
    if pages is not None:
        krows = idx_k[0].shape[0] if fp4 else idx_k.shape[0]
        if pages.rows > krows:
            raise ValueError(f"pages.rows ({pages.rows}) exceeds the key planes' {krows} rows")
        pg = pages.c()
        qs, ks = (qp[1], kp[1]) if fp4 else (None, None)
        args = (ctypes.byref(d), ctypes.byref(q), ctypes.byref(pg), qp[0], qs, idx_w.data_ptr(), kp[0], ks,
                pool_blocks.data_ptr(), pool_count.data_ptr(), topk_pos.data_ptr(), topk_count.data_ptr(),
                _ptr(topk_scores), wp, wn, _stream(dev))
        call = _issue(lib().csa2_index_reindex_paged, args, (d, q, pg, ws, pages.table), prepare)
        return call if prepare else (topk_pos, topk_count)
    fn = lib().csa2_index_reindex_fp4 if fp4 else lib().csa2_index_reindex
    call = _issue(fn, args, (d, q, ws), prepare)
    return call if prepare else (topk_pos, topk_count)


def attend(dims: Dims, b: Batch, q_lat: torch.Tensor, q_rope: torch.Tensor, softmax_scale: float,
           kv_codes: torch.Tensor, kv_scales: torch.Tensor, kv_rope: torch.Tensor,
           topk_pos: torch.Tensor, topk_count: torch.Tensor, swa_kv: torch.Tensor, swa_base: torch.Tensor,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           ws: Optional[torch.Tensor] = None, want_lse: bool = True, prepare: bool = False,
           pages: Optional[Pages] = None):
    """Sparse FP4 + window attention. Returns (out f32 [n_q, H, 512], lse).
    With `pages` the main-KV planes are paged (csa2_attend_paged)."""
    dev = q_lat.device
    _dev(q_lat, q_rope, kv_codes, kv_scales, kv_rope, topk_pos, topk_count, swa_kv, swa_base, out, lse)
    n_q, H = b.n_q, dims.n_heads
    if q_lat.shape != (n_q, H, 512) or q_rope.shape != (n_q, H, 64):
        raise ValueError("q_lat / q_rope shape mismatch")
    if q_lat.dtype != torch.bfloat16 or q_rope.dtype != torch.bfloat16 or swa_kv.dtype != torch.bfloat16:
        raise TypeError("q_lat, q_rope and swa_kv must be bfloat16")
    if topk_pos.shape != (n_q, dims.topk) or swa_base.dtype != torch.int64 or swa_base.shape != (n_q,):
        raise ValueError("topk_pos / swa_base shape mismatch")
    if swa_kv.dim() != 2 or swa_kv.shape[1] != 576:
        raise ValueError("swa_kv must be [rows, 576]")
    if out is None:
        out = torch.empty(n_q, H, 512, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(n_q, H, dtype=torch.float32, device=dev)
    ws = _workspace(workspace_attend(dims, b), dev, ws)
    wp, wn = _ws_ptr(ws)
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), q_lat.data_ptr(), q_rope.data_ptr(),
            float(softmax_scale), kv_codes.data_ptr(), kv_scales.data_ptr(), kv_rope.data_ptr(),
            topk_pos.data_ptr(), topk_count.data_ptr(), swa_kv.data_ptr(), swa_base.data_ptr(),
            out.data_ptr(), _ptr(lse), wp, wn, _stream(dev))
    if pages is not None:
        if pages.rows > min(kv_codes.shape[0], kv_scales.shape[0], kv_rope.shape[0]):
            raise ValueError(f"pages.rows ({pages.rows}) exceeds the main-KV planes' rows")
        pg = pages.c()
        call = _issue(lib().csa2_attend_paged, args[:2] + (ctypes.byref(pg),) + args[2:], (d, q, pg, ws, pages.table),
                      prepare)
        return call if prepare else (out, lse)
    call = _issue(lib().csa2_attend, args, (d, q, ws), prepare)
    return call if prepare else (out, lse)


def pool_topk_attend(dims: Dims, b: Batch, block_scores: torch.Tensor, pos_keys: torch.Tensor,
                     q_lat: torch.Tensor, q_rope: torch.Tensor, softmax_scale: float,
                     kv_codes: torch.Tensor, kv_scales: torch.Tensor, kv_rope: torch.Tensor,
                     swa_kv: torch.Tensor, swa_base: torch.Tensor,
                     pool_blocks: Optional[torch.Tensor] = None, pool_count: Optional[torch.Tensor] = None,
                     topk_pos: Optional[torch.Tensor] = None, topk_count: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, pool_ws: Optional[torch.Tensor] = None,
                     from_scan: bool = False, want_lse: bool = True, prepare: bool = False,
                     pages: Optional[Pages] = None):
    """The pool, the Full layer's Top-K and the attention on it, selected
    inside the attention kernel (csa2_pool_topk_attend; with `pages`,
    csa2_pool_topk_attend_paged).  `pool_ws`, `from_scan` as index_pool's
    `ws`, `from_scan` (read by the selection of queries past 16,384 blocks).
    Returns (pool_blocks, pool_count, topk_pos, topk_count, out, lse)."""
    dev = q_lat.device
    _dev(block_scores, pos_keys, q_lat, q_rope, kv_codes, kv_scales, kv_rope, swa_kv, swa_base, pool_blocks,
         pool_count, topk_pos, topk_count, out, lse)
    n_q, H = b.n_q, dims.n_heads
    if block_scores.dtype != torch.float32 or block_scores.dim() != 2 or block_scores.shape[0] != n_q:
        raise ValueError("block_scores must be float32 [n_q, ld]")
    if pos_keys.dim() != 2 or pos_keys.shape[0] != n_q or pos_keys.element_size() != 4:
        raise ValueError("pos_keys must be 32-bit [n_q, ld]")
    if q_lat.shape != (n_q, H, 512) or q_rope.shape != (n_q, H, 64):
        raise ValueError("q_lat / q_rope shape mismatch")
    if q_lat.dtype != torch.bfloat16 or q_rope.dtype != torch.bfloat16 or swa_kv.dtype != torch.bfloat16:
        raise TypeError("q_lat, q_rope and swa_kv must be bfloat16")
    if swa_base.dtype != torch.int64 or swa_base.shape != (n_q,):
        raise ValueError("swa_base must be int64 [n_q]")
    if swa_kv.dim() != 2 or swa_kv.shape[1] != 576:
        raise ValueError("swa_kv must be [rows, 576]")
    if pool_blocks is None:
        pool_blocks = torch.empty(n_q, dims.pool_blocks, dtype=torch.int32, device=dev)
    if pool_count is None:
        pool_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    if topk_pos is None:
        topk_pos = torch.empty(n_q, dims.topk, dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    if pool_blocks.shape != (n_q, dims.pool_blocks) or topk_pos.shape != (n_q, dims.topk):
        raise ValueError("pool_blocks / topk_pos shape mismatch")
    if out is None:
        out = torch.empty(n_q, H, 512, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(n_q, H, dtype=torch.float32, device=dev)
    if from_scan and pool_ws is None:
        raise ValueError("from_scan needs the workspace that index_scan prepared")
    ws = _workspace(workspace_attend(dims, b), dev, ws)
    wp, wn = _ws_ptr(ws)
    if n_blocks(dims, b) > 16384 or os.environ.get("CSA2_POOL_SMALL") == "0":
        pool_ws = _workspace(workspace_pool(dims, b), dev, pool_ws)
    pp, pn = _ws_ptr(pool_ws) if pool_ws is not None else (None, 0)
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), block_scores.data_ptr(), block_scores.shape[1], pos_keys.data_ptr(),
            pos_keys.shape[1], pool_blocks.data_ptr(), pool_count.data_ptr(), topk_pos.data_ptr(),
            topk_count.data_ptr(), q_lat.data_ptr(), q_rope.data_ptr(), float(softmax_scale), kv_codes.data_ptr(),
            kv_scales.data_ptr(), kv_rope.data_ptr(), swa_kv.data_ptr(), swa_base.data_ptr(), out.data_ptr(),
            _ptr(lse), pp, pn, POOL_WS_FROM_SCAN if from_scan else 0, wp, wn, _stream(dev))
    if pages is not None:
        if pages.rows > min(kv_codes.shape[0], kv_scales.shape[0], kv_rope.shape[0]):
            raise ValueError(f"pages.rows ({pages.rows}) exceeds the main-KV planes' rows")
        pg = pages.c()
        call = _issue(lib().csa2_pool_topk_attend_paged, args[:2] + (ctypes.byref(pg),) + args[2:],
                      (d, q, pg, ws, pool_ws, pages.table), prepare)
    else:
        call = _issue(lib().csa2_pool_topk_attend, args, (d, q, ws, pool_ws), prepare)
    return call if prepare else (pool_blocks, pool_count, topk_pos, topk_count, out, lse)


def reindex_attend(dims: Dims, b: Batch, idx_q, idx_w: torch.Tensor, idx_k,
                   pool_blocks: torch.Tensor, pool_count: torch.Tensor,
                   q_lat: torch.Tensor, q_rope: torch.Tensor, softmax_scale: float,
                   kv_codes: torch.Tensor, kv_scales: torch.Tensor, kv_rope: torch.Tensor,
                   swa_kv: torch.Tensor, swa_base: torch.Tensor,
                   topk_pos: Optional[torch.Tensor] = None, topk_count: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   reindex_ws: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                   want_lse: bool = True, prepare: bool = False, pages: Optional[Pages] = None):
    """A Reindex layer with the Top-K selected inside the attention kernel
    (csa2_reindex_attend; with `pages`, csa2_reindex_attend_paged).  idx_q /
    idx_k as in index_reindex (a (codes, scales) pair each for FP4 rows).
    Returns (topk_pos, topk_count, out, lse)."""
    dev = q_lat.device
    _dev(pool_blocks, pool_count, q_lat, q_rope, kv_codes, kv_scales, kv_rope, swa_kv, swa_base, topk_pos,
         topk_count, out, lse)
    fp4, qp, kp = _check_idx(dims, b, idx_q, idx_w, idx_k)
    (qc, qs), (kc, ksc) = (qp, kp) if fp4 else ((qp[0], None), (kp[0], None))
    n_q, H = b.n_q, dims.n_heads
    if q_lat.shape != (n_q, H, 512) or q_rope.shape != (n_q, H, 64):
        raise ValueError("q_lat / q_rope shape mismatch")
    if q_lat.dtype != torch.bfloat16 or q_rope.dtype != torch.bfloat16 or swa_kv.dtype != torch.bfloat16:
        raise TypeError("q_lat, q_rope and swa_kv must be bfloat16")
    if swa_base.dtype != torch.int64 or swa_base.shape != (n_q,):
        raise ValueError("swa_base must be int64 [n_q]")
    if pool_blocks.shape != (n_q, dims.pool_blocks):
        raise ValueError("pool_blocks shape mismatch")
    if topk_pos is None:
        topk_pos = torch.empty(n_q, dims.topk, dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    if topk_pos.shape != (n_q, dims.topk):
        raise ValueError("topk_pos shape mismatch")
    if out is None:
        out = torch.empty(n_q, H, 512, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(n_q, H, dtype=torch.float32, device=dev)
    reindex_ws = _workspace(workspace_reindex(dims, b), dev, reindex_ws)
    ws = _workspace(workspace_attend(dims, b), dev, ws)
    rp, rn = _ws_ptr(reindex_ws)
    wp, wn = _ws_ptr(ws)
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), qc, qs, idx_w.data_ptr(), kc, ksc,
            pool_blocks.data_ptr(), pool_count.data_ptr(), topk_pos.data_ptr(), topk_count.data_ptr(),
            q_lat.data_ptr(), q_rope.data_ptr(), float(softmax_scale), kv_codes.data_ptr(), kv_scales.data_ptr(),
            kv_rope.data_ptr(), swa_kv.data_ptr(), swa_base.data_ptr(), out.data_ptr(), _ptr(lse), rp, rn, wp, wn,
            _stream(dev))
    if pages is not None:
        if pages.rows > min(kv_codes.shape[0], kv_scales.shape[0], kv_rope.shape[0]):
            raise ValueError(f"pages.rows ({pages.rows}) exceeds the main-KV planes' rows")
        pg = pages.c()
        call = _issue(lib().csa2_reindex_attend_paged, args[:2] + (ctypes.byref(pg),) + args[2:],
                      (d, q, pg, ws, reindex_ws, pages.table), prepare)
    else:
        call = _issue(lib().csa2_reindex_attend, args, (d, q, ws, reindex_ws), prepare)
    return call if prepare else (topk_pos, topk_count, out, lse)


LAYER_FULL, LAYER_REINDEX, LAYER_REUSE = 0, 1, 2


def decode_step(dims: Dims, b: Batch, mode: int, idx_q, idx_w, idx_k,
                pool_blocks: torch.Tensor, pool_count: torch.Tensor,
                topk_pos: torch.Tensor, topk_count: torch.Tensor,
                q_lat: torch.Tensor, q_rope: torch.Tensor, softmax_scale: float,
                kv_codes: torch.Tensor, kv_scales: torch.Tensor, kv_rope: torch.Tensor,
                swa_kv: torch.Tensor, swa_base: torch.Tensor, out: torch.Tensor,
                lse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, prepare: bool = False,
                pages: Optional[Pages] = None):
    """One decode layer (csa2_decode_step; csa2_decode_step_paged with `pages`): LAYER_FULL writes the pool and the
    Top-K and attends; LAYER_REINDEX reads the pool, writes the Top-K and
    attends; LAYER_REUSE attends over the given Top-K.  Indexer rows as for
    index_full (None allowed for LAYER_REUSE).  `ws` must come from a
    zero-filled allocation of at least workspace_step bytes (+256 for
    alignment); it is allocated zero-filled when None."""
    if mode not in (LAYER_FULL, LAYER_REINDEX, LAYER_REUSE):
        raise ValueError("mode must be LAYER_FULL, LAYER_REINDEX or LAYER_REUSE")
    dev = q_lat.device
    n_q, H = b.n_q, dims.n_heads
    _dev(pool_blocks, pool_count, topk_pos, topk_count, q_lat, q_rope, kv_codes, kv_scales, kv_rope, swa_kv,
         swa_base, out, lse)
    if pool_blocks.shape != (n_q, dims.pool_blocks) or pool_count.shape != (n_q,):
        raise ValueError("pool shape mismatch")
    if topk_pos.shape != (n_q, dims.topk) or topk_count.shape != (n_q,):
        raise ValueError("topk shape mismatch")
    if q_lat.shape != (n_q, H, 512) or q_rope.shape != (n_q, H, 64) or out.shape != (n_q, H, 512):
        raise ValueError("q_lat / q_rope / out shape mismatch")
    if swa_kv.dim() != 2 or swa_kv.shape[1] != 576 or swa_base.shape != (n_q,):
        raise ValueError("swa_kv must be [rows, 576] and swa_base [n_q]")
    if mode == LAYER_REUSE and idx_q is None:
        qp, kp, wp_ = [None, None], [None, None], None
    else:
        fp4, qp, kp = _check_idx(dims, b, idx_q, idx_w, idx_k)
        if not fp4:
            qp, kp = [qp[0], None], [kp[0], None]
        wp_ = idx_w.data_ptr()
    ws = _workspace(workspace_step(dims, b), dev, ws)
    wsp, wn = _ws_ptr(ws)
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), mode, qp[0], qp[1], wp_, kp[0], kp[1], pool_blocks.data_ptr(),
            pool_count.data_ptr(), topk_pos.data_ptr(), topk_count.data_ptr(), q_lat.data_ptr(), q_rope.data_ptr(),
            float(softmax_scale), kv_codes.data_ptr(), kv_scales.data_ptr(), kv_rope.data_ptr(), swa_kv.data_ptr(),
            swa_base.data_ptr(), out.data_ptr(), _ptr(lse), wsp, wn, _stream(dev))
    if pages is not None:
        planes = [kv_codes, kv_scales, kv_rope]
        if idx_k is not None:
            planes += list(idx_k) if isinstance(idx_k, tuple) else [idx_k]
        _check_page_rows(pages, *planes)
        pg = pages.c()
        return _issue(lib().csa2_decode_step_paged, args[:2] + (ctypes.byref(pg),) + args[2:],
                      (d, q, pg, ws, pages.table), prepare)
    return _issue(lib().csa2_decode_step, args, (d, q, ws), prepare)


def stream_read(buf: torch.Tensor, sink: torch.Tensor, prepare: bool = False):
    """One nontemporal read of every byte of `buf` (csa2_stream_read): the
    streaming-read reference the Full scan's bandwidth is compared with.
    `sink` is an int32 device tensor of at least one element."""
    _dev(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    args = (buf.data_ptr(), nbytes - nbytes % 16, sink.data_ptr(), _stream(buf.device))
    return _issue(lib().csa2_stream_read, args, (), prepare)


def decode_step_noalloc(dims: Dims, b: Batch, mode: int, idx_q, idx_w, idx_k,
                        pool_blocks: torch.Tensor, pool_count: torch.Tensor,
                        topk_pos: torch.Tensor, topk_count: torch.Tensor,
                        q_lat: torch.Tensor, q_rope: torch.Tensor, softmax_scale: float,
                        kv_codes: torch.Tensor, kv_scales: torch.Tensor, kv_rope: torch.Tensor,
                        swa_kv: torch.Tensor, swa_base: torch.Tensor, out: torch.Tensor,
                        lse: Optional[torch.Tensor] = None, prepare: bool = False):
    """decode_step without a workspace (csa2_decode_step_noalloc): the
    library's own per-GPU scratch array serves the stages, and nothing is
    allocated, here or in the library.  Calls that may overlap on one GPU
    race on that array."""
    if mode not in (LAYER_FULL, LAYER_REINDEX, LAYER_REUSE):
        raise ValueError("mode must be LAYER_FULL, LAYER_REINDEX or LAYER_REUSE")
    n_q, H = b.n_q, dims.n_heads
    _dev(pool_blocks, pool_count, topk_pos, topk_count, q_lat, q_rope, kv_codes, kv_scales, kv_rope, swa_kv,
         swa_base, out, lse)
    if pool_blocks.shape != (n_q, dims.pool_blocks) or pool_count.shape != (n_q,):
        raise ValueError("pool shape mismatch")
    if topk_pos.shape != (n_q, dims.topk) or topk_count.shape != (n_q,):
        raise ValueError("topk shape mismatch")
    if q_lat.shape != (n_q, H, 512) or q_rope.shape != (n_q, H, 64) or out.shape != (n_q, H, 512):
        raise ValueError("q_lat / q_rope / out shape mismatch")
    if swa_kv.dim() != 2 or swa_kv.shape[1] != 576 or swa_base.shape != (n_q,):
        raise ValueError("swa_kv must be [rows, 576] and swa_base [n_q]")
    if mode == LAYER_REUSE and idx_q is None:
        qp, kp, wp_ = [None, None], [None, None], None
    else:
        fp4, qp, kp = _check_idx(dims, b, idx_q, idx_w, idx_k)
        if not fp4:
            qp, kp = [qp[0], None], [kp[0], None]
        wp_ = idx_w.data_ptr()
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), mode, qp[0], qp[1], wp_, kp[0], kp[1], pool_blocks.data_ptr(),
            pool_count.data_ptr(), topk_pos.data_ptr(), topk_count.data_ptr(), q_lat.data_ptr(), q_rope.data_ptr(),
            float(softmax_scale), kv_codes.data_ptr(), kv_scales.data_ptr(), kv_rope.data_ptr(), swa_kv.data_ptr(),
            swa_base.data_ptr(), out.data_ptr(), _ptr(lse), _stream(q_lat.device))
    return _issue(lib().csa2_decode_step_noalloc, args, (d, q), prepare)


def index_topk_keys(dims: Dims, b: Batch, pool_blocks: torch.Tensor, pool_count: torch.Tensor,
                    block_scores: torch.Tensor, pos_keys: torch.Tensor,
                    topk_pos: Optional[torch.Tensor] = None, topk_count: Optional[torch.Tensor] = None,
                    topk_scores: Optional[torch.Tensor] = None, prepare: bool = False):
    """A Full layer's Top-K from index_scan(..., pos_keys=...)'s scores
    (csa2_index_topk_keys): the same set as index_reindex with the scan's
    query.  Returns (topk_pos int32 [n_q, K], topk_count)."""
    dev = pool_blocks.device
    _dev(pool_blocks, pool_count, block_scores, pos_keys, topk_pos, topk_count, topk_scores)
    n_q = b.n_q
    if pool_blocks.shape != (n_q, dims.pool_blocks) or pool_count.shape != (n_q,):
        raise ValueError("pool shape mismatch")
    if topk_pos is None:
        topk_pos = torch.empty(n_q, dims.topk, dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty(n_q, dtype=torch.int32, device=dev)
    if topk_scores is not None and topk_scores.shape != (n_q, dims.topk):
        raise ValueError("topk_scores must be float32 [n_q, K]")
    d, q = dims.c(), b.c()
    args = (ctypes.byref(d), ctypes.byref(q), pool_blocks.data_ptr(), pool_count.data_ptr(), block_scores.data_ptr(),
            block_scores.shape[1], pos_keys.data_ptr(), pos_keys.shape[1], topk_pos.data_ptr(),
            topk_count.data_ptr(), _ptr(topk_scores), _stream(dev))
    call = _issue(lib().csa2_index_topk_keys, args, (d, q), prepare)
    return call if prepare else (topk_pos, topk_count)
