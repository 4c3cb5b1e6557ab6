"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/csa2.h declares, and
reject bad arguments synchronously with the documented status before it
touches a device.  Workspace-size queries are pure host arithmetic.
"""
import ctypes
import dataclasses
import os
import re

import pytest

import compressed_sparse_attention_decode_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_]\w*\s*\*?\s*(csa2_\w+)\s*\(", src, re.M)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    for n in ("csa2_encode_kv", "csa2_encode_kv_grouped", "csa2_index_full", "csa2_index_reindex", "csa2_attend",
              "csa2_index_scan", "csa2_index_pool", "csa2_status_string", "csa2_abi_version",
              "csa2_encode_fp4", "csa2_index_scan_fp4", "csa2_index_full_fp4", "csa2_index_reindex_fp4",
              "csa2_decode_step", "csa2_decode_step_workspace_size", "csa2_index_reindex_paged",
              "csa2_attend_paged", "csa2_page_rows", "csa2_index_full_paged", "csa2_decode_step_paged",
              "csa2_index_scan_paged"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(csa2.lib_path)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_abi_version_and_status_strings():
    L = csa2.lib()
    # the header's version, which the library was built from
    want = int(re.search(r"#define CSA2_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.csa2_abi_version() == want == 3
    for st in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIP):
        assert L.csa2_status_string(st)
    assert L.csa2_status_string(99)          # unknown codes still get text


def _dims(**kw):
    d = dict(n_heads=64, idx_heads=64, idx_dim=128, pool_blocks=2048, topk=512, swa=128)
    d.update(kw)
    return csa2.Dims(**d)


class _HostBatch:
    """Query batch for host-side calls: non-null placeholder device pointers
    that the argument checks never dereference."""

    def __init__(self, n_q=8, max_visible=131072, g=1):
        self.n_q, self.max_visible, self.g = n_q, max_visible, g

    def c(self):
        return csa2._Queries(self.n_q, self.g, self.max_visible, 0, 0x10000, 0x20000)


def _batch(**kw):
    return _HostBatch(**kw)


def _call_ws(fn, dims, batch):
    n = ctypes.c_size_t(0)
    d, q = dims.c(), batch.c()
    st = fn(ctypes.byref(d), ctypes.byref(q), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("bad", [
    dict(idx_dim=96), dict(n_heads=20), dict(n_heads=0), dict(n_heads=136), dict(n_heads=4),
    dict(idx_heads=0), dict(idx_heads=65),
    dict(pool_blocks=0), dict(pool_blocks=4096), dict(topk=0), dict(topk=8 * 16 + 1, pool_blocks=16),
    dict(swa=-1), dict(swa=2048), dict(kv_group=8), dict(kv_group=64),
])
def test_bad_dims_rejected(bad):
    L = csa2.lib()
    st, _ = _call_ws(L.csa2_attend_workspace_size, _dims(**bad), _batch())
    assert st == INVALID
    assert L.csa2_last_error()


@pytest.mark.parametrize("good", [dict(n_heads=8), dict(n_heads=24), dict(n_heads=120), dict(n_heads=128),
                                  dict(idx_heads=1), dict(idx_heads=40), dict(idx_heads=64), dict(idx_dim=64),
                                  dict(pool_blocks=1, topk=8), dict(topk=2048), dict(swa=0), dict(swa=1024),
                                  dict(kv_group=32)])
def test_documented_dims_accepted(good):
    """The ranges include/csa2.h documents: H a multiple of 8 up to 128,
    H_i 1..64, d_i 64 or 128, P 1..2048, K 1..min(8P, 2048), W 0..1024."""
    L = csa2.lib()
    for fn in (L.csa2_attend_workspace_size, L.csa2_index_full_workspace_size,
               L.csa2_index_reindex_workspace_size, L.csa2_decode_step_workspace_size):
        st, n = _call_ws(fn, _dims(**good), _batch())
        assert st == OK, L.csa2_last_error()


def test_attention_workspace_pads_heads_to_32():
    """Attention partials are laid out in 32-head workgroup blocks: 8, 24 and
    32 heads take the same workspace, 40 heads that of 64; a batch that fills
    the chip with one workgroup per (query, head group) needs none."""
    L = csa2.lib()
    sizes = {}
    for h in (8, 24, 32, 40, 64):
        st, sizes[h] = _call_ws(L.csa2_attend_workspace_size, _dims(n_heads=h), _batch(n_q=1))
        assert st == OK
    assert sizes[8] == sizes[24] == sizes[32] > 0
    assert sizes[40] == sizes[64] > sizes[32]
    st, big = _call_ws(L.csa2_attend_workspace_size, _dims(n_heads=64), _batch(n_q=128))
    assert st == OK and big == 0


def test_block_score_stride_at_least_four():
    """ld_block_scores must be >= 4 even when no query has candidates (the
    pool select reads 16-byte groups inside each row)."""
    L = csa2.lib()
    d = _dims().c()
    q = _batch(n_q=1, max_visible=100).c()          # n <= W: no blocks
    st = L.csa2_index_pool(ctypes.byref(d), ctypes.byref(q), 0x1000, 0, 0x2000, 0x3000, 0x4000, 1 << 30, 0, None)
    assert st == INVALID and b"ld_block_scores" in L.csa2_last_error()
    st = L.csa2_index_scan(ctypes.byref(d), ctypes.byref(q), 0x1000, 0x2000, 0x3000, 0x4000, 0, None, 0, None)
    assert st == INVALID and b"ld_block_scores" in L.csa2_last_error()


@pytest.mark.parametrize("kw", [dict(n_q=0), dict(max_visible=(1 << 21) + 1), dict(g=3), dict(n_q=130, g=65),
                                dict(max_visible=-1)])
def test_bad_queries_rejected(kw):
    L = csa2.lib()
    st, _ = _call_ws(L.csa2_index_full_workspace_size, _dims(), _batch(**kw))
    assert st == INVALID


def test_tokens_per_seq_up_to_64():
    L = csa2.lib()
    st, n = _call_ws(L.csa2_index_full_workspace_size, _dims(), _batch(n_q=128, g=64))
    assert st == OK and n > 0


def test_workspace_sizes_are_consistent():
    L = csa2.lib()
    dims = _dims()
    for n_q, mv in [(1, 4096), (8, 131072), (1, 1048576), (256, 524291)]:
        b = _batch(n_q=n_q, max_visible=mv, g=4 if n_q == 256 else 1)
        st, full = _call_ws(L.csa2_index_full_workspace_size, dims, b)
        assert st == OK
        st, pool = _call_ws(L.csa2_index_pool_workspace_size, dims, b)
        assert st == OK
        nb = -(-(mv - dims.swa) // 8)
        # full = pool workspace + a block-score array of at least nb floats per query
        assert full >= pool + n_q * nb * 4
        assert pool % 256 == 0 and full % 256 == 0
        st, rx = _call_ws(L.csa2_index_reindex_workspace_size, dims, b)
        assert st == OK and rx >= n_q * dims.pool_blocks * 8 * 4
        st, at = _call_ws(L.csa2_attend_workspace_size, dims, b)
        assert st == OK and at % 256 == 0


def test_null_pointers_rejected_before_any_device_work():
    L = csa2.lib()
    d, q = _dims().c(), _batch().c()
    st = L.csa2_index_scan(ctypes.byref(d), ctypes.byref(q), None, None, None, None, 0, None, 0, None)
    assert st == INVALID
    assert b"NULL" in L.csa2_last_error()
    st = L.csa2_encode_kv(-1, None, None, None, None, None, None, None)
    assert st == INVALID
    st = L.csa2_index_pool(ctypes.byref(d), ctypes.byref(q), 0x1000, 16384, 0x2000, 0x3000, 0x4000, 1 << 30,
                           2, None)
    assert st == INVALID and b"flags" in L.csa2_last_error()
    st = L.csa2_encode_kv(0, None, None, None, None, None, None, None)
    assert st in (OK, INVALID)


def test_fp4_indexer_calls_rejected_before_any_device_work():
    L = csa2.lib()
    q = _batch().c()
    # FP4 indexer rows need d_i = 128 and both scale planes
    d64 = dataclasses.replace(_dims(), idx_dim=64).c()
    st = L.csa2_index_full_fp4(ctypes.byref(d64), ctypes.byref(q), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000,
                               0x6000, 0x7000, None, 0, 0x8000, 1 << 30, None)
    assert st == INVALID and b"idx_dim 128" in L.csa2_last_error()
    d = _dims().c()
    st = L.csa2_index_reindex_fp4(ctypes.byref(d), ctypes.byref(q), 0x1000, None, 0x3000, 0x4000, 0x5000,
                                  0x6000, 0x7000, 0x8000, 0x9000, None, 0xA000, 1 << 30, None)
    assert st == INVALID and b"scale" in L.csa2_last_error()
    st = L.csa2_index_scan_fp4(ctypes.byref(d), ctypes.byref(q), 0x1000, 0x2004, 0x3000, 0x4000, 0x5000,
                               0x6000, 1 << 20, None, 0, None)
    assert st == INVALID and b"8-byte" in L.csa2_last_error()
    # encode: widths are 16 times a power of two up to 1024
    for width in (0, 48, 2048):
        assert L.csa2_encode_fp4(4, width, 0x1000, None, 0x2000, 0x3000, None) == INVALID
    assert L.csa2_encode_fp4(-1, 128, None, None, None, None, None) == INVALID
    assert L.csa2_encode_fp4(4, 128, None, None, 0x2000, 0x3000, None) == INVALID
    assert L.csa2_encode_fp4(0, 128, None, None, None, None, None) in (OK, INVALID)


def test_paged_calls_rejected_before_any_device_work():
    """Page descriptors are checked on the host: a power-of-two page of 16 to
    65536 positions, rows a multiple of it, and planes inside the gathers'
    32-bit byte range (256 B per row for the main-KV codes, d_i for fp8 keys)."""
    L = csa2.lib()
    d, q = _dims().c(), _batch().c()

    def attend(pg):
        return L.csa2_attend_paged(ctypes.byref(d), ctypes.byref(q), pg, 0x1000, 0x2000, 1.0, 0x3000, 0x4000,
                                   0x5000, 0x6000, 0x7000, 0x8000, 0x9000, 0xA000, None, 0xB000, 1 << 30, None)

    def reindex(pg):
        return L.csa2_index_reindex_paged(ctypes.byref(d), ctypes.byref(q), pg, 0x1000, None, 0x2000, 0x3000, None,
                                          0x4000, 0x5000, 0x6000, 0x7000, None, 0x8000, 1 << 30, None)

    assert attend(None) == INVALID and b"pages" in L.csa2_last_error()
    bad = [csa2._Pages(None, 64, 0, 1 << 10),          # no table
           csa2._Pages(0x1000, 48, 0, 1 << 10),        # not a power of two
           csa2._Pages(0x1000, 8, 0, 1 << 10),         # below 16
           csa2._Pages(0x1000, 1 << 17, 0, 1 << 17),   # above 65536
           csa2._Pages(0x1000, 64, 1, 1 << 10),        # reserved
           csa2._Pages(0x1000, 64, 0, 1000),           # rows not a multiple of the page
           csa2._Pages(0x1000, 64, 0, 0)]              # no rows
    for pg in bad:
        assert attend(ctypes.byref(pg)) == INVALID
        assert reindex(ctypes.byref(pg)) == INVALID
        assert L.csa2_page_rows(ctypes.byref(pg), 4, 0x1000, 0x2000, 0x3000, None) == INVALID
    # 2^24 rows: 4 GiB of 256-byte main-KV code rows is past the range, while
    # 128-byte fp8 key rows still fit
    big = csa2._Pages(0x1000, 64, 0, 1 << 24)
    assert attend(ctypes.byref(big)) == INVALID and b"4 GiB" in L.csa2_last_error()
    # (a NULL pool stops this call after the page check, before any launch)
    st = L.csa2_index_reindex_paged(ctypes.byref(d), ctypes.byref(q), ctypes.byref(big), 0x1000, None, 0x2000,
                                    0x3000, None, None, 0x5000, 0x6000, 0x7000, None, 0x8000, 1 << 30, None)
    assert st == INVALID and b"NULL" in L.csa2_last_error()
    ok = csa2._Pages(0x1000, 64, 0, 1 << 10)
    assert L.csa2_page_rows(ctypes.byref(ok), -1, None, None, None, None) == INVALID


def test_dims_struct_matches_header():
    # the binding's struct carries every csa2_dims field, in order
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct csa2_dims \{(.*?)\} csa2_dims;", src, re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [f for f, _ in csa2._Dims._fields_]


def test_grouped_encode_rejects_other_groups():
    L = csa2.lib()
    for g in (0, 8, 64):
        assert L.csa2_encode_kv_grouped(4, g, 0x1000, 0x2000, None, 0x3000, 0x4000, 0x5000, None) == INVALID
        assert b"group" in L.csa2_last_error()


def test_decode_step_rejected_before_any_device_work():
    L = csa2.lib()
    d, q = _dims().c(), _batch().c()
    args = [0x1000] * 17 + [None, 0x2000, 1 << 30, None]
    # bad mode
    st = L.csa2_decode_step(ctypes.byref(d), ctypes.byref(q), 7, 0x1000, None, 0x1000, 0x1000, None,
                            0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1.0, 0x1000, 0x1000, 0x1000,
                            0x1000, 0x1000, 0x1000, None, 0x2000, 1 << 30, None)
    assert st == INVALID and b"mode" in L.csa2_last_error()
    # one FP4 scale plane without the other
    st = L.csa2_decode_step(ctypes.byref(d), ctypes.byref(q), 0, 0x1000, 0x1100, 0x1000, 0x1000, None,
                            0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1.0, 0x1000, 0x1000, 0x1000,
                            0x1000, 0x1000, 0x1000, None, 0x2000, 1 << 30, None)
    assert st == INVALID and b"scales" in L.csa2_last_error()
    # workspace too small
    st = L.csa2_decode_step(ctypes.byref(d), ctypes.byref(q), 2, None, None, None, None, None,
                            0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1.0, 0x1000, 0x1000, 0x1000,
                            0x1000, 0x1000, 0x1000, None, 0x2000, 16, None)
    assert st == WORKSPACE
    del args
    n = ctypes.c_size_t(0)
    assert L.csa2_decode_step_workspace_size(ctypes.byref(d), ctypes.byref(q), ctypes.byref(n)) == OK
    parts = [_call_ws(f, _dims(), _batch())[1] for f in (L.csa2_index_full_workspace_size,
                                                         L.csa2_index_reindex_workspace_size,
                                                         L.csa2_attend_workspace_size)]
    assert n.value >= sum(parts)


def test_noalloc_step_rejects_batches_beyond_its_scratch():
    """csa2_decode_step_noalloc checks its scratch limit on the host: the
    speculative-verify batch (256 query tokens up to 512K) needs more than
    64 MiB, and more than 65,536 queries are refused outright."""
    L = csa2.lib()
    d = _dims().c()
    args = [0x1000] * 17 + [None, None]
    q = _batch(n_q=256, max_visible=524291, g=4).c()
    st = L.csa2_decode_step_noalloc(ctypes.byref(d), ctypes.byref(q), 2, None, None, None, None, None,
                                    0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1.0, 0x1000, 0x1000, 0x1000,
                                    0x1000, 0x1000, 0x1000, None, None)
    assert st == WORKSPACE and b"maximum" in L.csa2_last_error()
    q = _batch(n_q=65537, max_visible=4096).c()
    st = L.csa2_decode_step_noalloc(ctypes.byref(d), ctypes.byref(q), 2, None, None, None, None, None,
                                    0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1.0, 0x1000, 0x1000, 0x1000,
                                    0x1000, 0x1000, 0x1000, None, None)
    assert st == WORKSPACE and b"65536" in L.csa2_last_error()
    del args
