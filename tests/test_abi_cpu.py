"""The C-ABI library on the CPU: it loads, exports every declared symbol,
plans prefill chunks like the oracle and rejects bad arguments on the host
(no kernel is launched by any case here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import sparse_attention_indexer_decode_amd as idx
from sparse_attention_indexer_decode_amd import binding as B
from oracle import planner
from tests.conftest import ROOT, load_golden

HEADER = os.path.join(ROOT, "include", "idx.h")


@pytest.fixture(scope="module")
def lib():
    return idx.load()


def test_exports_match_header(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(idx_\w+)\s*\(", text, re.M))
    assert declared == set(B.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.idx_version().decode().count(".") == 2


def test_struct_layout_matches_c(tmp_path):
    """Field offsets and sizes of the ctypes mirrors equal the C compiler's."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for cls, cname in ((B.IdxCache, "idx_cache"), (B.IdxRows, "idx_rows"), (B.IdxChunk, "idx_chunk")):
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for cls, cname in ((B.IdxCache, "idx_cache"), (B.IdxRows, "idx_rows"), (B.IdxChunk, "idx_chunk")):
        assert int(got[cname]) == ctypes.sizeof(cls)
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)


def test_status_strings(lib):
    for s in range(5):
        assert lib.idx_status_string(s)
    assert lib.idx_status_string(99) == b"unknown status"


def _chunk_key(r):
    return [r["req_begin"], r["req_end"], r["q_begin"], r["q_end"], r["total_seq_lens"],
            r["token_begin"], r["token_end"], r["skip_kv_gather"]]


def test_planner_hand_cases(lib):
    g = load_golden("planner_cases.json")
    for c in g["cases"]:
        got = idx.idx_prefill_chunks(c["seq"], c["q"], c["workspace"], c["budget_bytes"])
        assert [_chunk_key(r) for r in got] == c["records"], c


def test_planner_matches_oracle_random(lib):
    rng = np.random.default_rng(19)
    for _ in range(500):
        n = int(rng.integers(0, 9))
        seq = rng.integers(0, 300, size=n)
        ql = np.minimum(rng.integers(0, 60, size=n), seq)
        ws = int(rng.integers(1, 700))
        budget = int(rng.integers(0, 40000))
        off = int(rng.integers(0, 5))
        got = idx.idx_prefill_chunks(seq, ql, ws, budget, off)
        ref = planner.chunk_records(seq, ql, ws, budget, off)
        assert [_chunk_key(r) for r in got] == [_chunk_key(r) for r in ref]
        for r in got:
            m = r["q_end"] - r["q_begin"]
            over = r["total_seq_lens"] > ws or m * r["total_seq_lens"] * 4 > budget
            assert r["over_budget"] == int(over and r["req_end"] - r["req_begin"] == 1)


def test_planner_c5(lib):
    got = idx.idx_prefill_chunks([65536, 65536], [16384, 16384], 65536, 512 << 20)
    ref = planner.chunk_records([65536, 65536], [16384, 16384], 65536, 512 << 20)
    assert len(got) == 16 and [_chunk_key(r) for r in got] == [_chunk_key(r) for r in ref]
    assert sum(r["skip_kv_gather"] for r in got) == 14


def test_planner_errors(lib):
    n_out = ctypes.c_int32(0)
    assert lib.idx_prefill_chunks(None, None, 1, 10, 10, 0, None, 0, ctypes.byref(n_out)) == B.IDX_EINVAL
    arr = (ctypes.c_int32 * 1)(-1)
    assert lib.idx_prefill_chunks(arr, arr, 1, 10, 10, 0, None, 0, ctypes.byref(n_out)) == B.IDX_EINVAL
    a = (ctypes.c_int32 * 2)(5, 5)
    out = (B.IdxChunk * 1)()
    assert lib.idx_prefill_chunks(a, a, 2, 5, 1000, 0, out, 1, ctypes.byref(n_out)) == B.IDX_ENOSPC
    assert n_out.value == 2


FAKE = 1 << 20   # a 256-aligned fake device address: never dereferenced, every case fails on the host


def _cache(**kw):
    c = dict(base=FAKE, num_pages=10, page_bytes=64 * 132, page_size=64, head_dim=128, fmt=0, reserved=0)
    c.update(kw)
    return B.IdxCache(**c)


def _rows(**kw):
    r = dict(kind=0, num_req=2, block_table=FAKE, bt_stride=8, bt_width=8, max_seq_len=300,
             seq_lens=FAKE, decode_lens=None, next_n=1, q_packed=0, query_start_loc=None, q_begin=0, q_end=0)
    r.update(kw)
    return B.IdxRows(**r)


def _logits(lib, cache, rows, heads=64, q=FAKE, w=FAKE, logits=FAKE, stride=512, ws=FAKE, wsb=1 << 20):
    return lib.idx_logits_paged(ctypes.byref(cache), ctypes.byref(rows), q, w, heads, logits, stride, ws, wsb, None)


def test_validation_rejects_before_launch(lib):
    E, U, S = B.IDX_EINVAL, B.IDX_EUNSUPPORTED, B.IDX_ENOSPC
    assert lib.idx_logits_paged(None, ctypes.byref(_rows()), FAKE, FAKE, 64, FAKE, 512, FAKE, 4096, None) == E
    assert _logits(lib, _cache(head_dim=96), _rows()) == U
    assert _logits(lib, _cache(fmt=1, head_dim=64, page_bytes=64 * 34 + 16 - (64 * 34) % 16), _rows()) == U
    assert _logits(lib, _cache(fmt=7), _rows()) == U
    assert _logits(lib, _cache(page_size=16), _rows()) == U
    assert _logits(lib, _cache(page_bytes=64 * 132 - 16), _rows()) == E      # rows do not fit a page
    assert _logits(lib, _cache(page_bytes=64 * 132 + 8), _rows()) == E       # not a multiple of 16
    assert _logits(lib, _cache(base=FAKE + 4), _rows()) == E                 # misaligned cache
    assert _logits(lib, _cache(reserved=1), _rows()) == E
    assert _logits(lib, _cache(), _rows(max_seq_len=8 * 64 + 1)) == E        # table too narrow
    assert _logits(lib, _cache(), _rows(bt_stride=4)) == E
    assert _logits(lib, _cache(), _rows(next_n=0)) == E
    assert _logits(lib, _cache(), _rows(kind=5)) == E
    assert _logits(lib, _cache(), _rows(), heads=65) == U
    assert _logits(lib, _cache(), _rows(), heads=0) == E
    assert _logits(lib, _cache(), _rows(), q=FAKE + 2) == E
    assert _logits(lib, _cache(), _rows(), stride=100) == E                  # < max_seq_len
    assert _logits(lib, _cache(), _rows(), wsb=16) == S
    assert _logits(lib, _cache(), _rows(), ws=FAKE + 8) == E
    assert _logits(lib, _cache(), _rows(num_req=5000)) == U                  # too many row groups
    assert _logits(lib, _cache(), _rows(kind=1, num_req=2, query_start_loc=None, q_begin=0, q_end=4)) == E
    # top-k
    r = _rows()
    assert lib.idx_topk(FAKE, 512, ctypes.byref(r), 0, FAKE, FAKE, 4096, None) == E
    assert lib.idx_topk(FAKE, 512, ctypes.byref(r), 5000, FAKE, FAKE, 4096, None) == U
    assert lib.idx_topk(None, 512, ctypes.byref(r), 16, FAKE, FAKE, 4096, None) == E
    # fused decode
    c = _cache()
    assert lib.idx_decode_topk(ctypes.byref(c), ctypes.byref(_rows(kind=1, query_start_loc=FAKE, q_end=2)),
                               FAKE, FAKE, 64, 16, FAKE, FAKE, 1 << 30, None) == E
    need = lib.idx_workspace_bytes(B.IDX_OP_DECODE_TOPK, ctypes.byref(c), ctypes.byref(r), 64, 16)
    assert need > 0
    assert lib.idx_decode_topk(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, 64, 16, FAKE, FAKE,
                               need - 1, None) == S


def test_workspace_sizes(lib):
    c = _cache()
    r = _rows(num_req=32, max_seq_len=300)
    wsb = lib.idx_workspace_bytes(B.IDX_OP_DECODE_TOPK, ctypes.byref(c), ctypes.byref(r), 64, 2048)
    # header + 32 rows x 320 fp32 row logits
    assert wsb == 256 + 32 * 320 * 4
    assert lib.idx_workspace_bytes(B.IDX_OP_LOGITS, ctypes.byref(c), ctypes.byref(r), 64, 0) == 256
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(r), 0, 16) == 256
    assert lib.idx_workspace_bytes(B.IDX_OP_DECODE_TOPK, ctypes.byref(c), ctypes.byref(r), 99, 16) == 0
    # k outside 1..4096: invalid for both selecting operations
    for k in (0, -3, 4097):
        assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(r), 0, k) == 0
        assert lib.idx_workspace_bytes(B.IDX_OP_DECODE_TOPK, ctypes.byref(c), ctypes.byref(r), 64, k) == 0
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(r), 0, 4096) == 256
    # long rows in a small batch: chunk candidates (2 x rows x chunks x 4096
    # 4-byte values and a count per chunk for k <= 2048; k values per chunk
    # above)
    rl = _rows(num_req=64, max_seq_len=131072, bt_width=2048, bt_stride=2048)
    split = 2 * 4 * 64 * 4 * 4096 + 4 * 64 * 4
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(rl), 0, 2048) == 256 + split
    assert lib.idx_workspace_bytes(B.IDX_OP_DECODE_TOPK, ctypes.byref(c), ctypes.byref(rl), 64, 2048) == \
        256 + 64 * 131072 * 4 + split
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(rl), 0, 3000) == 256 + 2 * 4 * 64 * 4 * 3000
    # many rows take the one-workgroup-per-row streaming path: no candidates
    rm = _rows(num_req=600, max_seq_len=131072, bt_width=2048)
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(rm), 0, 2048) == 256
    # rows are split only while all their chunks fit 256 workgroups: 64 rows of
    # four 32768-key chunks are split, 65 are not, nor are 128 MTP rows
    # (64 requests x next_n 2) of four chunks; 128 rows of two chunks are
    r65 = _rows(num_req=65, max_seq_len=131072, bt_width=2048, bt_stride=2048)
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(r65), 0, 2048) == 256
    r64x2 = _rows(num_req=64, next_n=2, max_seq_len=131072, bt_width=2048, bt_stride=2048)
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(r64x2), 0, 2048) == 256
    r128 = _rows(num_req=128, max_seq_len=65536, bt_width=1024, bt_stride=1024)
    assert lib.idx_workspace_bytes(B.IDX_OP_TOPK, None, ctypes.byref(r128), 0, 2048) == \
        256 + 2 * 4 * 128 * 2 * 4096 + 4 * 128 * 2
    assert lib.idx_num_rows(ctypes.byref(_rows(num_req=3, next_n=2))) == 6
    assert lib.idx_num_rows(ctypes.byref(_rows(kind=1, q_begin=4, q_end=9))) == 5
    assert lib.idx_num_rows(ctypes.byref(_rows(kind=1, q_begin=4, q_end=3))) == -1


def test_cache_write_validation_and_workspace(lib):
    E, U, S = B.IDX_EINVAL, B.IDX_EUNSUPPORTED, B.IDX_ENOSPC
    c = _cache()
    assert lib.idx_workspace_bytes(B.IDX_OP_CACHE_WRITE, ctypes.byref(c), None, 0, 0) == 256
    assert lib.idx_workspace_bytes(B.IDX_OP_CACHE_WRITE, ctypes.byref(_cache(head_dim=96)), None, 0, 0) == 0

    def w(cache=None, k=FAKE, stride=128, slots=FAKE, n=10, ws=FAKE, wsb=256):
        cache = cache or _cache()
        return lib.idx_cache_write(ctypes.byref(cache), k, stride, slots, n, ws, wsb, None)

    assert lib.idx_cache_write(None, FAKE, 128, FAKE, 10, FAKE, 256, None) == E
    assert w(cache=_cache(head_dim=96)) == U
    assert w(k=None) == E
    assert w(slots=None) == E
    assert w(k=FAKE + 8) == E                  # k not 16-byte aligned
    assert w(slots=FAKE + 4) == E              # slots not 8-byte aligned
    assert w(stride=64) == E                   # < head_dim
    assert w(stride=132) == E                  # not a multiple of 8
    assert w(n=-1) == E
    assert w(wsb=16) == S
    assert w(ws=FAKE + 8) == E
    assert w(n=0) == B.IDX_OK                  # nothing to enqueue


def test_compressed_cache_validation(lib):
    """Page size 256 and the compress ratio are checked on the host."""
    E, U = B.IDX_EINVAL, B.IDX_EUNSUPPORTED
    c256 = _cache(page_size=256, page_bytes=256 * 132)
    assert _logits(lib, _cache(page_size=128), _rows()) == U
    assert _logits(lib, _cache(page_size=256, page_bytes=64 * 132), _rows()) == E       # 256 rows do not fit
    assert _logits(lib, c256, _rows(max_seq_len=8 * 256 + 1)) == E                      # table too narrow
    assert _logits(lib, _cache(), _rows(max_seq_len=4 * 8 * 64 + 4, compress_ratio=4)) == E
    assert _logits(lib, _cache(), _rows(compress_ratio=-1)) == E
    assert _logits(lib, _cache(), _rows(compress_ratio=5000)) == U
    # the decode logits stride has to hold max_seq_len / ratio keys
    assert _logits(lib, _cache(), _rows(max_seq_len=400, compress_ratio=4), stride=99) == E
    assert b"compress_ratio" in lib.idx_last_error()


def test_noalloc_host_checks(lib):
    """idx_decode_topk_noalloc: argument checks and the static-scratch limit
    are decided on the host before anything is enqueued."""
    E, S = B.IDX_EINVAL, B.IDX_ENOSPC
    c = _cache()
    big = _rows(num_req=400, max_seq_len=131072, bt_width=2048, bt_stride=2048)
    assert lib.idx_decode_topk_noalloc(ctypes.byref(c), ctypes.byref(big), FAKE, FAKE, 64, 2048, FAKE, None,
                                       None) == S
    assert b"static scratch" in lib.idx_last_error()
    r = _rows()
    assert lib.idx_decode_topk_noalloc(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, 64, 16, None, None, None) == E
    assert lib.idx_decode_topk_noalloc(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, 64, 0, FAKE, None, None) == E
    assert lib.idx_decode_topk_noalloc(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, 64, 16, FAKE, FAKE + 2,
                                       None) == E
    empty = _rows(num_req=0)
    assert lib.idx_decode_topk_noalloc(ctypes.byref(c), ctypes.byref(empty), FAKE, FAKE, 64, 16, FAKE, None,
                                       None) == B.IDX_OK


def test_pool_host_checks(lib):
    """Pool selection: parameter checks on the host, workspace sizes."""
    E, U, S = B.IDX_EINVAL, B.IDX_EUNSUPPORTED, B.IDX_ENOSPC
    r = _rows(max_seq_len=300)

    def pt(pools, rows=r, out=FAKE, ws=FAKE, wsb=256, stride=512):
        return lib.idx_pool_topk(FAKE, stride, ctypes.byref(rows), ctypes.byref(pools) if pools else None, out,
                                 None, ws, wsb, None)

    assert pt(None) == E
    assert pt(B.IdxPools(48, 8, 0, 0)) == U                   # pool size
    assert pt(B.IdxPools(64, 0, 0, 0)) == E                   # no place
    assert pt(B.IdxPools(64, 513, 0, 0)) == U
    assert pt(B.IdxPools(64, 8, 5, 4)) == E                   # kept by position > topk
    assert pt(B.IdxPools(64, 8, -1, 0)) == E
    assert pt(B.IdxPools(64, 8, 1, 1), out=None) == E
    assert pt(B.IdxPools(64, 8, 1, 1), stride=100) == E       # stride < max_seq_len
    assert pt(B.IdxPools(64, 8, 1, 1), wsb=16) == S
    long_rows = _rows(max_seq_len=131072 + 16, bt_width=2049, bt_stride=2049)
    assert pt(B.IdxPools(16, 8, 1, 1), rows=long_rows, stride=1 << 20) == U   # 8193 pools
    assert pt(B.IdxPools(64, 8, 1, 1), rows=_rows(num_req=0)) == B.IDX_OK
    c = _cache()
    assert lib.idx_workspace_bytes(B.IDX_OP_POOL_TOPK, None, ctypes.byref(r), 0, 0) == 256
    assert lib.idx_workspace_bytes(B.IDX_OP_DECODE_POOL_TOPK, ctypes.byref(c), ctypes.byref(r), 64, 0) == \
        lib.idx_workspace_bytes(B.IDX_OP_DECODE_TOPK, ctypes.byref(c), ctypes.byref(r), 64, 16)
    need = lib.idx_workspace_bytes(B.IDX_OP_DECODE_POOL_TOPK, ctypes.byref(c), ctypes.byref(r), 64, 0)
    pl = B.IdxPools(64, 8, 1, 1)
    assert lib.idx_decode_pool_topk(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, 64, ctypes.byref(pl), FAKE, None,
                                    FAKE, need - 1, None) == S
    assert lib.idx_decode_pool_topk(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, 64, None, FAKE, None,
                                    FAKE, need, None) == E
