"""GPU parity of the decode path (idx_logits_paged, idx_topk, idx_decode_topk)
against the CPU oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev, check_logits, check_topk_e2e, fp32_rows, topk_workspace
from workloads import build_decode, config

pytestmark = pytest.mark.gpu

SEQS = [1, 63, 64, 65, 130, 700, 2000]


def _case(fmt, D, H, next_n, packed, seed):
    rng = np.random.default_rng(seed)
    dl = None
    if next_n > 1:
        dl = rng.integers(0, next_n + 1, size=len(SEQS)).astype(np.int32)
        dl[-1] = next_n      # at least one full request
    return build_decode(seed=seed, seq_lens=SEQS, heads=H, head_dim=D, topk=64, fmt=fmt,
                        next_n=next_n, decode_lens=dl, q_packed=packed, name=f"{fmt}-D{D}-H{H}-n{next_n}")


SHAPES = [
    ("fp8", 128, 64, 1, False),
    ("fp8", 128, 64, 2, False),
    ("fp8", 128, 64, 2, True),
    ("fp8", 128, 32, 3, False),
    ("fp8", 64, 64, 1, False),
    ("fp8", 64, 17, 2, True),
    ("fp8", 32, 4, 1, False),
    ("fp8", 32, 48, 2, False),
    ("mxfp4", 128, 64, 1, False),
    ("mxfp4", 128, 64, 2, False),
    ("mxfp4", 128, 8, 1, False),
    ("fp8", 128, 64, 4, False),
    ("fp8", 128, 64, 3, True),
    ("fp8", 64, 16, 5, False),
    ("mxfp4", 128, 64, 4, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_logits_and_topk_shapes(shape):
    fmt, D, H, nn, packed = shape
    wl = _case(fmt, D, H, nn, packed, seed=100 + SHAPES.index(shape))
    print(f"case {wl.name} packed={packed} seqs={SEQS} dl={wl.decode_lens}", flush=True)
    dev = Dev(wl)
    ref = oracle.pipeline.decode_logits(wl)
    got, _ = dev.logits_decode()
    check_logits(got, {r: v for r, v in ref.items() if len(v)}, label=wl.name)
    # rows with L = 0 are never written
    L, _ = oracle.pipeline.decode_row_info(wl)
    for r in np.nonzero(L == 0)[0]:
        assert np.isnan(got[r]).all()
    out, _ = dev.decode_topk()
    check_topk_e2e(out, ref, L, wl.topk, label=wl.name)


def test_c1_tiny_decode():
    wl = config("C1")
    dev = Dev(wl)
    ref = oracle.pipeline.decode_logits(wl)
    got, _ = dev.logits_decode()
    check_logits(got, ref, label="C1")
    out, _ = dev.decode_topk()
    L, _ = oracle.pipeline.decode_row_info(wl)
    check_topk_e2e(out, ref, L, wl.topk, label="C1")
    # the fused path selects exactly what the oracle's selection picks from
    # the GPU's own logits (same fp32 values, so bit-exact)
    exp = oracle.topk.topk_row(got[0, : L[0]].astype(np.float64), int(L[0]), wl.topk)
    assert out.shape == (1, 64) and np.array_equal(out[0], exp)
    # and idx_topk on the oracle's fp32-rounded logits is the oracle's selection
    buf = fp32_rows(ref, 1, got.shape[1])
    rows = dev.decode_rows()
    o2 = torch.full((1, wl.topk), -7, dtype=torch.int32, device=dev.device)
    idx.idx_topk(torch.from_numpy(buf).to(dev.device), rows, wl.topk, o2, topk_workspace(rows, wl.topk))
    exp2 = oracle.topk.topk_row(buf[0, : L[0]].astype(np.float64), int(L[0]), wl.topk)
    assert np.array_equal(o2.cpu().numpy()[0], exp2)


SEQS_LONG = [5000, 33000, 70001, 140001]
LONG_SHAPES = [("fp8", 128, 64, 1, False), ("fp8", 128, 64, 2, True), ("mxfp4", 128, 64, 1, False),
               ("fp8", 64, 16, 3, False)]


@pytest.mark.parametrize("shape", LONG_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_long_rows(shape):
    """Rows from 5000 to 140001 keys (past the selector's 32768-key register
    rows and its 131072-position bitmap), k = 2048, next_n 1..3."""
    fmt, D, H, nn, packed = shape
    rng = np.random.default_rng(300 + LONG_SHAPES.index(shape))
    dl = None if nn == 1 else rng.integers(1, nn + 1, size=len(SEQS_LONG)).astype(np.int32)
    wl = build_decode(seed=300 + LONG_SHAPES.index(shape), seq_lens=SEQS_LONG, heads=H, head_dim=D, topk=2048,
                      fmt=fmt, next_n=nn, decode_lens=dl, q_packed=packed, name=f"long-{fmt}-D{D}-H{H}-n{nn}")
    print(f"case {wl.name} packed={packed} seqs={SEQS_LONG} dl={dl}", flush=True)
    dev = Dev(wl)
    ref = oracle.pipeline.decode_logits(wl)
    got, _ = dev.logits_decode()
    check_logits(got, {r: v for r, v in ref.items() if len(v)}, label=wl.name)
    L, _ = oracle.pipeline.decode_row_info(wl)
    out, _ = dev.decode_topk()
    check_topk_e2e(out, ref, L, wl.topk, label=wl.name)


def _topk_rows(k):
    """Rows of every length class the selector distinguishes (empty, L <= k,
    register-resident up to 32768, streamed beyond) and value patterns that
    stress its digits: ties, signed zeros, one value, huge and infinite
    magnitudes, subnormals, 60 decades of range, tied levels at the top."""
    rng = np.random.default_rng(5)
    lens = [0, 1, k - 1, k, k + 1, 100, 1000, 5000, 33000, 131072, 3000, 20000, 32768, 32769, 9000, 12000]
    rows = []
    for i, L in enumerate(lens):
        kind = i % 8
        if kind == 0:
            v = rng.standard_normal(L).astype(np.float32) * 8
        elif kind == 1:
            v = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32), size=L)
        elif kind == 2:
            v = np.full(L, 3.25, dtype=np.float32)
        elif kind == 3:
            v = (rng.integers(-3, 4, size=L) * 0.125).astype(np.float32)
            v[::7] = -0.0
        elif kind == 4:
            v = np.clip(rng.standard_normal(L) * 1e38, -3.3e38, 3.3e38).astype(np.float32)
            v[::97] = np.inf
            v[5::89] = -np.inf
        elif kind == 5:
            v = (rng.standard_normal(L) * 1e-40).astype(np.float32)   # subnormals
        elif kind == 6:
            v = (rng.choice([-1.0, 1.0], size=L) * 10.0 ** rng.uniform(-30, 30, size=L)).astype(np.float32)
        else:
            v = (rng.integers(0, 50, size=L) * 0.1).astype(np.float32)
        rows.append(v)
    return lens, rows


@pytest.mark.parametrize("k", [1, 64, 2048])
def test_topk_bitexact_on_given_logits(k):
    lens, rows = _topk_rows(k)
    R = len(lens)
    stride = max(lens) + 3        # rows start at unaligned addresses too
    buf = np.full((R, stride), np.nan, dtype=np.float32)
    for r, v in enumerate(rows):
        buf[r, : len(v)] = v
    d = torch.device("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device=d)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=d)
    rows_d = idx.Rows.decode(bt, seq, max(lens))
    logits = torch.from_numpy(buf).to(d)
    out = torch.full((R, k), -7, dtype=torch.int32, device=d)
    ws = topk_workspace(rows_d, k, d)
    idx.idx_topk(logits, rows_d, k, out, ws)
    got = out.cpu().numpy()
    for r, v in enumerate(rows):
        exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
        assert np.array_equal(got[r], exp), f"row {r} (L={lens[r]}) differs"


@pytest.mark.parametrize("k", [64, 2048])
def test_topk_bitexact_many_rows_with_long_ones(k):
    """A batch with at least two rows per CU and rows past the register
    path: the selector runs its streaming-only kernel (several rows per CU)
    on every row, short ones included."""
    rng = np.random.default_rng(17)
    base = [0, 1, k - 1, k, k + 1, 100, 1000, 5000, 33000, 3000, 20000, 32768, 32769, 9000, 12000, 40000]
    R = 600
    lens = [base[i % len(base)] for i in range(R)]
    rows = []
    for i, L in enumerate(lens):
        kind = (i // len(base)) % 4
        if kind == 0:
            v = rng.standard_normal(L).astype(np.float32) * 8
        elif kind == 1:
            v = (rng.integers(-3, 4, size=L) * 0.125).astype(np.float32)
            v[::7] = -0.0
        elif kind == 2:
            v = (rng.choice([-1.0, 1.0], size=L) * 10.0 ** rng.uniform(-30, 30, size=L)).astype(np.float32)
        else:
            v = (rng.integers(0, 50, size=L) * 0.1).astype(np.float32)
        rows.append(v)
    stride = max(lens) + 3
    buf = np.full((R, stride), np.nan, dtype=np.float32)
    for r, v in enumerate(rows):
        buf[r, : len(v)] = v
    d = torch.device("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device=d)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=d)
    rows_d = idx.Rows.decode(bt, seq, max(lens))
    out = torch.full((R, k), -7, dtype=torch.int32, device=d)
    idx.idx_topk(torch.from_numpy(buf).to(d), rows_d, k, out, topk_workspace(rows_d, k, d))
    got = out.cpu().numpy()
    for r, v in enumerate(rows):
        exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
        assert np.array_equal(got[r], exp), f"row {r} (L={lens[r]}) differs"


def test_topk_bitexact_on_oracle_logits():
    wl = _case("fp8", 128, 64, 2, False, seed=7)
    ref = oracle.pipeline.decode_logits(wl)
    L, _ = oracle.pipeline.decode_row_info(wl)
    R = wl.num_req * wl.next_n
    stride = int(L.max())
    buf = fp32_rows(ref, R, stride)
    d = torch.device("cuda")
    dev = Dev(wl)
    out = torch.full((R, wl.topk), -7, dtype=torch.int32, device=d)
    idx.idx_topk(torch.from_numpy(buf).to(d), dev.decode_rows(), wl.topk, out,
                 topk_workspace(dev.decode_rows(), wl.topk, d))
    got = out.cpu().numpy()
    for r in range(R):
        exp = oracle.topk.topk_row(buf[r, : L[r]].astype(np.float64), int(L[r]), wl.topk)
        assert np.array_equal(got[r], exp), f"row {r}"


def test_decode_topk_workspace_reuse_and_determinism():
    wl = _case("fp8", 128, 64, 2, False, seed=9)
    dev = Dev(wl)
    out1, ws = dev.decode_topk()
    out2, _ = dev.decode_topk(ws)
    assert np.array_equal(out1, out2)
    # the status word stays clear on valid input
    assert int(ws[:4].view(torch.int32).cpu()[0]) == 0
    # a smaller batch reusing the same (larger) workspace
    wl2 = _case("fp8", 128, 64, 1, False, seed=10)
    dev2 = Dev(wl2)
    out3, _ = dev2.decode_topk(ws)
    ref = oracle.pipeline.decode_logits(wl2)
    L, _ = oracle.pipeline.decode_row_info(wl2)
    check_topk_e2e(out3, ref, L, wl2.topk, label="reuse")


def test_bad_page_id_flags_and_never_faults():
    wl = _case("fp8", 128, 64, 1, False, seed=11)
    bt = wl.block_table.copy()
    bt[3, 0] = wl.num_pages + 5          # request 3's first page points outside the pool
    wl.block_table = bt
    dev = Dev(wl)
    _, ws = dev.logits_decode()
    assert idx.idx_read_device_status(ws) & idx.IDX_DEV_BAD_PAGE
    assert idx.idx_read_device_status(ws) == 0      # read clears it


@pytest.mark.parametrize("rows_kind", ["short", "long"])
def test_decode_topk_in_a_hip_graph_replays(rows_kind):
    """idx_decode_topk captured in a HIP graph: every replay, with other
    eager work and synchronisation in between and new query contents each
    time, gives the eager result for those contents.  "long" rows exceed
    32768 keys, so the selector's chunk and merge launches are captured."""
    if rows_kind == "short":
        wl = _case("fp8", 128, 64, 2, False, seed=12)
    else:
        wl = build_decode(seed=13, seq_lens=[40000, 131072, 500, 70001], heads=16, head_dim=64, topk=256,
                          name="graph-long")
    dev = Dev(wl)
    rows = dev.decode_rows()
    k = wl.topk
    d = dev.device
    q_a = dev.q.clone()
    q_b = torch.roll(dev.q, shifts=1, dims=0).contiguous()   # other rows' queries
    qbuf = dev.q.clone()
    out = torch.full((rows.num_rows, k), -7, dtype=torch.int32, device=d)
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_TOPK, dev.cache, rows, wl.heads, k), d)
    refs = []
    for qv in (q_a, q_b):
        qbuf.copy_(qv)
        idx.idx_decode_topk(dev.cache, rows, qbuf, dev.w, k, out, ws)
        torch.cuda.synchronize()
        refs.append(out.clone())
    assert not torch.equal(refs[0], refs[1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        idx.idx_decode_topk(dev.cache, rows, qbuf, dev.w, k, out, ws)
    torch.cuda.synchronize()
    other = torch.full((rows.num_rows, max(dev.max_len, 1)), float("nan"), device=d)
    ows = idx.new_workspace(256, d)
    for i in range(6):
        qbuf.copy_(q_a if i % 2 == 0 else q_b)
        out.fill_(-7)
        idx.idx_logits_paged(dev.cache, rows, dev.q, dev.w, other, ows)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[i % 2]), f"replay {i}"


@pytest.mark.parametrize("k", [64, 2048, 4096])
def test_topk_long_rows_split_over_workgroups(k):
    """Rows past the register path in a small batch are selected chunk by
    chunk (32768 keys per workgroup) and merged: bit-exact against the
    oracle, with ties that straddle chunk boundaries."""
    rng = np.random.default_rng(41)
    lens = [32769, 65536, 98321, 131072, 40000, 131071, 70000, 5000]
    rows = []
    for i, L in enumerate(lens):
        kind = i % 4
        if kind == 0:
            v = np.full(L, -2.5, dtype=np.float32)                       # every key ties
        elif kind == 1:
            v = (rng.integers(0, 3, size=L) * 0.5).astype(np.float32)    # three levels
            v[32760:32780] = 1.0                                          # ties across the first boundary
        elif kind == 2:
            v = np.linspace(1.0, -1.0, L).astype(np.float32)             # largest keys first
            v[::2] = -0.0
        else:
            v = (rng.standard_normal(L) * 4).astype(np.float32)
            v[-k:] = 100.0                                                # the top-k sits in the last chunk
        rows.append(v)
    R = len(lens)
    stride = max(lens) + 5
    buf = np.full((R, stride), np.nan, dtype=np.float32)
    for r, v in enumerate(rows):
        buf[r, : len(v)] = v
    d = torch.device("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device=d)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=d)
    rows_d = idx.Rows.decode(bt, seq, max(lens))
    out = torch.full((R, k), -7, dtype=torch.int32, device=d)
    ws = topk_workspace(rows_d, k)
    assert ws.numel() > 256                 # the chunk candidates live in the workspace
    idx.idx_topk(torch.from_numpy(buf).to(d), rows_d, k, out, ws)
    o = out.cpu().numpy()
    for r, v in enumerate(rows):
        exp = oracle.topk.topk_row(v.astype(np.float64), len(v), k)
        assert np.array_equal(o[r], exp), f"row {r} (L={len(v)}, k={k})"


@pytest.mark.parametrize("k", [1, 100, 2048, 4096])
def test_topk_split_random_mix(k):
    """A seeded mix of short rows and rows split over workgroups (odd row
    count, lengths at and around the 32768-key chunk boundaries, tied and
    untied values): every row bit-exact against the oracle."""
    rng = np.random.default_rng(4000 + k)
    fixed = [32768, 32769, 65536, 65537, 98304, 131072, 1, k, k + 1]
    lens = fixed + [int(x) for x in rng.integers(1, 32769, size=10)] + \
        [int(x) for x in rng.integers(32769, 131073, size=18)]
    rows = []
    for i, L in enumerate(lens):
        if i % 3 == 0:
            v = (np.round(rng.standard_normal(L) * 4) / 4).astype(np.float32)   # many ties
        else:
            v = rng.standard_normal(L).astype(np.float32)
        rows.append(v)
    R = len(lens)
    assert R % 8 != 0
    stride = max(lens) + 1
    buf = np.full((R, stride), np.nan, dtype=np.float32)
    for r, v in enumerate(rows):
        buf[r, : len(v)] = v
    d = torch.device("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device=d)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=d)
    rows_d = idx.Rows.decode(bt, seq, max(lens))
    out = torch.full((R, k), -7, dtype=torch.int32, device=d)
    ws = topk_workspace(rows_d, k, d)
    assert ws.numel() > 256                 # the split path is taken
    print(f"split mix k={k}: {R} rows, lengths {min(lens)}..{max(lens)}", flush=True)
    idx.idx_topk(torch.from_numpy(buf).to(d), rows_d, k, out, ws)
    got = out.cpu().numpy()
    for r, v in enumerate(rows):
        exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
        assert np.array_equal(got[r], exp), f"row {r} (L={lens[r]}, k={k}) differs"
