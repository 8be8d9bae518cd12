"""GPU: the pool-level selection (idx_pool_topk, idx_decode_pool_topk)
against the oracle (oracle/pool.py), through the C ABI.

On given logits the selection is bit-exact (both sides take the pool maxima
of the same fp32 values); end to end, the kept pools equal the oracle's
except pools whose oracle score lies within the logits tolerance of the
score at the selection's boundary, and the fused path equals the oracle's
selection on the GPU's own logits exactly.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import ATOL, RTOL, Dev, check_logits
from workloads import build_decode, config

pytestmark = pytest.mark.gpu


def _values(kind, L, rng):
    if L == 0:
        return np.zeros(0, dtype=np.float32)
    if kind == 0:
        return (rng.standard_normal(L) * 3).astype(np.float32)
    if kind == 1:
        v = (rng.integers(-4, 5, size=L) * 0.5).astype(np.float32)
        v[rng.random(L) < 0.3] = -0.0
        return v
    if kind == 2:
        return np.full(L, -1.5, dtype=np.float32)
    if kind == 3:
        v = np.where(rng.random(L) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        v[rng.integers(0, L, size=max(1, L // 50))] = 2.0
        return v
    return np.clip(rng.standard_normal(L) * 1e37, -3e38, 3e38).astype(np.float32)


CASES = [  # pool_size, topk, init, local
    (64, 32, 1, 2), (16, 8, 0, 0), (32, 100, 4, 4), (128, 3, 1, 1), (64, 1, 0, 0), (16, 512, 10, 20),
    (64, 5, 2, 3), (32, 17, 0, 5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_pool_topk_bitexact_on_given_logits(case):
    B, k, init, local = case
    rng = np.random.default_rng(B * 1000 + k)
    lens = [0, 1, B - 1, B, B + 1, k * B, k * B + 7, (k + 1) * B, 5000, 32768, 40001, 131072 if B >= 16 else 8192,
            777, 3 * B + 2]
    lens += [int(x) for x in rng.integers(0, 60000, size=18)]
    R = len(lens)
    stride = max(lens) + 3
    buf = np.full((R, stride), np.nan, dtype=np.float32)
    vals = []
    for r, L in enumerate(lens):
        v = _values(r % 5, L, rng)
        buf[r, :L] = v
        vals.append(v)
    d = torch.device("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device=d)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=d)
    rows = idx.Rows.decode(bt, seq, max(lens))
    pl = idx.pools(B, k, init, local)
    W = (k + 1) * B
    toks = torch.full((R + 1, W), -7, dtype=torch.int32, device=d)   # one slack row
    pools = torch.full((R + 1, k), -7, dtype=torch.int32, device=d)
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_POOL_TOPK, None, rows, 0, 0), d)
    print(f"idx_pool_topk B={B} k={k} init={init} local={local}: {R} rows, max L {max(lens)}", flush=True)
    idx.idx_pool_topk(torch.from_numpy(buf).to(d), rows, pl, toks[:R], pools[:R], ws)
    gt, gp = toks.cpu().numpy(), pools.cpu().numpy()
    assert (gt[R] == -7).all() and (gp[R] == -7).all(), "wrote past the last row"
    for r, v in enumerate(vals):
        et, ep = oracle.pool.pool_topk_row(v.astype(np.float64), lens[r], B, k, init, local)
        assert np.array_equal(gp[r], ep), f"row {r} (L={lens[r]}) pools differ"
        assert np.array_equal(gt[r], et), f"row {r} (L={lens[r]}) tokens differ"
    # out_pools is optional
    toks2 = torch.full((R, W), -7, dtype=torch.int32, device=d)
    idx.idx_pool_topk(torch.from_numpy(buf).to(d), rows, pl, toks2, None, ws)
    assert np.array_equal(toks2.cpu().numpy(), gt[:R])


def test_pool_topk_prefill_rows():
    """Prefill chunk rows: each row's window starts at its request's column
    base; rows of the second request see columns past the first's keys."""
    rng = np.random.default_rng(77)
    seq, ql = [3000, 9000], [40, 25]
    q_begin, q_end = 10, 60
    N = sum(seq)
    M = q_end - q_begin
    buf = (rng.standard_normal((M, N)) * 2).astype(np.float32)
    buf[::3] = np.round(buf[::3])                  # ties
    d = torch.device("cuda")
    qsl = torch.tensor([0, 40, 65], dtype=torch.int32, device=d)
    bt = torch.zeros((2, 1), dtype=torch.int32, device=d)
    rows = idx.Rows.prefill(bt, torch.tensor(seq, dtype=torch.int32, device=d), qsl, q_begin, q_end, max(seq))
    B, k, init, local = 64, 12, 1, 2
    toks = torch.full((M, (k + 1) * B), -7, dtype=torch.int32, device=d)
    pools = torch.full((M, k), -7, dtype=torch.int32, device=d)
    ws = idx.new_workspace(256, d)
    idx.idx_pool_topk(torch.from_numpy(buf).to(d), rows, idx.pools(B, k, init, local), toks, pools, ws)
    gt, gp = toks.cpu().numpy(), pools.cpu().numpy()
    for r in range(M):
        tok = q_begin + r
        b = 0 if tok < 40 else 1
        j = tok - (0 if b == 0 else 40)
        L = seq[b] - ql[b] + j + 1
        ks = 0 if b == 0 else seq[0]
        et, ep = oracle.pool.pool_topk_row(buf[r, ks : ks + L].astype(np.float64), L, B, k, init, local)
        assert np.array_equal(gp[r], ep) and np.array_equal(gt[r], et), f"prefill row {r}"


def check_pools_e2e(got_pools, ref_logits, L, B, k, init, local, label=""):
    """Kept pools against the oracle's fp64 logits: the same count, the
    kept-by-position pools present, and any pool in the symmetric difference
    scoring within the tolerance of the boundary score."""
    for r in range(got_pools.shape[0]):
        Lr = int(L[r])
        lg = ref_logits.get(r, np.zeros(0))
        _, ep = oracle.pool.pool_topk_row(lg, Lr, B, k, init, local)
        g = set(got_pools[r][got_pools[r] >= 0].tolist())
        e = set(ep[ep >= 0].tolist())
        assert len(g) == len(e), f"{label} row {r}: {len(g)} pools, want {len(e)}"
        diff = g ^ e
        if not diff:
            continue
        n = Lr // B
        m = lg[: n * B].reshape(n, B).max(axis=1)
        a = min(init, n)
        z = min(local, n - a)
        forced = set(range(a)) | set(range(n - z, n))
        assert not (diff & forced), f"{label} row {r}: a kept-by-position pool is missing"
        cand = sorted(set(range(n)) - forced)
        order = sorted(cand, key=lambda p: (-m[p], p))
        edge = m[order[k - len(forced) - 1]]
        far = [p for p in diff if abs(m[p] - edge) > ATOL + RTOL * abs(edge)]
        assert not far, f"{label} row {r}: pools {far[:4]} differ beyond tolerance"


POOL_DECODE = [("fp8", 128, 64, 1, 64, 32, 1, 2), ("fp8", 128, 64, 2, 16, 64, 2, 4), ("mxfp4", 128, 32, 1, 128, 8, 1, 1),
               ("fp8", 64, 16, 3, 32, 10, 0, 3)]


@pytest.mark.parametrize("shape", POOL_DECODE, ids=lambda s: "-".join(map(str, s)))
def test_decode_pool_topk_end_to_end(shape):
    fmt, D, H, nn, B, k, init, local = shape
    rng = np.random.default_rng(900 + POOL_DECODE.index(shape))
    seqs = [1, B - 1, B, 3 * B + 5, k * B, k * B + B + 3, 5000, 33000, 70001, 131072 if B >= 32 else 120000]
    dl = None if nn == 1 else rng.integers(0, nn + 1, size=len(seqs)).astype(np.int32)
    wl = build_decode(seed=900 + POOL_DECODE.index(shape), seq_lens=seqs, heads=H, head_dim=D, topk=2048, fmt=fmt,
                      next_n=nn, decode_lens=dl, name=f"pool-{fmt}-D{D}-n{nn}-B{B}")
    print(f"case {wl.name} k={k} init={init} local={local} dl={dl}", flush=True)
    dev = Dev(wl)
    rows = dev.decode_rows()
    R = rows.num_rows
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_POOL_TOPK, dev.cache, rows, H, 0), dev.device)
    pl = idx.pools(B, k, init, local)
    toks = torch.full((R, (k + 1) * B), -7, dtype=torch.int32, device=dev.device)
    pools = torch.full((R, k), -7, dtype=torch.int32, device=dev.device)
    idx.idx_decode_pool_topk(dev.cache, rows, dev.q, dev.w, pl, toks, pools, ws)
    torch.cuda.synchronize()
    assert idx.idx_read_device_status(ws) == 0
    gt, gp = toks.cpu().numpy(), pools.cpu().numpy()
    ref = oracle.pipeline.decode_logits(wl)
    L, _ = oracle.pipeline.decode_row_info(wl)
    got, _ = dev.logits_decode()
    check_logits(got, {r: v for r, v in ref.items() if len(v)}, label=wl.name)
    check_pools_e2e(gp, ref, L, B, k, init, local, label=wl.name)
    # the fused selection is the oracle's selection on the GPU's own logits
    for r in range(R):
        et, ep = oracle.pool.pool_topk_row(got[r, : L[r]].astype(np.float64), int(L[r]), B, k, init, local)
        assert np.array_equal(gp[r], ep) and np.array_equal(gt[r], et), f"{wl.name} row {r}"


def test_pool_workload_p2_every_row():
    """The benchmark's pool workload: the C2 batch with pools of 64 keys,
    32 kept, the first and the last two always kept."""
    wl = config("C2")
    B, k, init, local = 64, 32, 1, 2
    dev = Dev(wl)
    rows = dev.decode_rows()
    R = rows.num_rows
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_POOL_TOPK, dev.cache, rows, wl.heads, 0),
                           dev.device)
    toks = torch.full((R, (k + 1) * B), -7, dtype=torch.int32, device=dev.device)
    pools = torch.full((R, k), -7, dtype=torch.int32, device=dev.device)
    idx.idx_decode_pool_topk(dev.cache, rows, dev.q, dev.w, idx.pools(B, k, init, local), toks, pools, ws)
    gp = pools.cpu().numpy()
    ref = oracle.pipeline.decode_logits(wl)
    L, _ = oracle.pipeline.decode_row_info(wl)
    check_pools_e2e(gp, ref, L, B, k, init, local, label="P2")
