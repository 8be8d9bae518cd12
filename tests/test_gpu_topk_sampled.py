"""GPU: the one-read selection of long rows, bit-exact against the oracle.

Rows of 16384..131072 keys with k <= 2048 first try one read: a systematic
sample (every S-th 64-key block, S = 16 up to 65536 keys and 32 up to
131072) in linear bins gives a threshold bin, one pass collects the keys
whose bin value reaches it, and the exact selection runs on those
candidates (linear bins over their range, then the keys of the threshold
bin by rank or by radix passes).  A degenerate or infinite sample range, or
too few or too many candidates, falls back to the two-read path.  The rows
here aim at each branch: infinities kept off the sampled blocks (so the
candidates' range is infinite and their exact selection runs on one bin),
infinities on the sampled blocks (fallback), values a few ulps apart,
three levels with signed zeros (heavy ties in the threshold bin), the top
keys crowded at one end of the row, and plain random rows.  Both selector
kernels are covered: one 1024-thread workgroup per row (80 rows whose
split would take more than 256 workgroups) and the 512-thread
streaming-only kernel (512 rows); and a batch small enough that its long
rows are split over workgroups that share the sample threshold, each
collecting one 32768-key chunk, with one workgroup per row selecting among
the chunks' candidates (or from the whole row when the chunks together hold
too few or too many).  Every output row carries a slack row after it that
must stay untouched.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import topk_workspace

pytestmark = pytest.mark.gpu


def _off_sample(L):
    """Positions of the 64-key blocks the sample never reads (block index 5
    mod 16: not a multiple of 16 or 32)."""
    pos = np.arange(L)
    return (pos // 64) % 16 == 5


def _pattern(kind, L, k, rng):
    if kind == 0:
        return (rng.standard_normal(L) * 3).astype(np.float32)
    if kind == 1:   # a few +inf and many -inf, all off the sampled blocks
        v = (rng.standard_normal(L) * 3).astype(np.float32)
        off = np.flatnonzero(_off_sample(L))
        v[rng.choice(off, size=min(len(off), max(1, k // 3)), replace=False)] = np.inf
        v[rng.choice(off, size=len(off) // 2, replace=False)] = -np.inf
        return v
    if kind == 2:   # infinities on the sampled blocks too
        v = (rng.standard_normal(L) * 3).astype(np.float32)
        v[::997] = np.inf
        v[3::991] = -np.inf
        return v
    if kind == 3:   # eight values a few ulps apart
        vals = [np.float32(1.0)]
        for _ in range(7):
            vals.append(np.nextafter(vals[-1], np.float32(2)))
        return np.array(vals, dtype=np.float32)[rng.integers(0, 8, size=L)]
    if kind == 4:   # three levels and signed zeros
        v = (rng.integers(-1, 2, size=L) * 0.75).astype(np.float32)
        v[v == 0] = np.where(rng.random(int((v == 0).sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
        return v
    if kind == 5:   # the largest keys crowded at the end of the row
        v = (rng.standard_normal(L) * 0.1).astype(np.float32)
        v[-(2 * k + 7):] += np.float32(5.0)
        return v
    if kind == 6:   # k/2 clear winners above a flat field
        v = np.full(L, 2.0, dtype=np.float32)
        v[rng.choice(L, size=max(1, k // 2), replace=False)] = 3.0
        return v
    return np.linspace(-1.0, 1.0, L, dtype=np.float32)[rng.permutation(L)]


def _run(lens, vals, k):
    R = len(lens)
    stride = max(lens) + 3          # rows at unaligned addresses too
    buf = np.full((R, stride), np.nan, dtype=np.float32)
    for r, v in enumerate(vals):
        buf[r, : len(v)] = v
    d = torch.device("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device=d)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=d)
    rows = idx.Rows.decode(bt, seq, max(lens))
    out = torch.full((R + 1, k), -7, dtype=torch.int32, device=d)
    ws = topk_workspace(rows, k, d)
    print(f"idx_topk: {R} rows, L {min(lens)}..{max(lens)}, k {k}", flush=True)
    idx.idx_topk(torch.from_numpy(buf).to(d), rows, k, out[:R], ws)
    got = out.cpu().numpy()
    assert (got[R] == -7).all(), "the selector wrote past the last output row"
    for r, v in enumerate(vals):
        exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
        assert np.array_equal(got[r], exp), f"row {r} (L={lens[r]}, pattern {r % 8}) differs"


@pytest.mark.parametrize("k", [1, 100, 2048])
def test_one_read_selection_workgroup_per_row(k):
    rng = np.random.default_rng(5000 + k)
    lens = [int(x) for x in rng.integers(32769, 131073, size=72)] + [32769, 65536, 98304, 131072, 40000,
                                                                     131071, 70001, 100000]
    vals = [_pattern(i % 8, L, k, rng) for i, L in enumerate(lens)]
    _run(lens, vals, k)


@pytest.mark.parametrize("k", [1, 100, 2048])
def test_one_read_selection_lean_kernel(k):
    rng = np.random.default_rng(6000 + k)
    lens = [int(x) for x in rng.integers(16384, 65537, size=504)] + [16384, 16385, 32768, 32769, 65535,
                                                                      65536, 20000, 50001]
    vals = [_pattern(i % 8, L, k, rng) for i, L in enumerate(lens)]
    _run(lens, vals, k)


@pytest.mark.parametrize("k", [1, 100, 2048])
def test_one_read_selection_split_rows(k):
    rng = np.random.default_rng(7000 + k)
    lens = [32769, 65536, 98304, 131072, 40000, 131071, 70001, 100000, 5000, 32768, 2 * k + 9, 65537, 120000,
            90001, 33000, 131072]
    vals = [_pattern(i % 8, L, k, rng) for i, L in enumerate(lens)]
    _run(lens, vals, k)
