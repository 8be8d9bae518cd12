"""GPU: seeded random batches through idx_topk, bit-exact against the oracle.

Each case draws a batch shape that picks one of the selector's launches --
a small batch of long rows (split over workgroups: one shared threshold for
k <= 2048, a top-k per chunk above), a medium batch with rows past the
bitmap (one 1024-thread workgroup per row: register, one-read and two-read
paths), a batch of at least 512 rows (the 512-thread streaming kernel), or
short rows (the register path and the causal fill) -- a k among 1..4096,
a row stride that leaves most rows unaligned, and per row one of the value
patterns of the one-read tests (infinities on and off the sampled blocks,
ulp-close values, three levels with signed zeros, crowded tops, a flat field
with a few winners, a permuted ramp) or plain and quantized normal values.
Every row must equal the oracle's top-k (ties to the lower position) and
the slack row after the output must stay untouched.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import topk_workspace
from tests.test_gpu_topk_sampled import _pattern

pytestmark = pytest.mark.gpu

KS = [1, 7, 64, 100, 1000, 2047, 2048, 2049, 3000, 4096]


def _case(rng, mode):
    k = int(rng.choice(KS))
    if mode == 0:      # small batch of long rows: split over workgroups
        R, hi = int(rng.integers(1, 65)), 131072
    elif mode == 1:    # mixed, rows past the bitmap too
        R, hi = int(rng.integers(65, 300)), 140000
    elif mode == 2:    # at least 512 rows: the streaming-only kernel
        R, hi = int(rng.integers(512, 700)), 70000
    else:              # short rows
        R, hi = int(rng.integers(1, 200)), 33000
    lens = [int(x) for x in rng.integers(1, hi + 1, size=R)]
    vals = []
    for L in lens:
        kind = int(rng.integers(0, 10))
        if kind < 8 and L >= max(16, k):
            v = _pattern(kind, L, k, rng)
        elif kind == 8:
            v = (np.round(rng.standard_normal(L) * 2) / 2).astype(np.float32)
        else:
            v = rng.standard_normal(L).astype(np.float32)
        vals.append(v)
    return k, lens, vals


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_random_batches_bitexact(mode):
    rng = np.random.default_rng(9100 + mode)
    d = torch.device("cuda")
    for case in range(8):
        k, lens, vals = _case(rng, mode)
        R = len(lens)
        stride = max(lens) + int(rng.integers(0, 5))
        buf = np.full((R, stride), np.nan, dtype=np.float32)
        for r, v in enumerate(vals):
            buf[r, : len(v)] = v
        seq = torch.tensor(lens, dtype=torch.int32, device=d)
        rows = idx.Rows.decode(torch.zeros((R, 1), dtype=torch.int32, device=d), seq, max(lens))
        out = torch.full((R + 1, k), -7, dtype=torch.int32, device=d)
        ws = topk_workspace(rows, k, d)
        print(f"mode {mode} case {case}: {R} rows, L {min(lens)}..{max(lens)}, k {k}, stride {stride}", flush=True)
        idx.idx_topk(torch.from_numpy(buf).to(d), rows, k, out[:R], ws)
        got = out.cpu().numpy()
        assert (got[R] == -7).all(), "the selector wrote past the last output row"
        for r, v in enumerate(vals):
            exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
            assert np.array_equal(got[r], exp), f"mode {mode} case {case} row {r} (L={lens[r]}, k={k}) differs"
