"""GPU: seeded random decode batches through idx_logits_paged and
idx_decode_topk, against the oracle.

Each case draws every argument the decode path takes from its legal range:
key format (fp8 e4m3 at head_dim 32/64/128, MXFP4 at 128), 1..64 heads, next_n
1..5 with per-request decode_lens 0..next_n (packed queries or the padded
grid), 1..32 requests whose lengths mix page-boundary values (64 j - 1,
64 j, 64 j + 1), short rows, rows around k and a few rows past the
selector's 32768-key register rows, a block table wider than needed over a
pool with spare pages, and k in 1..4096.  The logits must match the oracle
within |gpu - oracle| <= 1e-4 + 2e-3 |oracle| (columns past a row's length
untouched, padded rows never written), the device status word must stay
clear, and the top-k rows must be the oracle's up to keys within that
tolerance of the k-th largest logit.
"""

import numpy as np
import pytest

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev, check_logits, check_topk_e2e
from workloads import build_decode

pytestmark = pytest.mark.gpu

KS = [1, 5, 64, 300, 2048, 4096]


def _lengths(rng, n, k):
    out = []
    for _ in range(n):
        kind = int(rng.integers(0, 6))
        if kind == 0:    # a page boundary
            L = 64 * int(rng.integers(1, 40)) + int(rng.integers(-1, 2))
        elif kind == 1:  # short
            L = int(rng.integers(1, 130))
        elif kind == 2:  # around k
            L = max(1, k + int(rng.integers(-2, 3)))
        elif kind == 3:  # long: register rows and past them
            L = int(rng.integers(20000, 40001))
        else:            # medium
            L = int(rng.integers(130, 6000))
        out.append(L)
    return np.array(out, dtype=np.int32)


def _case(i):
    rng = np.random.default_rng(9200 + i)
    fmt = "mxfp4" if rng.random() < 0.35 else "fp8"
    D = int(rng.choice([32, 64, 128])) if fmt == "fp8" else 128
    H = int(rng.integers(1, 65))
    nn = int(rng.integers(1, 6))
    k = int(rng.choice(KS))
    B = int(rng.integers(1, 33))
    seq = _lengths(rng, B, k)
    dl = None
    packed = False
    if nn > 1:
        dl = np.minimum(rng.integers(0, nn + 1, size=B), seq).astype(np.int32)
        packed = bool(rng.random() < 0.5)
    pages = -(-seq // 64)
    width = int(pages.max()) + int(rng.integers(0, 4))
    slack = float(rng.choice([0.0, 0.1, 0.5]))
    name = f"rand{i}-{fmt}-D{D}-H{H}-n{nn}-{'packed' if packed else 'grid'}-k{k}-B{B}"
    wl = build_decode(seed=9200 + i, seq_lens=seq, heads=H, head_dim=D, topk=k, fmt=fmt, next_n=nn,
                      decode_lens=dl, q_packed=packed, pool_slack=slack, width=width, w_std=1.0 / 8,
                      name=name)
    return wl


@pytest.mark.parametrize("i", range(16))
def test_random_decode_batch(i):
    wl = _case(i)
    print(f"case {wl.name}: seq_lens {wl.seq_lens.tolist()} decode_lens "
          f"{None if wl.decode_lens is None else wl.decode_lens.tolist()}", flush=True)
    dev = Dev(wl)
    ref = oracle.pipeline.decode_logits(wl)
    L, _ = oracle.pipeline.decode_row_info(wl)
    got, ws = dev.logits_decode()
    check_logits(got, {r: v for r, v in ref.items() if len(v)}, label=wl.name)
    for r in np.nonzero(L == 0)[0]:
        assert np.isnan(got[r]).all(), f"{wl.name}: padded row {r} was written"
    assert idx.idx_read_device_status(ws) == 0
    out, ws2 = dev.decode_topk()
    assert idx.idx_read_device_status(ws2) == 0
    check_topk_e2e(out, ref, L, wl.topk, label=wl.name)
