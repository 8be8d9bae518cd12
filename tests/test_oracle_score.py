"""Pins for the oracle's cache addressing, dequantisation and score (CPU only)."""

from fractions import Fraction

import numpy as np
import torch

from oracle import cache, score
from tests.conftest import load_golden
from workloads import build_decode
from workloads.gen import _bf16_bits


class _WL:
    """A minimal workload-like holder for hand-built caches."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def _one_page_wl(fmt, head_dim, rows_bytes):
    rb = rows_bytes.shape[1]
    cache_arr = np.full((1, 64 * rb), 0xFF, dtype=np.uint8)
    cache_arr[0, : rows_bytes.size] = rows_bytes.reshape(-1)
    return _WL(cache=cache_arr, block_table=np.zeros((1, 1), dtype=np.int32), fmt=fmt,
               head_dim=head_dim, page_size=64, page_bytes=64 * rb)


def _bits(vals):
    return _bf16_bits(np.asarray(vals, dtype=np.float32))


def test_e1_fp8_hand_example():
    g = load_golden("e1_fp8_two_heads.json")
    D, H = g["head_dim"], g["heads"]
    rows = np.zeros((4, D + 4), dtype=np.uint8)
    for t, (c0, c1) in enumerate(g["key_codes"]):
        rows[t, 0], rows[t, 1] = c0, c1
        rows[t, D:] = np.array([g["key_scales"][t]], dtype="<f4").view(np.uint8)
    wl = _one_page_wl("fp8", D, rows)
    k = cache.keys(wl, 0, 4)
    q = np.zeros((H, D), dtype=np.float32)
    q[:, :2] = g["q_rows"]
    got = score.logits(_bits(q), np.array(g["w"], dtype=np.float32), k)
    assert got.tolist() == g["logits"]


def test_e3_mxfp4_nibble_order():
    g = load_golden("e3_mxfp4_nibbles.json")
    D, H = g["head_dim"], g["heads"]
    row = np.zeros((1, D // 2 + D // 32), dtype=np.uint8)
    row[0, 0] = g["packed_byte0"]
    row[0, D // 2] = g["scale_byte"]
    wl = _one_page_wl("mxfp4", D, row)
    k = cache.keys(wl, 0, 1)
    assert k[0, :2].tolist() == g["dequantized_prefix"]
    assert not k[0, 2:].any()
    q = np.zeros((H, D), dtype=np.float32)
    q[:, :2] = g["q_rows"]
    got = score.logits(_bits(q), np.array(g["w"], dtype=np.float32), k)
    assert got.tolist() == [g["logit"]]


def _fraction_logits(q_bits, w, codes_f, scales_f, L, H, D):
    """Exact rational evaluation of sum_h w_h relu(q_h . k_t): every input is
    converted to a Fraction from an independent decoder (torch casts)."""
    qf = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    out = []
    for t in range(L):
        acc = Fraction(0)
        for h in range(H):
            dot = Fraction(0)
            for d in range(D):
                dot += Fraction(float(qf[h, d])) * Fraction(float(codes_f[t, d])) * scales_f(t, d)
            if dot > 0:
                acc += Fraction(float(w[h])) * dot
        out.append(acc)
    return out


def test_fp8_score_exact_fraction_bruteforce():
    H, D, L = 3, 32, 70          # two pages
    wl = build_decode(seed=21, seq_lens=[L], heads=H, head_dim=D, topk=8, fmt="fp8")
    rows = cache.key_rows(wl.cache, wl.block_table, 0, L, fmt="fp8", head_dim=D,
                          page_size=64, page_bytes=wl.page_bytes)
    codes = torch.from_numpy(np.ascontiguousarray(rows[:, :D])).view(torch.float8_e4m3fn).double().numpy()
    sc = np.ascontiguousarray(rows[:, D:]).view("<f4")[:, 0]
    q = wl.q[0]
    w = wl.w[0]
    exact = _fraction_logits(q, w, codes, lambda t, d: Fraction(float(sc[t])), L, H, D)
    got = score.logits(q, w, cache.keys(wl, 0, L))
    for t in range(L):
        # float64 evaluation is within a few ulps of the exact value
        assert abs(Fraction(float(got[t])) - exact[t]) <= abs(exact[t]) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 80)


def test_mxfp4_score_exact_fraction_bruteforce():
    H, D, L = 2, 64, 40
    wl = build_decode(seed=22, seq_lens=[L], heads=H, head_dim=D, topk=8, fmt="mxfp4")
    rows = cache.key_rows(wl.cache, wl.block_table, 0, L, fmt="mxfp4", head_dim=D,
                          page_size=64, page_bytes=wl.page_bytes)
    packed = rows[:, : D // 2]
    nib = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(L, D)
    # independent e2m1 decode straight from the OCP MX value table
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = np.vectorize(lambda n: (-1.0 if n & 8 else 1.0) * table[n & 7])(nib)
    sb = rows[:, D // 2 :].astype(np.int64)
    exact = _fraction_logits(wl.q[0], wl.w[0], codes,
                             lambda t, d: Fraction(2) ** int(sb[t, d // 32] - 127), L, H, D)
    got = score.logits(wl.q[0], wl.w[0], cache.keys(wl, 0, L))
    for t in range(L):
        assert abs(Fraction(float(got[t])) - exact[t]) <= abs(exact[t]) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 80)


def test_single_head_positive_reduces_to_matvec():
    rng = np.random.default_rng(2)
    D, L = 128, 200
    k = np.abs(rng.standard_normal((L, D))) + 0.01
    q = np.abs(rng.standard_normal((1, D))).astype(np.float32)
    qb = _bits(q)
    qf = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = score.logits(qb, np.ones(1, dtype=np.float32), k)
    assert np.allclose(got, np.matmul(k, qf[0]), rtol=1e-14, atol=0)


def test_cache_read_back_matches_generated_keys():
    """Addressing pin: the keys the generator drew (re-drawn from the same
    seed and draw order) come back through block table + dequantisation
    within the quantisation error of each format."""
    for fmt, D in (("fp8", 64), ("mxfp4", 128)):
        seq = [130, 64, 1]
        wl = build_decode(seed=31, seq_lens=seq, heads=2, head_dim=D, topk=4, fmt=fmt)
        rng = np.random.Generator(np.random.PCG64(31))
        rng.permutation(wl.num_pages)            # same draw order: pages first
        for b, L in enumerate(seq):
            orig = rng.standard_normal((L, D), dtype=np.float32).astype(np.float64)
            got = cache.keys(wl, b, L)
            if fmt == "fp8":
                amax = np.abs(orig).max(axis=1, keepdims=True)
                # e4m3: relative step 2^-3 above 2^-6 of the scale range, absolute below
                bound = np.maximum(np.abs(orig) * 2.0 ** -4, amax / 448.0 * 2.0 ** -9) * 1.0001
            else:
                blocks = np.abs(orig).reshape(L, D // 32, 32).max(axis=2)
                e = np.floor(np.log2(blocks)) - 2
                step = np.repeat(np.exp2(e), 32, axis=1)     # half the largest e2m1 gap is 1 * 2^e
                bound = step * 1.0001 + np.maximum(np.abs(orig) - 6 * step, 0)
            assert np.all(np.abs(got - orig) <= bound), (fmt, b)


def test_page256_cache_reads_same_keys_as_page64():
    """Keys are drawn in token order whatever the page size, so a workload
    stored in 256-token pages and one in 64-token pages (same seed) hold the
    same keys; the oracle's block-table reader must return them equally."""
    from oracle import cache
    from workloads import build_decode
    kw = dict(seed=31, seq_lens=[1, 255, 256, 257, 700], heads=4, head_dim=64, topk=16)
    # explicit tables (request r owns a run of pages, in reverse order) so that
    # both draw their keys from the same generator state
    bt64 = np.array([[r * 11 + 10 - i for i in range(11)] for r in range(5)], dtype=np.int32)
    bt256 = np.array([[r * 3 + 2 - i for i in range(3)] for r in range(5)], dtype=np.int32)
    a = build_decode(**kw, block_table=bt64, num_pages=55)
    b = build_decode(**kw, block_table=bt256, num_pages=15, page_size=256)
    assert b.page_bytes == 256 * 68 and b.block_table.shape[1] == 3
    for r, L in enumerate(kw["seq_lens"]):
        assert np.array_equal(cache.keys(a, r, L), cache.keys(b, r, L))
