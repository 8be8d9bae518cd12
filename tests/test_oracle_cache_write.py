"""Pins for the oracle's index-cache write (quantisers and slot scatter), CPU only."""

import math

import numpy as np
import torch

from oracle import cache as ocache
from oracle import cache_write as cw
from oracle import formats
from workloads.gen import encode_fp8_rows


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3_probe_values():
    """Every midpoint between adjacent non-negative e4m3 values, the fp32
    neighbours of each midpoint, the code values themselves, with both signs."""
    v = formats.e4m3(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)   # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    pos = np.concatenate([v, mids, up, dn, np.float32([1e-30, 2.0 ** -10, 447.99997])])
    pos = pos[pos <= 448]
    return np.concatenate([pos, -pos]).astype(np.float32)


def test_e4m3_encoder_matches_torch_cast_at_every_tie():
    x = _e4m3_probe_values()
    ours = cw.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encoder_random_values_match_torch():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-12, 9, 200_000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = cw.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e2m1_encoder_tie_table():
    # OCP FP4 values 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); a magnitude
    # halfway between two values goes to the even code (mantissa bit 0).
    table = {0.0: 0, 0.2: 0, 0.25: 0, 0.3: 1, 0.5: 1, 0.75: 2, 1.0: 2, 1.25: 2, 1.3: 3, 1.5: 3,
             1.75: 4, 2.0: 4, 2.5: 4, 2.6: 5, 3.0: 5, 3.5: 6, 4.0: 6, 5.0: 6, 5.01: 7, 6.0: 7}
    for x, code in table.items():
        assert cw.e2m1_encode(np.array([x]))[0] == code, x
        assert cw.e2m1_encode(np.array([-x]))[0] == code | 0x8, -x
    # every value decodes back to itself
    v = formats.e2m1(np.arange(16, dtype=np.uint8))
    assert np.array_equal(formats.e2m1(cw.e2m1_encode(v)), v)


def test_fp8_row_closed_forms():
    D = 128
    k = np.zeros((3, D), dtype=np.float32)
    k[1, 5] = -3.0
    k[1, 7] = 1.5
    k[2, :] = 2.0
    rows = cw.fp8_rows(_bf16_bits(k))
    # all-zero row: scale 1, codes 0
    assert formats.f32le(rows[0:1, D:])[0] == 1.0 and not rows[0, :D].any()
    # the absmax element maps to -448 exactly; scale = 3/448 in fp32
    assert rows[1, 5] == 0xFE
    assert formats.f32le(rows[1:2, D:])[0] == float(np.float32(3.0) / np.float32(448.0))
    x = np.float32(1.5) / (np.float32(3.0) / np.float32(448.0))
    assert rows[1, 7] == cw.e4m3_encode(np.array([float(x)]))[0]
    # a constant row: every code is 448
    assert (rows[2, :D] == 0x7E).all()


def test_fp8_rows_match_generator_encoding():
    """The workload generator encodes with torch's float8 cast (an
    independent implementation of the same reading)."""
    rng = np.random.default_rng(3)
    for D in (32, 64, 128):
        k = rng.standard_normal((500, D)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (500, 1)))
        bits = _bf16_bits(k)
        kq = formats.bf16(bits).astype(np.float32)
        assert np.array_equal(cw.fp8_rows(bits), encode_fp8_rows(kq))


def test_fp8_rows_error_bound():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2000, 128)).astype(np.float32)
    bits = _bf16_bits(k)
    exact = formats.bf16(bits)
    back = ocache.dequantize(cw.fp8_rows(bits), fmt="fp8", head_dim=128)
    scale = np.abs(exact).max(axis=1, keepdims=True) / 448
    # half an e4m3 ulp: 2^-4 relative for normal codes, 2^-10 * scale below 2^-6 * scale
    bound = np.maximum(np.abs(exact) * 2.0 ** -4, scale * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(back - exact) <= bound).all()


def test_mx_block_exponent_closed_forms():
    a = np.array([0.0, 1.0, 4.0, 7.99, 8.0, 0.3, 2.0 ** -126, 2.0 ** -140, 3.0e38])
    e = cw.mx_block_exponent(a)
    assert list(e) == [-127, -2, 0, 0, 1, -4, -127, -127, 125]


def test_mxfp4_rows_closed_forms_and_error_bound():
    D = 128
    k = np.zeros((2, D), dtype=np.float32)
    k[1, 0] = 1.0       # block 0: amax 1 -> e = -2, x = 4 -> code 6 (value 4)
    k[1, 1] = -0.25     # x = -1 -> code 0xA
    k[1, 40] = 7.0      # block 1: amax 7 -> e = 0, 7 saturates to 6 -> code 7
    k[1, 41] = 2.5      # tie between 2 and 3 -> 2 (code 4)
    rows = cw.mxfp4_rows(_bf16_bits(k))
    assert not rows[0, : D // 2].any() and (rows[0, D // 2 :] == 0).all()
    assert rows[1, 0] == (6 | (0xA << 4))
    assert rows[1, 20] == (7 | (4 << 4))
    assert list(rows[1, D // 2 :]) == [125, 127, 0, 0]

    rng = np.random.default_rng(6)
    k = rng.standard_normal((1000, D)).astype(np.float32)
    bits = _bf16_bits(k)
    exact = formats.bf16(bits)
    back = ocache.dequantize(cw.mxfp4_rows(bits), fmt="mxfp4", head_dim=D)
    blocks = np.abs(exact).reshape(1000, 4, 32)
    step = np.exp2(cw.mx_block_exponent(blocks.max(axis=2)).astype(np.float64))   # 2^e
    err = np.abs(back - exact).reshape(1000, 4, 32)
    # |x| <= 6: half the e2m1 spacing (at most 1 at magnitudes 4..6); above 6: saturation
    x = blocks / step[:, :, None]
    bound = np.where(x <= 6, np.where(x < 2, 0.25, np.where(x < 4, 0.5, 1.0)), x - 6) * step[:, :, None]
    assert (err <= bound * (1 + 1e-12)).all()


def test_write_scatter_readback_and_skips():
    D, ps = 64, 64
    rb = D + 4
    page_bytes = ps * rb + 16
    num_pages = 5
    cache = np.full(num_pages * page_bytes, 0xA5, dtype=np.uint8)
    rng = np.random.default_rng(8)
    k = rng.standard_normal((7, D)).astype(np.float32)
    bits = _bf16_bits(k)
    slots = np.array([3 * ps + 10, -1, 0, 4 * ps + 63, 2 * ps, 5 * ps, 1 * ps + 1], dtype=np.int64)
    flat, bad = cw.write(cache, bits, slots, fmt="fp8", page_size=ps, page_bytes=page_bytes)
    assert bad                        # slot 5*64 is past the 5-page pool
    rows = cw.fp8_rows(bits)
    # read back through the oracle's cache reader: request 0 owns pages 3, 0, 4, 2, 1
    bt = np.array([[3, 0, 4, 2, 1]], dtype=np.int32)
    L = 5 * ps
    got = ocache.key_rows(flat, bt, 0, L, fmt="fp8", head_dim=D, page_size=ps, page_bytes=page_bytes)
    pos_of_slot = {3 * ps + 10: 0 * ps + 10, 0: 1 * ps + 0, 4 * ps + 63: 2 * ps + 63, 2 * ps: 3 * ps,
                   1 * ps + 1: 4 * ps + 1}
    written = set()
    for t, s in enumerate(slots):
        if s in pos_of_slot:
            assert np.array_equal(got[pos_of_slot[s]], rows[t])
            written.add(pos_of_slot[s])
    # every other byte is untouched
    mask = np.ones(flat.size, dtype=bool)
    for s in pos_of_slot:
        start = (s // ps) * page_bytes + (s % ps) * rb
        mask[start : start + rb] = False
    assert (flat[mask] == 0xA5).all()
    assert math.isclose(len(written), 5)
