"""Pins for the oracle's number-format decoders (CPU only)."""

import math

import numpy as np
import torch

from oracle import formats


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2            # S.1111.111 only
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_closed_form_landmarks():
    v = formats.e4m3(np.array([0x00, 0x01, 0x08, 0x38, 0x40, 0x7E, 0xFE, 0x80], dtype=np.uint8))
    assert list(v[:7]) == [0.0, 2.0 ** -9, 2.0 ** -6, 1.0, 2.0, 448.0, -448.0]
    assert v[7] == 0.0 and math.copysign(1.0, v[7]) == -1.0


def test_e2m1_table():
    # OCP MX v1.0 FP4 (E2M1) value table
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    v = formats.e2m1(np.arange(16, dtype=np.uint8))
    assert list(v[:8]) == table
    assert list(-v[8:]) == table


def test_ue8m0():
    e = np.arange(255, dtype=np.uint8)
    v = formats.ue8m0(e)
    for i in (0, 1, 126, 127, 128, 200, 254):
        assert v[i] == math.ldexp(1.0, i - 127)
    assert np.isnan(formats.ue8m0(np.array([255], dtype=np.uint8)))[0]


def test_bf16_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ours = formats.bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f32le():
    x = np.array([1.5, -0.25, 3.0e-5, 448.0], dtype="<f4")
    b = x.view(np.uint8).reshape(4, 4)
    assert list(formats.f32le(b)) == [float(v) for v in x]
