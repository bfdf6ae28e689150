"""Pins for oracle.formats against the OCP specs and torch's dtype casts."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


def test_e4m3_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_golden_points():
    for code, val in _table("e4m3_points.txt"):
        got = F.e4m3_to_f64(np.uint8(code))
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_encode_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.e4m3_to_f64(codes)
    assert np.array_equal(F.f64_to_e4m3_bits(vals), codes)
    # midpoints between consecutive positive codes go to the even mantissa
    pos = F.e4m3_to_f64(np.arange(0, 127, dtype=np.uint8))
    mids = 0.5 * (pos[:-1] + pos[1:])
    got = F.f64_to_e4m3_bits(mids)
    lower = np.arange(0, 126)
    want = np.where(lower % 2 == 0, lower, lower + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    # saturation instead of NaN
    assert F.f64_to_e4m3_bits(np.array([1e6, -1e6, 460.0, 480.0])).tolist() == [0x7E, 0xFE, 0x7E, 0x7E]


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    x = x[np.abs(x) < 440]
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.f64_to_e4m3_bits(x32.astype(np.float64)), ref)


def test_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(F.bf16_to_f64(ref), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_e2m1_table():
    for code, val in _table("e2m1_table.txt"):
        got = F.e2m1_to_f64(code)
        assert got == val and np.signbit(got) == np.signbit(val)


def test_e2m1_rounding_ties_even_and_saturation():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.25, -5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -0.0, -4.0])
    assert np.array_equal(F.round_e2m1(x), want)


def test_mxfp4_scale_rule_and_roundtrip():
    rng = np.random.default_rng(11)
    # values already on the grid of one block scale come back exactly
    for shared in (-3, 0, 2):
        codes = rng.integers(0, 16, size=(5, 64))
        v = F.e2m1_to_f64(codes) * 2.0 ** shared
        v[:, 0] = 6.0 * 2.0 ** shared      # pins amax so floor(log2 amax) - 2 == shared
        v[:, 32] = -4.0 * 2.0 ** shared
        rows = F.mxfp4_encode(v)
        assert rows.shape == (5, 32 + 2)
        assert np.all(rows[:, 32:] == 127 + shared)
        assert np.array_equal(F.mxfp4_decode(rows, 64), v)
    # zero block
    rows = F.mxfp4_encode(np.zeros((1, 32)))
    assert rows.tolist() == [[0] * 17]
    # error bound: |x - q(x)| <= half the top spacing (1.0 * scale) and amax maps into [4, 8) * scale
    x = rng.standard_normal((200, 128))
    dq = F.mxfp4_decode(F.mxfp4_encode(x), 128)
    blk = np.abs(x).reshape(200, 4, 32).max(-1)
    scale = 2.0 ** (np.floor(np.log2(blk)) - 2)
    err = np.abs(x - dq).reshape(200, 4, 32).max(-1)
    assert np.all(err <= scale * 2.0 + 1e-12)     # saturation of [6, 8) costs at most 2 * scale
    inside = np.abs(x).reshape(200, 4, 32) <= 6 * scale[..., None]
    e_in = np.where(inside, np.abs(x - dq).reshape(200, 4, 32), 0).max(-1)
    assert np.all(e_in <= scale * 1.0 + 1e-12)


def test_split_row_layout():
    D, R = 512, 64
    assert F.split_row_bytes(D, R) == 576
    with open(os.path.join(GOLD, "pages_constants.json")) as f:
        assert json.load(f)["split_entry_bytes"]["value"] == F.split_row_bytes(D, R)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, D))
    rows = F.split_encode(x, R)
    assert rows.shape == (3, 576)
    dec = F.split_decode(rows, D, R)
    assert np.array_equal(dec[:, : D - R], F.round_e4m3(x[:, : D - R]))
    assert np.array_equal(dec[:, D - R:], F.round_bf16(x[:, D - R:]))
    # the BF16 part is little-endian uint16 right after the FP8 bytes
    b = rows[0, D - R: D - R + 2].astype(np.uint16)
    assert F.bf16_to_f64(b[0] | (b[1] << 8)) == dec[0, D - R]
