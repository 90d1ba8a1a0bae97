"""Pins of the oracle's number formats (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _hexfloat(s):
    if s in ("inf", "-inf", "nan"):
        return float(s)
    return float.fromhex(s)


def test_bf16_golden_cases():
    rows = _read("bf16_rounding.txt")
    assert len(rows) >= 10
    x = np.array([_hexfloat(a) for a, _ in rows])
    want = np.array([_hexfloat(b) for _, b in rows])
    got = codecs.bf16_round(x)
    np.testing.assert_array_equal(got, want)


def test_bf16_matches_torch_cast_random_and_edges():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(50_000) * 1e37).astype(np.float32),    # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4e38, -3.4e38], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_encode(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    # decode is exact widening
    np.testing.assert_array_equal(codecs.bf16_decode(ref),
                                  torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_bf16_nan():
    assert np.isnan(codecs.bf16_decode(codecs.bf16_encode(np.array([np.nan])))[0])


def test_e4m3_golden_codes():
    for code, val in _read("e4m3fn_codes.txt"):
        c = int(code, 16)
        v = float(val)
        got = codecs.e4m3_decode(np.array([c], np.uint8))[0]
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), (code, got, v)


def test_e4m3_exhaustive_roundtrip_and_torch_decode():
    codes = np.arange(256, dtype=np.uint8)
    vals = codecs.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    assert ok.sum() == 254                      # only S.1111.111 are NaN
    np.testing.assert_array_equal(codecs.e4m3_encode(vals[ok]), codes[ok])
    tv = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(tv), ~ok)
    np.testing.assert_array_equal(tv[ok], vals[ok])
    assert vals[ok].max() == 448.0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.uniform(-448, 448, 100_000),
        rng.standard_normal(100_000),
        rng.standard_normal(50_000) * 2.0 ** -8,                    # subnormals
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.e4m3_encode(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_e4m3_rne_ties_and_saturation():
    # 1 + 1/16 sits halfway between 1.0 (mantissa 0, even) and 1.125 -> 1.0
    assert codecs.e4m3_decode(codecs.e4m3_encode(np.array([1.0625])))[0] == 1.0
    # 1.1875 halfway between 1.125 (odd) and 1.25 (even) -> 1.25
    assert codecs.e4m3_decode(codecs.e4m3_encode(np.array([1.1875])))[0] == 1.25
    # 1.5 * 2^-9 halfway between subnormal codes 1 and 2 -> 2 (even)
    assert codecs.e4m3_encode(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    # saturating encoder: beyond 448 clamps (torch's cast would give NaN here)
    assert codecs.e4m3_encode(np.array([1000.0, -600.0])).tolist() == [0x7E, 0xFE]
    assert codecs.e4m3_encode(np.array([np.nan]))[0] == 0x7F
