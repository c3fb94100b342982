"""Pins for the oracle's number formats (CPU only).

Each check compares the oracle with something other than itself: the OCP
E4M3 code points, torch's independent CPU casts (fp32 -> bf16, fp32 ->
float8_e4m3fn, float8_e4m3fn -> fp32), exact rational arithmetic, and
hand-derived rounding cases.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.txt")


def _golden_points():
    pts = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        c, v = line.split()
        pts.append((int(c, 16), float(v)))
    return pts


# ------------------------------------------------------------------ e4m3
def test_e4m3_decode_matches_ocp_points():
    for code, val in _golden_points():
        got = F.e4m3_decode(np.uint8(code))
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def test_e4m3_roundtrip_every_code():
    c = np.arange(256, dtype=np.uint8)
    v = F.e4m3_decode(c)
    ok = ~np.isnan(v)
    assert (F.e4m3_encode(v[ok]) == c[ok]).all()
    assert F.e4m3_encode(np.nan) == 0x7F
    assert F.e4m3_encode(-np.nan) == 0xFF


def test_e4m3_midpoints_round_to_even():
    # every midpoint between consecutive positive finite codes goes to the
    # code with an even mantissa (the even one of the two neighbours)
    v = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = (v[c] + v[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode(mid) == want, (c, mid)
        assert F.e4m3_encode(-mid) == want | 0x80
        # just off the midpoint goes to the nearer neighbour
        eps = (v[c + 1] - v[c]) * 2.0 ** -20
        assert F.e4m3_encode(mid - eps) == c
        assert F.e4m3_encode(mid + eps) == c + 1


def test_e4m3_saturation_and_specials():
    assert F.e4m3_encode(448.0) == 0x7E
    assert F.e4m3_encode(460.0) == 0x7E
    assert F.e4m3_encode(464.0) == 0x7E
    assert F.e4m3_encode(1e30) == 0x7E
    assert F.e4m3_encode(np.inf) == 0x7E
    assert F.e4m3_encode(-np.inf) == 0xFE
    assert F.e4m3_encode(2.0 ** -10) == 0x00          # tie between 0 and 2^-9 -> even (0)
    assert F.e4m3_encode(1.5 * 2.0 ** -10) == 0x01
    assert F.e4m3_encode(3 * 2.0 ** -10) == 0x02       # tie between 1 and 2 -> 2
    assert F.e4m3_encode(-0.0) == 0x80
    assert F.e4m3_encode(-1e-30) == 0x80
    assert F.e4m3_encode(15.5 * 2.0 ** -10) == 0x08    # top subnormal tie -> min normal


def test_e4m3_encode_matches_torch_in_range():
    # torch's fp32 -> float8_e4m3fn cast is RNE but does not saturate above
    # 464, so the comparison is restricted to |v| <= 448.
    g = np.random.default_rng(123)
    bf = np.arange(65536, dtype=np.uint32)
    vals = [(bf << 16).view(np.float32)]
    for s in (1.0, 2.0 ** 5, 448.0 / 13.7, 0.37, 2.0 ** -7):
        vals.append((vals[0].astype(np.float64) * s).astype(np.float32))
    vals.append((g.standard_normal(400000) * 50).astype(np.float32))
    vals.append((g.standard_normal(400000) * 1e-3).astype(np.float32))
    v = np.concatenate(vals)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(v.astype(np.float64))
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, (v[bad[:5]], ref[bad[:5]], got[bad[:5]])


# ------------------------------------------------------------------ bf16
def test_bf16_round_matches_torch_fp32_patterns():
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x = bits.view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.bf16_round(x.astype(np.float64))
    nan = np.isnan(x)
    assert (got[~nan] == ref[~nan]).all()
    assert (F.bf16_to_f64(got[nan]) != F.bf16_to_f64(got[nan])).all()


def test_bf16_round_from_f64_is_single_rounding():
    # just above a tie in bf16 but a tie in fp32: via fp32 it would go to
    # even (1.0); rounded once from fp64 it goes up.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16(x) == 1.0 + 2.0 ** -7
    assert F.bf16(1.0 + 2.0 ** -8) == 1.0                    # exact tie -> even
    assert F.bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # tie -> even (up)
    assert F.bf16(2.0 ** -134) == 0.0                        # half min-subnormal tie -> 0
    assert F.bf16(1.5 * 2.0 ** -133) == 2.0 ** -132
    assert np.isinf(F.bf16(3.5e38))
    assert F.bf16(-3.0) == -3.0


def test_bf16_decode_exact():
    assert F.bf16_to_f64(np.uint16(0x3F80)) == 1.0
    assert F.bf16_to_f64(np.uint16(0xC040)) == -3.0
    assert F.bf16_to_f64(np.uint16(0x0001)) == 2.0 ** -133


# ------------------------------------------------------------------ fp32
def test_fl32_is_correctly_rounded():
    g = np.random.default_rng(5)
    for x in g.standard_normal(200) * 10.0 ** g.integers(-20, 20, 200):
        r = F.fl32(x)
        q = Fraction(float(x))
        lo = np.nextafter(np.float32(r), np.float32(-np.inf))
        hi = np.nextafter(np.float32(r), np.float32(np.inf))
        err = abs(Fraction(float(r)) - q)
        assert err <= abs(Fraction(float(lo)) - q)
        assert err <= abs(Fraction(float(hi)) - q)
