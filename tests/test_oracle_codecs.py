"""Pins of the oracle's scalar codecs against things other than itself.

E2M1: the value set printed on the pages, and a brute-force nearest-value
search.  E4M3: torch's float8_e4m3fn cast (a library routine).  E8M0 exponent:
an exact integer search and torch's float8_e8m0fnu cast.  bf16 storage:
torch's bfloat16 cast.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import read_golden

pytestmark = pytest.mark.filterwarnings("ignore")


def all_bf16_finite():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_e2m1_value_set_matches_page():
    expect = [float(v) for v in read_golden("e2m1_value_set.txt")["values"].split()]
    got = [oracle.e2m1_value(c) for c in range(8)]
    assert got == expect
    assert [oracle.e2m1_value(8 + c) for c in range(8)] == [-v for v in expect]


def _e2m1_nearest_even(v):
    """Brute force: nearest of the 8 magnitudes; ties to the even code; >= 6 saturates."""
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - mags[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates prefer an even code
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a >= 6, 7, pick)
    sign = np.signbit(v).astype(np.uint8) * 8
    return (pick.astype(np.uint8) | sign)


def test_e2m1_encode_brute_force_dense():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        all_bf16_finite(),
        rng.uniform(-8, 8, 200000).astype(np.float32),
        # every midpoint of the value set and its float32 neighbours
        np.array([m for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
                  for m in (mid, np.nextafter(np.float32(mid), np.float32(0)),
                            np.nextafter(np.float32(mid), np.float32(9)))], np.float32),
    ]).astype(np.float32)
    v = np.concatenate([v, -v])
    got = oracle.e2m1_encode_array(v)
    np.testing.assert_array_equal(got, _e2m1_nearest_even(v))


def test_e2m1_worked_tie_225_goes_to_2():
    # the page's worked example: 2.25 rounds deterministically to 2
    assert oracle.e2m1_value(oracle.e2m1_encode(2.25)) == 2.0


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes], np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def _torch_e4m3_sat(v):
    t = torch.from_numpy(np.clip(v, -448, 448).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_all_bf16_and_dense():
    rng = np.random.default_rng(2)
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float32)
    mids = ((grid[1:].astype(np.float64) + grid[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    v = np.concatenate([
        all_bf16_finite(),
        near,
        np.exp2(rng.uniform(-14, 10, 300000)).astype(np.float32),
        np.array([448, 448.0001, 460, 464, 464.5, 1e30, 3e38], np.float32),
    ]).astype(np.float32)
    v = np.concatenate([v, -v])
    got = oracle.e4m3_encode_array(v)
    np.testing.assert_array_equal(got, _torch_e4m3_sat(v))


def _smallest_k_exact(a: float) -> int:
    """Smallest integer k with a <= 448 * 2**k, by exact rational comparison."""
    fa = Fraction(a)
    k = -200
    while fa > Fraction(448) * (Fraction(2) ** k):
        k += 1
    return max(-127, min(119, k))


def test_e8m0_exponent_brute_force_all_bf16():
    f = all_bf16_finite()
    f = np.unique(np.abs(f))
    got = oracle.mxfp8_block_exponent_array(f.astype(np.float32))
    # exact search on a subsample spread over the whole range plus all boundaries
    idx = np.unique(np.concatenate([np.arange(0, f.size, 7), np.arange(f.size - 50, f.size)]))
    for i in idx:
        assert got[i] == _smallest_k_exact(float(f[i])), float(f[i])
    # boundary family: 448 * 2^j and its bf16 neighbours
    for j in range(-100, 110):
        a = np.float32(448.0 * 2.0 ** j)
        up = np.nextafter(a, np.float32(np.inf))
        assert oracle.mxfp8_block_exponent(float(a)) == max(-127, min(119, j))
        assert oracle.mxfp8_block_exponent(float(up)) == max(-127, min(119, j + 1))


def test_e8m0_exponent_matches_torch_cast_where_rounding_agrees():
    # torch's e8m0 cast rounds a/448 to the nearest power of two (half up).  It
    # agrees with "smallest k with a <= 448 * 2^k" (a ceiling) exactly when the
    # significand of a/448 is 1 or lies in [1.5, 2); check those values.
    f = all_bf16_finite()
    f = f[(f > 0) & (f > 448 * 2.0 ** -120) & (f <= 448 * 2.0 ** 119)]
    r = (f / np.float32(448)).astype(np.float32)
    sig, _ = np.frexp(r.astype(np.float64))
    f = f[(sig == 0.5) | (sig >= 0.75)]
    ratio = torch.from_numpy((f / np.float32(448)).astype(np.float32))
    code = ratio.to(torch.float8_e8m0fnu).view(torch.uint8).numpy().astype(np.int32)
    got = oracle.mxfp8_block_exponent_array(f)
    np.testing.assert_array_equal(got, code - 127)


def test_e8m0_value():
    for c in (0, 1, 100, 127, 200, 254):
        assert oracle.e8m0_value(c) == 2.0 ** (c - 127)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10) ** rng.uniform(-30, 30, 200000).astype(np.float32),
        # exact halfway cases between bf16 neighbours
        ((np.arange(1, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
    ]).astype(np.float32)
    v = v[np.isfinite(v)]
    got = oracle.f32_to_bf16_array(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
