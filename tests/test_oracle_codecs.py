"""Pins for the oracle's number codecs (BF16, E4M3, E2M1).

Each codec is checked against something other than itself: torch's own
conversions (library routines), brute-force nearest-value search over the
format's finite values in exact rational arithmetic, and the hand tables in
tests/golden/.
"""
import bisect
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_table

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f32(x):
    return float(np.float32(x))


# ---------------------------------------------------------------- BF16 ----

def test_bf16_decode_all_patterns_vs_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = np.array([orc.bf16_decode(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # sign of zero
    assert np.signbit(orc.bf16_decode(0x8000)) and not np.signbit(orc.bf16_decode(0x0000))


def _torch_bf16_bits(vals_f32):
    t = torch.from_numpy(np.asarray(vals_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_encode_random_vs_torch(orc):
    rng = np.random.default_rng(7)
    mags = np.ldexp(rng.random(20000) + 0.5, rng.integers(-140, 127, 20000)).astype(np.float32)
    vals = np.where(rng.random(20000) < 0.5, -mags, mags).astype(np.float32)
    # exact f32 ties: bf16 pattern followed by 0x8000 in the low half
    tb = rng.integers(0, 0x7F7F, 3000).astype(np.uint32)
    ties = ((tb << 16) | 0x8000).view(np.float32)
    extra = np.array([0.0, -0.0, 1.0, 3.3895314e38, 1e-45, -1e-45, 1.1754942e-38], dtype=np.float32)
    allv = np.concatenate([vals, ties, -ties, extra]).astype(np.float32)
    want = _torch_bf16_bits(allv)
    got = np.array([orc.bf16_encode(float(v)) for v in allv], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(allv[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_bf16_encode_double_inputs_round_once(orc):
    """The oracle rounds the exact double once; a value a hair above a BF16 tie
    must round up even though its f32 rounding would be the tie itself."""
    rng = np.random.default_rng(11)
    for p in rng.integers(0x0080, 0x7F00, 500):
        lo = orc.bf16_decode(int(p))
        hi = orc.bf16_decode(int(p) + 1)
        ulp = hi - lo
        for t, expect in ((0.25, p), (0.75, p + 1), (0.5 + 2.0 ** -30, p + 1), (0.5 - 2.0 ** -30, p),
                          (0.5, p if p % 2 == 0 else p + 1)):
            v = lo + t * ulp  # exact in double: t has few significant bits
            assert Fraction(v) == Fraction(lo) + Fraction(t) * Fraction(ulp)
            assert orc.bf16_encode(v) == expect, (hex(p), t)
            assert orc.bf16_encode(-v) == (expect | 0x8000), (hex(p), t)


def test_bf16_encode_range_vs_torch(orc):
    """The range form (codec 2, used to sweep the device's BF16 converter)
    against torch's f32 -> BF16 cast (round to nearest even) on every f32
    pattern of several stretches: around 1, the subnormals, the overflow
    edge, both signs, and random starts; NaN patterns must come back NaN with
    the sign kept."""
    starts = [0x3F800000 - (1 << 19), 0x00000000, 0x7F7F0000, 0x80000000, 0xFF7F0000, 0x7F800000 - (1 << 16)]
    rng = np.random.default_rng(11)
    starts += [int(x) for x in rng.integers(0, (1 << 32) - (1 << 20), 8, dtype=np.uint64)]
    for first in starts:
        n = min(1 << 20, (1 << 32) - first)
        got = orc.encode_range(2, first, n)
        assert got.dtype == np.uint16
        u = (np.arange(n, dtype=np.uint64) + first).astype(np.uint32)
        f = u.view(np.float32)
        want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        assert np.array_equal(got[~nan], want[~nan]), hex(first)
        g = got[nan]
        assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x007F) != 0), hex(first)
        assert np.array_equal(g >> 15, (u[nan] >> 31).astype(np.uint16)), hex(first)


def test_bf16_encode_overflow_and_subnormal(orc):
    assert orc.bf16_encode(float("inf")) == 0x7F80
    assert orc.bf16_encode(3.5e38) == 0x7F80  # above max + half ulp -> inf
    assert orc.bf16_encode(2.0 ** -133) == 0x0001  # smallest subnormal
    assert orc.bf16_encode(2.0 ** -134) == 0x0000  # tie with zero -> even (0)
    assert orc.bf16_encode(3 * 2.0 ** -134) == 0x0002  # tie 1/2 -> even
    assert orc.bf16_encode(-2.0 ** -140) == 0x8000


# ---------------------------------------------------------------- E4M3 ----

def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def test_e4m3_decode_all_codes_vs_torch(orc):
    want = _torch_e4m3_values()
    got = np.array([orc.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(want)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def _e4m3_nearest(v, mags, codes_for_mag):
    """Brute force: nearest finite E4M3 magnitude in exact arithmetic, ties to the
    even code, saturating at 448, sign copied from the input."""
    sign = 0x80 if np.signbit(v) else 0
    a = Fraction(abs(float(v)))
    if a >= 448:
        return sign | 0x7E
    i = bisect.bisect_left(mags, a)
    cands = [j for j in (i - 1, i) if 0 <= j < len(mags)]
    best = min(cands, key=lambda j: (abs(mags[j] - a), codes_for_mag[j] & 1))
    return sign | codes_for_mag[best]


def _e4m3_table():
    vals = _torch_e4m3_values()
    pairs = sorted((Fraction(vals[c]), c) for c in range(0x7F))  # 0x00..0x7E, finite, >= 0
    return [p[0] for p in pairs], [p[1] for p in pairs]


def test_e4m3_encode_golden_table(orc):
    for val, code, *_ in read_table("e4m3_encode.txt"):
        v = float(eval(val))
        assert orc.e4m3_encode(v) == int(code, 16), val


def test_e4m3_encode_bruteforce(orc):
    mags, cm = _e4m3_table()
    rng = np.random.default_rng(3)
    vals = list(np.ldexp(rng.random(6000) + 0.5, rng.integers(-13, 10, 6000)).astype(np.float32))
    # every midpoint between neighbours, and one f32 ulp either side of it
    for a, b in zip(mags[:-1], mags[1:]):
        mid = np.float32(float((a + b) / 2))
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    vals += [np.float32(x) for x in (449.0, 463.99, 464.0, 479.0, 480.0, 1e6, 2.0 ** -12, 1e-30)]
    for v in vals:
        for s in (v, -v):
            assert orc.e4m3_encode(float(s)) == _e4m3_nearest(s, mags, cm), float(s)


def test_e4m3_encode_vs_torch_cast(orc):
    """torch's float8_e4m3fn cast rounds to nearest even but does not saturate:
    compare where no saturation is involved."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(50000) * np.ldexp(1.0, rng.integers(-12, 8, 50000))).astype(np.float32)
    v = v[np.abs(v) <= 448]
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_encode_nan_inf(orc):
    assert orc.e4m3_encode(float("nan")) & 0x7F == 0x7F
    assert orc.e4m3_encode(float("inf")) == 0x7E
    assert orc.e4m3_encode(float("-inf")) == 0xFE


# ---------------------------------------------------------------- E2M1 ----

def test_e2m1_decode_all_codes_golden(orc):
    rows = read_table("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = orc.e2m1_decode(int(code, 16))
        assert got == float(val) and np.signbit(got) == np.signbit(float(val)), code


def test_e2m1_encode_golden_table(orc):
    for val, code, *_ in read_table("e2m1_encode.txt"):
        assert orc.e2m1_encode(float(val)) == int(code, 16), val


def test_e2m1_encode_bruteforce(orc):
    table = [(Fraction(float(v)), int(c, 16)) for c, v in read_table("e2m1_values.txt")[:8]]
    mags = [t[0] for t in table]
    rng = np.random.default_rng(9)
    vals = list((rng.random(20000) * 8).astype(np.float32))
    for a, b in zip(mags[:-1], mags[1:]):
        mid = np.float32(float((a + b) / 2))
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(9))]
    for v in vals:
        a = Fraction(float(v))
        if a >= 6:
            want = 7
        else:
            want = min(range(8), key=lambda j: (abs(mags[j] - a), table[j][1] & 1))
        assert orc.e2m1_encode(float(v)) == want, float(v)
        assert orc.e2m1_encode(-float(v)) == (want | 8), float(v)
