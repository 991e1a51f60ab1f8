"""Pins for the oracle's FP8 and NVFP4 weight quantizers.

Checked against hand-worked examples (tests/golden/), special cases whose
answer follows from the recipe by hand, invariants (the absmax element encodes
to the largest code), error bounds, and a brute-force nearest-code search with
numpy's IEEE float32 division standing in for the scale arithmetic.
"""
import bisect
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_table

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    out = t.view(torch.int16).numpy().view(np.uint16)
    # the fixtures only use BF16-exact values
    assert np.array_equal(t.to(torch.float32).numpy(), np.asarray(vals, dtype=np.float32))
    return out


def bf16_vals(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(
        torch.float32).numpy().astype(np.float64)


E2M1 = {int(c, 16): float(v) for c, v in read_table("e2m1_values.txt")}


# ------------------------------------------------------------------ FP8 ----

def test_fp8_golden_row(orc):
    rows = read_table("fp8_row_example.txt")
    vals = [float(eval(r[0])) for r in rows]
    want = [int(r[1], 16) for r in rows]
    w = bf16_bits(vals).reshape(1, -1)
    codes, scale = orc.quantize_fp8(w)
    assert scale[0] == np.float32(1.0)
    assert list(codes[0]) == want


def test_fp8_zero_row_and_single_nonzero(orc):
    w = np.zeros((3, 32), dtype=np.uint16)
    w[1, 5] = bf16_bits([-3.0])[0]
    w[2, :] = 0x8000  # all -0
    codes, scale = orc.quantize_fp8(w)
    assert scale[0] == 1.0 and not codes[0].any()
    assert scale[1] == np.float32(3.0) / np.float32(448.0)
    assert codes[1, 5] == 0xFE and codes[1].sum() == 0xFE
    assert scale[2] == 1.0 and np.all(codes[2] == 0x80)


def test_fp8_subnormal_bf16_row(orc):
    """BF16 subnormals (exponent field 0): a flush-to-zero anywhere would zero
    the scale and the codes."""
    w = np.array([[0x0001, 0x0040, 0x807F, 0x0002] + [0] * 12], dtype=np.uint16)
    codes, scale = orc.quantize_fp8(w)
    a = float(bf16_vals([0x807F])[0])
    assert a != 0.0
    assert scale[0] == np.float32(abs(a)) / np.float32(448.0)
    assert codes[0, 2] == 0xFE  # the absmax element
    assert codes[0, 0] != 0 and codes[0, 1] != 0


def _nearest_e4m3(t):
    vals = e4m3_values()
    pairs = sorted((Fraction(vals[c]), c) for c in range(0x7F))
    mags = [p[0] for p in pairs]
    sign = 0x80 if np.signbit(t) else 0
    a = Fraction(abs(float(t)))
    if a >= 448:
        return sign | 0x7E
    i = bisect.bisect_left(mags, a)
    cands = [j for j in (i - 1, i) if 0 <= j < len(mags)]
    best = min(cands, key=lambda j: (abs(mags[j] - a), pairs[j][1] & 1))
    return sign | pairs[best][1]


def test_fp8_random_rows_invariants_and_bruteforce(orc):
    rng = np.random.default_rng(1)
    n, k = 24, 64
    f = (rng.standard_normal((n, k)) * np.ldexp(1.0, rng.integers(-20, 10, (n, 1)))).astype(np.float32)
    w = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wv = bf16_vals(w).reshape(n, k)
    codes, scale = orc.quantize_fp8(w)
    dec = e4m3_values()
    for r in range(n):
        a = np.float32(np.abs(wv[r]).max())
        s = np.float32(a / np.float32(448.0))  # IEEE float32 division (numpy)
        assert scale[r] == s
        j = int(np.abs(wv[r]).argmax())
        assert codes[r, j] & 0x7F == 0x7E
        for i in range(k):
            t = np.float32(wv[r, i] / s)
            assert codes[r, i] == _nearest_e4m3(t), (r, i)
            # error bound: half the E4M3 spacing at t, times s (f32 division adds < 1 f32 ulp)
            if wv[r, i] != 0:
                e = max(int(np.floor(np.log2(abs(float(t))))), -6)
                half = 2.0 ** (e - 3) / 2
                assert abs(dec[codes[r, i]] * float(s) - float(wv[r, i])) <= (half + abs(float(t)) * 2 ** -23) * float(s)


def test_fp8_threads_do_not_change_result(orc):
    rng = np.random.default_rng(2)
    w = torch.from_numpy(rng.standard_normal((300, 48)).astype(np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    c1, s1 = orc.quantize_fp8(w, threads=1)
    c8, s8 = orc.quantize_fp8(w, threads=7)
    assert np.array_equal(c1, c8) and np.array_equal(s1, s8)


# ---------------------------------------------------------------- NVFP4 ----

def _read_nvfp4_example():
    d = {}
    for row in read_table("nvfp4_example.txt"):
        d[row[0]] = row[1:]
    return d


def test_nvfp4_golden_example(orc):
    d = _read_nvfp4_example()
    w = bf16_bits([float(v) for v in d["row"]]).reshape(1, -1)
    codes, bscale, g = orc.quantize_nvfp4(w)
    assert g[0] == np.float32(d["global_scale"][0])
    assert [int(x, 16) for x in d["block_scales"]] == list(bscale[0])
    assert [int(x, 16) for x in d["packed"]] == list(codes[0])


def test_nvfp4_nibble_order_and_layout(orc):
    """Two rows, two blocks each: element 2j low nibble, 2j+1 high nibble; block
    scales row-major [n, k/16]."""
    d = _read_nvfp4_example()
    row = [float(v) for v in d["row"]]
    row2 = [x / 2 for x in row[16:]] + [x / 4 for x in row[:16]]
    w = bf16_bits(row + row2).reshape(2, 32)
    codes, bscale, g = orc.quantize_nvfp4(w)
    assert g[0] == np.float32(1.0)  # G is still 2688, in row 0
    want = [int(x, 16) for x in d["codes"]]
    for j in range(32):
        q = (codes[0, j // 2] >> (4 * (j & 1))) & 0xF
        assert q == want[j], j
    assert list(bscale[0]) == [0x7E, 0x40]
    # row 1 block 0 = block B / 2 (max 6 -> a/d = 1 -> 0x38); block 1 = block A / 4
    # (max 672 -> a/d = 112 = 1.75 * 2^6 -> exponent field 13, mantissa 6 -> 0x6E)
    assert list(bscale[1]) == [0x38, 0x6E]


def test_nvfp4_invariants_and_error_bound(orc):
    rng = np.random.default_rng(4)
    n, k = 16, 256
    f = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    m = rng.random((n, k)) < 0.01
    f[m] *= 20
    w = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wv = bf16_vals(w).reshape(n, k).astype(np.float64)
    codes, bscale, g = orc.quantize_nvfp4(w)
    G = np.abs(wv).max()
    assert orc.global_absmax(w) == np.float32(G)
    assert g[0] == np.float32(np.float32(G) / np.float32(2688.0))
    r0, c0 = np.unravel_index(np.abs(wv).argmax(), wv.shape)
    assert bscale[r0, c0 // 16] == 0x7E
    q0 = (codes[r0, c0 // 2] >> (4 * (c0 & 1))) & 0xF
    assert q0 == (0xF if wv[r0, c0] < 0 else 0x7)
    dec = e4m3_values()
    for r in range(n):
        for c in range(k):
            q = (codes[r, c // 2] >> (4 * (c & 1))) & 0xF
            S = float(np.float32(np.float32(dec[bscale[r, c // 16]]) * g[0]))
            what = E2M1[int(q)] * S
            t = abs(wv[r, c]) / S if S else 0.0
            # spacing of E2M1 at |t|: 0.5 below 2, 1 in [2, 4), 2 in [4, 6]
            sp = 0.5 if t < 2 else (1.0 if t < 4 else 2.0)
            if t <= 6:
                assert abs(what - wv[r, c]) <= (sp / 2) * S * (1 + 2 ** -20) + 1e-30, (r, c)


def test_nvfp4_zero_matrix(orc):
    w = np.zeros((2, 32), dtype=np.uint16)
    w[1, 3] = 0x8000
    codes, bscale, g = orc.quantize_nvfp4(w)
    assert g[0] == 1.0 and not bscale.any()
    assert codes[0].sum() == 0 and codes[1, 1] == 0x80  # -0 keeps its sign (element 3: high nibble)


# ------------------------------------------- NVFP4 at s_g != 1 (f32 steps) ----

def _read_sg_examples():
    ex = {}
    for row in read_table("nvfp4_example_sg.txt"):
        name, key = row[0].split(".", 1)
        ex.setdefault(name, {})[key] = row[1:]
    return ex


def _nibbles(codes_row, k):
    return [(int(codes_row[j // 2]) >> (4 * (j & 1))) & 0xF for j in range(k)]


@pytest.mark.parametrize("name", ["A", "B"])
def test_nvfp4_golden_example_nonunit_global_scale(orc, name):
    """Hand-worked examples with s_g = f32(13/14) and f32(11/12): block maxima
    whose a / d falls on or within an f32 ulp of an E4M3 tie, elements whose
    w / S does the same for E2M1 (the worked f32 steps are in the fixture)."""
    ex = _read_sg_examples()[name]
    rows = sorted(k for k in ex if k.startswith("row"))
    w = np.stack([bf16_bits([float(v) for v in ex[r]]) for r in rows])
    k = w.shape[1]
    codes, bscale, g = orc.quantize_nvfp4(w)
    assert g.view(np.uint32)[0] == int(ex["global_scale_bits"][0], 16)
    for i, r in enumerate(rows):
        idx = r[len("row"):]
        assert list(bscale[i]) == [int(x, 16) for x in ex["block_scales" + idx]], (name, r)
        assert _nibbles(codes[i], k) == [int(x, 16) for x in ex["codes" + idx]], (name, r)


E4M3_FINITE = sorted((Fraction(float(v)), c) for c, v in enumerate(e4m3_values()) if c < 0x7F)
E2M1_MAGS = sorted((Fraction(v), c) for c, v in E2M1.items() if c < 8)


def _nearest_code(table, t):
    """Nearest code of |t| in a sorted (value, code) table: ties to the even code,
    saturating at the largest value; the sign bit of t on top."""
    mags = [p[0] for p in table]
    sign_bit = 0x80 if table is E4M3_FINITE else 0x8
    sign = sign_bit if np.signbit(t) else 0
    a = Fraction(abs(float(t)))
    if a >= mags[-1]:
        return sign | table[-1][1]
    i = bisect.bisect_left(mags, a)
    cands = [j for j in (i - 1, i) if 0 <= j < len(mags)]
    best = min(cands, key=lambda j: (abs(mags[j] - a), table[j][1] & 1))
    return sign | table[best][1]


def _nvfp4_expected(wv):
    """Block scales and codes of the recipe, with numpy's IEEE f32 division and
    multiplication for the scale arithmetic and a nearest-code search in exact
    rationals for the encoders."""
    n, k = wv.shape
    G = np.float32(np.abs(wv).max())
    sg = np.float32(G / np.float32(2688.0)) if G != 0 else np.float32(1.0)
    d = np.float32(np.float32(6.0) * sg)
    bs = np.zeros((n, k // 16), dtype=np.uint8)
    q = np.zeros((n, k), dtype=np.uint8)
    for r in range(n):
        for b in range(k // 16):
            blk = wv[r, 16 * b:16 * b + 16]
            a = np.float32(np.abs(blk).max())
            sb = _nearest_code(E4M3_FINITE, np.float32(a / d))
            bs[r, b] = sb
            S = np.float32(np.float32(e4m3_values()[sb]) * sg)
            for i in range(16):
                wi = np.float32(blk[i])
                if S == 0:
                    q[r, 16 * b + i] = 0x8 if np.signbit(wi) else 0
                else:
                    q[r, 16 * b + i] = _nearest_code(E2M1_MAGS, np.float32(wi / S))
    return sg, bs, q


def test_nvfp4_bruteforce_block_scales_and_codes(orc):
    """Every block scale and code against a brute-force nearest search, on random
    heads with 1 % outliers x20 at several magnitudes and on the worked examples
    scaled by powers of two (the ties and near-ties scale with them)."""
    rng = np.random.default_rng(11)
    mats = []
    for s in (-12, -3, 0, 5):
        f = (rng.standard_normal((6, 256)) * 0.02 * 2.0 ** s).astype(np.float32)
        m = rng.random(f.shape) < 0.01
        f[m] *= 20
        mats.append(torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    ex = _read_sg_examples()
    for name in ("A", "B"):
        rows = sorted(k for k in ex[name] if k.startswith("row"))
        base = np.stack([np.asarray([float(v) for v in ex[name][r]]) for r in rows])
        for e in (-20, -7, 0, 9):
            mats.append(bf16_bits(np.ldexp(base, e).ravel()).reshape(base.shape))
    for w in mats:
        n, k = w.shape
        wv = bf16_vals(w).reshape(n, k)
        codes, bscale, g = orc.quantize_nvfp4(w)
        sg, bs, q = _nvfp4_expected(wv)
        assert g[0] == sg
        assert np.array_equal(bscale, bs), np.argwhere(bscale != bs)[:5]
        got = np.stack([np.asarray(_nibbles(codes[r], k)) for r in range(n)])
        assert np.array_equal(got, q), np.argwhere(got != q)[:5]
