"""Pins for the oracle's top-1 log-probability, grammar-masked argmax and the
combiner variants (fc stored in FP8 / NVFP4, and the split e_proj / h_proj
form).

The log-probability is checked against closed forms and a 50-digit decimal
evaluation; the masked argmax against the plain argmax and masks whose answer
is known by construction; the quantized-fc combine against the BF16 combine on
weights every precision represents exactly and against exact rational sums;
the split combine against exact rational arithmetic with its two extra
rounding points.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from test_oracle_math import _exact_weights, exact_rms, nearest_bf16, rand_bf16, val

getcontext().prec = 50


# ---- top-1 log-probability --------------------------------------------------

@pytest.mark.parametrize("n", [1, 7, 1000])
def test_logprob_uniform_closed_form(orc, n):
    assert orc.top1_logprob(np.full(n, -3.5)) == pytest.approx(-math.log(n), abs=1e-14)


@pytest.mark.parametrize("a,b", [(2.0, -1.0), (0.0, 0.0), (1000.0, 999.0), (-1e3, -1e3 - 30.0)])
def test_logprob_two_point_closed_form(orc, a, b):
    d = abs(a - b)
    expect = -math.log1p(math.exp(-d))
    assert orc.top1_logprob(np.array([a, b])) == pytest.approx(expect, abs=1e-14)
    assert orc.top1_logprob(np.array([b, a])) == pytest.approx(expect, abs=1e-14)


def _decimal_logp(v):
    ds = [Decimal(float(x)) for x in v]
    m = max(ds)
    s = sum((d - m).exp() for d in ds)
    return float(-s.ln())


def test_logprob_decimal_brute_force_and_shift(orc):
    rng = np.random.default_rng(21)
    for trial in range(20):
        n = int(rng.integers(2, 60))
        v = rng.standard_normal(n) * (0.5 + 4 * trial)
        lp = orc.top1_logprob(v)
        assert lp == pytest.approx(_decimal_logp(v), abs=1e-12)
        assert orc.top1_logprob(v + 123.25) == pytest.approx(lp, abs=1e-12)
        assert lp <= 0.0


def test_logprob_non_finite(orc):
    assert orc.top1_logprob(np.array([0.5])) == 0.0
    assert orc.top1_logprob(np.array([1.0, -np.inf, 2.0])) == orc.top1_logprob(np.array([1.0, 2.0]))
    assert math.isnan(orc.top1_logprob(np.array([1.0, np.nan, 2.0])))
    assert math.isnan(orc.top1_logprob(np.array([-np.inf, -np.inf])))


# ---- grammar-masked argmax ----------------------------------------------------

def _mask_from(allowed, n, words=None):
    words = (n + 31) // 32 if words is None else words
    m = np.zeros(words, dtype=np.uint32)
    for i in allowed:
        if i // 32 < words:
            m[i // 32] |= np.uint32(1) << np.uint32(i % 32)
    return m.view(np.int32)


def _brute(v, allowed):
    allowed = sorted(allowed)
    if not allowed:
        return 0, 0
    best, bv = 0, -np.inf
    for i in allowed:
        if v[i] > bv:
            best, bv = i, v[i]
    return best, 1


def test_masked_full_mask_is_plain_argmax(orc):
    rng = np.random.default_rng(31)
    for n in (1, 31, 32, 33, 100, 1000):
        v = rng.standard_normal(n)
        assert orc.argmax_masked(v, _mask_from(range(n), n)) == (orc.argmax(v), 1)


def test_masked_empty_and_short(orc):
    v = np.arange(10, dtype=np.float64)
    assert orc.argmax_masked(v, np.zeros(1, dtype=np.int32)) == (0, 0)
    assert orc.argmax_masked(v, np.full(1, -1, dtype=np.int32), mask_words=0) == (0, 0)
    w = np.zeros(100)
    w[70] = 5.0  # the maximum lies past a 2-word mask
    assert orc.argmax_masked(w, np.full(2, -1, dtype=np.int32)) == (0, 1)
    assert orc.argmax_masked(w, np.full(3, -1, dtype=np.int32)) == (70, 1)


def test_masked_known_answers(orc):
    rng = np.random.default_rng(32)
    n = 300
    for _ in range(30):
        v = rng.standard_normal(n)
        allowed = set(rng.choice(n, size=int(rng.integers(1, n)), replace=False).tolist())
        allowed.discard(int(np.argmax(v)))  # the global maximum is masked out
        assert orc.argmax_masked(v, _mask_from(allowed, n)) == _brute(v, allowed)
    i = 77
    assert orc.argmax_masked(rng.standard_normal(n), _mask_from([i], n)) == (i, 1)


def test_masked_ties_nan_inf_and_bit31(orc):
    v = np.zeros(64)
    v[5] = v[40] = 3.0
    assert orc.argmax_masked(v, _mask_from(range(64), 64)) == (5, 1)
    assert orc.argmax_masked(v, _mask_from([i for i in range(64) if i != 5], 64)) == (40, 1)
    u = np.full(64, -np.inf)
    u[9] = np.nan
    assert orc.argmax_masked(u, _mask_from([9, 12], 64)) == (0, 1)  # allowed, nothing above -inf
    w = np.zeros(64)
    w[31] = -2.0
    m = np.array([np.int32(-2 ** 31), 0], dtype=np.int32)  # only bit 31 of word 0
    assert orc.argmax_masked(w, m) == (31, 1)


# ---- combine with a quantized fc ---------------------------------------------

def _step_inputs(rng, V, h, b):
    E = rand_bf16(rng, (V, h))
    H = rand_bf16(rng, (b, h))
    ge, gh, gf = (rand_bf16(rng, h, 0.1, 1.0) for _ in range(3))
    tok = rng.integers(0, V, size=b).astype(np.int32)
    return E, H, ge, gh, gf, tok


def _fp8_exact_fc(rng, h):
    """Rows with absmax exactly 448 and E4M3-representable entries: scale 1."""
    mags = np.array([0.0, 0.015625, 0.25, 0.5, 0.75, 1.0, 1.5, 3.0, 10.0, 26.0, 96.0, 224.0, 448.0], dtype=np.float32)
    W = rng.choice(mags, size=(h, 2 * h)) * rng.choice([-1.0, 1.0], size=(h, 2 * h)).astype(np.float32)
    W[np.arange(h), rng.integers(0, 2 * h, size=h)] = 448.0
    return W.astype(np.float32)


def _nvfp4_exact_fc(rng, h):
    """Global max 2688 (global scale 1); every 16-block has absmax 6 * 2^e and
    entries E2M1 * 2^e, so every value is represented exactly."""
    e2m1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
    W = np.zeros((h, 2 * h), dtype=np.float32)
    for r in range(h):
        for blk in range(2 * h // 16):
            e = float(2.0 ** int(rng.integers(-6, 6)))
            vals = rng.choice(e2m1, size=16) * rng.choice([-1.0, 1.0], size=16)
            vals[int(rng.integers(0, 16))] = 6.0
            W[r, blk * 16:(blk + 1) * 16] = vals * e
    W[0, 3] = 2688.0  # its block: absmax 2688 -> block scale 448
    W[0, 0:16] = np.where(np.arange(16) == 3, 2688.0, 448.0 * rng.choice(e2m1[:6], size=16))
    return W


@pytest.mark.parametrize("wd", ["fp8", "nvfp4"])
def test_combine_q_exact_weights_equal_bf16(orc, wd):
    from test_oracle_math import bf16_from_f32

    rng = np.random.default_rng({"fp8": 41, "nvfp4": 42}[wd])
    V, h, b = 9, 32, 3
    E, H, ge, gh, gf, tok = _step_inputs(rng, V, h, b)
    Wf = _fp8_exact_fc(rng, h) if wd == "fp8" else _nvfp4_exact_fc(rng, h)
    W = bf16_from_f32(Wf)
    assert np.array_equal(np.asarray(val(W.ravel()), dtype=float), Wf.ravel().astype(float))
    if wd == "fp8":
        codes, s = orc.quantize_fp8(W)
        g = None
        assert np.all(s == 1.0)
    else:
        codes, s, g = orc.quantize_nvfp4(W)
        assert g[0] == 1.0
    x_q, u_q = orc.draft_combine_q(E, tok, H, ge, gh, wd, codes, s, g, gf, 1e-6, 0.0, with_u=True)
    x, c, u = orc.draft_combine(E, tok, H, ge, gh, W, gf, 1e-6, 0.0, intermediates=True)
    assert np.array_equal(u_q, u) and np.array_equal(x_q, x)
    x_b = orc.draft_combine_q(E, tok, H, ge, gh, "bf16", W, None, None, gf, 1e-6, 0.0)
    assert np.array_equal(x_b, x)


@pytest.mark.parametrize("wd", ["fp8", "nvfp4"])
def test_combine_q_exact_rational(orc, wd):
    rng = np.random.default_rng({"fp8": 43, "nvfp4": 44}[wd])
    V, h, b = 7, 16, 2
    E, H, ge, gh, gf, tok = _step_inputs(rng, V, h, b)
    W = rand_bf16(rng, (h, 2 * h), 0.2)
    if wd == "fp8":
        codes, s = orc.quantize_fp8(W)
        g = None
    else:
        codes, s, g = orc.quantize_nvfp4(W)
    x, u = orc.draft_combine_q(E, tok, H, ge, gh, wd, codes, s, g, gf, 1e-6, 0.0, with_u=True)
    What = _exact_weights(wd, codes, s, g, 2 * h)
    for bi in range(b):
        cv = val(np.concatenate([exact_rms(E[tok[bi]], ge, 1e-6, 0.0), exact_rms(H[bi], gh, 1e-6, 0.0)]))
        uu = np.array([nearest_bf16(sum(What[j][i] * cv[i] for i in range(2 * h))) for j in range(h)], dtype=np.uint16)
        assert np.array_equal(u[bi], uu)
        assert np.array_equal(x[bi], exact_rms(uu, gf, 1e-6, 0.0))


# ---- split combine ---------------------------------------------------------

def test_combine_split_exact_rational(orc):
    rng = np.random.default_rng(51)
    V, h, b = 6, 16, 3
    E, H, ge, gh, gf, tok = _step_inputs(rng, V, h, b)
    Ep = rand_bf16(rng, (h, h), 0.3)
    Hp = rand_bf16(rng, (h, h), 0.3)
    x, u = orc.draft_combine_split(E, tok, H, ge, gh, Ep, Hp, gf, 1e-6, 0.0, with_u=True)
    Epv = [val(Ep[j]) for j in range(h)]
    Hpv = [val(Hp[j]) for j in range(h)]
    for bi in range(b):
        ne = val(exact_rms(E[tok[bi]], ge, 1e-6, 0.0))
        nh = val(exact_rms(H[bi], gh, 1e-6, 0.0))
        uu = []
        for j in range(h):
            be = val([nearest_bf16(sum(Epv[j][i] * ne[i] for i in range(h)))])[0]
            bh = val([nearest_bf16(sum(Hpv[j][i] * nh[i] for i in range(h)))])[0]
            uu.append(nearest_bf16(be + bh))
        uu = np.array(uu, dtype=np.uint16)
        assert np.array_equal(u[bi], uu)
        assert np.array_equal(x[bi], exact_rms(uu, gf, 1e-6, 0.0))
    # the two projections are not interchangeable
    _, u_sw = orc.draft_combine_split(E, tok, H, ge, gh, Hp, Ep, gf, 1e-6, 0.0, with_u=True)
    assert not np.array_equal(u_sw, u)


def test_combine_split_zero_branch_is_one_rounding(orc):
    rng = np.random.default_rng(52)
    V, h, b = 4, 16, 2
    E, H, ge, gh, gf, tok = _step_inputs(rng, V, h, b)
    Ep = rand_bf16(rng, (h, h), 0.3)
    Z = np.zeros((h, h), dtype=np.uint16)
    _, u = orc.draft_combine_split(E, tok, H, ge, gh, Ep, Z, gf, 1e-6, 0.0, with_u=True)
    Epv = [val(Ep[j]) for j in range(h)]
    for bi in range(b):
        ne = val(exact_rms(E[tok[bi]], ge, 1e-6, 0.0))
        assert np.array_equal(u[bi], [nearest_bf16(sum(Epv[j][i] * ne[i] for i in range(h))) for j in range(h)])
