"""Pins for the oracle's RMSNorm, combine (norms + concat + fc + final norm),
lm_head logits / tolerance, argmax, and the whole draft on a case whose token
is known in closed form.

RMSNorm, fc and the lm_head sums are checked against exact rational arithmetic
(fractions, with a 60-digit decimal square root) on small shapes; the argmax
against planted maxima, duplicates, permutations and prefixes. Operands are
deliberately non-symmetric so that a transposed weight, a swapped concat order,
a dropped gamma or a wrong offset changes the answer.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_table

getcontext().prec = 60


def bf16_from_f32(f):
    return torch.from_numpy(np.asarray(f, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def val(bits):
    """BF16 bits -> Fraction, via torch's bfloat16 -> float32 cast."""
    f = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float32)
    return [Fraction(float(x)) for x in f.numpy().ravel()]


_BF16_POS = None


def _bf16_grid():
    global _BF16_POS
    if _BF16_POS is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint16)  # all finite non-negative patterns, ascending
        _BF16_POS = (bits, val(bits))
    return _BF16_POS


def nearest_bf16(x: Fraction) -> int:
    """Brute force: the BF16 pattern nearest to the exact value x, ties to even."""
    import bisect

    bits, vals = _bf16_grid()
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    i = bisect.bisect_left(vals, a)
    cands = [j for j in (i - 1, i) if 0 <= j < len(vals)]
    best = min(cands, key=lambda j: (abs(vals[j] - a), int(bits[j]) & 1))
    return sign | int(bits[best])


def exact_rms(v_bits, g_bits, eps, off):
    v = val(v_bits)
    g = val(g_bits)
    h = len(v)
    ms = sum(x * x for x in v) / h + Fraction(float(np.float32(eps)))
    d = Decimal(ms.numerator) / Decimal(ms.denominator)
    r = Fraction(1 / d.sqrt())  # 60 digits, far beyond BF16's rounding needs
    return np.array([nearest_bf16(v[i] * r * (g[i] + Fraction(float(off)))) for i in range(h)], dtype=np.uint16)


def rand_bf16(rng, shape, std=1.0, mean=0.0):
    return bf16_from_f32(rng.standard_normal(shape).astype(np.float32) * std + mean)


@pytest.mark.parametrize("h,off", [(8, 0.0), (16, 0.0), (16, 1.0), (32, 0.0)])
def test_rms_norm_exact(orc, h, off):
    rng = np.random.default_rng(h + int(off))
    for _ in range(5):
        v = rand_bf16(rng, h)
        g = rand_bf16(rng, h, 0.1, 0.0 if off else 1.0)
        got = orc.rms_norm(v, g, 1e-6, off)
        assert np.array_equal(got, exact_rms(v, g, 1e-6, off))


def test_rms_norm_eps_matters_and_scale_invariance(orc):
    rng = np.random.default_rng(3)
    h = 64
    g = rand_bf16(rng, h, 0.1, 1.0)
    tiny = bf16_from_f32(rng.standard_normal(h).astype(np.float32) * 1e-4)
    # with ms ~ 1e-8 an eps of 1e-6 dominates: result far from the eps-free norm
    a = val(orc.rms_norm(tiny, g, 1e-6, 0.0))
    b = val(orc.rms_norm(tiny, g, 1e-12, 0.0))
    assert max(abs(x) for x in a) < max(abs(x) for x in b) / 5
    assert np.array_equal(orc.rms_norm(tiny, g, 1e-6, 0.0), exact_rms(tiny, g, 1e-6, 0.0))
    # scaling the input by a power of two leaves the norm unchanged when eps is negligible
    v = rand_bf16(rng, h)
    v4 = bf16_from_f32(np.asarray(val(v), dtype=np.float64).astype(np.float32) * 4)
    d = np.abs(np.asarray(val(orc.rms_norm(v, g, 1e-12, 0.0)), dtype=float) -
               np.asarray(val(orc.rms_norm(v4, g, 1e-12, 0.0)), dtype=float))
    assert d.max() == 0.0


def test_rms_norm_gamma_offset(orc):
    """offset 1 with gamma w equals offset 0 with gamma 1 + w (when 1 + w is BF16 exact)."""
    rng = np.random.default_rng(5)
    h = 32
    v = rand_bf16(rng, h)
    w = bf16_from_f32(np.round(rng.standard_normal(h) * 8) / 64)  # multiples of 1/64: 1 + w exact in BF16
    one_plus = bf16_from_f32(np.asarray(val(w), dtype=float).astype(np.float32) + 1)
    assert np.array_equal(orc.rms_norm(v, w, 1e-6, 1.0), orc.rms_norm(v, one_plus, 1e-6, 0.0))


def test_combine_exact_composition(orc):
    """Embedding gather, both norms, concat with the embedding first, fc [h, 2h]
    row-major, bf16 after fc, final norm: each intermediate against exact
    arithmetic."""
    rng = np.random.default_rng(8)
    V, h, b = 11, 16, 3
    E = rand_bf16(rng, (V, h))
    H = rand_bf16(rng, (b, h))
    ge, gh, gf = (rand_bf16(rng, h, 0.1, 1.0) for _ in range(3))
    W = rand_bf16(rng, (h, 2 * h), 0.2)
    tok = np.array([7, 0, 10], dtype=np.int32)
    x, c, u = orc.draft_combine(E, tok, H, ge, gh, W, gf, 1e-6, 0.0, intermediates=True)
    Wv = [val(W[j]) for j in range(h)]
    for bi in range(b):
        ce = exact_rms(E[tok[bi]], ge, 1e-6, 0.0)
        ch = exact_rms(H[bi], gh, 1e-6, 0.0)
        assert np.array_equal(c[bi], np.concatenate([ce, ch]))
        cv = val(c[bi])
        uu = np.array([nearest_bf16(sum(Wv[j][i] * cv[i] for i in range(2 * h))) for j in range(h)], dtype=np.uint16)
        assert np.array_equal(u[bi], uu)
        assert np.array_equal(x[bi], exact_rms(uu, gf, 1e-6, 0.0))


def test_combine_catches_swapped_concat_and_transposed_fc(orc):
    """Sanity of the pin itself: the obvious mistakes give different u."""
    rng = np.random.default_rng(9)
    V, h = 5, 16
    E = rand_bf16(rng, (V, h))
    H = rand_bf16(rng, (1, h))
    ge, gh, gf = (rand_bf16(rng, h, 0.1, 1.0) for _ in range(3))
    W = rand_bf16(rng, (h, 2 * h), 0.2)
    x, c, u = orc.draft_combine(E, np.array([2], np.int32), H, ge, gh, W, gf, intermediates=True)
    cv = np.asarray(val(c[0]), dtype=float)
    Wf = np.asarray(val(W), dtype=float).reshape(h, 2 * h)
    swapped = np.concatenate([cv[h:], cv[:h]])
    good = Wf @ cv
    assert np.allclose(np.asarray(val(u[0]), dtype=float), good, rtol=1e-2, atol=1e-3)
    assert not np.allclose(good, Wf @ swapped, rtol=1e-2, atol=1e-3)


# ------------------------------------------------------------- lm_head ----

def _e4m3_dec():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(
        torch.float32).numpy().astype(np.float64)


E2M1 = {int(c, 16): Fraction(float(v)) for c, v in read_table("e2m1_values.txt")}


def _exact_weights(wd, w, scale, g, h):
    """Dequantized weights as Fractions, from independent decode tables."""
    n = w.shape[0]
    if wd == "bf16":
        return [val(w[r]) for r in range(n)]
    dec = _e4m3_dec()
    if wd == "fp8":
        return [[Fraction(dec[w[r, i]]) * Fraction(float(scale[r])) for i in range(h)] for r in range(n)]
    out = []
    for r in range(n):
        row = []
        for i in range(h):
            q = (int(w[r, i // 2]) >> (4 * (i & 1))) & 0xF
            row.append(E2M1[q] * Fraction(dec[scale[r, i // 16]]) * Fraction(float(g[0])))
        out.append(row)
    return out


@pytest.mark.parametrize("wd", ["bf16", "fp8", "nvfp4"])
def test_lmhead_logits_exact(orc, wd):
    rng = np.random.default_rng({"bf16": 1, "fp8": 2, "nvfp4": 3}[wd])
    n, h, b = 40, 64, 3
    W = rand_bf16(rng, (n, h), 0.02)
    x = rand_bf16(rng, (b, h))
    if wd == "bf16":
        w, s, g = W, None, None
    elif wd == "fp8":
        w, s = orc.quantize_fp8(W)
        g = None
    else:
        w, s, g = orc.quantize_nvfp4(W)
    logits, tau = orc.lmhead_logits(x, wd, w, s, g, with_tau=True)
    What = _exact_weights(wd, w, s, g, h)
    for bi in range(b):
        xv = val(x[bi])
        for r in range(n):
            terms = [What[r][i] * xv[i] for i in range(h)]
            L = sum(terms)
            T = Fraction(1, 1000) * sum(abs(t) for t in terms)
            assert abs(Fraction(logits[bi, r]) - L) <= abs(L) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)
            assert abs(Fraction(tau[bi, r]) - T) <= T * Fraction(1, 10 ** 12)


def test_lmhead_truncation_and_batch_rows(orc):
    rng = np.random.default_rng(4)
    n, h = 100, 32
    W = rand_bf16(rng, (n, h), 0.02)
    x = rand_bf16(rng, (4, h))
    assert orc.effective_vocab(n, 0) == n
    assert orc.effective_vocab(n, 37) == 37
    assert orc.effective_vocab(n, 1000) == n
    tok, lg = orc.lmhead_argmax(x, "bf16", W, mtp_vocab_size=37)
    assert lg.shape == (4, 37)
    full = orc.lmhead_logits(x, "bf16", W)
    assert np.array_equal(lg, full[:, :37])
    for bi in range(4):
        t1, l1 = orc.lmhead_argmax(x[bi:bi + 1], "bf16", W, mtp_vocab_size=37)
        assert t1[0] == tok[bi] and np.array_equal(l1[0], lg[bi])


# --------------------------------------------------------------- argmax ----

def test_argmax_rules(orc):
    assert orc.argmax(np.array([1.0, 3.0, 3.0, 2.0])) == 1  # lowest index of the max
    assert orc.argmax(np.array([-0.0, 0.0])) == 0  # -0 == +0: the first wins
    assert orc.argmax(np.array([0.0, -0.0])) == 0
    assert orc.argmax(np.array([np.nan, 1.0, np.nan])) == 1  # NaN never wins
    assert orc.argmax(np.array([np.nan, np.nan])) == 0
    assert orc.argmax(np.array([-np.inf, -np.inf, -np.inf])) == 0
    assert orc.argmax(np.array([-np.inf, -5.0])) == 1
    assert orc.argmax(np.full(17, 2.5)) == 0
    assert orc.argmax(np.array([np.inf, np.inf])) == 0


def test_argmax_permutation_and_random(orc):
    rng = np.random.default_rng(6)
    for _ in range(50):
        v = rng.standard_normal(257)
        i = orc.argmax(v)
        assert v[i] == v.max() and i == int(np.flatnonzero(v == v.max())[0])
        p = rng.permutation(257)
        assert p[orc.argmax(v[p])] == i


def test_planted_row_wins_and_duplicate_lower_index(orc):
    """A row equal to bf16(alpha * sign(x)) with large alpha maximises w . x; a copy
    of it at a lower index takes over; truncation before it hides it."""
    rng = np.random.default_rng(12)
    n, h = 300, 64
    W = rand_bf16(rng, (n, h), 0.02)
    x = rand_bf16(rng, (1, h))
    xs = np.sign(np.asarray(val(x[0]), dtype=float))
    plant = bf16_from_f32(xs * 0.5)
    W[211] = plant
    tok, lg = orc.lmhead_argmax(x, "bf16", W)
    assert tok[0] == 211
    W[64] = plant
    tok, lg = orc.lmhead_argmax(x, "bf16", W)
    assert tok[0] == 64 and lg[0, 64] == lg[0, 211]
    tok, _ = orc.lmhead_argmax(x, "bf16", W, mtp_vocab_size=64)  # rows 0..63: plant excluded
    assert tok[0] != 64 and tok[0] < 64
    tok, _ = orc.lmhead_argmax(x, "bf16", W, mtp_vocab_size=65)  # the plant is the last row kept
    assert tok[0] == 64


# ---------------------------------------------------------- whole step ----

@pytest.mark.parametrize("wd", ["bf16", "fp8", "nvfp4"])
def test_step_closed_form_token(orc, wd):
    """The whole draft (combine, then the lm_head argmax) on a case whose token
    is known without arithmetic: each hidden row has one large planted element,
    every embedding row one at a different place, fc = [0 | I] keeps only the
    normalized hidden half of the concat, unit gammas, and the head's first h
    rows are the unit vectors in a shuffled order above rows of small noise.
    Then x keeps the hidden row's peak, and the token is the head row that
    holds the unit vector at the peak. A swapped concat would pick the
    embedding's peak instead."""
    rng = np.random.default_rng(31)
    V, h, n = 9, 32, 80
    peaks = [5, 17, 30]
    b = len(peaks)
    E = rand_bf16(rng, (V, h), 0.05)
    E[:, 11] = bf16_from_f32(np.full(V, 4.0))
    H = rand_bf16(rng, (b, h), 0.05)
    for bi, p in enumerate(peaks):
        H[bi, p] = bf16_from_f32(np.float32(4.0))
    one = bf16_from_f32(np.ones(h, dtype=np.float32))
    fc = np.zeros((h, 2 * h), dtype=np.uint16)
    fc[np.arange(h), h + np.arange(h)] = bf16_from_f32(np.ones(h, dtype=np.float32))
    perm = rng.permutation(h)  # head row r < h is the unit vector e_perm[r]
    W = np.zeros((n, h), dtype=np.float32)
    W[np.arange(h), perm] = 1.0
    W[h:] = rng.standard_normal((n - h, h)).astype(np.float32) * 0.01
    W = bf16_from_f32(W)
    if wd == "bf16":
        w, s, g = W, None, None
    elif wd == "fp8":
        (w, s), g = orc.quantize_fp8(W), None
    else:
        w, s, g = orc.quantize_nvfp4(W)
    toks = np.array([2, 7, 0], dtype=np.int32)
    x = orc.draft_combine(E, toks, H, one, one, fc, one, 1e-6, 0.0)
    tok, _ = orc.lmhead_argmax(x, wd, w, s, g)
    want = [int(np.flatnonzero(perm == p)[0]) for p in peaks]
    assert tok.tolist() == want
