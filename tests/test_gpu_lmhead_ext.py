"""GPU parity of the lm_head entry points with extra outputs, through the C ABI:

- mtp_lmhead_argmax_logprob: the token, each row's top-1 log-probability and
  the running chain confidence. The log-probability is checked against the
  oracle's (fp64 logits) within 2 max_r tau_r + 2e-4 (the log-sum-exp moves by
  at most the largest logit error, the maximum by at most its own), and
  against the oracle's log-probability of the GPU's own f32 logits within 1e-4
  (f32 online sums and exponentials only).
- mtp_lmhead_argmax_masked: the argmax over the rows a grammar bitmask allows
  and the "any allowed" flag; bit-exact against the oracle's masked argmax of
  the GPU's own f32 logits, and within the tolerance rule against the oracle's
  fp64 logits restricted to the allowed rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity import DEV, head_host, log, mtp

pytestmark = pytest.mark.gpu


def make_head(wdtype, vocab, h, seed, outlier_p=0.0):
    m = mtp()
    W = si.normal_bf16(seed, si.TAG_LM, vocab, h, std=0.02, outlier_p=outlier_p, device=DEV)
    head = m.quantize_head(W, wdtype)
    torch.cuda.synchronize()
    return W, head


def own_logits(x, head, mvs):
    """The plain entry point's f32 logits (same kernel arithmetic) and token."""
    m = mtp()
    tok, lg = m.lmhead_argmax(x, head, mtp_vocab_size=mvs, with_logits=True)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lg.cpu().numpy()


def check_logprob(x, head, vocab, mvs, tok, lp, label):
    hh = head_host(head)
    name, w, s, g = hh
    n_eff = oracle.effective_vocab(vocab, mvs)
    L, tau = oracle.lmhead_logits(si.bits(x), name, w, s, g, n_eff=n_eff, with_tau=True)
    tok0, lg = own_logits(x, head, mvs)
    assert np.array_equal(tok, tok0), f"{label}: token differs from mtp_lmhead_argmax"
    for bi in range(x.shape[0]):
        mine = oracle.top1_logprob(lg[bi].astype(np.float64))
        ref = oracle.top1_logprob(L[bi])
        assert abs(lp[bi] - mine) <= 1e-4, f"{label}: row {bi} lp {lp[bi]} vs own-logit {mine}"
        tol = 2 * tau[bi].max() + 2e-4
        assert abs(lp[bi] - ref) <= tol, f"{label}: row {bi} lp {lp[bi]} vs oracle {ref} (tol {tol})"
        assert lp[bi] <= 0.0


LP_CASES = [
    ("bf16", 4099, 256, 1, 0),
    ("bf16", 4099, 4096, 3, 0),
    ("bf16", 5000, 4096, 2, 2050),
    ("bf16", 3, 16, 5, 0),
    ("fp8", 4099, 4096, 1, 0),
    ("fp8", 5001, 5120, 8, 0),
    ("nvfp4", 4099, 4096, 1, 0),
    ("nvfp4", 3333, 5120, 4, 0),
    ("nvfp4", 2048, 256, 8, 1000),
    ("nvfp4", 3001, 5120, 1, 2000),  # one pass of 3 chunks per lane per row
    ("bf16", 4099, 4096, 1, 0),      # static 4-wave blocks, one row per group
    # wide batches (the matrix-core form of the sweep)
    ("bf16", 2050, 4096, 5, 0),
    ("fp8", 4099, 4096, 6, 3000),
    ("nvfp4", 3001, 5120, 8, 0),
    ("nvfp4", 4099, 4096, 2, 0),
]


@pytest.mark.parametrize("wdtype,vocab,h,b,mvs", LP_CASES)
def test_logprob_small(wdtype, vocab, h, b, mvs):
    m = mtp()
    log(f"logprob small {wdtype} V={vocab} h={h} b={b} mvs={mvs}")
    W, head = make_head(wdtype, vocab, h, seed=vocab + 3 * h + b, outlier_p=0.01 if wdtype == "nvfp4" else 0.0)
    # x scaled so that the softmax is neither flat nor one-hot
    x = si.normal_bf16(11 + b, si.TAG_X, b, h, std=4.0, device=DEV)
    conf = torch.tensor([1.0, 0.5, 1e-30, 0.9, 1.0, 0.2, 1.0, 0.7][:b], dtype=torch.float32, device=DEV)
    conf0 = conf.cpu().numpy().copy()
    tok, lp = m.lmhead_argmax_logprob(x, head, mtp_vocab_size=mvs, conf=conf)
    torch.cuda.synchronize()
    lp = lp.cpu().numpy()
    check_logprob(x, head, vocab, mvs, tok.cpu().numpy(), lp, wdtype)
    np.testing.assert_allclose(conf.cpu().numpy(), np.minimum(conf0, np.exp(lp.astype(np.float64))), rtol=2e-6)


def test_logprob_chain_confidence_and_planted_rows():
    """Three drafts lower a running confidence; a planted dominant row gives a
    log-probability near 0; two planted equal rows give about -log 2."""
    m = mtp()
    vocab, h = 4096, 1024
    W, head = make_head("bf16", vocab, h, seed=5)
    x = si.normal_bf16(6, si.TAG_X, 1, h, device=DEV)
    conf = torch.ones(1, dtype=torch.float32, device=DEV)
    lps = []
    for i in range(3):
        xi = si.normal_bf16(60 + i, si.TAG_X, 1, h, std=3.0, device=DEV)
        _, lp = m.lmhead_argmax_logprob(xi, head, conf=conf)
        lps.append(float(lp.cpu()[0]))
    torch.cuda.synchronize()
    assert float(conf.cpu()[0]) == pytest.approx(min(np.exp(lps)), rel=2e-6)
    # planted rows: bf16(alpha * sign(x)) dominates every Gaussian row
    sgn = torch.where(x[0].float() >= 0, 1.0, -1.0)
    W2 = W.clone()
    W2[1234] = (0.05 * sgn).to(torch.bfloat16)
    head2 = m.quantize_head(W2, "bf16")
    tok, lp = m.lmhead_argmax_logprob(x, head2)
    torch.cuda.synchronize()
    assert int(tok.cpu()[0]) == 1234 and float(lp.cpu()[0]) > -1e-3
    check_logprob(x, head2, vocab, 0, tok.cpu().numpy(), lp.cpu().numpy(), "planted")
    W2[77] = W2[1234]
    head3 = m.quantize_head(W2, "bf16")
    tok, lp = m.lmhead_argmax_logprob(x, head3)
    torch.cuda.synchronize()
    assert int(tok.cpu()[0]) == 77
    assert float(lp.cpu()[0]) == pytest.approx(-np.log(2.0), abs=2e-3)


def test_logprob_nan_row():
    m = mtp()
    vocab, h = 1000, 256
    W, _ = make_head("bf16", vocab, h, seed=8)
    W[500, 3] = float("nan")
    head = m.quantize_head(W, "bf16")
    x = si.normal_bf16(9, si.TAG_X, 2, h, device=DEV)
    tok, lp = m.lmhead_argmax_logprob(x, head)
    torch.cuda.synchronize()
    assert np.all(np.isnan(lp.cpu().numpy()))
    tok0, _ = own_logits(x, head, 0)
    assert np.array_equal(tok.cpu().numpy(), tok0)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "nvfp4"])
def test_logprob_full_size(wdtype):
    m = mtp()
    wl = si.WORKLOADS[f"{wdtype}_154880x4096_b1"]
    log(f"logprob full {wl.name}")
    W = si.lm_weight(wl, 3, device=DEV)
    head = m.quantize_head(W, wdtype)
    del W
    x = si.normal_bf16(4, si.TAG_X, 1, wl.hidden, std=3.0, device=DEV)
    tok, lp = m.lmhead_argmax_logprob(x, head)
    torch.cuda.synchronize()
    check_logprob(x, head, wl.vocab, 0, tok.cpu().numpy(), lp.cpu().numpy(), wl.name)


# ---- grammar-masked argmax ----------------------------------------------------

def random_masks(seed, b, words, density):
    g = torch.Generator(device="cpu").manual_seed(seed)
    bits = (torch.rand((b, words * 32), generator=g) < density).to(torch.int64)
    w = (bits.view(b, words, 32) << torch.arange(32)).sum(-1)
    return w.to(torch.int64).apply_(lambda v: v - (1 << 32) if v >= (1 << 31) else v).to(torch.int32)


def check_masked(x, head, vocab, mvs, mask, tok, allowed, label):
    hh = head_host(head)
    name, w, s, g = hh
    n_eff = oracle.effective_vocab(vocab, mvs)
    _, lg = own_logits(x, head, mvs)
    L, tau = oracle.lmhead_logits(si.bits(x), name, w, s, g, n_eff=n_eff, with_tau=True)
    mk = np.zeros((x.shape[0], 0), dtype=np.int32) if mask is None else mask.cpu().numpy()
    for bi in range(x.shape[0]):
        t_own, a_own = oracle.argmax_masked(lg[bi].astype(np.float64), mk[bi], mk.shape[1])
        assert (int(tok[bi]), int(allowed[bi])) == (t_own, a_own), f"{label}: row {bi} vs own logits"
        t_ref, a_ref = oracle.argmax_masked(L[bi], mk[bi], mk.shape[1])
        assert int(allowed[bi]) == a_ref
        if a_ref and t_ref != int(tok[bi]):
            gt = int(tok[bi])
            assert L[bi, t_ref] - L[bi, gt] <= tau[bi, t_ref] + tau[bi, gt], f"{label}: row {bi} not within tau"


MASK_CASES = [
    # wdtype, vocab, h, b, mvs, density
    ("bf16", 4099, 256, 1, 0, 0.5),
    ("bf16", 4099, 4096, 3, 0, 0.1),
    ("bf16", 5000, 4096, 2, 2050, 0.5),
    ("fp8", 4099, 4096, 1, 0, 0.01),
    ("fp8", 5001, 5120, 8, 0, 0.5),
    ("nvfp4", 4099, 4096, 1, 0, 0.5),
    ("nvfp4", 3333, 5120, 4, 0, 0.002),
    ("nvfp4", 3001, 5120, 1, 0, 0.3),  # one pass of 3 chunks per lane per row
    ("bf16", 4099, 4096, 1, 0, 0.2),   # static 4-wave blocks, one row per group
    ("fp8", 4099, 4096, 8, 0, 0.3),    # matrix-core split schedule
    # wide batches (the matrix-core form of the sweep)
    ("bf16", 4099, 4096, 8, 2050, 0.3),
    ("fp8", 3001, 4096, 4, 0, 0.002),
    ("nvfp4", 4099, 4096, 8, 0, 0.5),
]


@pytest.mark.parametrize("wdtype,vocab,h,b,mvs,density", MASK_CASES)
def test_masked_small(wdtype, vocab, h, b, mvs, density):
    m = mtp()
    log(f"masked small {wdtype} V={vocab} h={h} b={b} mvs={mvs} density={density}")
    W, head = make_head(wdtype, vocab, h, seed=vocab + 5 * h + b)
    x = si.normal_bf16(13 + b, si.TAG_X, b, h, device=DEV)
    mask = random_masks(vocab + b, b, (vocab + 31) // 32, density).to(DEV)
    tok, allowed = m.lmhead_argmax_masked(x, head, mask, mtp_vocab_size=mvs)
    torch.cuda.synchronize()
    check_masked(x, head, vocab, mvs, mask, tok.cpu().numpy(), allowed.cpu().numpy(), wdtype)


def test_masked_edges():
    m = mtp()
    vocab, h, b = 3000, 512, 4
    W, head = make_head("bf16", vocab, h, seed=17)
    x = si.normal_bf16(18, si.TAG_X, b, h, device=DEV)
    words = (vocab + 31) // 32
    cases = {}
    cases["no words"] = None
    cases["empty"] = torch.zeros((b, words), dtype=torch.int32)
    full = torch.full((b, words), -1, dtype=torch.int32)
    cases["full"] = full
    cases["short"] = torch.full((b, 3), -1, dtype=torch.int32)            # rows >= 96 rejected
    only31 = torch.zeros((b, words), dtype=torch.int32)
    only31[:, 40] = -2 ** 31                                               # row 40 * 32 + 31 only
    cases["bit31"] = only31
    tok0, lg = own_logits(x, head, 0)
    knock = full.clone()
    for bi in range(b):                                                    # mask out each row's winner
        knock[bi, int(tok0[bi]) // 32] &= ~(1 << (int(tok0[bi]) % 32)) if int(tok0[bi]) % 32 != 31 else 0x7FFFFFFF
    cases["winner masked"] = knock
    for label, mk in cases.items():
        mk_dev = None if mk is None else mk.to(DEV)
        tok, allowed = m.lmhead_argmax_masked(x, head, mk_dev)
        torch.cuda.synchronize()
        check_masked(x, head, vocab, 0, mk_dev, tok.cpu().numpy(), allowed.cpu().numpy(), label)
    tok, allowed = m.lmhead_argmax_masked(x, head, cases["full"].to(DEV))
    assert np.array_equal(tok.cpu().numpy(), tok0) and np.all(allowed.cpu().numpy() == 1)
    tok, allowed = m.lmhead_argmax_masked(x, head, cases["empty"].to(DEV))
    assert np.all(tok.cpu().numpy() == 0) and np.all(allowed.cpu().numpy() == 0)
    # rows past n_eff do not count even when allowed
    beyond = torch.zeros((b, words), dtype=torch.int32)
    beyond[:, 80:] = -1
    tok, allowed = m.lmhead_argmax_masked(x, head, beyond.to(DEV), mtp_vocab_size=2000)
    assert np.all(tok.cpu().numpy() == 0) and np.all(allowed.cpu().numpy() == 0)


def test_masked_all_allowed_rows_nan():
    """Allowed rows whose logits are all NaN: token 0, allowed 1 (as on the pages)."""
    m = mtp()
    vocab, h = 640, 256
    W, _ = make_head("bf16", vocab, h, seed=19)
    W[100:200, 0] = float("nan")
    head = m.quantize_head(W, "bf16")
    x = si.normal_bf16(20, si.TAG_X, 1, h, device=DEV)
    mask = torch.zeros((1, vocab // 32), dtype=torch.int32)
    mask[0, 4] = -1  # rows 128..159, all NaN
    tok, allowed = m.lmhead_argmax_masked(x, head, mask.to(DEV))
    torch.cuda.synchronize()
    assert int(tok.cpu()[0]) == 0 and int(allowed.cpu()[0]) == 1


@pytest.mark.parametrize("wdtype", ["bf16", "nvfp4"])
def test_masked_full_size(wdtype):
    m = mtp()
    wl = si.WORKLOADS[f"{wdtype}_154880x4096_b1"]
    log(f"masked full {wl.name}")
    W = si.lm_weight(wl, 5, device=DEV)
    head = m.quantize_head(W, wdtype)
    del W
    x = si.normal_bf16(6, si.TAG_X, 1, wl.hidden, device=DEV)
    mask = random_masks(7, 1, (wl.vocab + 31) // 32, 0.3).to(DEV)
    tok, allowed = m.lmhead_argmax_masked(x, head, mask)
    torch.cuda.synchronize()
    check_masked(x, head, wl.vocab, 0, mask, tok.cpu().numpy(), allowed.cpu().numpy(), wl.name)


def _draw_ext(rng, kind):
    """One masked or log-probability call within the header's limits: format,
    vocab, h (a multiple of 16; of 256 for NVFP4; half the draws on the 1,024
    grid with b >= 3, the matrix-core form), b, truncation one time in three,
    mask density over three decades."""
    wdtype = str(rng.choice(["bf16", "fp8", "nvfp4"]))
    if rng.random() < 0.5:
        h = 1024 * int(rng.integers(1, 9))
        b = int(rng.integers(3, 9))
    else:
        h = 256 * int(rng.integers(1, 33)) if wdtype == "nvfp4" else 16 * int(rng.integers(1, 513))
        b = int(rng.integers(1, 9))
    vocab = int(rng.integers(1, 6001))
    mvs = int(rng.integers(1, vocab + 1)) if rng.random() < 1 / 3 else 0
    density = float(10.0 ** rng.uniform(-3, 0))
    return kind, wdtype, vocab, h, b, mvs, density


RANDOM_EXT = [_draw_ext(np.random.default_rng(9850 + i), ("masked", "logprob")[i % 2]) for i in range(18)]


@pytest.mark.parametrize("case", range(len(RANDOM_EXT)))
def test_masked_and_logprob_random_shapes(case):
    """Seeded random shapes through the masked and log-probability entry
    points, checked as the hand-picked cases are; each case logs its draw."""
    m = mtp()
    kind, wdtype, vocab, h, b, mvs, density = RANDOM_EXT[case]
    log(f"{kind} random #{case}: {wdtype} V={vocab} h={h} b={b} mvs={mvs} density={density:.4f} "
        f"form={m.lmhead_kernel_form(b, h, wdtype)}")
    W, head = make_head(wdtype, vocab, h, seed=9860 + case, outlier_p=0.01 if wdtype == "nvfp4" else 0.0)
    if kind == "masked":
        x = si.normal_bf16(9870 + case, si.TAG_X, b, h, device=DEV)
        mask = random_masks(9880 + case, b, (vocab + 31) // 32, density).to(DEV)
        tok, allowed = m.lmhead_argmax_masked(x, head, mask, mtp_vocab_size=mvs)
        torch.cuda.synchronize()
        check_masked(x, head, vocab, mvs, mask, tok.cpu().numpy(), allowed.cpu().numpy(), f"random #{case}")
    else:
        x = si.normal_bf16(9870 + case, si.TAG_X, b, h, std=4.0, device=DEV)
        conf = torch.rand(b, generator=torch.Generator().manual_seed(9890 + case)).to(DEV)
        conf0 = conf.cpu().numpy().astype(np.float64)
        tok, lp = m.lmhead_argmax_logprob(x, head, mtp_vocab_size=mvs, conf=conf)
        torch.cuda.synchronize()
        lp = lp.cpu().numpy()
        check_logprob(x, head, vocab, mvs, tok.cpu().numpy(), lp, f"random #{case}")
        np.testing.assert_allclose(conf.cpu().numpy(), np.minimum(conf0, np.exp(lp.astype(np.float64))), rtol=2e-6)
