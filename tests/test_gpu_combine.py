"""GPU parity of the combine (mtp_draft_combine: embedding gather, two RMSNorms,
concat, fc [h, 2h], final RMSNorm) and of the whole draft step (combine, then
lm_head + argmax), against the oracle, through the C ABI.

Each stage of the combine is checked from the intermediates the call leaves in
its workspace (parity.check_combine_stages): the concat c against the oracle's,
u against the double-precision fc of the GPU's own c, x against the oracle's
RMSNorm of the GPU's own u, each within one BF16 unit with the share of
elements one unit off bounded. The end-to-end x is also compared with the
oracle's x within a bound derived from the arithmetic
(parity.combine_tolerance). The step's logits and token use the lm_head rules,
with the oracle's own x as the reference input.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity import (DEV, check_combine, check_combine_stages, check_lmhead, combine_tolerance, fmt_stages, head_host,
                    log, mtp)

pytestmark = pytest.mark.gpu


def run_step(wl, seed, gamma_offset=0.0, tokens=None, W=None, check_tokens=True):
    m = mtp()
    inp = si.step_inputs(wl, seed, device=DEV)
    if tokens is not None:
        inp["tokens"] = np.asarray(tokens, dtype=np.int32)
    b, h = wl.batch, wl.hidden
    ws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, h), DEV)
    x = m.draft_combine(inp["embed"], inp["tokens"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"],
                        inp["gamma_f"], eps=wl.eps, gamma_offset=gamma_offset, ws=ws)
    if W is None:
        W = si.lm_weight(wl, seed, device=DEV)
    head = m.quantize_head(W, wl.wdtype)
    tok, lg = m.lmhead_argmax(x, head, mtp_vocab_size=wl.mtp_vocab_size, with_logits=True)
    torch.cuda.synchronize()
    c_g, u_g = m.combine_intermediates(ws, b, h)
    stg = check_combine_stages(inp, gamma_offset, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(x), label=wl.name)
    xo, tol = combine_tolerance(inp, gamma_offset, wl.eps)
    d = check_combine(si.bits(x), xo, tol, label=wl.name)
    log(f"  {wl.name}: stages {fmt_stages(stg)}; x vs oracle x: exact {d['exact']:.4f} max {d['max_ulps']} ulps")
    if check_tokens:
        st = check_lmhead(xo, head_host(head), wl.vocab, wl.mtp_vocab_size, tok.cpu().numpy(), lg.cpu().numpy(),
                          label=wl.name)
    else:
        st = {}
    return x, xo, tok, lg, inp, W, st, d


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_step(seed):
    wl = si.WORKLOADS["tiny_step"]
    log(f"tiny step seed {seed}")
    run_step(wl, seed)


def test_tiny_step_gamma_offset_one():
    """The shared-norm convention (gamma applied as 1 + w)."""
    wl = si.WORKLOADS["tiny_step"]
    run_step(wl, 3, gamma_offset=1.0)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_step_batches(b):
    wl = si.Workload("step_b", "step", vocab=4096, hidden=256, batch=b)
    run_step(wl, 10 + b, tokens=[0, 4095, 17, 17, 1, 2, 3, 4][:b])


def test_step_h4096_b8_and_h8192_b4():
    run_step(si.Workload("s4096", "step", vocab=2000, hidden=4096, batch=8), 5)
    run_step(si.Workload("s8192", "step", vocab=1000, hidden=8192, batch=4), 6)
    run_step(si.Workload("s8192b8", "step", vocab=1000, hidden=8192, batch=8), 7)


def test_tiny_step_planted_tie():
    """Copy the winning row to a lower index in another block (the copy wins) and
    to a higher index (the original still wins)."""
    m = mtp()
    wl = si.WORKLOADS["tiny_step"]
    x, xo, tok, lg, inp, W, st, d = run_step(wl, 0)
    i_star = int(tok[0])
    for j, want in ((i_star // 2, i_star // 2), (min(wl.vocab - 1, i_star + 700), i_star)):
        if j == i_star:
            continue
        W2 = W.clone()
        W2[j] = W[i_star]
        t2, l2 = m.lmhead_argmax(x, m.quantize_head(W2, "bf16"), with_logits=True)
        assert int(t2[0]) == want, (i_star, j, int(t2[0]))


@pytest.mark.parametrize("h,b", [(5120, 1), (5120, 2), (2064, 5)])
def test_combine_hidden_off_the_grid(h, b):
    """The two-entry-point path (combine with its own final norm, then the
    lm_head) at hidden sizes off the 4,096 grid: 5,120 (a VALU combine from
    b = 2, fc rows of a pass and a quarter) and 2,064 (ragged fc rows)."""
    log(f"combine h={h} b={b}")
    run_step(si.Workload(f"c{h}b{b}", "step", vocab=2500, hidden=h, batch=b), 60 + b)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "nvfp4"])
def test_step_32000x4096(wdtype):
    wl = si.Workload(f"step_32000x4096_{wdtype}", "step", vocab=32000, hidden=4096, batch=1, wdtype=wdtype)
    log(f"step 32000x4096 {wdtype}")
    for seed in (0, 1):
        run_step(wl, seed)


def test_step_154880x4096():
    wl = si.WORKLOADS["step_154880x4096"]
    log("step 154880x4096")
    run_step(wl, 0)


@pytest.mark.parametrize("b", [2, 3, 5, 7])
def test_combine_wide_batches_h4096(b):
    """Batch widths from 2 on take the matrix-core fc (at h = 4096): parity
    within the combine bound, and each vector's x the same bits whatever else
    shares the call."""
    m = mtp()
    wl = si.Workload("cw", "step", vocab=1000, hidden=4096, batch=8)
    inp = si.step_inputs(wl, 40 + b, device=DEV)
    args = (inp["embed"], inp["tokens"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"], inp["gamma_f"])
    x8 = m.draft_combine(*args, eps=wl.eps)
    sub = dict(inp)
    sub["tokens"] = inp["tokens"][:b]
    sub["hidden"] = inp["hidden"][:b].contiguous()
    ws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, wl.hidden), DEV)
    xb = m.draft_combine(sub["embed"], sub["tokens"], sub["hidden"], sub["gamma_e"], sub["gamma_h"], sub["fc"],
                         sub["gamma_f"], eps=wl.eps, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(xb.view(torch.int16), x8[:b].view(torch.int16))
    c_g, u_g = m.combine_intermediates(ws, b, wl.hidden)
    stg = check_combine_stages(sub, 0.0, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(xb), label=f"b={b}")
    xo, tol = combine_tolerance(sub, 0.0, wl.eps)
    d = check_combine(si.bits(xb), xo, tol, label=f"b={b}")
    log(f"  combine b={b}: stages {fmt_stages(stg)}; x vs oracle x: exact {d['exact']:.4f} max {d['max_ulps']}")
