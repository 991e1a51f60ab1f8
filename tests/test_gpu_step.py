"""GPU parity of the draft step (mtp_draft_step) through the C ABI.

The step computes what mtp_draft_combine followed by mtp_lmhead_argmax
computes; its lm_head blocks apply the final norm to the combine's u. Its x_out is checked against the oracle's
combine within parity.combine_tolerance; its token against the oracle's
lm_head logits of the GPU's own x with the tolerance rule; its log-probability
as in tests/test_gpu_lmhead_ext.py. Chained steps take the previous step's
token on the device. Each case runs twice on one workspace (the counters it
leaves must be zero).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity import DEV, check_combine, check_lmhead, combine_tolerance, head_host, log, mtp

pytestmark = pytest.mark.gpu


def run_step(wl, seed, wdtype, b, with_lp=False, tokens=None, ws=None):
    m = mtp()
    from dataclasses import replace

    wl = replace(wl, batch=b)
    inp = si.step_inputs(wl, seed, device=DEV)
    if tokens is not None:
        inp["tokens"] = tokens
    head = m.quantize_head(si.lm_weight(wl, seed, device=DEV), wdtype)
    if ws is None:
        ws = m.zeroed_workspace(m.mtp_draft_step_workspace_bytes(b, wl.hidden), DEV)
    outs = []
    for rep in range(2):
        r = m.draft_step(inp["embed"], inp["tokens"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"],
                         inp["gamma_f"], head, eps=wl.eps, with_x=True, with_logprob=with_lp, ws=ws)
        outs.append(r)
    torch.cuda.synchronize()
    tok, x = outs[0][0], outs[0][1]
    assert torch.equal(outs[1][0], tok) and torch.equal(outs[1][1].view(torch.int16), x.view(torch.int16))
    assert int(ws[:4].view(torch.int32).cpu()[0]) == 0
    step = dict(inp)
    step["tokens"] = np.asarray(inp["tokens"]) if not isinstance(inp["tokens"], torch.Tensor) else \
        inp["tokens"].cpu().numpy()
    xo, tol = combine_tolerance(step, 0.0, wl.eps)
    d = check_combine(si.bits(x), xo, tol, label=f"step x {wdtype}")
    st = check_lmhead(si.bits(x), head_host(head), wl.vocab, 0, tok.cpu().numpy(), None, label=f"step {wdtype}")
    log(f"  step {wl.name} {wdtype} b={b}: x exact {d['exact']:.4f}, decidable {st['decidable']}/{st['rows']}")
    if with_lp:
        name, w, s, g = head_host(head)
        L, tau = oracle.lmhead_logits(si.bits(x), name, w, s, g, with_tau=True)
        lp = outs[0][2].cpu().numpy()
        for bi in range(b):
            ref = oracle.top1_logprob(L[bi])
            assert abs(lp[bi] - ref) <= 2 * tau[bi].max() + 2e-4, (bi, lp[bi], ref)
    return inp, head, tok, x


CASES = [
    ("tiny_step", "bf16", 1), ("tiny_step", "bf16", 3), ("tiny_step", "fp8", 8), ("tiny_step", "nvfp4", 2),
    ("step_32000x4096", "bf16", 1), ("step_32000x4096", "fp8", 4), ("step_32000x4096", "nvfp4", 8),
    ("step_32000x4096", "bf16", 5),
]


@pytest.mark.parametrize("wname,wdtype,b", CASES)
def test_step(wname, wdtype, b):
    log(f"step {wname} {wdtype} b={b}")
    run_step(si.WORKLOADS[wname], 20 + b, wdtype, b, with_lp=(b % 2 == 1))


def test_step_matches_two_launches():
    """Same inputs through mtp_draft_combine + mtp_lmhead_argmax: the tokens agree
    wherever the oracle decides them, and x agrees within the combine bound."""
    m = mtp()
    wl = si.WORKLOADS["step_32000x4096"]
    inp, head, tok, x = run_step(wl, 31, "bf16", 1)
    x2 = m.draft_combine(inp["embed"], inp["tokens"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"],
                         inp["gamma_f"], eps=wl.eps)
    tok2 = m.lmhead_argmax(x2, head)
    torch.cuda.synchronize()
    from parity import bf16_ulp_diff

    d = bf16_ulp_diff(si.bits(x), si.bits(x2))
    log(f"  step vs two launches: x max {int(d.max())} ulps, tokens {tok.tolist()} {tok2.tolist()}")
    assert d.max() <= 2


def test_step_154880x4096_nvfp4_and_bf16():
    for wdtype in ("bf16", "nvfp4"):
        log(f"step 154880x4096 {wdtype}")
        run_step(si.WORKLOADS["step_154880x4096"], 41, wdtype, 1, with_lp=True)


def test_step_h8192_b4():
    from dataclasses import replace

    wl = replace(si.WORKLOADS["step_32000x4096"], hidden=8192, vocab=6000)
    run_step(wl, 43, "bf16", 4)


def test_chained_steps_device_tokens():
    """Four steps, each taking the previous step's token on the device, one host
    synchronization at the end; each step against the oracle given its inputs."""
    m = mtp()
    wl = si.WORKLOADS["tiny_step"]
    inp = si.step_inputs(wl, 50, device=DEV)
    head = m.quantize_head(si.lm_weight(wl, 50, device=DEV), "bf16")
    ws = m.zeroed_workspace(m.mtp_draft_step_workspace_bytes(1, wl.hidden), DEV)
    conf = torch.ones(1, dtype=torch.float32, device=DEV)
    ids = [torch.as_tensor(inp["tokens"], dtype=torch.int32).to(DEV)]
    xs, lps = [], []
    for i in range(4):
        tok, x, lp = m.draft_step(inp["embed"], ids[i], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"],
                                  inp["gamma_f"], head, eps=wl.eps, with_x=True, with_logprob=True, conf=conf, ws=ws)
        ids.append(tok)
        xs.append(x)
        lps.append(lp)
    torch.cuda.synchronize()
    for i in range(4):
        step = dict(inp)
        step["tokens"] = ids[i].cpu().numpy()
        xo, tol = combine_tolerance(step, 0.0, wl.eps)
        check_combine(si.bits(xs[i]), xo, tol, label=f"chained step {i}")
        check_lmhead(si.bits(xs[i]), head_host(head), wl.vocab, 0, ids[i + 1].cpu().numpy(), None,
                     label=f"chained step {i}")
    assert float(conf.cpu()[0]) == pytest.approx(min(float(np.exp(l.cpu()[0])) for l in lps), rel=2e-6)
    log(f"  chain {[int(t.cpu()[0]) for t in ids]}")
