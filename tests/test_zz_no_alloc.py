"""mtp_draft_step_noalloc (the draft step on the library's fixed scratch, for
callers that cannot allocate) against mtp_draft_step, through the C ABI: two
calls in a row, the second with a smaller input; tokens and x bit-identical to
mtp_draft_step's on the same inputs (the same kernels), the log-probability
within 2e-5 (its sums follow the run-time order of the row groups), and the
tokens against the oracle's logits where the oracle decides the row."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from parity import DEV, check_lmhead, combine_tolerance, head_host, log, mtp

pytestmark = pytest.mark.gpu


def _one(wname, wdtype, b, seed):
    m = mtp()
    wl = replace(si.WORKLOADS[wname], batch=b)
    log(f"noalloc {wname} {wdtype} b={b}")
    inp = si.step_inputs(wl, seed, device=DEV)
    head = m.quantize_head(si.lm_weight(wl, seed, device=DEV), wdtype)
    args = (inp["embed"], inp["tokens"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"], inp["gamma_f"],
            head)
    tok_n, x_n, lp_n = m.draft_step(*args, eps=wl.eps, with_x=True, with_logprob=True, noalloc=True)
    tok_w, x_w, lp_w = m.draft_step(*args, eps=wl.eps, with_x=True, with_logprob=True)
    torch.cuda.synchronize()
    assert torch.equal(tok_n, tok_w), (tok_n.tolist(), tok_w.tolist())
    assert torch.equal(x_n.view(torch.int16), x_w.view(torch.int16))
    # the log-probability's online softmax sums run in the order the waves take
    # row groups (a run-time counter), so two calls agree to rounding: -log S
    # moves by the relative change of S, a few f32 ulps of each block's sum
    assert torch.allclose(lp_n, lp_w, rtol=0.0, atol=2e-5), (lp_n.tolist(), lp_w.tolist())
    step = dict(inp)
    step["tokens"] = np.asarray(inp["tokens"])
    xo, _ = combine_tolerance(step, 0.0, wl.eps)
    st = check_lmhead(xo, head_host(head), wl.vocab, 0, tok_n.cpu().numpy(), None, label=f"noalloc {wname}")
    log(f"  tokens {tok_n.tolist()}, decidable {st['decidable']}/{st['rows']}")


def test_noalloc_matches_step_two_calls():
    _one("step_32000x4096", "fp8", 4, 71)
    _one("tiny_step", "bf16", 1, 72)
