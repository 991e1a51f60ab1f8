"""mtp_draft_step_noalloc (the draft step on the library's fixed scratch, for
callers that cannot allocate) against mtp_draft_step, through the C ABI: two
calls in a row, the second with a smaller input; tokens, x and log-probability
bit-identical to mtp_draft_step's on the same inputs (the same kernels), and
the tokens against the oracle's logits where the oracle decides the row."""
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
    assert torch.equal(lp_n.view(torch.int32), lp_w.view(torch.int32))
    step = dict(inp)
    step["tokens"] = np.asarray(inp["tokens"])
    xo, _ = combine_tolerance(step, 0.0, wl.eps)
    st = check_lmhead(xo, head_host(head), wl.vocab, 0, tok_n.cpu().numpy(), None, label=f"noalloc {wname}")
    log(f"  tokens {tok_n.tolist()}, decidable {st['decidable']}/{st['rows']}")


def test_noalloc_matches_step_two_calls():
    _one("step_32000x4096", "fp8", 4, 71)
    _one("tiny_step", "bf16", 1, 72)
