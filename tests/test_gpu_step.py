"""GPU parity of the draft step (mtp_draft_step) through the C ABI.

The step computes what mtp_draft_combine followed by mtp_lmhead_argmax
computes; its lm_head blocks apply the final norm to the combine's u. The
concat c and u it leaves in its workspace and its x_out are checked stage by
stage (parity.check_combine_stages), x_out also against the oracle's x within
parity.combine_tolerance; its token against the oracle's lm_head logits of the
oracle's own x (the end-to-end draft) and of the GPU's x, with the tolerance
rule; its log-probability as in tests/test_gpu_lmhead_ext.py. Chained steps
take the previous step's token on the device. Each case runs twice on one
workspace (the counters it leaves must be zero). One family of cases needs no
oracle at all: its token is fixed in closed form by the construction.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity import (DEV, bf16_ulp_diff, check_combine, check_combine_stages, check_lmhead, combine_tolerance,
                    fmt_stages, head_host, log, mtp)

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
    c_g, u_g = m.step_intermediates(ws, b, wl.hidden)
    stg = check_combine_stages(step, 0.0, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(x), label=f"step {wdtype}")
    xo, tol = combine_tolerance(step, 0.0, wl.eps)
    d = check_combine(si.bits(x), xo, tol, label=f"step x {wdtype}")
    hh = head_host(head)
    st = check_lmhead(si.bits(x), hh, wl.vocab, 0, tok.cpu().numpy(), None, label=f"step {wdtype} (gpu x)")
    st_o = check_lmhead(xo, hh, wl.vocab, 0, tok.cpu().numpy(), None, label=f"step {wdtype} (oracle x)")
    log(f"  step {wl.name} {wdtype} b={b}: stages {fmt_stages(stg)}; x vs oracle x exact {d['exact']:.4f}; "
        f"decidable rows {st_o['decidable']}/{st_o['rows']} (oracle x), {st['decidable']}/{st['rows']} (gpu x)")
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


@pytest.mark.parametrize("b", [1, 4])
def test_step_matches_two_launches(b):
    """Same inputs through mtp_draft_combine + mtp_lmhead_argmax: u is the same
    bits (the same combine kernel), x within one unit (the final norm's sum of
    squares is reduced over a different block shape), and the tokens agree
    wherever the oracle decides the row."""
    m = mtp()
    wl = si.WORKLOADS["step_32000x4096"]
    ws = m.zeroed_workspace(m.mtp_draft_step_workspace_bytes(b, wl.hidden), DEV)
    inp, head, tok, x = run_step(wl, 31, "bf16", b, ws=ws)
    wc = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, wl.hidden), DEV)
    x2 = m.draft_combine(inp["embed"], inp["tokens"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"],
                         inp["gamma_f"], eps=wl.eps, ws=wc)
    tok2 = m.lmhead_argmax(x2, head)
    torch.cuda.synchronize()
    _, u1 = m.step_intermediates(ws, b, wl.hidden)
    _, u2 = m.combine_intermediates(wc, b, wl.hidden)
    assert torch.equal(u1.view(torch.int16), u2.view(torch.int16))
    d = bf16_ulp_diff(si.bits(x), si.bits(x2))
    log(f"  step vs two launches: x max {int(d.max())} ulps, tokens {tok.tolist()} {tok2.tolist()}")
    assert d.max() <= 1
    step = dict(inp)
    step["tokens"] = np.asarray(inp["tokens"])
    xo, _ = combine_tolerance(step, 0.0, wl.eps)
    hh = head_host(head)
    L, tau = oracle.lmhead_logits(xo, "bf16", hh[1], with_tau=True)
    for bi in range(b):
        i1 = oracle.argmax(L[bi])
        others = np.delete(L[bi] + tau[bi], i1)
        if others.max() < L[bi, i1] - tau[bi, i1]:
            assert int(tok[bi]) == int(tok2[bi]) == i1, (bi, int(tok[bi]), int(tok2[bi]), i1)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "nvfp4"])
def test_step_154880x4096(wdtype):
    log(f"step 154880x4096 {wdtype}")
    run_step(si.WORKLOADS["step_154880x4096"], 41, wdtype, 1, with_lp=True)


def test_step_154880x4096_fp8_b8():
    log("step 154880x4096 fp8 b=8")
    run_step(si.WORKLOADS["step_154880x4096"], 42, "fp8", 8)


def test_step_h8192_b4():
    from dataclasses import replace

    wl = replace(si.WORKLOADS["step_32000x4096"], hidden=8192, vocab=6000)
    run_step(wl, 43, "bf16", 4)


@pytest.mark.parametrize("h,wdtype,b", [(5120, "nvfp4", 1), (5120, "nvfp4", 4), (5120, "fp8", 6), (2064, "bf16", 3),
                                     (2064, "fp8", 1)])
def test_step_hidden_off_the_grid(h, wdtype, b):
    """Hidden sizes off the 4,096 grid: 5,120 (the width of the 131,072 x 5,120
    head: fc rows of a pass and a quarter, and from b = 2 a combine that stays
    on the VALU form, 320 tiles of 16 rows being more than one per CU) and
    2,064 (ragged fc rows and ragged lm_head passes)."""
    from dataclasses import replace

    log(f"step h={h} {wdtype} b={b}")
    wl = replace(si.WORKLOADS["step_32000x4096"], hidden=h, vocab=3001)
    run_step(wl, 44 + b, wdtype, b)


def _draw_step(rng):
    """One draft-step shape within the header's limits: format, vocab, h (a
    multiple of 16, of 256 for NVFP4), b with b (4h + 16) <= 131584."""
    wdtype = str(rng.choice(["bf16", "fp8", "nvfp4"]))
    h = 256 * int(rng.integers(1, 33)) if wdtype == "nvfp4" else 16 * int(rng.integers(1, 513))
    b = int(rng.integers(1, min(8, 131584 // (4 * h + 16)) + 1))
    vocab = int(rng.integers(1, 5001))
    return wdtype, vocab, h, b


RANDOM_STEPS = [_draw_step(np.random.default_rng(9500 + i)) for i in range(10)]


@pytest.mark.parametrize("case", range(len(RANDOM_STEPS)))
def test_step_random_shapes(case):
    """Seeded random draft-step shapes (combine form, lm_head form, ragged fc
    rows and passes); each case logs its draw."""
    from dataclasses import replace

    wdtype, vocab, h, b = RANDOM_STEPS[case]
    log(f"step random #{case}: {wdtype} V={vocab} h={h} b={b}")
    wl = replace(si.WORKLOADS["step_32000x4096"], hidden=h, vocab=vocab)
    run_step(wl, 9600 + case, wdtype, b)


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


@pytest.mark.parametrize("wname,wdtype,b", [("step_32000x4096", "bf16", 2), ("tiny_step", "nvfp4", 1),
                                            ("step_32000x4096", "fp8", 8)])
def test_chained_steps_in_a_hip_graph(wname, wdtype, b):
    """Four chained drafts (each taking the previous draft's token on the
    device, with log-probability and chain confidence) captured once into a
    HIP graph through torch.cuda.graph and replayed three times, with eager
    work of its own (another draft on other inputs) and a host
    synchronization between replays: every replay's tokens, x, log-
    probabilities and confidence equal the eager chain's bit for bit. The
    library enqueues only kernels (no memset nodes, no host synchronization),
    and each call leaves its workspace counters at zero, so a replay needs no
    reset."""
    from dataclasses import replace

    m = mtp()
    K = 4
    wl = replace(si.WORKLOADS[wname], batch=b)
    inp = si.step_inputs(wl, 52, device=DEV)
    head = m.quantize_head(si.lm_weight(wl, 52, device=DEV), wdtype)
    ws = m.zeroed_workspace(m.mtp_draft_step_workspace_bytes(b, wl.hidden), DEV)
    ids = [torch.as_tensor(inp["tokens"], dtype=torch.int32).to(DEV)] + \
          [torch.zeros(b, dtype=torch.int32, device=DEV) for _ in range(K)]
    xs = [torch.zeros((b, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in range(K)]
    lps = [torch.zeros(b, dtype=torch.float32, device=DEV) for _ in range(K)]
    conf = torch.ones(b, dtype=torch.float32, device=DEV)

    def chain():
        for i in range(K):
            m.mtp_draft_step(inp["embed"], ids[i], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"],
                             inp["gamma_f"], wl.eps, 0.0, head, 0, ids[i + 1], xs[i], lps[i], conf, ws)

    def reset():
        for t in ids[1:] + xs + lps:
            t.zero_()
        conf.fill_(1.0)

    def snapshot():
        return ([t.clone() for t in ids[1:]], [t.view(torch.int16).clone() for t in xs],
                [t.view(torch.int32).clone() for t in lps], conf.view(torch.int32).clone())

    chain()
    torch.cuda.synchronize()
    ref = snapshot()
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    other = si.step_inputs(wl, 53, device=DEV)
    for rep in range(3):
        # eager work of the program's own between replays, then a fresh start
        t2 = m.draft_step(other["embed"], other["tokens"], other["hidden"], other["gamma_e"], other["gamma_h"],
                          other["fc"], other["gamma_f"], head, eps=wl.eps)
        torch.cuda.synchronize()
        assert t2.shape == (b,)
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for i in range(K):
            assert torch.equal(got[0][i], ref[0][i]), (rep, i, "token")
            assert torch.equal(got[1][i], ref[1][i]), (rep, i, "x")
            assert torch.equal(got[2][i], ref[2][i]), (rep, i, "log-probability")
        assert torch.equal(got[3], ref[3]), (rep, "confidence")
        assert int(ws[:4].view(torch.int32).cpu()[0]) == 0
    log(f"  graph chain {wname} {wdtype} b={b}: tokens {[t.cpu().tolist() for t in ref[0]]}")


def test_helpers_on_a_side_stream():
    """The helpers given a stream other than the current one allocate, zero-fill
    and launch on it: results against the oracle, with the current stream kept
    busy meanwhile (a long unrelated fill) so nothing is ordered by accident."""
    m = mtp()
    wl = si.WORKLOADS["step_32000x4096"]
    inp = si.step_inputs(wl, 61, device=DEV)
    head = m.quantize_head(si.lm_weight(wl, 61, device=DEV), "fp8")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    busy = torch.empty(1 << 28, dtype=torch.float32, device=DEV)
    busy.fill_(1.0)  # on the current stream
    tok, x = m.draft_step(inp["embed"], inp["tokens"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"],
                          inp["gamma_f"], head, eps=wl.eps, with_x=True, stream=side)
    tok2 = m.lmhead_argmax(x, head, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    step = dict(inp)
    step["tokens"] = np.asarray(inp["tokens"])
    xo, tol = combine_tolerance(step, 0.0, wl.eps)
    check_combine(si.bits(x), xo, tol, label="side stream x")
    hh = head_host(head)
    check_lmhead(xo, hh, wl.vocab, 0, tok.cpu().numpy(), None, label="side stream step")
    check_lmhead(si.bits(x), hh, wl.vocab, 0, tok2.cpu().numpy(), None, label="side stream lm_head")
    log(f"  side stream: tokens {tok.tolist()} {tok2.tolist()}")


@pytest.mark.parametrize("wdtype,b", [("bf16", 1), ("bf16", 8), ("fp8", 1), ("fp8", 6), ("nvfp4", 1),
                                      ("nvfp4", 8)])
def test_step_closed_form_token(wdtype, b):
    """A draft whose token is known without the oracle: each hidden row has one
    large planted element, every embedding row one at another place, fc = [0 | I]
    keeps only the normalized hidden half of the concat, the gammas are 1, and
    the head (40,000 × 4,096) holds each unit vector e_i in its own random row
    among rows of small noise. Then x peaks where the hidden row does, and the
    token is the row holding that unit vector."""
    log(f"step closed form {wdtype} b={b}")
    m = mtp()
    h, n, V = 4096, 40000, 512
    g = torch.Generator().manual_seed(77 + b)
    rng = np.random.default_rng(77 + b)
    peaks = rng.choice(np.setdiff1d(np.arange(h - 1), [11]), b - 1, replace=False).tolist() + [h - 1]
    E = torch.randn(V, h, generator=g) * 0.05
    E[:, 11] = 4.0
    Hd = torch.randn(b, h, generator=g) * 0.05
    Hd[torch.arange(b), torch.tensor(peaks)] = 4.0
    fc = torch.zeros(h, 2 * h)
    fc[torch.arange(h), h + torch.arange(h)] = 1.0
    unit_rows = rng.choice(n, h, replace=False)  # row unit_rows[i] is e_i
    W = torch.randn(n, h, generator=g) * 0.01
    W[torch.from_numpy(unit_rows)] = torch.eye(h)
    one = torch.ones(h, dtype=torch.bfloat16, device=DEV)
    bf = lambda t: t.to(torch.bfloat16).to(DEV)
    head = m.quantize_head(bf(W), wdtype)
    toks = rng.integers(0, V, b).astype(np.int32)
    tok, x = m.draft_step(bf(E), toks, bf(Hd), one, one, bf(fc), one, head, eps=1e-6, with_x=True)
    torch.cuda.synchronize()
    want = [int(unit_rows[p]) for p in peaks]
    assert x.float().argmax(dim=1).cpu().tolist() == peaks
    assert tok.cpu().tolist() == want, (tok.cpu().tolist(), want)


def test_step_host_threads_on_their_own_streams():
    """Three host threads, each on its own stream with its own workspaces, run
    draft steps (all three head formats, b = 1 and 5, so both combine forms
    and both lm_head forms) at once: every step gives the token and x of the
    same step run alone."""
    import threading

    from dataclasses import replace

    m = mtp()
    wl = si.WORKLOADS["step_32000x4096"]
    heads = {wd: m.quantize_head(si.lm_weight(wl, 90 + i, device=DEV), wd)
             for i, wd in enumerate(("bf16", "fp8", "nvfp4"))}
    inps = {b: si.step_inputs(replace(wl, batch=b), 95 + b, device=DEV) for b in (1, 5)}
    jobs = [(wd, b) for wd in heads for b in (1, 5)]

    def run(wd, b, stream=None):
        i = inps[b]
        return m.draft_step(i["embed"], i["tokens"], i["hidden"], i["gamma_e"], i["gamma_h"], i["fc"], i["gamma_f"],
                            heads[wd], eps=wl.eps, with_x=True, stream=stream)

    ref = {j: tuple(t.clone() for t in run(*j)) for j in jobs}
    torch.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            outs = [(jobs[(k + it) % len(jobs)], run(*jobs[(k + it) % len(jobs)], stream=s)) for it in range(8)]
            s.synchronize()
            for key, (tok, x) in outs:
                if not (torch.equal(tok, ref[key][0]) and torch.equal(x.view(torch.int16), ref[key][1].view(torch.int16))):
                    errors.append((k, key))
        except Exception as e:  # reported below; a thread's exception is otherwise lost
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
