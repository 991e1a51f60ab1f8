"""GPU parity of the combine variants through the C ABI:

- mtp_draft_combine_dev: token ids read on the device. Bit-identical to
  mtp_draft_combine with the same ids; out-of-range ids clamp; K drafts
  chained on the device (each draft's token feeds the next draft's embedding
  gather, no host synchronization in between), each draft checked against the
  oracle given the ids and hidden it was fed.
- mtp_draft_combine_q: the fc quantized to FP8 / NVFP4 on the GPU (codes
  checked byte-exact against the oracle quantizers), x against the oracle's
  quantized-fc combine within the combine bound taken over the dequantized fc.
- mtp_draft_combine_split: two [h, h] projections, x against the oracle's split
  combine within a bound that adds the two branch roundings
  (parity.combine_split_tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity import (DEV, check_combine, check_combine_stages, check_lmhead, check_quantized, combine_q_tolerance,
                    combine_split_tolerance, combine_tolerance, fmt_stages, head_host, log, mtp)

pytestmark = pytest.mark.gpu


def combine_args(inp):
    return inp["embed"], inp["hidden"], inp["gamma_e"], inp["gamma_h"], inp["fc"], inp["gamma_f"]


@pytest.mark.parametrize("wname,b", [("tiny_step", 1), ("tiny_step", 5), ("step_32000x4096", 3)])
def test_combine_dev_equals_host_ids(wname, b):
    m = mtp()
    from dataclasses import replace

    wl = replace(si.WORKLOADS[wname], batch=b)
    inp = si.step_inputs(wl, 3, device=DEV)
    E, H, ge, gh, fc, gf = combine_args(inp)
    x_host = m.draft_combine(E, inp["tokens"], H, ge, gh, fc, gf, eps=wl.eps)
    tok_dev = torch.as_tensor(inp["tokens"], dtype=torch.int32).to(DEV)
    ws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, wl.hidden), DEV)
    x_dev = torch.empty_like(x_host)
    m.mtp_draft_combine_dev(E, tok_dev, H, ge, gh, fc, gf, wl.eps, 0.0, x_dev, ws)
    torch.cuda.synchronize()
    assert torch.equal(x_dev.view(torch.int16), x_host.view(torch.int16))
    # out-of-range ids clamp into [0, vocab)
    bad = torch.tensor([-5, wl.vocab + 7, wl.vocab - 1, 0, 2 ** 31 - 1][:b] + [1] * max(0, b - 5),
                       dtype=torch.int32).to(DEV)
    clamped = np.clip(bad.cpu().numpy().astype(np.int64), 0, wl.vocab - 1).astype(np.int32)
    m.mtp_draft_combine_dev(E, bad, H, ge, gh, fc, gf, wl.eps, 0.0, x_dev, ws)
    x_ref = m.draft_combine(E, clamped, H, ge, gh, fc, gf, eps=wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(x_dev.view(torch.int16), x_ref.view(torch.int16))


@pytest.mark.parametrize("wname,b,k", [("tiny_step", 1, 4), ("tiny_step", 3, 4), ("step_32000x4096", 1, 3)])
def test_device_chained_drafts(wname, b, k):
    """Draft i: combine(ids_i on the device, hidden_i) -> lm_head -> ids_{i+1}
    left on the device; hidden_{i+1} = x_i (identity body). K drafts, one host
    synchronization at the end, then every draft against the oracle given the
    ids and hidden it was fed."""
    m = mtp()
    from dataclasses import replace

    wl = replace(si.WORKLOADS[wname], batch=b)
    inp = si.step_inputs(wl, 4, device=DEV)
    E, H, ge, gh, fc, gf = combine_args(inp)
    head = m.quantize_head(si.lm_weight(wl, 4, device=DEV), "bf16")
    ws_c = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, wl.hidden), DEV)
    ws_l = m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(wl.vocab, wl.hidden, b, 0), DEV)
    ids = [torch.as_tensor(inp["tokens"], dtype=torch.int32).to(DEV)]
    hid = [H]
    xs, lgs = [], []
    for i in range(k):
        x = torch.empty((b, wl.hidden), dtype=torch.bfloat16, device=DEV)
        m.mtp_draft_combine_dev(E, ids[i], hid[i], ge, gh, fc, gf, wl.eps, 0.0, x, ws_c)
        t = torch.empty(b, dtype=torch.int32, device=DEV)
        lg = torch.empty((b, wl.vocab), dtype=torch.float32, device=DEV)
        m.mtp_lmhead_argmax(x, head.wd, head.w, None, None, wl.vocab, 0, t, lg, ws_l)
        ids.append(t)
        hid.append(x)
        xs.append(x)
        lgs.append(lg)
    torch.cuda.synchronize()
    for i in range(k):
        step = dict(inp)
        step["tokens"] = ids[i].cpu().numpy()
        step["hidden"] = hid[i]
        xo, tol = combine_tolerance(step, 0.0, wl.eps)
        check_combine(si.bits(xs[i]), xo, tol, label=f"draft {i}")
        check_lmhead(si.bits(xs[i]), head_host(head), wl.vocab, 0, ids[i + 1].cpu().numpy(), lgs[i].cpu().numpy(),
                     label=f"draft {i}")
    log(f"  chain tokens {[t.cpu().tolist() for t in ids]}")


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("wname,b", [("tiny_step", 1), ("tiny_step", 4), ("step_32000x4096", 1),
                                     ("step_32000x4096", 3)])
def test_combine_quantized_fc(wdtype, wname, b):
    m = mtp()
    from dataclasses import replace

    wl = replace(si.WORKLOADS[wname], batch=b)
    log(f"combine_q {wdtype} {wname} b={b}")
    inp = si.step_inputs(wl, 5 + b, device=DEV)
    E, H, ge, gh, fc, gf = combine_args(inp)
    fq = m.quantize_head(fc, wdtype)  # [h, 2h] through the same quantizers as the head
    torch.cuda.synchronize()
    check_quantized(fq, si.bits(fc))
    _, codes, sc, g = head_host(fq)
    x = torch.empty((b, wl.hidden), dtype=torch.bfloat16, device=DEV)
    ws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, wl.hidden), DEV)
    m.mtp_draft_combine_q(E, inp["tokens"], H, ge, gh, fq.wd, fq.w, fq.scale, fq.gscale, gf, wl.eps, 0.0, x, ws)
    torch.cuda.synchronize()
    c_g, u_g = m.combine_intermediates(ws, b, wl.hidden)
    fcq = ("bf16", None) if wdtype == "bf16" else (wdtype, codes, sc, g)
    stg = check_combine_stages(inp, 0.0, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(x), fc=fcq,
                               label=f"combine_q {wdtype}")
    xo, tol = combine_q_tolerance(inp, wdtype, codes, sc, g, 0.0, wl.eps)
    d = check_combine(si.bits(x), xo, tol, label=f"combine_q {wdtype}")
    log(f"  stages {fmt_stages(stg)}; x vs oracle x: exact {d['exact']:.4f} max {d['max_ulps']} ulps")
    if wdtype == "bf16":  # the BF16 path of combine_q is the plain combine
        x0 = m.draft_combine(E, inp["tokens"], H, ge, gh, fc, gf, eps=wl.eps)
        assert torch.equal(x.view(torch.int16), x0.view(torch.int16))


@pytest.mark.parametrize("wname,b,off", [("tiny_step", 1, 0.0), ("tiny_step", 2, 1.0), ("tiny_step", 7, 0.0),
                                         ("step_32000x4096", 1, 0.0), ("step_32000x4096", 4, 0.0)])
def test_combine_split(wname, b, off):
    m = mtp()
    from dataclasses import replace

    wl = replace(si.WORKLOADS[wname], batch=b)
    log(f"combine_split {wname} b={b} offset={off}")
    inp = si.step_inputs(wl, 9 + b, device=DEV)
    E, H, ge, gh, fc, gf = combine_args(inp)
    h = wl.hidden
    Ep = si.normal_bf16(100 + b, si.TAG_LM, h, h, std=0.02, device=DEV)
    Hp = si.normal_bf16(200 + b, si.TAG_LM, h, h, std=0.02, device=DEV)
    x = torch.empty((b, h), dtype=torch.bfloat16, device=DEV)
    ws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, h), DEV)
    m.mtp_draft_combine_split(E, inp["tokens"], H, ge, gh, Ep, Hp, gf, wl.eps, off, x, ws)
    torch.cuda.synchronize()
    c_g, u_g = m.combine_intermediates(ws, b, h)
    stg = check_combine_stages(inp, off, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(x),
                               split=(si.bits(Ep), si.bits(Hp)), label="combine_split")
    xo, tol = combine_split_tolerance(inp, si.bits(Ep), si.bits(Hp), off, wl.eps)
    d = check_combine(si.bits(x), xo, tol, label="combine_split")
    log(f"  stages {fmt_stages(stg)}; x vs oracle x: exact {d['exact']:.4f} max {d['max_ulps']} ulps")
    assert d["within1ulp"] > 0.9


def _draw_combine(rng):
    """One combine call within the header's limits: variant (BF16 fc, FP8 fc,
    NVFP4 fc, split), h (a multiple of 16; of 128 for the NVFP4 fc), b (wide
    b x h run as several row groups), vocab of the embedding table, gamma
    offset 0 or 1."""
    variant = str(rng.choice(["bf16", "fp8", "nvfp4", "split"]))
    h = 128 * int(rng.integers(1, 65)) if variant == "nvfp4" else 16 * int(rng.integers(1, 513))
    b = int(rng.integers(1, 9))
    vocab = int(rng.integers(1, 3001))
    off = float(rng.integers(0, 2))
    return variant, h, b, vocab, off


RANDOM_COMBINES = [_draw_combine(np.random.default_rng(9700 + i)) for i in range(12)]


@pytest.mark.parametrize("case", range(len(RANDOM_COMBINES)))
def test_combine_variants_random_shapes(case):
    """Seeded random shapes through the combine entry points; each stage
    against the oracle given the GPU's own input to it, x end to end within
    the variant's bound."""
    from dataclasses import replace

    m = mtp()
    variant, h, b, vocab, off = RANDOM_COMBINES[case]
    log(f"combine random #{case}: {variant} h={h} b={b} vocab={vocab} offset={off}")
    wl = replace(si.WORKLOADS["step_32000x4096"], hidden=h, vocab=vocab, batch=b)
    inp = si.step_inputs(wl, 9800 + case, device=DEV)
    E, H, ge, gh, fc, gf = combine_args(inp)
    x = torch.empty((b, h), dtype=torch.bfloat16, device=DEV)
    ws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, h), DEV)
    if variant == "split":
        Ep = si.normal_bf16(9900 + case, si.TAG_LM, h, h, std=0.02, device=DEV)
        Hp = si.normal_bf16(9950 + case, si.TAG_LM, h, h, std=0.02, device=DEV)
        m.mtp_draft_combine_split(E, inp["tokens"], H, ge, gh, Ep, Hp, gf, wl.eps, off, x, ws)
        torch.cuda.synchronize()
        c_g, u_g = m.combine_intermediates(ws, b, h)
        stg = check_combine_stages(inp, off, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(x),
                                   split=(si.bits(Ep), si.bits(Hp)), label="split")
        xo, tol = combine_split_tolerance(inp, si.bits(Ep), si.bits(Hp), off, wl.eps)
    elif variant == "bf16":
        m.mtp_draft_combine(E, inp["tokens"], H, ge, gh, fc, gf, wl.eps, off, x, ws)
        torch.cuda.synchronize()
        c_g, u_g = m.combine_intermediates(ws, b, h)
        stg = check_combine_stages(inp, off, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(x), label="bf16")
        xo, tol = combine_tolerance(inp, off, wl.eps)
    else:
        fq = m.quantize_head(fc, variant)
        torch.cuda.synchronize()
        check_quantized(fq, si.bits(fc))
        _, codes, sc, g = head_host(fq)
        m.mtp_draft_combine_q(E, inp["tokens"], H, ge, gh, fq.wd, fq.w, fq.scale, fq.gscale, gf, wl.eps, off, x, ws)
        torch.cuda.synchronize()
        c_g, u_g = m.combine_intermediates(ws, b, h)
        stg = check_combine_stages(inp, off, wl.eps, si.bits(c_g), si.bits(u_g), si.bits(x),
                                   fc=(variant, codes, sc, g), label=variant)
        xo, tol = combine_q_tolerance(inp, variant, codes, sc, g, off, wl.eps)
    d = check_combine(si.bits(x), xo, tol, label=f"combine random #{case}")
    log(f"  stages {fmt_stages(stg)}; x vs oracle x: exact {d['exact']:.4f} max {d['max_ulps']} ulps")
