"""Helpers for the GPU parity tests: run the HIP path through the C ABI (via the
Python binding) and compare with the oracle on the same seeded inputs.

The comparison rules:
  - codes, scales, tokens that the tolerance decides: bit-exact;
  - logits: |L_gpu - L| <= tau = 1e-3 * sum_i |w^_i x_i| per (row, batch row);
  - argmax: when the oracle's winner i1 beats every other row by more than
    tau[i1] + tau[j], the GPU must return i1; otherwise the GPU's token g must
    satisfy L[i1] - L[g] <= tau[i1] + tau[g]. In every case the GPU token must be
    the lowest index attaining the max of the GPU's own f32 logits.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synthetic_inputs as si

DEV = "cuda:0"


def lm_form(wdtype: str, b: int, h: int) -> str:
    """Which kernel form an lm_head call of this shape takes ('valu' or 'mfma',
    the library's own answer): the two sum in different orders, so rows agree
    bit for bit between calls of the same form and within tau across forms."""
    return mtp().lmhead_kernel_form(b, h, wdtype)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def mtp():
    import mtp_draft_head_02_amd as m

    return m


def head_host(head) -> tuple:
    """(wdtype name, w, scale, gscale) as host numpy arrays for the oracle."""
    name = {0: "bf16", 1: "fp8", 2: "nvfp4"}[head.wd]
    if head.wd == 0:
        return name, si.bits(head.w), None, None
    w = head.w.cpu().numpy()
    s = head.scale.cpu().numpy()
    g = None if head.gscale is None else head.gscale.cpu().numpy()
    return name, w, s, g


def check_quantized(head, W_bits: np.ndarray) -> None:
    """GPU codes/scales == oracle codes/scales, byte for byte."""
    if head.wd == 1:
        c, s = oracle.quantize_fp8(W_bits)
        gc = head.w.cpu().numpy()
        gs = head.scale.cpu().numpy()
        bad_rows = np.nonzero((gc != c).any(axis=1) | (gs.view(np.uint32) != s.view(np.uint32)))[0]
        assert bad_rows.size == 0, f"FP8 mismatch in {bad_rows.size} rows, first {bad_rows[:5]}"
    elif head.wd == 2:
        c, bs, g = oracle.quantize_nvfp4(W_bits)
        assert head.gscale.cpu().numpy().view(np.uint32)[0] == g.view(np.uint32)[0], "global scale"
        gbs = head.scale.cpu().numpy()
        assert np.array_equal(gbs, bs), f"block scales differ in {(gbs != bs).sum()} places"
        gc = head.w.cpu().numpy()
        assert np.array_equal(gc, c), f"codes differ in {(gc != c).sum()} bytes"


def argmax_f32_lowest(v: np.ndarray) -> int:
    """Lowest index of the max of an f32 vector (NaN never wins; all -inf/NaN -> 0)."""
    v = np.asarray(v, dtype=np.float32)
    ok = ~np.isnan(v)
    if not ok.any():
        return 0
    m = v[ok].max()
    if m == -np.inf:
        return 0
    return int(np.flatnonzero(v == m)[0])


def check_lmhead(x_bits, hh, vocab, mvs, tok_gpu, logits_gpu, label="", threads=None) -> dict:
    """Compare one GPU lm_head call with the oracle. Returns stats."""
    name, w, s, g = hh
    n_eff = oracle.effective_vocab(vocab, mvs)
    L, tau = oracle.lmhead_logits(x_bits, name, w, s, g, n_eff=n_eff, with_tau=True, threads=threads)
    b = x_bits.shape[0]
    stats = {"decidable": 0, "rows": b}
    tok_gpu = np.asarray(tok_gpu)
    if logits_gpu is not None:
        lg = np.asarray(logits_gpu, dtype=np.float64)
        assert lg.shape == L.shape
        err = np.abs(lg - L)
        bad = err > tau
        assert not bad.any(), (f"{label}: {bad.sum()} logits outside tau; worst "
                               f"{np.unravel_index(np.argmax(err - tau), err.shape)} err {err.max()}")
        for bi in range(b):
            assert tok_gpu[bi] == argmax_f32_lowest(logits_gpu[bi]), f"{label}: token vs own logits, row {bi}"
    for bi in range(b):
        i1 = oracle.argmax(L[bi])
        gt = int(tok_gpu[bi])
        assert 0 <= gt < n_eff, f"{label}: token {gt} out of range"
        others = np.delete(L[bi] + tau[bi], i1)
        decidable = others.size == 0 or others.max() < L[bi, i1] - tau[bi, i1]
        if decidable:
            stats["decidable"] += 1
            assert gt == i1, f"{label}: row {bi} decidable, oracle {i1}, gpu {gt}"
        else:
            assert L[bi, i1] - L[bi, gt] <= tau[bi, i1] + tau[bi, gt], f"{label}: row {bi} gpu {gt} not within tau"
    return stats


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in BF16 units in the last place (same-sign finite values; ordered integer map)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)

    return np.abs(ordered(a_bits) - ordered(b_bits))


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 values at |v| (2^(e-7) for normals; the subnormal spacing below)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, np.exp2(e - 7), 2.0 ** -133)


def embed_rows(inp: dict):
    """(the gathered embedding rows as host bits, tokens 0..b-1 into them): the
    oracle's combine gets the same vectors without the whole table on the host."""
    tok = torch.as_tensor(np.asarray(inp["tokens"], dtype=np.int64), device=inp["embed"].device)
    b = int(tok.numel())
    return si.bits(inp["embed"][tok]), np.arange(b, dtype=np.int32)


def combine_tolerance(inp: dict, gamma_offset: float, eps: float):
    """Oracle x and a per-element bound for the GPU's x.

    x_j = bf16(u_j * r * (g_j + o)) with u = bf16(W_fc . c). The GPU sums in f32
    and the oracle in double, so c can round differently in a few elements; that
    moves u_j by an absolute amount bounded, like any GEMV here, by
    tau_j = 1e-3 * sum_i |W_ji c_i| (the logit tolerance applied to fc), which
    is many BF16 ulps when u_j is near zero. Bound:
      |x_gpu_j - x_j| <= r |g_j + o| (tau_j + ulp(u_j)) + 2 ulp(x_j).
    """
    rows, toks = embed_rows(inp)
    xo, co, uo = oracle.draft_combine(rows, toks, si.bits(inp["hidden"]),
                                      si.bits(inp["gamma_e"]), si.bits(inp["gamma_h"]), si.bits(inp["fc"]),
                                      si.bits(inp["gamma_f"]), eps, gamma_offset, intermediates=True)
    _, tau_fc = oracle.lmhead_logits(co, "bf16", si.bits(inp["fc"]), with_tau=True)
    u = oracle.bf16_decode_array(uo)
    r = 1.0 / np.sqrt((u * u).mean(axis=1, keepdims=True) + np.float64(np.float32(eps)))
    g = np.abs(oracle.bf16_decode_array(si.bits(inp["gamma_f"])) + gamma_offset)[None, :]
    x = oracle.bf16_decode_array(xo)
    tol = r * g * (tau_fc + bf16_ulp(u)) + 2 * bf16_ulp(x)
    return xo, tol


def check_combine(x_gpu_bits: np.ndarray, xo: np.ndarray, tol: np.ndarray, label="") -> dict:
    xg = oracle.bf16_decode_array(x_gpu_bits)
    xv = oracle.bf16_decode_array(xo)
    err = np.abs(xg - xv)
    bad = err > tol
    assert not bad.any(), (f"{label}: {bad.sum()} combine outputs outside the bound; worst at "
                           f"{np.unravel_index(np.argmax(err - tol), err.shape)}")
    d = bf16_ulp_diff(x_gpu_bits, xo)
    return {"exact": float((d == 0).mean()), "within1ulp": float((d <= 1).mean()), "max_ulps": int(d.max())}


def _x_bound(u, x, gamma_f_bits, gamma_offset, eps, u_err):
    r = 1.0 / np.sqrt((u * u).mean(axis=1, keepdims=True) + np.float64(np.float32(eps)))
    g = np.abs(oracle.bf16_decode_array(gamma_f_bits) + gamma_offset)[None, :]
    return r * g * u_err + 2 * bf16_ulp(x)


def combine_q_tolerance(inp: dict, wdtype: str, codes, scale, gscale, gamma_offset: float, eps: float):
    """Oracle x of the quantized-fc combine and the bound of combine_tolerance
    with tau_fc taken over the dequantized fc."""
    _, co, _ = oracle.draft_combine(si.bits(inp["embed"]), inp["tokens"], si.bits(inp["hidden"]),
                                    si.bits(inp["gamma_e"]), si.bits(inp["gamma_h"]), si.bits(inp["fc"]),
                                    si.bits(inp["gamma_f"]), eps, gamma_offset, intermediates=True)
    xo, uo = oracle.draft_combine_q(si.bits(inp["embed"]), inp["tokens"], si.bits(inp["hidden"]),
                                    si.bits(inp["gamma_e"]), si.bits(inp["gamma_h"]), wdtype, codes, scale, gscale,
                                    si.bits(inp["gamma_f"]), eps, gamma_offset, with_u=True)
    _, tau_fc = oracle.lmhead_logits(co, wdtype, codes, scale, gscale, with_tau=True)
    u = oracle.bf16_decode_array(uo)
    tol = _x_bound(u, oracle.bf16_decode_array(xo), si.bits(inp["gamma_f"]), gamma_offset, eps, tau_fc + bf16_ulp(u))
    return xo, tol


def combine_split_tolerance(inp: dict, e_proj_bits, h_proj_bits, gamma_offset: float, eps: float):
    """Oracle x of the split combine and a bound: each branch's f32 sum is within
    its tau of the exact one, then three BF16 roundings (each branch, the sum)
    can each land one unit apart:
      |u_gpu - u| <= tau_e + tau_h + ulp(ue) + ulp(uh) + ulp(u)."""
    _, co, _ = oracle.draft_combine(si.bits(inp["embed"]), inp["tokens"], si.bits(inp["hidden"]),
                                    si.bits(inp["gamma_e"]), si.bits(inp["gamma_h"]), si.bits(inp["fc"]),
                                    si.bits(inp["gamma_f"]), eps, gamma_offset, intermediates=True)
    h = e_proj_bits.shape[0]
    se, tau_e = oracle.lmhead_logits(np.ascontiguousarray(co[:, :h]), "bf16", e_proj_bits, with_tau=True)
    sh, tau_h = oracle.lmhead_logits(np.ascontiguousarray(co[:, h:]), "bf16", h_proj_bits, with_tau=True)
    xo, uo = oracle.draft_combine_split(si.bits(inp["embed"]), inp["tokens"], si.bits(inp["hidden"]),
                                        si.bits(inp["gamma_e"]), si.bits(inp["gamma_h"]), e_proj_bits, h_proj_bits,
                                        si.bits(inp["gamma_f"]), eps, gamma_offset, with_u=True)
    u = oracle.bf16_decode_array(uo)
    err = tau_e + tau_h + bf16_ulp(se) + bf16_ulp(sh) + bf16_ulp(u)
    tol = _x_bound(u, oracle.bf16_decode_array(xo), si.bits(inp["gamma_f"]), gamma_offset, eps, err)
    return xo, tol


# -------------------------------------------------- combine, stage by stage ----
#
# The combine and the draft step leave the concat c [b, 2h] and the fc output
# u [b, h] in their workspaces (include/mtp_draft.h). Each stage is checked
# against the oracle given the GPU's own input to that stage, so a rounding
# point dropped or added anywhere shows up where it happens:
#   c: the oracle's c (same inputs);
#   u: bf16 of the fc row times the GPU's c, summed in double;
#   x: the oracle's RMSNorm of the GPU's u.
# The GPU sums in f32 where the oracle sums in double, so an element can land
# one BF16 unit off where the exact value sits within the f32 error of a
# rounding midpoint; that is rare (a few per 10^4 for c and x, about 10^-3 for
# u), so at most STAGE_C_X_OFF / STAGE_U_OFF of the elements (and at least a
# handful) may be off, each by at most one unit, except that u elements whose
# exact sum is so near zero that the f32 error bound (gamma_k * sum |w c|,
# gamma_k = (k / 64 + 48) 2^-24 for the k-term sums done per lane, then
# across lanes and waves) exceeds an ulp are held to that bound instead. A
# dropped BF16 rounding of c or u moves about half the elements by one unit.

STAGE_C_X_OFF = 0.005
STAGE_U_OFF = 0.01


def bf16_encode_array(v) -> np.ndarray:
    """The oracle's round-to-nearest-even BF16 encoder over an array of doubles."""
    v = np.asarray(v, dtype=np.float64)
    return np.vectorize(oracle.bf16_encode, otypes=[np.uint16])(v).reshape(v.shape)


def _stage(label, got_bits, want_bits, frac, extra_ok=None) -> dict:
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    want_bits = np.asarray(want_bits, dtype=np.uint16)
    d = bf16_ulp_diff(got_bits, want_bits)
    far = d > 1
    if extra_ok is not None:
        far &= ~extra_ok
    assert not far.any(), (f"{label}: {int(far.sum())} elements more than one BF16 unit off, first at "
                           f"{np.argwhere(far)[0]}")
    off = int((d != 0).sum())
    allowed = max(4, int(frac * d.size))
    assert off <= allowed, f"{label}: {off} of {d.size} elements off by one unit (at most {allowed})"
    return {"n": int(d.size), "off": off, "max_ulps": int(d.max()) if d.size else 0}


def check_combine_stages(inp: dict, gamma_offset: float, eps: float, c_gpu, u_gpu, x_gpu, fc=("bf16", None),
                         split=None, label="") -> dict:
    """Stage-by-stage parity of one combine. c_gpu, u_gpu, x_gpu: BF16 bit
    arrays [b, 2h], [b, h], [b, h] from the GPU. fc: (wdtype, codes, scale,
    gscale) of a quantized fc, or ("bf16", None) for inp["fc"]; split:
    (e_proj bits, h_proj bits) for the split combiner."""
    c_gpu = np.asarray(c_gpu, dtype=np.uint16)
    u_gpu = np.asarray(u_gpu, dtype=np.uint16)
    x_gpu = np.asarray(x_gpu, dtype=np.uint16)
    b, h = u_gpu.shape
    rows, toks = embed_rows(inp)
    _, co, _ = oracle.draft_combine(rows, toks, si.bits(inp["hidden"]),
                                    si.bits(inp["gamma_e"]), si.bits(inp["gamma_h"]), si.bits(inp["fc"]),
                                    si.bits(inp["gamma_f"]), eps, gamma_offset, intermediates=True)
    st = {"c": _stage(f"{label} c", c_gpu, co, STAGE_C_X_OFF)}
    u = oracle.bf16_decode_array(u_gpu)
    if split is None:
        wdtype = fc[0]
        if wdtype == "bf16":
            U, tau = oracle.lmhead_logits(c_gpu, "bf16", si.bits(inp["fc"]), with_tau=True)
        else:
            U, tau = oracle.lmhead_logits(c_gpu, wdtype, fc[1], fc[2], fc[3], with_tau=True)
        gamma_k = (2 * h / 64 + 48) * 2.0 ** -24
        near_zero_ok = np.abs(u - U) <= bf16_ulp(u) + gamma_k * tau * 1e3
        st["u"] = _stage(f"{label} u", u_gpu, bf16_encode_array(U), STAGE_U_OFF, near_zero_ok)
    else:
        e_proj, h_proj = split
        Ue, te = oracle.lmhead_logits(np.ascontiguousarray(c_gpu[:, :h]), "bf16", e_proj, with_tau=True)
        Uh, th = oracle.lmhead_logits(np.ascontiguousarray(c_gpu[:, h:]), "bf16", h_proj, with_tau=True)
        ue = oracle.bf16_decode_array(bf16_encode_array(Ue))
        uh = oracle.bf16_decode_array(bf16_encode_array(Uh))
        gamma_k = (h / 64 + 48) * 2.0 ** -24
        near_zero_ok = (np.abs(u - (Ue + Uh)) <= bf16_ulp(u) + bf16_ulp(ue) + bf16_ulp(uh) +
                        gamma_k * (te + th) * 1e3)
        st["u"] = _stage(f"{label} u", u_gpu, bf16_encode_array(ue + uh), 3 * STAGE_U_OFF, near_zero_ok)
    gf = si.bits(inp["gamma_f"])
    xr = np.stack([oracle.rms_norm(u_gpu[i], gf, eps, gamma_offset) for i in range(b)])
    st["x"] = _stage(f"{label} x", x_gpu, xr, STAGE_C_X_OFF)
    return st


def fmt_stages(st: dict) -> str:
    return ", ".join(f"{k} {v['off']}/{v['n']} off (max {v['max_ulps']})" for k, v in st.items())
