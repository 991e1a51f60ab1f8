"""C-ABI checks that run without a GPU: the library loads, exports every symbol
include/mtp_draft.h declares, and every call rejects bad arguments on the host
with the documented status before any HIP call (fake, never-dereferenced
device addresses are passed; token ids are real host memory).
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mtp_draft.h")

OK, NULL, SHAPE, ALIGN, DTYPE, WS, OVERLAP, HIP, RANGE = range(9)


@pytest.fixture(scope="module")
def L():
    import mtp_draft_head_02_amd as m

    return m.lib


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"MTP_API\s+[\w\s\*]+?\b(mtp_\w+)\s*\(", src)))


def test_exports_match_header(L):
    import mtp_draft_head_02_amd as m

    names = declared_symbols()
    assert len(names) == 20
    assert sorted(m.EXPORTED) == names
    for n in names:
        assert hasattr(L, n), n
    # and nothing else named mtp_ is exported
    so = open(m.LIB_PATH, "rb").read()
    for n in names:
        assert n.encode() in so


def test_version_and_status_strings(L):
    assert L.mtp_abi_version() == 1
    seen = set()
    for st in range(9):
        s = L.mtp_status_string(st).decode()
        assert s and s not in seen
        seen.add(s)
    assert L.mtp_status_string(99).decode() == "unknown status"


def test_lmhead_kernel_form(L):
    """The documented choice between the VALU and the matrix-core lm_head sweep
    (host logic only): BF16 from b = 3 where its split schedule (4 waves per
    tile: h a multiple of 1024, 8 staged vectors, tiles and partial sums in LDS)
    applies; FP8 from b = 5, NVFP4 from b = 3 (FP8 3 and NVFP4 2 when
    h % 4096 != 0), when h is a multiple of 512 (FP8) or 1024 (NVFP4) and the
    staged vectors and weight tiles fit in LDS (b <= 5 at h = 8192)."""
    form = L.mtp_lmhead_kernel_form
    form.argtypes = [C.c_int64, C.c_int64, C.c_int]
    form.restype = C.c_int

    def fits(b, h):
        # b staged vectors (row stride k/8 chunks rounded up to 1 mod 16) + 8 waves' 16 x 33-chunk weight tiles
        cx = h // 8
        return b * (cx + ((1 - cx) % 16)) * 16 + 8 * 16 * 33 * 16 <= 152 * 1024

    for b in range(1, 9):
        for h in (1024, 2048, 4096):
            assert form(b, h, 0) == (1 if b >= 3 else 0)
        for h in (256, 768, 4352, 5120, 8192, 48, 272):
            assert form(b, h, 0) == 0
        assert form(b, 4096, 1) == (1 if b >= 5 else 0)
        assert form(b, 8192, 1) == (1 if 5 <= b <= 5 else 0) and fits(5, 8192) and not fits(6, 8192)
        assert form(b, 5120, 1) == (1 if b >= 3 else 0)
        assert form(b, 512, 1) == (1 if b >= 3 else 0)
        assert form(b, 256, 1) == 0 and form(b, 48, 1) == 0
        assert form(b, 4096, 2) == (1 if b >= 3 else 0)
        assert form(b, 8192, 2) == (1 if 3 <= b <= 5 else 0)
        assert form(b, 5120, 2) == (1 if b >= 2 else 0)
        assert form(b, 1024, 2) == (1 if b >= 2 else 0)
        assert form(b, 256, 2) == 0 and form(b, 768, 2) == 0
    for b, h, wd in ((0, 4096, 1), (9, 4096, 1), (1, 8, 0), (1, 8208, 1), (1, 4100, 0), (1, 272, 2), (1, 4096, 3),
                     (1, 4096, -1)):
        assert form(b, h, wd) == -1, (b, h, wd)


def test_workspace_queries(L):
    assert L.mtp_lmhead_argmax_workspace_bytes(154880, 4096, 8, 2) >= 128
    assert L.mtp_quantize_nvfp4_workspace_bytes(131072, 5120) >= 4
    a = L.mtp_draft_combine_workspace_bytes(1, 4096)
    b = L.mtp_draft_combine_workspace_bytes(8, 4096)
    assert a >= 4 + 2 * 4096 * 2 + 4096 * 2 and b > a
    assert L.mtp_draft_combine_workspace_bytes(9, 4096) == 0
    assert L.mtp_draft_combine_workspace_bytes(1, 99999) == 0


# fake, aligned, far-apart device addresses (never dereferenced: every call below fails validation)
A = 0x7F0000000000
GB = 1 << 30


def P(i, off=0):
    return C.c_void_p(A + i * 64 * GB + off)


def lm(L, **kw):
    args = dict(x=P(0), b=1, h=4096, wd=0, w=P(1), scale=None, gscale=None, vocab=1000, mvs=0, tok=P(2),
                logits=None, ws=P(3), ws_bytes=L.mtp_lmhead_argmax_workspace_bytes(1000, 4096, 1, 0))
    args.update(kw)
    return L.mtp_lmhead_argmax(args["x"], args["b"], args["h"], args["wd"], args["w"], args["scale"],
                               args["gscale"], args["vocab"], args["mvs"], args["tok"], args["logits"],
                               args["ws"], args["ws_bytes"], None)


def test_lmhead_validation(L):
    assert lm(L, wd=3) == DTYPE
    assert lm(L, wd=-1) == DTYPE
    assert lm(L, x=None) == NULL
    assert lm(L, w=None) == NULL
    assert lm(L, tok=None) == NULL
    assert lm(L, ws=None) == WS
    assert lm(L, scale=P(4)) == DTYPE                      # BF16 takes no scale
    assert lm(L, gscale=P(4)) == DTYPE
    assert lm(L, wd=1) == NULL                             # FP8 needs a row scale
    assert lm(L, wd=1, scale=P(4), gscale=P(5)) == DTYPE   # ... and no global scale
    assert lm(L, wd=2, scale=P(4)) == NULL                 # NVFP4 needs both
    assert lm(L, wd=2, gscale=P(5)) == NULL
    for b in (0, 9, -1):
        assert lm(L, b=b) == SHAPE
    for v in (0, -5, 1 << 31):
        assert lm(L, vocab=v) == SHAPE
    assert lm(L, mvs=-1) == SHAPE
    for h in (0, 8, 4100, 8208, 16384):
        assert lm(L, h=h) == SHAPE
    assert lm(L, wd=2, scale=P(4), gscale=P(5), h=4112) == SHAPE  # NVFP4 needs h % 256
    assert lm(L, x=P(0, 8)) == ALIGN
    assert lm(L, w=P(1, 4)) == ALIGN
    assert lm(L, tok=P(2, 2)) == ALIGN
    assert lm(L, ws=P(3, 8)) == ALIGN
    assert lm(L, logits=P(4, 2)) == ALIGN
    assert lm(L, wd=1, scale=P(4, 2)) == ALIGN
    assert lm(L, wd=2, scale=P(4, 4), gscale=P(5)) == ALIGN
    assert lm(L, wd=2, scale=P(4), gscale=P(5, 2)) == ALIGN
    assert lm(L, ws_bytes=100) == WS
    assert lm(L, tok=P(1, 4096)) == OVERLAP                # token_out inside the weights
    assert lm(L, logits=P(0, 4096)) == OVERLAP             # logits over x
    assert lm(L, ws=P(2)) == OVERLAP                       # workspace over token_out
    assert lm(L, logits=P(2, 0)) == OVERLAP                # two outputs
    # truncation does not shrink the weight range the overlap check protects
    assert lm(L, mvs=10, tok=P(1, 999 * 8192)) == OVERLAP


def lmx(L, fn, extra, **kw):
    """Call the logprob or masked entry point: common arguments as lm(), then `extra`."""
    args = dict(x=P(0), b=1, h=4096, wd=0, w=P(1), scale=None, gscale=None, vocab=1000, mvs=0, tok=P(2),
                ws=P(3), ws_bytes=L.mtp_lmhead_argmax_workspace_bytes(1000, 4096, 1, 0))
    args.update(kw)
    e = dict(extra)
    e.update({k: v for k, v in kw.items() if k in e})
    head = (args["x"], args["b"], args["h"], args["wd"], args["w"], args["scale"], args["gscale"], args["vocab"],
            args["mvs"])
    if fn == "logprob":
        return L.mtp_lmhead_argmax_logprob(*head, args["tok"], e["lp"], e["conf"], args["ws"], args["ws_bytes"], None)
    return L.mtp_lmhead_argmax_masked(*head, e["mask"], e["mw"], args["tok"], e["allowed"], args["ws"],
                                      args["ws_bytes"], None)


def test_logprob_validation(L):
    ok = dict(lp=P(4), conf=None)
    assert lmx(L, "logprob", ok, lp=None) == NULL
    assert lmx(L, "logprob", ok, lp=P(4, 2)) == ALIGN
    assert lmx(L, "logprob", ok, conf=P(5, 1)) == ALIGN
    assert lmx(L, "logprob", ok, lp=P(1, 64)) == OVERLAP       # log-probabilities written into the weights
    assert lmx(L, "logprob", ok, conf=P(0, 16)) == OVERLAP     # conf over x
    assert lmx(L, "logprob", ok, conf=P(2)) == OVERLAP         # conf over token_out
    assert lmx(L, "logprob", ok, lp=P(3, 128)) == OVERLAP      # into the workspace
    assert lmx(L, "logprob", ok, wd=5) == DTYPE
    assert lmx(L, "logprob", ok, b=9) == SHAPE
    assert lmx(L, "logprob", ok, ws_bytes=1000) == WS


def test_masked_validation(L):
    ok = dict(mask=P(4), mw=32, allowed=P(5))
    assert lmx(L, "masked", ok, allowed=None) == NULL
    assert lmx(L, "masked", ok, mask=None) == NULL
    assert lmx(L, "masked", ok, mw=-1) == SHAPE
    assert lmx(L, "masked", ok, mw=(1 << 26) + 1) == SHAPE
    assert lmx(L, "masked", ok, mask=P(4, 2)) == ALIGN
    assert lmx(L, "masked", ok, allowed=P(5, 1)) == ALIGN
    assert lmx(L, "masked", ok, allowed=P(4, 64)) == OVERLAP   # allowed_out over the mask
    assert lmx(L, "masked", ok, allowed=P(2)) == OVERLAP       # allowed_out over token_out
    assert lmx(L, "masked", ok, tok=P(4, 8)) == OVERLAP        # token_out over the mask
    assert lmx(L, "masked", ok, x=None) == NULL
    assert lmx(L, "masked", ok, h=4100) == SHAPE


def test_quantize_validation(L):
    q8 = L.mtp_quantize_fp8
    assert q8(None, 10, 64, P(1), P(2), None) == NULL
    assert q8(P(0), 10, 64, None, P(2), None) == NULL
    assert q8(P(0), 10, 64, P(1), None, None) == NULL
    assert q8(P(0), 0, 64, P(1), P(2), None) == SHAPE
    assert q8(P(0), 10, 8, P(1), P(2), None) == SHAPE
    assert q8(P(0), 10, 40, P(1), P(2), None) == SHAPE
    assert q8(P(0), 10, 65552, P(1), P(2), None) == SHAPE
    assert q8(P(0, 2), 10, 64, P(1), P(2), None) == ALIGN
    assert q8(P(0), 10, 64, P(1, 8), P(2), None) == ALIGN
    assert q8(P(0), 10, 64, P(1), P(2, 1), None) == ALIGN
    assert q8(P(0), 10, 64, P(0, 128), P(2), None) == OVERLAP
    assert q8(P(0), 10, 64, P(1), P(1, 16), None) == OVERLAP
    q4 = L.mtp_quantize_nvfp4
    ok = dict(w=P(0), n=10, k=256, c=P(1), s=P(2), g=P(3), ws=P(4), wsb=256)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return q4(a["w"], a["n"], a["k"], a["c"], a["s"], a["g"], a["ws"], a["wsb"], None)

    assert call(w=None) == NULL and call(c=None) == NULL and call(s=None) == NULL and call(g=None) == NULL
    assert call(ws=None) == WS
    assert call(wsb=3) == WS
    assert call(k=128) == SHAPE and call(k=272) == SHAPE and call(n=0) == SHAPE
    assert call(s=P(2, 8)) == ALIGN and call(g=P(3, 1)) == ALIGN and call(ws=P(4, 4)) == ALIGN
    assert call(g=P(0, 64)) == OVERLAP and call(ws=P(1)) == OVERLAP


def test_combine_validation(L):
    tok = np.array([3, 0], dtype=np.int32)
    tptr = C.c_void_p(tok.ctypes.data)
    ok = dict(E=P(0), V=100, t=tptr, H=P(1), ge=P(2), gh=P(3), fc=P(4), gf=P(5), b=2, h=256, eps=1e-6,
              off=0.0, x=P(6), ws=P(7), wsb=L.mtp_draft_combine_workspace_bytes(2, 256))

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.mtp_draft_combine(a["E"], a["V"], a["t"], a["H"], a["ge"], a["gh"], a["fc"], a["gf"], a["b"],
                                   a["h"], C.c_float(a["eps"]), C.c_float(a["off"]), a["x"], a["ws"], a["wsb"], None)

    for k in ("E", "t", "H", "ge", "gh", "fc", "gf", "x"):
        assert call(**{k: None}) == NULL, k
    assert call(ws=None) == WS
    assert call(b=0) == SHAPE and call(b=9) == SHAPE and call(h=8) == SHAPE and call(h=264) == SHAPE
    assert call(V=0) == SHAPE
    assert call(eps=0.0) == SHAPE and call(eps=float("nan")) == SHAPE and call(off=float("inf")) == SHAPE
    bad = np.array([3, 100], dtype=np.int32)
    assert call(t=C.c_void_p(bad.ctypes.data)) == RANGE
    neg = np.array([-1, 0], dtype=np.int32)
    assert call(t=C.c_void_p(neg.ctypes.data)) == RANGE
    assert call(E=P(0, 2)) == ALIGN and call(x=P(6, 8)) == ALIGN and call(ws=P(7, 4)) == ALIGN
    assert call(wsb=16) == WS
    assert call(x=P(4, 512)) == OVERLAP  # x_out inside fc
    assert call(ws=P(6)) == OVERLAP      # workspace over x_out


def test_combine_variant_validation(L):
    tok = np.array([3, 0], dtype=np.int32)
    tptr = C.c_void_p(tok.ctypes.data)
    base = dict(E=P(0), V=100, t=tptr, H=P(1), ge=P(2), gh=P(3), gf=P(5), b=2, h=256, eps=1e-6, off=0.0, x=P(6),
                ws=P(7), wsb=L.mtp_draft_combine_workspace_bytes(2, 256))

    def dev(**kw):
        a = dict(base, t=P(8), fc=P(4))
        a.update(kw)
        return L.mtp_draft_combine_dev(a["E"], a["V"], a["t"], a["H"], a["ge"], a["gh"], a["fc"], a["gf"], a["b"],
                                       a["h"], C.c_float(a["eps"]), C.c_float(a["off"]), a["x"], a["ws"], a["wsb"],
                                       None)

    assert dev(t=None) == NULL
    assert dev(t=P(8, 2)) == ALIGN
    assert dev(x=P(8, 0)) == OVERLAP        # x_out over the device token ids
    assert dev(fc=None) == NULL
    assert dev(h=264) == SHAPE

    def q(**kw):
        a = dict(base, wd=1, fc=P(4), sc=P(9), gs=None)
        a.update(kw)
        return L.mtp_draft_combine_q(a["E"], a["V"], a["t"], a["H"], a["ge"], a["gh"], a["wd"], a["fc"], a["sc"],
                                     a["gs"], a["gf"], a["b"], a["h"], C.c_float(a["eps"]), C.c_float(a["off"]),
                                     a["x"], a["ws"], a["wsb"], None)

    assert q(wd=3) == DTYPE
    assert q(sc=None) == NULL                         # FP8 needs row scales
    assert q(gs=P(10)) == DTYPE                       # ... and no global scale
    assert q(wd=0) == DTYPE                           # BF16 takes no scale
    assert q(wd=2, gs=None) == NULL                   # NVFP4 needs both
    assert q(wd=2, gs=P(10), h=64) == SHAPE           # NVFP4 needs 2h % 256
    assert q(wd=2, gs=P(10), sc=P(9, 4)) == ALIGN
    assert q(sc=P(9, 2)) == ALIGN
    assert q(x=P(9, 16)) == OVERLAP                   # x_out over the scales
    bad = np.array([3, 100], dtype=np.int32)
    assert q(t=C.c_void_p(bad.ctypes.data)) == RANGE

    def sp(**kw):
        a = dict(base, ep=P(4), hp=P(9))
        a.update(kw)
        return L.mtp_draft_combine_split(a["E"], a["V"], a["t"], a["H"], a["ge"], a["gh"], a["ep"], a["hp"], a["gf"],
                                         a["b"], a["h"], C.c_float(a["eps"]), C.c_float(a["off"]), a["x"], a["ws"],
                                         a["wsb"], None)

    assert sp(ep=None) == NULL and sp(hp=None) == NULL
    assert sp(hp=P(9, 8)) == ALIGN
    assert sp(ws=P(9, 256)) == OVERLAP                # workspace over h_proj
    assert sp(x=P(4, 1024)) == OVERLAP                # x_out inside e_proj


def test_step_validation(L):
    tok = np.array([3, 0], dtype=np.int32)
    tptr = C.c_void_p(tok.ctypes.data)
    base = dict(E=P(0), EV=100, t=tptr, dev=0, H=P(1), ge=P(2), gh=P(3), fc=P(4), gf=P(5), b=2, h=256, eps=1e-6,
                off=0.0, wd=0, w=P(6), sc=None, gs=None, V=1000, mvs=0, tok=P(7), x=None, lp=None, conf=None, ws=P(8),
                wsb=L.mtp_draft_step_workspace_bytes(2, 256))

    def st(**kw):
        a = dict(base)
        a.update(kw)
        return L.mtp_draft_step(a["E"], a["EV"], a["t"], a["dev"], a["H"], a["ge"], a["gh"], a["fc"], a["gf"], a["b"],
                                a["h"], C.c_float(a["eps"]), C.c_float(a["off"]), a["wd"], a["w"], a["sc"], a["gs"],
                                a["V"], a["mvs"], a["tok"], a["x"], a["lp"], a["conf"], a["ws"], a["wsb"], None)

    assert L.mtp_draft_step_workspace_bytes(2, 256) > L.mtp_lmhead_argmax_workspace_bytes(1000, 256, 2, 0)
    assert L.mtp_draft_step_workspace_bytes(9, 256) == 0
    assert st(fc=None) == NULL and st(w=None) == NULL and st(tok=None) == NULL and st(E=None) == NULL
    assert st(ws=None) == WS and st(wsb=1000) == WS
    assert st(wd=4) == DTYPE and st(sc=P(9)) == DTYPE and st(wd=1) == NULL
    assert st(b=9) == SHAPE and st(h=264) == SHAPE and st(V=0) == SHAPE
    assert st(wd=2, sc=P(9), gs=P(10), h=4112) == SHAPE              # NVFP4 h % 256
    assert st(h=8192, b=5, wsb=L.mtp_draft_step_workspace_bytes(5, 8192), t=C.c_void_p(
        np.zeros(5, np.int32).ctypes.data)) == SHAPE                   # concat vectors past the LDS budget
    bad = np.array([3, 100], dtype=np.int32)
    assert st(t=C.c_void_p(bad.ctypes.data)) == RANGE                 # host ids are checked
    assert st(dev=1, t=P(11, 2)) == ALIGN                             # device ids: 4-byte aligned, not range-checked
    assert st(x=P(12, 8)) == ALIGN and st(lp=P(12, 2)) == ALIGN
    assert st(x=P(6, 64)) == OVERLAP                                  # x_out inside the lm_head weights
    assert st(lp=P(4, 16)) == OVERLAP                                 # log-probabilities inside fc
    assert st(conf=P(7)) == OVERLAP                                   # conf over token_out
    assert st(tok=P(8, 512)) == OVERLAP                               # token_out inside the workspace


def test_step_noalloc_validation(L):
    """mtp_draft_step_noalloc: mtp_draft_step's checks, with no workspace
    argument (its scratch holds the largest workspace any accepted shape needs)."""
    import mtp_draft_head_02_amd as m

    tok = np.array([3, 0], dtype=np.int32)
    tptr = C.c_void_p(tok.ctypes.data)
    base = dict(E=P(0), EV=100, t=tptr, dev=0, H=P(1), ge=P(2), gh=P(3), fc=P(4), gf=P(5), b=2, h=256, eps=1e-6,
                off=0.0, wd=0, w=P(6), sc=None, gs=None, V=1000, mvs=0, tok=P(7), x=None, lp=None, conf=None)

    def st(**kw):
        a = dict(base)
        a.update(kw)
        return L.mtp_draft_step_noalloc(a["E"], a["EV"], a["t"], a["dev"], a["H"], a["ge"], a["gh"], a["fc"],
                                        a["gf"], a["b"], a["h"], C.c_float(a["eps"]), C.c_float(a["off"]), a["wd"],
                                        a["w"], a["sc"], a["gs"], a["V"], a["mvs"], a["tok"], a["x"], a["lp"],
                                        a["conf"], None)

    assert st(fc=None) == NULL and st(w=None) == NULL and st(tok=None) == NULL and st(E=None) == NULL
    assert st(wd=4) == DTYPE and st(sc=P(9)) == DTYPE and st(wd=1) == NULL
    assert st(b=0) == SHAPE and st(b=9) == SHAPE and st(h=264) == SHAPE and st(h=8208) == SHAPE
    assert st(eps=0.0) == SHAPE and st(V=0) == SHAPE
    assert st(h=8192, b=5, t=C.c_void_p(np.zeros(5, np.int32).ctypes.data)) == SHAPE   # concat past the LDS budget
    bad = np.array([3, 100], dtype=np.int32)
    assert st(t=C.c_void_p(bad.ctypes.data)) == RANGE
    assert st(dev=1, t=P(11, 2)) == ALIGN
    assert st(x=P(6, 64)) == OVERLAP and st(conf=P(7)) == OVERLAP
    # the scratch serves every accepted shape: the largest step workspace
    assert L.mtp_draft_step_workspace_bytes(8, 8192) == 786944
    assert m.MTP_STEP_WS_U_OFFSET == 393728 and m.MTP_COMBINE_WS_C_OFFSET == 256


def test_workspace_layout_constants_match_header():
    src = open(HEADER).read()
    import mtp_draft_head_02_amd as m

    assert re.search(r"#define MTP_STEP_WS_U_OFFSET (\d+)", src).group(1) == str(m.MTP_STEP_WS_U_OFFSET)
    assert re.search(r"#define MTP_COMBINE_WS_C_OFFSET (\d+)", src).group(1) == str(m.MTP_COMBINE_WS_C_OFFSET)
    for name in ("MTP_CODEC_E4M3", "MTP_CODEC_E2M1", "MTP_CODEC_BF16"):
        assert re.search(name + r" = (\d+)", src).group(1) == str(getattr(m, name)), name


def test_codec_range_validation(L):
    f = L.mtp_codec_encode_range
    assert f(3, 0, 10, P(0), None) == DTYPE
    assert f(-1, 0, 10, P(0), None) == DTYPE
    assert f(2, 0, 10, None, None) == NULL
    assert f(2, 0xFFFFFFFF, 2, P(0), None) == SHAPE
    assert f(2, 0, 10, P(0, 2), None) == ALIGN
    assert f(0, 0, 10, None, None) == NULL
    assert f(0, 0, 0, P(0), None) == SHAPE
    assert f(0, 0xFFFFFFFF, 2, P(0), None) == SHAPE
    assert f(1, 0, 10, P(0, 1), None) == ALIGN


def test_stream_read_validation(L):
    """The streaming-read reference: NULL pointers, a size under one 8 KB unit
    and misalignment are refused before any launch."""
    f = L.mtp_stream_read
    assert f(None, 8192, 0, 0, P(0), None) == NULL
    assert f(P(0), 8192, 0, 0, None, None) == NULL
    assert f(P(0), 8191, 0, 0, P(0), None) == SHAPE
    assert f(P(0), 8192, 6, 0, P(0), None) == SHAPE
    assert f(P(0), 8192, -1, 0, P(0), None) == SHAPE
    assert f(P(0, 8), 8192, 0, 0, P(0), None) == ALIGN
    assert f(P(0), 8192, 0, 0, P(0, 2), None) == ALIGN


def test_python_dtype_parser():
    import mtp_draft_head_02_amd as m

    assert m.parse_wdtype("NVFP4") == m.parse_wdtype("fp4") == m.MTP_W_NVFP4
    assert m.parse_wdtype("Fp8") == m.MTP_W_FP8_E4M3_ROW
    assert m.parse_wdtype("bf16") == m.MTP_W_BF16
    with pytest.raises(ValueError, match="Expected: nvfp4, fp8, bf16"):
        m.parse_wdtype("int4")


def test_plain_c_consumer(L, tmp_path):
    """The header compiles as strict C99 and a C program linked against the
    library passes its host-only checks (tests/abi_consumer.c: version, status
    texts, workspace layout, kernel forms, argument errors before any device
    work)."""
    import subprocess

    libdir = os.path.dirname(L._name)
    exe = str(tmp_path / "abi_consumer")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-o", exe, os.path.join(ROOT, "tests", "abi_consumer.c"), "-L", libdir, "-lmtpdraft",
                    f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
