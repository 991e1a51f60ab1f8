"""Property-based checks of the C ABI's host validation, without a GPU.

Every example starts from a valid argument set for one entry point and
applies one or more of the argument errors that include/mtp_draft.h documents
(a bad format, a NULL pointer, a shape out of range, a misalignment, a short
workspace, a host token id out of range, an output overlapping an input).
The call must return a documented status: with one error exactly that
error's status, with several one of theirs (the checks run in a fixed
order). Since every example carries an error, no call reaches a launch; the
fake device addresses are never dereferenced.
"""
import ctypes as C

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

OK, NULL, SHAPE, ALIGN, DTYPE, WS, OVERLAP, HIP, RANGE = range(9)
A = 0x7F0000000000
GB = 1 << 30


def P(i, off=0):
    """A fake, 16-byte aligned device address; bases 64 GB apart."""
    return A + i * 64 * GB + off


@pytest.fixture(scope="module")
def L():
    import mtp_draft_head_02_amd as m

    return m.lib


SETTINGS = settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])

# ----------------------------------------------------------------- lm_head --

LM_ERRORS = ["format", "null_x", "null_w", "null_tok", "null_ws", "scales", "b", "vocab", "mvs", "h", "align_x",
             "align_tok", "align_ws", "align_logits", "ws_small", "overlap"]


@st.composite
def lm_case(draw):
    wd = draw(st.sampled_from([0, 1, 2]))
    h = 256 * draw(st.integers(1, 32)) if wd == 2 else 16 * draw(st.integers(1, 512))
    a = dict(x=P(0), b=draw(st.integers(1, 8)), h=h, wd=wd, w=P(1), scale=P(4) if wd else None,
             gscale=P(5) if wd == 2 else None, vocab=draw(st.integers(1, 2_000_000)),
             mvs=draw(st.sampled_from([0, 1, 7, 10 ** 6])), tok=P(2),
             logits=P(6) if draw(st.booleans()) else None, ws=P(3), ws_bytes=None)
    errs = draw(st.sets(st.sampled_from(sorted(LM_ERRORS)), min_size=1, max_size=3))
    return a, errs


def apply_lm(L, a, errs):
    a = dict(a)
    a["ws_bytes"] = L.mtp_lmhead_argmax_workspace_bytes(a["vocab"], a["h"], a["b"], a["wd"])
    codes = set()
    for e in sorted(errs):
        if e == "format":
            a["wd"] = 3
            codes.add(DTYPE)
        elif e == "null_x":
            a["x"] = None
            codes.add(NULL)
        elif e == "null_w":
            a["w"] = None
            codes.add(NULL)
        elif e == "null_tok":
            a["tok"] = None
            codes.add(NULL)
        elif e == "null_ws":
            a["ws"] = None
            codes.add(WS)
        elif e == "scales":  # BF16 given a scale: DTYPE; FP8 / NVFP4 missing one: NULL
            if a["wd"] == 0:
                a["scale"] = P(4)
                codes.add(DTYPE)
            elif a["wd"] == 1:
                a["scale"] = None
                codes.add(NULL)
            else:
                a["gscale"] = None
                codes.add(NULL)
        elif e == "b":
            a["b"] = 0 if a["b"] % 2 else 9
            codes.add(SHAPE)
        elif e == "vocab":
            a["vocab"] = 0 if a["vocab"] % 2 else 1 << 31
            codes.add(SHAPE)
        elif e == "mvs":
            a["mvs"] = -1
            codes.add(SHAPE)
        elif e == "h":
            a["h"] = a["h"] + 8 if a["h"] < 8192 else 8208
            codes.add(SHAPE)
        elif e == "align_x":
            a["x"] = (a["x"] or P(0)) + 2
            codes.add(ALIGN)
        elif e == "align_tok":
            a["tok"] = (a["tok"] or P(2)) + 2
            codes.add(ALIGN)
        elif e == "align_ws":
            a["ws"] = (a["ws"] or P(3)) + 8
            codes.add(ALIGN)
        elif e == "align_logits":
            a["logits"] = P(6, 2)
            codes.add(ALIGN)
        elif e == "ws_small":
            a["ws_bytes"] = a["ws_bytes"] - 1
            codes.add(WS)
        elif e == "overlap":
            a["tok"] = P(1)  # token_out at the start of the weights
            codes.add(OVERLAP)
    vp = lambda v: None if v is None else C.c_void_p(v)
    rc = L.mtp_lmhead_argmax(vp(a["x"]), a["b"], a["h"], a["wd"], vp(a["w"]), vp(a["scale"]), vp(a["gscale"]),
                             a["vocab"], a["mvs"], vp(a["tok"]), vp(a["logits"]), vp(a["ws"]), a["ws_bytes"], None)
    return rc, codes


@SETTINGS
@given(case=lm_case())
def test_lmhead_rejects_every_documented_error(L, case):
    a, errs = case
    rc, codes = apply_lm(L, a, errs)
    assert rc not in (OK, HIP), (errs, rc)
    assert rc in codes, (sorted(errs), rc, codes)
    if len(errs) == 1:
        assert rc == next(iter(codes))


def test_lmhead_valid_base_passes_validation_here(L):
    """The fuzz's base cases are valid: with no error applied, the only
    possible failure on this GPU-less host is the HIP call itself (no launch
    happens; the status is MTP_ERR_HIP)."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a valid call would launch on the fake addresses; host-only check")
    a = dict(x=P(0), b=3, h=4096, wd=1, w=P(1), scale=P(4), gscale=None, vocab=5000, mvs=0, tok=P(2),
             logits=None, ws=P(3))
    rc, _ = apply_lm(L, a, set())
    assert rc == HIP


# -------------------------------------------------------------- draft step --

STEP_ERRORS = ["null_embed", "null_fc", "null_w", "null_tok", "null_ws", "ws_small", "format", "b", "h", "vocab",
               "embed_vocab", "lds", "eps", "token_range", "align_x", "align_lp", "overlap_x", "overlap_conf"]


@st.composite
def step_case(draw):
    wd = draw(st.sampled_from([0, 1, 2]))
    h = 256 * draw(st.integers(1, 32)) if wd == 2 else 16 * draw(st.integers(1, 512))
    bmax = min(8, 131584 // (4 * h + 16))
    a = dict(b=draw(st.integers(1, bmax)), h=h, wd=wd, EV=draw(st.integers(1, 100_000)),
             V=draw(st.integers(1, 1_000_000)), eps=1e-6, x=P(12) if draw(st.booleans()) else None,
             lp=P(13) if draw(st.booleans()) else None, conf=P(14) if draw(st.booleans()) else None)
    a["tokens"] = draw(st.lists(st.integers(0, a["EV"] - 1), min_size=8, max_size=8))
    errs = draw(st.sets(st.sampled_from(sorted(STEP_ERRORS)), min_size=1, max_size=3))
    return a, errs


@SETTINGS
@given(case=step_case())
def test_step_rejects_every_documented_error(L, case):
    a, errs = case
    a = dict(a)
    p = dict(E=P(0), fc=P(4), w=P(6), tok=P(7), ws=P(8), sc=P(9) if a["wd"] else None,
             gs=P(10) if a["wd"] == 2 else None, ge=P(2), gh=P(3), gf=P(5), H=P(1))
    wsb = L.mtp_draft_step_workspace_bytes(a["b"], a["h"])
    toks = np.asarray(a["tokens"], dtype=np.int32)
    codes = set()
    for e in sorted(errs):
        if e in ("null_embed", "null_fc", "null_w", "null_tok"):
            p[{"null_embed": "E", "null_fc": "fc", "null_w": "w", "null_tok": "tok"}[e]] = None
            codes.add(NULL)
        elif e == "null_ws":
            p["ws"] = None
            codes.add(WS)
        elif e == "ws_small":
            wsb = wsb - 1
            codes.add(WS)
        elif e == "format":
            a["wd"] = 4
            codes.add(DTYPE)
        elif e == "b":
            a["b"] = 9
            codes.add(SHAPE)
        elif e == "h":
            a["h"] = a["h"] + 8 if a["h"] < 8192 else 8208
            codes.add(SHAPE)
        elif e == "vocab":
            a["V"] = 0
            codes.add(SHAPE)
        elif e == "embed_vocab":
            a["EV"] = 0
            codes.add(SHAPE)
        elif e == "lds":  # the concat vectors past the LDS budget
            a["h"], a["b"] = 8192, 5
            codes.add(SHAPE)
        elif e == "eps":
            a["eps"] = 0.0
            codes.add(SHAPE)
        elif e == "token_range":
            toks[0] = a["EV"]
            codes.add(RANGE)
        elif e == "align_x":
            a["x"] = P(12, 8)
            codes.add(ALIGN)
        elif e == "align_lp":
            a["lp"] = P(13, 2)
            codes.add(ALIGN)
        elif e == "overlap_x":
            a["x"] = P(6)  # x_out at the start of the lm_head weights
            codes.add(OVERLAP)
        elif e == "overlap_conf":
            a["conf"] = P(7)  # conf over token_out
            codes.add(OVERLAP)
    vp = lambda v: None if v is None else C.c_void_p(v)
    rc = L.mtp_draft_step(vp(p["E"]), a["EV"], C.c_void_p(toks.ctypes.data), 0, vp(p["H"]), vp(p["ge"]),
                          vp(p["gh"]), vp(p["fc"]), vp(p["gf"]), a["b"], a["h"], C.c_float(a["eps"]), C.c_float(0.0),
                          a["wd"], vp(p["w"]), vp(p["sc"]), vp(p["gs"]), a["V"], 0, vp(p["tok"]), vp(a["x"]),
                          vp(a["lp"]), vp(a["conf"]), vp(p["ws"]), wsb, None)
    assert rc not in (OK, HIP), (sorted(errs), rc)
    assert rc in codes, (sorted(errs), rc, codes, a["b"], a["h"], a["wd"])
    if len(errs) == 1:
        assert rc == next(iter(codes))
