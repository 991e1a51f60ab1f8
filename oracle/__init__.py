"""CPU oracle for the MTP draft step -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The HIP product path never imports it and it never imports the
HIP path; they share no code.

This is a thin ctypes wrapper over oracle/mtp_oracle.c (plain C, fp64
accumulation, its own codecs). Each C function documents the passage of the
pages it follows and how it is pinned. Nothing here does arithmetic of its own
beyond array marshalling.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mtp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Another build of mtp_oracle.c to load instead (the mutation tests point this
# at copies with a planted mistake, to show that the pins catch it).
_LIB_OVERRIDE = os.environ.get("MTP_ORACLE_LIB")

W_BF16, W_FP8, W_NVFP4 = 0, 1, 2
_WD = {"bf16": W_BF16, "fp8": W_FP8, "nvfp4": W_NVFP4}

GCC_CMD = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB, _SRC, "-lm", "-lpthread"]


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    tmp = _LIB + ".tmp"
    cmd = list(GCC_CMD)
    cmd[cmd.index(_LIB)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = C.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build()
            L = C.CDLL(_LIB)
        p = C.c_void_p
        i64 = C.c_int64
        L.oracle_bf16_decode.argtypes = [C.c_uint16]
        L.oracle_bf16_decode.restype = C.c_double
        L.oracle_bf16_encode.argtypes = [C.c_double]
        L.oracle_bf16_encode.restype = C.c_uint16
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_decode.restype = C.c_double
        L.oracle_e2m1_decode.argtypes = [C.c_uint8]
        L.oracle_e2m1_decode.restype = C.c_double
        L.oracle_e4m3_encode.argtypes = [C.c_float]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e2m1_encode.argtypes = [C.c_float]
        L.oracle_e2m1_encode.restype = C.c_uint8
        L.oracle_quantize_fp8.argtypes = [p, i64, i64, p, p, C.c_int]
        L.oracle_quantize_fp8.restype = None
        L.oracle_global_absmax.argtypes = [p, i64, i64, C.c_int]
        L.oracle_global_absmax.restype = C.c_float
        L.oracle_quantize_nvfp4.argtypes = [p, i64, i64, p, p, p, C.c_int]
        L.oracle_quantize_nvfp4.restype = None
        L.oracle_rms_norm.argtypes = [p, p, i64, C.c_float, C.c_float, p]
        L.oracle_rms_norm.restype = None
        L.oracle_draft_combine.argtypes = [p, i64, p, p, p, p, p, p, i64, i64, C.c_float, C.c_float, p, p, p]
        L.oracle_draft_combine.restype = None
        L.oracle_effective_vocab.argtypes = [i64, i64]
        L.oracle_effective_vocab.restype = i64
        L.oracle_lmhead_logits.argtypes = [p, i64, i64, C.c_int, p, p, p, i64, p, p, C.c_int]
        L.oracle_lmhead_logits.restype = None
        L.oracle_argmax.argtypes = [p, i64]
        L.oracle_argmax.restype = C.c_int32
        L.oracle_lmhead_argmax.argtypes = [p, i64, i64, C.c_int, p, p, p, i64, i64, p, p, C.c_int]
        L.oracle_top1_logprob.argtypes = [p, i64]
        L.oracle_top1_logprob.restype = C.c_double
        L.oracle_argmax_masked.argtypes = [p, i64, p, i64, p]
        L.oracle_argmax_masked.restype = C.c_int32
        L.oracle_draft_combine_q.argtypes = [p, p, p, p, p, C.c_int, p, p, p, p, i64, i64, C.c_float, C.c_float,
                                             p, p]
        L.oracle_draft_combine_q.restype = None
        L.oracle_draft_combine_split.argtypes = [p, p, p, p, p, p, p, p, i64, i64, C.c_float, C.c_float, p, p]
        L.oracle_draft_combine_split.restype = None
        L.oracle_lmhead_argmax.restype = i64
        L.oracle_encode_range.argtypes = [C.c_int, C.c_uint32, i64, p, C.c_int]
        L.oracle_encode_range.restype = None
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


# ---- scalar codecs -------------------------------------------------------

def bf16_decode(bits: int) -> float:
    return lib().oracle_bf16_decode(int(bits))


def bf16_encode(v: float) -> int:
    return int(lib().oracle_bf16_encode(float(v)))


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(int(code))


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(np.float32(v))))


def e2m1_encode(v: float) -> int:
    return int(lib().oracle_e2m1_encode(float(np.float32(v))))


def encode_range(codec: int, first_bits: int, count: int, threads: int | None = None) -> np.ndarray:
    """Codes of the f32 patterns first_bits .. first_bits + count - 1 (codec 0 E4M3, 1 E2M1: uint8;
    2 BF16: uint16)."""
    out = np.empty(count, dtype=np.uint16 if codec == 2 else np.uint8)
    lib().oracle_encode_range(int(codec), int(first_bits), int(count), _ptr(out), threads or default_threads())
    return out


def bf16_decode_array(bits: np.ndarray) -> np.ndarray:
    """Vectorised BF16 decode (the same closed form: bits are the upper half of an f32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- quantizers ----------------------------------------------------------

def quantize_fp8(w: np.ndarray, threads: int | None = None):
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    scale = np.empty(n, dtype=np.float32)
    lib().oracle_quantize_fp8(_ptr(w), n, k, _ptr(codes), _ptr(scale), threads or default_threads())
    return codes, scale


def global_absmax(w: np.ndarray, threads: int | None = None) -> float:
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n, k = w.shape
    return float(lib().oracle_global_absmax(_ptr(w), n, k, threads or default_threads()))


def quantize_nvfp4(w: np.ndarray, threads: int | None = None):
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n, k = w.shape
    assert k % 16 == 0
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    bscale = np.empty((n, k // 16), dtype=np.uint8)
    g = np.empty(1, dtype=np.float32)
    lib().oracle_quantize_nvfp4(_ptr(w), n, k, _ptr(codes), _ptr(bscale), _ptr(g), threads or default_threads())
    return codes, bscale, g


# ---- combine -------------------------------------------------------------

def rms_norm(v: np.ndarray, gamma: np.ndarray, eps: float, gamma_offset: float = 0.0) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    out = np.empty_like(v)
    lib().oracle_rms_norm(_ptr(v), _ptr(gamma), v.shape[-1], eps, gamma_offset, _ptr(out))
    return out


def draft_combine(embed, tokens, hidden, gamma_e, gamma_h, fc, gamma_f, eps=1e-6, gamma_offset=0.0,
                  intermediates=False):
    embed = np.ascontiguousarray(embed, dtype=np.uint16)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    hidden = np.ascontiguousarray(hidden, dtype=np.uint16)
    vocab, h = embed.shape
    b = tokens.shape[0]
    assert hidden.shape == (b, h) and fc.shape == (h, 2 * h)
    x = np.empty((b, h), dtype=np.uint16)
    c = np.empty((b, 2 * h), dtype=np.uint16) if intermediates else None
    u = np.empty((b, h), dtype=np.uint16) if intermediates else None
    lib().oracle_draft_combine(_ptr(embed), vocab, _ptr(tokens), _ptr(hidden),
                               _ptr(np.ascontiguousarray(gamma_e, dtype=np.uint16)),
                               _ptr(np.ascontiguousarray(gamma_h, dtype=np.uint16)),
                               _ptr(np.ascontiguousarray(fc, dtype=np.uint16)),
                               _ptr(np.ascontiguousarray(gamma_f, dtype=np.uint16)),
                               b, h, eps, gamma_offset, _ptr(x), _ptr(c), _ptr(u))
    if intermediates:
        return x, c, u
    return x


# ---- lm_head -------------------------------------------------------------

def effective_vocab(vocab: int, mtp_vocab_size: int) -> int:
    return int(lib().oracle_effective_vocab(vocab, mtp_vocab_size))


def lmhead_logits(x, wdtype, w, scale=None, gscale=None, n_eff=None, with_tau=False, threads=None):
    """Double logits [b, n_eff] (and tau = 1e-3 * sum |w^ x| if with_tau)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    b, h = x.shape
    wd = _WD[wdtype]
    w = np.ascontiguousarray(w)
    n = w.shape[0] if n_eff is None else n_eff
    logits = np.empty((b, n), dtype=np.float64)
    tau = np.empty((b, n), dtype=np.float64) if with_tau else None
    lib().oracle_lmhead_logits(_ptr(x), b, h, wd, _ptr(w),
                               _ptr(None if scale is None else np.ascontiguousarray(scale)),
                               _ptr(None if gscale is None else np.ascontiguousarray(gscale, dtype=np.float32)),
                               n, _ptr(logits), _ptr(tau), threads or default_threads())
    return (logits, tau) if with_tau else logits


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, dtype=np.float64)
    return int(lib().oracle_argmax(_ptr(v), v.shape[0]))


def lmhead_argmax(x, wdtype, w, scale=None, gscale=None, vocab=None, mtp_vocab_size=0, threads=None):
    """token[b] (int32) and double logits [b, n_eff]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    b, h = x.shape
    w = np.ascontiguousarray(w)
    vocab = w.shape[0] if vocab is None else vocab
    n = effective_vocab(vocab, mtp_vocab_size)
    tok = np.empty(b, dtype=np.int32)
    logits = np.empty((b, n), dtype=np.float64)
    lib().oracle_lmhead_argmax(_ptr(x), b, h, _WD[wdtype], _ptr(w),
                               _ptr(None if scale is None else np.ascontiguousarray(scale)),
                               _ptr(None if gscale is None else np.ascontiguousarray(gscale, dtype=np.float32)),
                               vocab, mtp_vocab_size, _ptr(tok), _ptr(logits), threads or default_threads())
    return tok, logits


# ---- top-1 log-probability, masked argmax --------------------------------

def top1_logprob(v) -> float:
    """-log sum exp(v - max v) of one row of logits (NaN for a NaN or all -inf row)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    return float(lib().oracle_top1_logprob(_ptr(v), v.shape[0]))


def argmax_masked(v, mask, mask_words=None):
    """(token, any_allowed) of the argmax over the entries the int32 bitmask allows."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    mask = np.ascontiguousarray(mask, dtype=np.int32)
    mw = mask.shape[0] if mask_words is None else mask_words
    any_allowed = np.zeros(1, dtype=np.int32)
    tok = lib().oracle_argmax_masked(_ptr(v), v.shape[0], _ptr(mask), mw, _ptr(any_allowed))
    return int(tok), int(any_allowed[0])


# ---- combiner variants ---------------------------------------------------

def draft_combine_q(embed, tokens, hidden, gamma_e, gamma_h, fc_wdtype, fc, fc_scale, fc_gscale, gamma_f,
                    eps=1e-6, gamma_offset=0.0, with_u=False):
    """The combine with the fc [h, 2h] in BF16 / FP8 / NVFP4 (layouts as the lm_head)."""
    embed = np.ascontiguousarray(embed, dtype=np.uint16)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    hidden = np.ascontiguousarray(hidden, dtype=np.uint16)
    b, h = hidden.shape
    x = np.empty((b, h), dtype=np.uint16)
    u = np.empty((b, h), dtype=np.uint16)
    lib().oracle_draft_combine_q(_ptr(embed), _ptr(tokens), _ptr(hidden),
                                 _ptr(np.ascontiguousarray(gamma_e, dtype=np.uint16)),
                                 _ptr(np.ascontiguousarray(gamma_h, dtype=np.uint16)), _WD[fc_wdtype],
                                 _ptr(np.ascontiguousarray(fc)),
                                 _ptr(None if fc_scale is None else np.ascontiguousarray(fc_scale)),
                                 _ptr(None if fc_gscale is None else np.ascontiguousarray(fc_gscale, dtype=np.float32)),
                                 _ptr(np.ascontiguousarray(gamma_f, dtype=np.uint16)), b, h, eps, gamma_offset,
                                 _ptr(x), _ptr(u))
    return (x, u) if with_u else x


def draft_combine_split(embed, tokens, hidden, gamma_e, gamma_h, e_proj, h_proj, gamma_f, eps=1e-6,
                        gamma_offset=0.0, with_u=False):
    """The split combiner: u = bf16(bf16(e_proj . rms(e)) + bf16(h_proj . rms(h))), x = rms(u)."""
    embed = np.ascontiguousarray(embed, dtype=np.uint16)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    hidden = np.ascontiguousarray(hidden, dtype=np.uint16)
    b, h = hidden.shape
    x = np.empty((b, h), dtype=np.uint16)
    u = np.empty((b, h), dtype=np.uint16)
    lib().oracle_draft_combine_split(_ptr(embed), _ptr(tokens), _ptr(hidden),
                                     _ptr(np.ascontiguousarray(gamma_e, dtype=np.uint16)),
                                     _ptr(np.ascontiguousarray(gamma_h, dtype=np.uint16)),
                                     _ptr(np.ascontiguousarray(e_proj, dtype=np.uint16)),
                                     _ptr(np.ascontiguousarray(h_proj, dtype=np.uint16)),
                                     _ptr(np.ascontiguousarray(gamma_f, dtype=np.uint16)), b, h, eps, gamma_offset,
                                     _ptr(x), _ptr(u))
    return (x, u) if with_u else x
