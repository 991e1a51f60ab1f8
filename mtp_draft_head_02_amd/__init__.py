"""MI355X (gfx950) MTP draft step: Python binding of libmtpdraft.so.

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the draft path runs in the library's HIP kernels.
The functions carry the C ABI's names (include/mtp_draft.h) and raise MtpError
on a non-zero status. There is no CPU fallback: importing this package fails
if the library has not been built (python mtp_draft_head_02_amd/build.py).

Higher-level helpers (`quantize_head`, `draft_step`, ...) only allocate outputs
and workspaces with torch and call the same entry points. Given a `stream`,
they allocate and zero-fill on that stream (the caching allocator then ties
the memory to it), so the fills are ordered before the kernels and no
temporary is reused while the kernels still run.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmtpdraft.so")

MTP_OK = 0
STATUS_NAMES = {0: "MTP_OK", 1: "MTP_ERR_NULL", 2: "MTP_ERR_SHAPE", 3: "MTP_ERR_ALIGN", 4: "MTP_ERR_DTYPE",
                5: "MTP_ERR_WORKSPACE", 6: "MTP_ERR_OVERLAP", 7: "MTP_ERR_HIP", 8: "MTP_ERR_RANGE"}
MTP_W_BF16, MTP_W_FP8_E4M3_ROW, MTP_W_NVFP4 = 0, 1, 2
MTP_CODEC_E4M3, MTP_CODEC_E2M1, MTP_CODEC_BF16 = 0, 1, 2
EXPORTED = ("mtp_abi_version", "mtp_status_string", "mtp_quantize_fp8", "mtp_quantize_nvfp4_workspace_bytes",
            "mtp_quantize_nvfp4", "mtp_draft_combine_workspace_bytes", "mtp_draft_combine",
            "mtp_draft_combine_dev", "mtp_draft_combine_q", "mtp_draft_combine_split",
            "mtp_lmhead_argmax_workspace_bytes", "mtp_lmhead_kernel_form", "mtp_lmhead_argmax", "mtp_lmhead_argmax_logprob",
            "mtp_lmhead_argmax_masked", "mtp_draft_step_workspace_bytes", "mtp_draft_step",
            "mtp_draft_step_noalloc", "mtp_codec_encode_range", "mtp_stream_read")
# Documented workspace layouts (include/mtp_draft.h): where a completed call
# leaves the intermediates c [b, 2h] and u [b, h].
MTP_COMBINE_WS_C_OFFSET = 256
MTP_STEP_WS_U_OFFSET = 393728


class MtpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python mtp_draft_head_02_amd/build.py` "
                          "(the draft step has no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    p, i64, sz, i32 = C.c_void_p, C.c_int64, C.c_size_t, C.c_int
    sig = {
        "mtp_abi_version": ([], i32),
        "mtp_status_string": ([i32], C.c_char_p),
        "mtp_quantize_fp8": ([p, i64, i64, p, p, p], i32),
        "mtp_quantize_nvfp4_workspace_bytes": ([i64, i64], sz),
        "mtp_quantize_nvfp4": ([p, i64, i64, p, p, p, p, sz, p], i32),
        "mtp_draft_combine_workspace_bytes": ([i64, i64], sz),
        "mtp_draft_combine": ([p, i64, p, p, p, p, p, p, i64, i64, C.c_float, C.c_float, p, p, sz, p], i32),
        "mtp_draft_combine_dev": ([p, i64, p, p, p, p, p, p, i64, i64, C.c_float, C.c_float, p, p, sz, p], i32),
        "mtp_draft_combine_q": ([p, i64, p, p, p, p, i32, p, p, p, p, i64, i64, C.c_float, C.c_float, p, p, sz, p],
                                i32),
        "mtp_draft_combine_split": ([p, i64, p, p, p, p, p, p, p, i64, i64, C.c_float, C.c_float, p, p, sz, p], i32),
        "mtp_lmhead_argmax_workspace_bytes": ([i64, i64, i64, i32], sz),
        "mtp_lmhead_kernel_form": ([i64, i64, i32], i32),
        "mtp_lmhead_argmax": ([p, i64, i64, i32, p, p, p, i64, i64, p, p, p, sz, p], i32),
        "mtp_lmhead_argmax_logprob": ([p, i64, i64, i32, p, p, p, i64, i64, p, p, p, p, sz, p], i32),
        "mtp_lmhead_argmax_masked": ([p, i64, i64, i32, p, p, p, i64, i64, p, i64, p, p, p, sz, p], i32),
        "mtp_draft_step_workspace_bytes": ([i64, i64], sz),
        "mtp_draft_step": ([p, i64, p, i32, p, p, p, p, p, i64, i64, C.c_float, C.c_float, i32, p, p, p, i64, i64,
                            p, p, p, p, p, sz, p], i32),
        "mtp_draft_step_noalloc": ([p, i64, p, i32, p, p, p, p, p, i64, i64, C.c_float, C.c_float, i32, p, p, p,
                                    i64, i64, p, p, p, p, p], i32),
        "mtp_codec_encode_range": ([i32, C.c_uint32, i64, p, p], i32),
        "mtp_stream_read": ([p, i64, i32, C.c_uint32, p, p], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def status_string(st: int) -> str:
    return lib.mtp_status_string(int(st)).decode()


def _check(st: int, where: str) -> None:
    if st != MTP_OK:
        raise MtpError(st, where)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _on(stream):
    """Make `stream` current for the helpers' allocations, fills and launches."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _need(t, dtypes, name):
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8, torch.float8_e4m3fn)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


# ---------------------------------------------------------------- C-ABI names ----

def mtp_abi_version() -> int:
    return lib.mtp_abi_version()


def mtp_quantize_fp8(w, codes, row_scale, stream=None) -> None:
    _need(w, _BF16, "w"); _need(codes, _U8, "codes"); _need(row_scale, _F32, "row_scale")
    n, k = w.shape
    _check(lib.mtp_quantize_fp8(_ptr(w), n, k, _ptr(codes), _ptr(row_scale), _stream(stream)), "mtp_quantize_fp8")


def mtp_quantize_nvfp4_workspace_bytes(n: int, k: int) -> int:
    return lib.mtp_quantize_nvfp4_workspace_bytes(n, k)


def mtp_quantize_nvfp4(w, codes, block_scale, global_scale, ws, stream=None) -> None:
    _need(w, _BF16, "w"); _need(codes, _U8, "codes"); _need(block_scale, _U8, "block_scale")
    _need(global_scale, _F32, "global_scale")
    n, k = w.shape
    _check(lib.mtp_quantize_nvfp4(_ptr(w), n, k, _ptr(codes), _ptr(block_scale), _ptr(global_scale), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "mtp_quantize_nvfp4")


def mtp_draft_combine_workspace_bytes(b: int, h: int) -> int:
    return lib.mtp_draft_combine_workspace_bytes(b, h)


def mtp_draft_combine(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps, gamma_offset,
                      x_out, ws, stream=None) -> None:
    for t, nm in ((embed, "embed"), (hidden, "hidden"), (gamma_embed, "gamma_embed"), (gamma_hidden, "gamma_hidden"),
                  (fc, "fc"), (gamma_final, "gamma_final"), (x_out, "x_out")):
        _need(t, _BF16, nm)
    tok = torch.as_tensor(token_ids, dtype=torch.int32, device="cpu").contiguous()
    vocab, h = embed.shape
    b = tok.numel()
    _check(lib.mtp_draft_combine(_ptr(embed), vocab, C.c_void_p(tok.data_ptr()), _ptr(hidden), _ptr(gamma_embed),
                                 _ptr(gamma_hidden), _ptr(fc), _ptr(gamma_final), b, h, float(eps),
                                 float(gamma_offset), _ptr(x_out), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "mtp_draft_combine")


def mtp_draft_combine_dev(embed, token_ids_dev, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps,
                          gamma_offset, x_out, ws, stream=None) -> None:
    """token_ids_dev: int32 [b] on the device (e.g. the previous draft's token_out)."""
    for t, nm in ((embed, "embed"), (hidden, "hidden"), (gamma_embed, "gamma_embed"), (gamma_hidden, "gamma_hidden"),
                  (fc, "fc"), (gamma_final, "gamma_final"), (x_out, "x_out")):
        _need(t, _BF16, nm)
    _need(token_ids_dev, _I32, "token_ids_dev")
    vocab, h = embed.shape
    b = token_ids_dev.numel()
    _check(lib.mtp_draft_combine_dev(_ptr(embed), vocab, _ptr(token_ids_dev), _ptr(hidden), _ptr(gamma_embed),
                                     _ptr(gamma_hidden), _ptr(fc), _ptr(gamma_final), b, h, float(eps),
                                     float(gamma_offset), _ptr(x_out), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "mtp_draft_combine_dev")


def mtp_draft_combine_q(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc_wd, fc, fc_scale, fc_gscale,
                        gamma_final, eps, gamma_offset, x_out, ws, stream=None) -> None:
    for t, nm in ((embed, "embed"), (hidden, "hidden"), (gamma_embed, "gamma_embed"), (gamma_hidden, "gamma_hidden"),
                  (gamma_final, "gamma_final"), (x_out, "x_out")):
        _need(t, _BF16, nm)
    tok = torch.as_tensor(token_ids, dtype=torch.int32, device="cpu").contiguous()
    vocab, h = embed.shape
    b = tok.numel()
    _check(lib.mtp_draft_combine_q(_ptr(embed), vocab, C.c_void_p(tok.data_ptr()), _ptr(hidden), _ptr(gamma_embed),
                                   _ptr(gamma_hidden), int(fc_wd), _ptr(fc), _ptr(fc_scale), _ptr(fc_gscale),
                                   _ptr(gamma_final), b, h, float(eps), float(gamma_offset), _ptr(x_out), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "mtp_draft_combine_q")


def mtp_draft_combine_split(embed, token_ids, hidden, gamma_embed, gamma_hidden, e_proj, h_proj, gamma_final, eps,
                            gamma_offset, x_out, ws, stream=None) -> None:
    for t, nm in ((embed, "embed"), (hidden, "hidden"), (gamma_embed, "gamma_embed"), (gamma_hidden, "gamma_hidden"),
                  (e_proj, "e_proj"), (h_proj, "h_proj"), (gamma_final, "gamma_final"), (x_out, "x_out")):
        _need(t, _BF16, nm)
    tok = torch.as_tensor(token_ids, dtype=torch.int32, device="cpu").contiguous()
    vocab, h = embed.shape
    b = tok.numel()
    _check(lib.mtp_draft_combine_split(_ptr(embed), vocab, C.c_void_p(tok.data_ptr()), _ptr(hidden),
                                       _ptr(gamma_embed), _ptr(gamma_hidden), _ptr(e_proj), _ptr(h_proj),
                                       _ptr(gamma_final), b, h, float(eps), float(gamma_offset), _ptr(x_out), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)), "mtp_draft_combine_split")


def mtp_lmhead_argmax_workspace_bytes(vocab: int, h: int, b: int, wd: int) -> int:
    return lib.mtp_lmhead_argmax_workspace_bytes(vocab, h, b, wd)


def mtp_lmhead_kernel_form(b: int, h: int, wd: int) -> int:
    """0: VALU sweep, 1: matrix-core sweep, -1: outside the lm_head's limits."""
    return lib.mtp_lmhead_kernel_form(int(b), int(h), int(wd))


def lmhead_kernel_form(b: int, h: int, wdtype) -> str:
    """'valu' or 'mfma': the kernel form an lm_head call of this shape takes."""
    wd = parse_wdtype(wdtype) if isinstance(wdtype, str) else int(wdtype)
    f = mtp_lmhead_kernel_form(b, h, wd)
    if f < 0:
        raise ValueError(f"no lm_head kernel for b={b}, h={h}, wd={wdtype}")
    return "mfma" if f == 1 else "valu"


def mtp_lmhead_argmax(x, wd, w, scale, gscale, vocab, mtp_vocab_size, token_out, logits_out, ws,
                      stream=None) -> None:
    _need(x, _BF16, "x"); _need(token_out, _I32, "token_out"); _need(logits_out, _F32, "logits_out")
    b, h = x.shape
    _check(lib.mtp_lmhead_argmax(_ptr(x), b, h, int(wd), _ptr(w), _ptr(scale), _ptr(gscale), int(vocab),
                                 int(mtp_vocab_size), _ptr(token_out), _ptr(logits_out), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "mtp_lmhead_argmax")


def mtp_lmhead_argmax_logprob(x, wd, w, scale, gscale, vocab, mtp_vocab_size, token_out, logprob_out, conf_inout,
                              ws, stream=None) -> None:
    _need(x, _BF16, "x"); _need(token_out, _I32, "token_out"); _need(logprob_out, _F32, "logprob_out")
    _need(conf_inout, _F32, "conf_inout")
    b, h = x.shape
    _check(lib.mtp_lmhead_argmax_logprob(_ptr(x), b, h, int(wd), _ptr(w), _ptr(scale), _ptr(gscale), int(vocab),
                                         int(mtp_vocab_size), _ptr(token_out), _ptr(logprob_out), _ptr(conf_inout),
                                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "mtp_lmhead_argmax_logprob")


def mtp_lmhead_argmax_masked(x, wd, w, scale, gscale, vocab, mtp_vocab_size, mask, token_out, allowed_out, ws,
                             stream=None) -> None:
    """mask: int32 [b, mask_words] (or None with 0 words)."""
    _need(x, _BF16, "x"); _need(token_out, _I32, "token_out"); _need(allowed_out, _I32, "allowed_out")
    _need(mask, _I32, "mask")
    b, h = x.shape
    mw = 0 if mask is None else mask.shape[-1]
    _check(lib.mtp_lmhead_argmax_masked(_ptr(x), b, h, int(wd), _ptr(w), _ptr(scale), _ptr(gscale), int(vocab),
                                        int(mtp_vocab_size), _ptr(mask), mw, _ptr(token_out), _ptr(allowed_out),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "mtp_lmhead_argmax_masked")


def mtp_draft_step_workspace_bytes(b: int, h: int) -> int:
    return lib.mtp_draft_step_workspace_bytes(b, h)


def mtp_draft_step(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps, gamma_offset, head,
                   mtp_vocab_size, token_out, x_out, logprob_out, conf_inout, ws, stream=None) -> None:
    """token_ids: a host sequence (checked) or an int32 device tensor (clamped)."""
    for t, nm in ((embed, "embed"), (hidden, "hidden"), (gamma_embed, "gamma_embed"), (gamma_hidden, "gamma_hidden"),
                  (fc, "fc"), (gamma_final, "gamma_final"), (x_out, "x_out")):
        _need(t, _BF16, nm)
    _need(token_out, _I32, "token_out"); _need(logprob_out, _F32, "logprob_out"); _need(conf_inout, _F32, "conf_inout")
    on_dev = isinstance(token_ids, torch.Tensor) and token_ids.is_cuda
    if on_dev:
        _need(token_ids, _I32, "token_ids")
        tok_ptr, keep = _ptr(token_ids), None
    else:
        keep = torch.as_tensor(token_ids, dtype=torch.int32, device="cpu").contiguous()
        tok_ptr = C.c_void_p(keep.data_ptr())
    embed_vocab, h = embed.shape
    b = hidden.shape[0]
    _check(lib.mtp_draft_step(_ptr(embed), embed_vocab, tok_ptr, 1 if on_dev else 0, _ptr(hidden), _ptr(gamma_embed),
                              _ptr(gamma_hidden), _ptr(fc), _ptr(gamma_final), b, h, float(eps), float(gamma_offset),
                              int(head.wd), _ptr(head.w), _ptr(head.scale), _ptr(head.gscale), int(head.vocab),
                              int(mtp_vocab_size), _ptr(token_out), _ptr(x_out), _ptr(logprob_out), _ptr(conf_inout),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "mtp_draft_step")


def mtp_draft_step_noalloc(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps, gamma_offset,
                           head, mtp_vocab_size, token_out, x_out, logprob_out, conf_inout, stream=None) -> None:
    """mtp_draft_step on the library's fixed scratch: no workspace argument."""
    for t, nm in ((embed, "embed"), (hidden, "hidden"), (gamma_embed, "gamma_embed"), (gamma_hidden, "gamma_hidden"),
                  (fc, "fc"), (gamma_final, "gamma_final"), (x_out, "x_out")):
        _need(t, _BF16, nm)
    _need(token_out, _I32, "token_out"); _need(logprob_out, _F32, "logprob_out"); _need(conf_inout, _F32, "conf_inout")
    on_dev = isinstance(token_ids, torch.Tensor) and token_ids.is_cuda
    if on_dev:
        _need(token_ids, _I32, "token_ids")
        tok_ptr, keep = _ptr(token_ids), None
    else:
        keep = torch.as_tensor(token_ids, dtype=torch.int32, device="cpu").contiguous()
        tok_ptr = C.c_void_p(keep.data_ptr())
    embed_vocab, h = embed.shape
    b = hidden.shape[0]
    _check(lib.mtp_draft_step_noalloc(_ptr(embed), embed_vocab, tok_ptr, 1 if on_dev else 0, _ptr(hidden),
                                      _ptr(gamma_embed), _ptr(gamma_hidden), _ptr(fc), _ptr(gamma_final), b, h,
                                      float(eps), float(gamma_offset), int(head.wd), _ptr(head.w), _ptr(head.scale),
                                      _ptr(head.gscale), int(head.vocab), int(mtp_vocab_size), _ptr(token_out),
                                      _ptr(x_out), _ptr(logprob_out), _ptr(conf_inout), _stream(stream)),
           "mtp_draft_step_noalloc")


def mtp_codec_encode_range(codec: int, first_bits: int, count: int, out, stream=None) -> None:
    """out: uint8 [count] for E4M3 / E2M1 (codec 0 / 1), 16-bit [count] for BF16 (codec 2)."""
    _need(out, _BF16 if int(codec) == MTP_CODEC_BF16 else _U8, "out")
    if out is not None and out.numel() < int(count):
        raise ValueError(f"mtp_codec_encode_range: count {count} past the buffer's {out.numel()} codes")
    _check(lib.mtp_codec_encode_range(int(codec), int(first_bits), int(count), _ptr(out), _stream(stream)),
           "mtp_codec_encode_range")


def mtp_stream_read(buf, nbytes: int, magic: int, sink, stream=None, shape: int = 0) -> None:
    """The streaming-read reference kernel over the first nbytes of buf (any
    device tensor) in launch shape 0..3; sink: device int32/uint32 [1]."""
    if int(nbytes) > buf.numel() * buf.element_size():
        raise ValueError(f"mtp_stream_read: {nbytes} bytes past the buffer's {buf.numel() * buf.element_size()}")
    _check(lib.mtp_stream_read(_ptr(buf), int(nbytes), int(shape), int(magic) & 0xFFFFFFFF, _ptr(sink),
                               _stream(stream)),
           "mtp_stream_read")


# ------------------------------------------------------------------- helpers ----

WDTYPES = {"bf16": MTP_W_BF16, "fp8": MTP_W_FP8_E4M3_ROW, "nvfp4": MTP_W_NVFP4}


def parse_wdtype(s: str) -> int:
    """'nvfp4' or 'fp4', 'fp8', 'bf16', case-insensitive (mtp_head.rs,
    `MtpQuantization::from_str`)."""
    k = s.lower()
    if k == "fp4":
        k = "nvfp4"
    if k not in WDTYPES:
        raise ValueError(f"Unknown MTP quantization: {s}. Expected: nvfp4, fp8, bf16")
    return WDTYPES[k]


@dataclass
class LmHead:
    """A draft lm_head in one of the three precisions (device tensors)."""
    wd: int
    w: torch.Tensor                 # bf16 [V, h] | u8 [V, h] | u8 [V, h/2]
    scale: torch.Tensor | None      # None | f32 [V] | u8 [V, h/16]
    gscale: torch.Tensor | None     # None | f32 [1]
    vocab: int
    hidden: int


def zeroed_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace (16-byte aligned: torch allocations are)."""
    return torch.zeros(max(16, (nbytes + 15) // 16 * 16), dtype=torch.uint8, device=device)


def quantize_head(w_bf16: torch.Tensor, wdtype: str, stream=None) -> LmHead:
    wd = parse_wdtype(wdtype)
    V, h = w_bf16.shape
    dev = w_bf16.device
    if wd == MTP_W_BF16:
        return LmHead(wd, w_bf16, None, None, V, h)
    with _on(stream):
        if wd == MTP_W_FP8_E4M3_ROW:
            codes = torch.empty((V, h), dtype=torch.uint8, device=dev)
            scale = torch.empty(V, dtype=torch.float32, device=dev)
            mtp_quantize_fp8(w_bf16, codes, scale)
            return LmHead(wd, codes, scale, None, V, h)
        codes = torch.empty((V, h // 2), dtype=torch.uint8, device=dev)
        bs = torch.empty((V, h // 16), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(mtp_quantize_nvfp4_workspace_bytes(V, h), dtype=torch.uint8, device=dev)
        mtp_quantize_nvfp4(w_bf16, codes, bs, g, ws)
        return LmHead(wd, codes, bs, g, V, h)


def lmhead_argmax(x: torch.Tensor, head: LmHead, mtp_vocab_size: int = 0, with_logits: bool = False,
                  ws: torch.Tensor | None = None, token_out: torch.Tensor | None = None, stream=None):
    b = x.shape[0]
    dev = x.device
    n_eff = min(mtp_vocab_size, head.vocab) if mtp_vocab_size > 0 else head.vocab
    with _on(stream):
        if ws is None:
            ws = zeroed_workspace(mtp_lmhead_argmax_workspace_bytes(head.vocab, head.hidden, b, head.wd), dev)
        if token_out is None:
            token_out = torch.empty(b, dtype=torch.int32, device=dev)
        logits = torch.empty((b, n_eff), dtype=torch.float32, device=dev) if with_logits else None
        mtp_lmhead_argmax(x, head.wd, head.w, head.scale, head.gscale, head.vocab, mtp_vocab_size, token_out, logits,
                          ws)
    return (token_out, logits) if with_logits else token_out


def lmhead_argmax_logprob(x: torch.Tensor, head: LmHead, mtp_vocab_size: int = 0, conf: torch.Tensor | None = None,
                          ws: torch.Tensor | None = None, stream=None):
    """(token [b] int32, top-1 log-probability [b] f32); `conf` [b] f32, if given, is
    lowered to the top-1 probability where that is smaller."""
    b = x.shape[0]
    dev = x.device
    with _on(stream):
        if ws is None:
            ws = zeroed_workspace(mtp_lmhead_argmax_workspace_bytes(head.vocab, head.hidden, b, head.wd), dev)
        tok = torch.empty(b, dtype=torch.int32, device=dev)
        lp = torch.empty(b, dtype=torch.float32, device=dev)
        mtp_lmhead_argmax_logprob(x, head.wd, head.w, head.scale, head.gscale, head.vocab, mtp_vocab_size, tok, lp,
                                  conf, ws)
    return tok, lp


def lmhead_argmax_masked(x: torch.Tensor, head: LmHead, mask: torch.Tensor | None, mtp_vocab_size: int = 0,
                         ws: torch.Tensor | None = None, stream=None):
    """(token [b] int32, allowed [b] int32) of the argmax over the rows `mask`
    ([b, words] int32, bit r % 32 of word r / 32) allows."""
    b = x.shape[0]
    dev = x.device
    with _on(stream):
        if ws is None:
            ws = zeroed_workspace(mtp_lmhead_argmax_workspace_bytes(head.vocab, head.hidden, b, head.wd), dev)
        tok = torch.empty(b, dtype=torch.int32, device=dev)
        allowed = torch.empty(b, dtype=torch.int32, device=dev)
        mtp_lmhead_argmax_masked(x, head.wd, head.w, head.scale, head.gscale, head.vocab, mtp_vocab_size, mask, tok,
                                 allowed, ws)
    return tok, allowed


def draft_step(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, head: LmHead, eps=1e-6,
               gamma_offset=0.0, mtp_vocab_size=0, with_x=False, with_logprob=False, conf=None, ws=None, stream=None,
               noalloc=False):
    """One draft in one call (mtp_draft_step: the combine, then the lm_head sweep
    with the final norm applied per block): token [b] (and x [b, h],
    log-probability [b] when asked). noalloc=True takes mtp_draft_step_noalloc
    (the library's fixed scratch instead of a workspace)."""
    b, h = hidden.shape
    dev = hidden.device
    with _on(stream):
        if ws is None and not noalloc:
            ws = zeroed_workspace(mtp_draft_step_workspace_bytes(b, h), dev)
        tok = torch.empty(b, dtype=torch.int32, device=dev)
        x = torch.empty((b, h), dtype=hidden.dtype, device=dev) if with_x else None
        lp = torch.empty(b, dtype=torch.float32, device=dev) if (with_logprob or conf is not None) else None
        if noalloc:
            mtp_draft_step_noalloc(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps,
                                   gamma_offset, head, mtp_vocab_size, tok, x, lp, conf)
        else:
            mtp_draft_step(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps, gamma_offset,
                           head, mtp_vocab_size, tok, x, lp, conf, ws)
    out = [tok]
    if with_x:
        out.append(x)
    if with_logprob:
        out.append(lp)
    return tok if len(out) == 1 else tuple(out)


def draft_combine(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps=1e-6,
                  gamma_offset=0.0, ws=None, x_out=None, stream=None):
    b, h = hidden.shape
    dev = hidden.device
    with _on(stream):
        if ws is None:
            ws = zeroed_workspace(mtp_draft_combine_workspace_bytes(b, h), dev)
        if x_out is None:
            x_out = torch.empty((b, h), dtype=hidden.dtype, device=dev)
        mtp_draft_combine(embed, token_ids, hidden, gamma_embed, gamma_hidden, fc, gamma_final, eps, gamma_offset,
                          x_out, ws)
    return x_out


def _round256(n: int) -> int:
    return (n + 255) // 256 * 256


def combine_intermediates(ws: torch.Tensor, b: int, h: int):
    """(c [b, 2h], u [b, h]) as BF16 views of a combine workspace after the call
    (the layout include/mtp_draft.h documents)."""
    c0 = MTP_COMBINE_WS_C_OFFSET
    u0 = c0 + _round256(4 * b * h)
    c = ws[c0:c0 + 4 * b * h].view(torch.bfloat16).view(b, 2 * h)
    u = ws[u0:u0 + 2 * b * h].view(torch.bfloat16).view(b, h)
    return c, u


def step_intermediates(ws: torch.Tensor, b: int, h: int):
    """(c [b, 2h], u [b, h]) as BF16 views of a draft-step workspace after the call."""
    u0 = MTP_STEP_WS_U_OFFSET
    c0 = u0 + _round256(2 * b * h)
    u = ws[u0:u0 + 2 * b * h].view(torch.bfloat16).view(b, h)
    c = ws[c0:c0 + 4 * b * h].view(torch.bfloat16).view(b, 2 * h)
    return c, u
