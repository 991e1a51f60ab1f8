"""GPU parity of the matrix-core (MFMA) form of the lm_head sweep + fused argmax,
the form wide batches take, against the oracle, through the C ABI.

Shapes (BF16, FP8, NVFP4): row counts that leave a partial last 16-row tile, a
single row, row lengths of one and several MFMA units (h = 256 .. 8192),
truncation; planted
exact duplicates at different positions inside and across tiles; vector order
and batch width not changing a vector's logits; NVFP4 vectors whose
magnitudes sit far from 1 (the F16 staging scales each vector by a power of 2).
The full-size heads at b = 4 and 8 (test_gpu_lmhead.py) take this form too.
"""
import pytest
import torch

import synthetic_inputs as si
from parity import DEV, check_lmhead, head_host, lm_form, log, mtp

pytestmark = pytest.mark.gpu


def make_head(wdtype, vocab, h, seed, outlier_p=0.0):
    m = mtp()
    W = si.normal_bf16(seed, si.TAG_LM, vocab, h, std=0.02, outlier_p=outlier_p, device=DEV)
    head = m.quantize_head(W, wdtype)
    torch.cuda.synchronize()
    return W, head


CASES = [
    # wdtype, vocab, h, b, mtp_vocab_size
    ("fp8", 4099, 4096, 8, 0),
    ("fp8", 4100, 5120, 3, 0),
    ("fp8", 1001, 512, 6, 777),
    ("fp8", 1, 4096, 8, 0),
    ("nvfp4", 4099, 4096, 8, 0),
    ("nvfp4", 3001, 5120, 3, 0),
    ("nvfp4", 1037, 1024, 5, 1000),
    ("nvfp4", 17, 4096, 8, 0),
    ("nvfp4", 2049, 8192, 5, 0),
    ("fp8", 1500, 8192, 5, 0),
    # BF16 (four waves per tile: h a multiple of 1024 up to 4096)
    ("bf16", 4099, 4096, 8, 0),
    ("bf16", 1037, 1024, 3, 1000),
    ("bf16", 2049, 2048, 6, 0),
    ("bf16", 17, 4096, 5, 0),
    ("bf16", 1, 3072, 4, 0),
]


@pytest.mark.parametrize("wdtype,vocab,h,b,mvs", CASES)
def test_mfma_small(wdtype, vocab, h, b, mvs):
    assert lm_form(wdtype, b, h) == "mfma"
    m = mtp()
    log(f"mfma small {wdtype} V={vocab} h={h} b={b} mvs={mvs}")
    W, head = make_head(wdtype, vocab, h, seed=3 * vocab + h + b, outlier_p=0.01 if wdtype == "nvfp4" else 0.0)
    x = si.normal_bf16(17 + b, si.TAG_X, b, h, device=DEV)
    tok, lg = m.lmhead_argmax(x, head, mtp_vocab_size=mvs, with_logits=True)
    torch.cuda.synchronize()
    check_lmhead(si.bits(x), head_host(head), vocab, mvs, tok.cpu().numpy(), lg.cpu().numpy(), label=wdtype)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "nvfp4"])
def test_mfma_planted_duplicates(wdtype):
    """Copies of vector 0's winning row at other tile positions give the same
    bits for every vector; the lowest copy wins."""
    m = mtp()
    V, h, b = 20011, 4096, 8
    log(f"mfma duplicates {wdtype}")
    W = si.normal_bf16(51, si.TAG_LM, V, h, std=0.02, device=DEV)
    x = si.normal_bf16(52, si.TAG_X, b, h, device=DEV)
    head = m.quantize_head(W, wdtype)
    tok0, _ = m.lmhead_argmax(x, head, with_logits=True)
    i_star = int(tok0[0])
    for j in (3, 16 + 9, 4096 + 15, V - 2, i_star - 1, i_star + 1):
        if j < 0 or j >= V or j == i_star:
            continue
        W2 = W.clone()
        W2[j] = W[i_star]
        head2 = m.quantize_head(W2, wdtype)
        tok, lg = m.lmhead_argmax(x, head2, with_logits=True)
        torch.cuda.synchronize()
        bits = lg.view(torch.int32)
        assert torch.equal(bits[:, j], bits[:, i_star]), j
        assert int(tok[0]) == min(i_star, j), (j, i_star, int(tok[0]))


@pytest.mark.parametrize("wdtype,h", [("fp8", 5120), ("nvfp4", 5120), ("fp8", 4096), ("nvfp4", 4096), ("bf16", 4096),
                                     ("bf16", 1024)])
def test_mfma_vector_order_and_width(wdtype, h):
    """A vector's logits do not depend on its position in the call or on how
    many other vectors share the call (within the MFMA form; FP8 at h = 4096
    takes the split schedule, two waves per tile, BF16 four)."""
    m = mtp()
    V = 3001
    W, head = make_head(wdtype, V, h, seed=61)
    x = si.normal_bf16(62, si.TAG_X, 8, h, device=DEV)
    _, l8 = m.lmhead_argmax(x, head, with_logits=True)
    perm = torch.tensor([5, 2, 7, 0, 3, 6, 1, 4], device=DEV)
    _, lp = m.lmhead_argmax(x[perm].contiguous(), head, with_logits=True)
    assert torch.equal(lp.view(torch.int32), l8[perm].view(torch.int32))
    for b in range(8, 0, -1):
        if lm_form(wdtype, b, h) != "mfma":
            break
        _, lb = m.lmhead_argmax(x[8 - b:].contiguous(), head, with_logits=True)
        assert torch.equal(lb.view(torch.int32), l8[8 - b:].view(torch.int32)), b


def test_mfma_nvfp4_vector_scales():
    """NVFP4 vectors far from unit magnitude (2^-100, 2^60, all zero) stage in
    F16 exactly (power-of-2 scaling) and take the MFMA form; a vector F16
    cannot hold (one huge entry beside small ones) sends the call to the VALU
    sweep, whose rows are the same bits as a narrower VALU call's."""
    m = mtp()
    V, h = 2053, 4096
    W, head = make_head("nvfp4", V, h, seed=71, outlier_p=0.01)
    base = si.normal_bf16(72, si.TAG_X, 4, h, device=DEV).float()
    x = torch.empty_like(base)
    x[0] = base[0] * 2.0 ** -100
    x[1] = base[1] * 2.0 ** 60
    x[2] = base[2]
    x[3] = 0.0
    x = x.to(torch.bfloat16)
    assert lm_form("nvfp4", 4, h) == "mfma"
    tok, lg = m.lmhead_argmax(x, head, with_logits=True)
    torch.cuda.synchronize()
    assert torch.isfinite(lg).all()
    assert (lg[3] == 0).all() and int(tok[3]) == 0
    check_lmhead(si.bits(x), head_host(head), V, 0, tok.cpu().numpy(), lg.cpu().numpy(), label="nvfp4 scales")
    # the staged F16 vectors of x[0], x[1] equal those of base[0], base[1]: logits differ by the power of 2
    _, lb = m.lmhead_argmax(x[2:3].expand(4, h).contiguous(), head, with_logits=True)
    _, l01 = m.lmhead_argmax(torch.stack([base[0], base[1], base[2], base[2]]).to(torch.bfloat16), head,
                             with_logits=True)
    assert torch.equal(lb[0].view(torch.int32), lg[2].view(torch.int32))
    assert torch.equal((lg[0].double() * 2.0 ** 100), l01[0].double())
    assert torch.equal((lg[1].double() * 2.0 ** -60), l01[1].double())
    # one entry 2^101 above the others' scale: the VALU sweep, bit-equal to the b = 2 VALU call
    y = base[:3].clone()
    y[0] = base[0] * 1e-3
    y[0, 5] = 3e30
    y = y.to(torch.bfloat16)
    assert lm_form("nvfp4", 3, h) == "mfma" and lm_form("nvfp4", 2, h) == "valu"
    t3, l3 = m.lmhead_argmax(y, head, with_logits=True)
    t2, l2 = m.lmhead_argmax(y[:2].contiguous(), head, with_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(l3[:2].view(torch.int32), l2.view(torch.int32))
    assert torch.equal(t3[:2], t2)
    check_lmhead(si.bits(y), head_host(head), V, 0, t3.cpu().numpy(), l3.cpu().numpy(), label="nvfp4 fallback")
