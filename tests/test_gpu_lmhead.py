"""GPU parity of the draft lm_head sweep + fused argmax (mtp_lmhead_argmax) and
of the weight quantizers that feed it, against the oracle, through the C ABI.

Shapes span several blocks and waves with ragged tails (odd row counts, row
lengths that leave lanes idle), all batch widths 1..8, truncation, planted
exact duplicates, a NaN row, and the full-size heads of the workload list.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity import DEV, check_lmhead, check_quantized, head_host, lm_form, log, mtp

pytestmark = pytest.mark.gpu


def make_head(wdtype, vocab, h, seed, outlier_p=0.0):
    m = mtp()
    W = si.normal_bf16(seed, si.TAG_LM, vocab, h, std=0.02, outlier_p=outlier_p, device=DEV)
    head = m.quantize_head(W, wdtype)
    torch.cuda.synchronize()
    return W, head


SMALL = [
    # wdtype, vocab, h, b, mtp_vocab_size
    ("bf16", 4099, 256, 1, 0),
    ("bf16", 4099, 4096, 3, 0),
    ("bf16", 777, 5120, 8, 0),
    ("bf16", 5000, 4096, 2, 2050),
    ("bf16", 1, 4096, 1, 0),
    ("bf16", 3, 16, 5, 0),
    ("fp8", 4099, 4096, 1, 0),
    ("fp8", 5001, 5120, 8, 0),
    ("fp8", 3001, 48, 2, 0),
    ("fp8", 4099, 4096, 6, 4000),
    ("nvfp4", 4099, 4096, 1, 0),
    ("nvfp4", 3333, 5120, 4, 0),
    ("nvfp4", 2048, 256, 8, 1000),
    ("nvfp4", 4097, 8192, 7, 0),
    # single-vector NVFP4 rows of 129..192 chunks take one pass of 3 chunks per lane
    ("nvfp4", 4099, 5120, 1, 0),
    ("nvfp4", 3001, 4608, 1, 1500),
    ("nvfp4", 2999, 6144, 1, 0),
    ("nvfp4", 1000, 1280, 1, 300),
    ("nvfp4", 2003, 6400, 1, 0),
]


@pytest.mark.parametrize("wdtype,vocab,h,b,mvs", SMALL)
def test_lmhead_small(wdtype, vocab, h, b, mvs):
    m = mtp()
    log(f"lmhead small {wdtype} V={vocab} h={h} b={b} mvs={mvs}")
    W, head = make_head(wdtype, vocab, h, seed=vocab + h + b, outlier_p=0.01 if wdtype == "nvfp4" else 0.0)
    Wb = si.bits(W)
    check_quantized(head, Wb)
    x = si.normal_bf16(7 + b, si.TAG_X, b, h, device=DEV)
    tok, lg = m.lmhead_argmax(x, head, mtp_vocab_size=mvs, with_logits=True)
    torch.cuda.synchronize()
    check_lmhead(si.bits(x), head_host(head), vocab, mvs, tok.cpu().numpy(), lg.cpu().numpy(), label=wdtype)


def _draw_lmhead(rng):
    """One shape within the header's limits: format, vocab, h (a multiple of 16,
    of 256 for NVFP4, up to 8192), b and, one time in three, a truncation. Half
    the draws take h on the 1,024 grid and b >= 3, where the matrix-core form
    runs (the library's own choice decides; the log names it)."""
    wdtype = str(rng.choice(["bf16", "fp8", "nvfp4"]))
    if rng.random() < 0.5:
        h = 1024 * int(rng.integers(1, 9))
        b = int(rng.integers(3, 9))
    else:
        h = 256 * int(rng.integers(1, 33)) if wdtype == "nvfp4" else 16 * int(rng.integers(1, 513))
        b = int(rng.integers(1, 9))
    vocab = int(rng.integers(1, 6001))
    mvs = int(rng.integers(1, vocab + 1)) if rng.random() < 1 / 3 else 0
    return wdtype, vocab, h, b, mvs


RANDOM = [_draw_lmhead(np.random.default_rng(9000 + i)) for i in range(24)]


@pytest.mark.parametrize("case", range(len(RANDOM)))
def test_lmhead_random_shapes(case):
    """Seeded random shapes, so kernel forms, ragged passes and tile tails meet
    shapes that no hand-picked case names; each case logs its draw."""
    wdtype, vocab, h, b, mvs = RANDOM[case]
    m = mtp()
    log(f"lmhead random #{case}: {wdtype} V={vocab} h={h} b={b} mvs={mvs} form={lm_form(wdtype, b, h)}")
    W, head = make_head(wdtype, vocab, h, seed=9100 + case, outlier_p=0.01 if wdtype == "nvfp4" else 0.0)
    check_quantized(head, si.bits(W))
    x = si.normal_bf16(9200 + case, si.TAG_X, b, h, device=DEV)
    tok, lg = m.lmhead_argmax(x, head, mtp_vocab_size=mvs, with_logits=True)
    torch.cuda.synchronize()
    check_lmhead(si.bits(x), head_host(head), vocab, mvs, tok.cpu().numpy(), lg.cpu().numpy(),
                 label=f"random #{case}")


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "nvfp4"])
def test_batch_rows_bit_identical_within_a_kernel_form(wdtype):
    """Row b of a call gives the same f32 logits, bit for bit, in every call of
    a width that takes the same kernel form (the VALU sweep below the format's
    matrix-core threshold, the MFMA sweep from it on); across the two forms
    every row agrees with the oracle within tau."""
    m = mtp()
    W, head = make_head(wdtype, 3001, 4096, seed=11)
    x = si.normal_bf16(12, si.TAG_X, 8, 4096, device=DEV)
    calls = {}
    for b in range(1, 9):
        calls[b] = m.lmhead_argmax(x[:b].contiguous(), head, with_logits=True)
    for form in ("valu", "mfma"):
        widths = [b for b in calls if lm_form(wdtype, b, 4096) == form]
        if not widths:
            continue
        tw, lw = calls[max(widths)]
        check_lmhead(si.bits(x[:max(widths)]), head_host(head), 3001, 0, tw.cpu().numpy(), lw.cpu().numpy(),
                     label=f"{wdtype} {form} b={max(widths)}")
        for b in widths:
            tb, lb = calls[b]
            assert torch.equal(lb.view(torch.int32), lw[:b].view(torch.int32)), (form, b)
            assert torch.equal(tb, tw[:b]), (form, b)
    # any single vector alone, in the VALU form: the same bits as in a wider VALU call
    valu = [b for b in calls if lm_form(wdtype, b, 4096) == "valu"]
    if valu:
        tw, lw = calls[max(valu)]
        for bi in range(max(valu)):
            t1, l1 = m.lmhead_argmax(x[bi:bi + 1].contiguous(), head, with_logits=True)
            assert torch.equal(l1[0].view(torch.int32), lw[bi].view(torch.int32)), bi
            assert int(t1[0]) == int(tw[bi])


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "nvfp4"])
def test_planted_duplicate_lowest_index(wdtype):
    """Copy the winning row to a lower index in another block: the copy wins;
    copy it to a higher index: the original still wins. Duplicates give
    bit-identical logits wherever they sit."""
    m = mtp()
    V, h = 20011, 4096
    W = si.normal_bf16(21, si.TAG_LM, V, h, std=0.02, device=DEV)
    x = si.normal_bf16(22, si.TAG_X, 1, h, device=DEV)
    head = m.quantize_head(W, wdtype)
    tok0, lg0 = m.lmhead_argmax(x, head, with_logits=True)
    i_star = int(tok0[0])
    for j in (3, V - 2, i_star - 1, i_star + 1):
        if j < 0 or j >= V or j == i_star:
            continue
        W2 = W.clone()
        W2[j] = W[i_star]
        head2 = m.quantize_head(W2, wdtype)
        tok, lg = m.lmhead_argmax(x, head2, with_logits=True)
        torch.cuda.synchronize()
        if wdtype == "nvfp4":
            # a copied row keeps its codes only if the global scale is unchanged (it is: same max)
            assert torch.equal(head2.w[j], head2.w[i_star])
        bits = lg[0].view(torch.int32)
        assert int(bits[j]) == int(bits[i_star]), j
        assert int(tok[0]) == min(i_star, j), (j, i_star, int(tok[0]))


def test_nan_row_never_wins_and_equal_rows():
    m = mtp()
    V, h = 600, 256
    W = si.normal_bf16(31, si.TAG_LM, V, h, std=0.02, device=DEV)
    x = si.normal_bf16(32, si.TAG_X, 2, h, device=DEV)
    W[0, 5] = float("nan")
    head = m.quantize_head(W, "bf16")
    tok, lg = m.lmhead_argmax(x, head, with_logits=True)
    assert torch.isnan(lg[:, 0]).all()
    assert (tok != 0).all()
    Wb = si.bits(W)
    tok_o, _ = oracle.lmhead_argmax(si.bits(x), "bf16", Wb)
    assert tok.cpu().numpy().tolist() == tok_o.tolist()
    # every row equal -> every logit equal -> token 0
    Weq = W[1:2].expand(V, h).contiguous()
    tok, lg = m.lmhead_argmax(x, m.quantize_head(Weq, "bf16"), with_logits=True)
    assert (tok == 0).all() and (lg == lg[:, :1]).all()


def test_truncation_boundary():
    """A planted maximum at row n_eff is excluded; at row n_eff - 1 it wins."""
    m = mtp()
    V, h, n_eff = 9000, 512, 4096
    W = si.normal_bf16(41, si.TAG_LM, V, h, std=0.02, device=DEV)
    x = si.normal_bf16(42, si.TAG_X, 1, h, device=DEV)
    plant = (torch.sign(x[0].float()) * 0.5).to(torch.bfloat16)
    W[n_eff] = plant
    head = m.quantize_head(W, "bf16")
    tok = m.lmhead_argmax(x, head, mtp_vocab_size=n_eff)
    assert int(tok[0]) != n_eff and int(tok[0]) < n_eff
    tok = m.lmhead_argmax(x, head, mtp_vocab_size=0)
    assert int(tok[0]) == n_eff
    W[n_eff - 1] = plant
    tok = m.lmhead_argmax(x, m.quantize_head(W, "bf16"), mtp_vocab_size=n_eff)
    assert int(tok[0]) == n_eff - 1
    tok = m.lmhead_argmax(x, m.quantize_head(W, "bf16"), mtp_vocab_size=10 ** 9)
    assert int(tok[0]) == n_eff - 1


def test_workspace_reuse_and_streams():
    """The workspace is left ready for the next call: many calls on one
    workspace, and calls on another stream with its own workspace, give the
    same tokens."""
    m = mtp()
    V, h = 10007, 4096
    W, head = make_head("fp8", V, h, seed=51)
    x = si.normal_bf16(52, si.TAG_X, 4, h, device=DEV)
    ws = m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(V, h, 4, head.wd), DEV)
    ref = m.lmhead_argmax(x, head, ws=ws).clone()
    for _ in range(20):
        assert torch.equal(m.lmhead_argmax(x, head, ws=ws), ref)
    assert int(ws[:256].count_nonzero()) == 0  # the completion counter is back at zero
    s = torch.cuda.Stream()
    ws2 = m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(V, h, 4, head.wd), DEV)
    with torch.cuda.stream(s):
        t2 = m.lmhead_argmax(x, head, ws=ws2)
    s.synchronize()
    assert torch.equal(t2, ref)


@pytest.mark.parametrize("wdtype,b", [("bf16", 1), ("bf16", 2), ("bf16", 4), ("fp8", 1), ("fp8", 2), ("fp8", 8),
                                       ("nvfp4", 1), ("nvfp4", 2), ("nvfp4", 8)])
def test_running_max_reset_between_calls(wdtype, b):
    """Each call leaves the workspace's running keys and counter at zero: a
    second call on the same workspace whose winners have smaller logits (x2 =
    -x1 / 2, so each winner is the first call's loser) returns what it returns
    on a fresh workspace, for every kernel form (static and shared-group VALU
    blocks, the matrix-core sweep)."""
    m = mtp()
    V, h = 4099, 4096
    log(f"running max reset {wdtype} b={b} form={lm_form(wdtype, b, h)}")
    W, head = make_head(wdtype, V, h, seed=61 + b)
    x1 = si.normal_bf16(62 + b, si.TAG_X, b, h, device=DEV)
    x2 = (x1.float() * -0.5).to(torch.bfloat16)
    fresh = lambda x: m.lmhead_argmax(
        x, head, ws=m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(V, h, b, head.wd), DEV)).clone()
    r1, r2 = fresh(x1), fresh(x2)
    assert not torch.equal(r1, r2)
    ws = m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(V, h, b, head.wd), DEV)
    for _ in range(3):
        assert torch.equal(m.lmhead_argmax(x1, head, ws=ws), r1)
        assert torch.equal(m.lmhead_argmax(x2, head, ws=ws), r2)
    torch.cuda.synchronize()
    assert int(ws[:256].count_nonzero()) == 0


# ------------------------------------------------------------ full size ----

_CACHE = {}


def full_head(vocab, h, wdtype, outlier_p):
    key = (vocab, h, outlier_p)
    if key not in _CACHE:
        _CACHE.clear()
        log(f"  generating W {vocab}x{h} outliers={outlier_p}")
        W = si.normal_bf16(0, si.TAG_LM, vocab, h, std=0.02, outlier_p=outlier_p, device=DEV)
        _CACHE[key] = (W, si.bits(W), {})
    W, Wb, heads = _CACHE[key]
    if wdtype not in heads:
        log(f"  quantizing {wdtype} on the GPU and checking codes against the oracle")
        head = mtp().quantize_head(W, wdtype)
        torch.cuda.synchronize()
        check_quantized(head, Wb)
        heads[wdtype] = (head, head_host(head))
    return heads[wdtype]


FULL = [
    # name in the workload list, wdtype, vocab, h, b, mtp_vocab_size, outliers
    ("bf16_154880x4096_b1", "bf16", 154880, 4096, 1, 0, 0.0),
    ("bf16_154880x4096_b4", "bf16", 154880, 4096, 4, 0, 0.0),
    ("fp8_154880x4096_b1", "fp8", 154880, 4096, 1, 0, 0.0),
    ("fp8_154880x4096_b2", "fp8", 154880, 4096, 2, 0, 0.0),
    ("fp8_154880x4096_b4", "fp8", 154880, 4096, 4, 0, 0.0),
    ("fp8_154880x4096_b8", "fp8", 154880, 4096, 8, 0, 0.0),
    ("nvfp4_154880x4096_b1", "nvfp4", 154880, 4096, 1, 0, 0.0),
    ("nvfp4_131072x5120_b1", "nvfp4", 131072, 5120, 1, 0, 0.01),
    ("nvfp4_131072x5120_b4", "nvfp4", 131072, 5120, 4, 0, 0.01),
    ("nvfp4_131072x5120_b8", "nvfp4", 131072, 5120, 8, 0, 0.01),
    ("nvfp4_131072x5120_t32768_b1", "nvfp4", 131072, 5120, 1, 32768, 0.01),
    ("nvfp4_131072x5120_t32768_b4", "nvfp4", 131072, 5120, 4, 32768, 0.01),
    ("nvfp4_131072x5120_t32768_b8", "nvfp4", 131072, 5120, 8, 32768, 0.01),
]


@pytest.mark.parametrize("name,wdtype,vocab,h,b,mvs,outl", FULL, ids=[f[0] for f in FULL])
def test_lmhead_full_size(name, wdtype, vocab, h, b, mvs, outl):
    m = mtp()
    log(f"lmhead full {name}")
    head, hh = full_head(vocab, h, wdtype, outl)
    stats = {"decidable": 0, "rows": 0}
    for seed in (0, 1):
        x = si.normal_bf16(seed, si.TAG_X, b, h, device=DEV)
        tok, lg = m.lmhead_argmax(x, head, mtp_vocab_size=mvs, with_logits=True)
        torch.cuda.synchronize()
        st = check_lmhead(si.bits(x), hh, vocab, mvs, tok.cpu().numpy(), lg.cpu().numpy(), label=name)
        stats["decidable"] += st["decidable"]
        stats["rows"] += st["rows"]
    log(f"  {name}: decidable rows {stats['decidable']}/{stats['rows']}")


@pytest.mark.parametrize("wdtype", ["bf16", "fp8"])
def test_max_vocab_closed_form(wdtype):
    """The largest vocabulary the call accepts (2^31 - 1 rows, at h = 16: 64 GiB
    of BF16 or 32 GiB of FP8 codes), all rows zero except planted ones, so the
    tokens and the log-probability are known in closed form: vector 0 meets
    two equal top rows at the very end of the head (the lower index wins),
    vector 1 one top row in the middle; truncating before the last two rows
    leaves vector 0 with all-zero logits but one (the first row wins)."""
    m = mtp()
    V, h = 2 ** 31 - 1, 16
    need = V * h * (2 if wdtype == "bf16" else 1) + (V * 4 if wdtype == "fp8" else 0)
    if torch.cuda.mem_get_info()[0] < need + (8 << 30):
        pytest.skip("not enough device memory for the largest head")
    log(f"max vocab {wdtype}: {V} rows x {h}")
    s = torch.tensor([1.0, -1.0] * (h // 2))
    x = torch.stack([s, -s]).to(torch.bfloat16).to(DEV)
    mid = 2 ** 30 + 5
    if wdtype == "bf16":
        w = torch.zeros((V, h), dtype=torch.bfloat16, device=DEV)
        w[V - 2] = s.to(torch.bfloat16)
        w[V - 1] = s.to(torch.bfloat16)
        w[mid] = (-s).to(torch.bfloat16)
        head = m.LmHead(m.MTP_W_BF16, w, None, None, V, h)
    else:  # E4M3 codes of +-1 (0x38, 0xB8), every row scale 1
        code = lambda v: torch.where(v > 0, torch.tensor(0x38), torch.tensor(0xB8)).to(torch.uint8)
        w = torch.zeros((V, h), dtype=torch.uint8, device=DEV)
        w[V - 2] = code(s)
        w[V - 1] = code(s)
        w[mid] = code(-s)
        head = m.LmHead(m.MTP_W_FP8_E4M3_ROW, w, torch.ones(V, dtype=torch.float32, device=DEV), None, V, h)
    tok = m.lmhead_argmax(x, head)
    tok_t = m.lmhead_argmax(x, head, mtp_vocab_size=V - 2)
    tok_lp, lp = m.lmhead_argmax_logprob(x, head)
    torch.cuda.synchronize()
    assert tok.cpu().tolist() == [V - 2, mid]
    assert tok_t.cpu().tolist() == [0, mid]
    assert tok_lp.cpu().tolist() == [V - 2, mid]
    # top logit 16; the rest 0 but one at -16 (vector 0: two tops; vector 1: one)
    e = np.exp(-16.0)
    want = [-np.log(2 + (V - 3) * e + e * e), -np.log(1 + (V - 3) * e + 2 * e * e)]
    got = lp.cpu().numpy().astype(np.float64)
    log(f"  log-probability {got.tolist()} closed form {want}")
    assert np.allclose(got, want, atol=2e-3), (got, want)
    del w, head
    torch.cuda.empty_cache()


def test_host_threads_on_their_own_streams():
    """Four host threads, each with its own stream and workspaces, call the
    lm_head entry point on heads of all three formats and both kernel forms at
    once (the library's per-device caches shared among them): every call gives
    the tokens and logits that the same call gives alone."""
    import threading

    m = mtp()
    V, h = 20011, 4096
    heads = {wd: make_head(wd, V, h, seed=71 + i)[1] for i, wd in enumerate(("bf16", "fp8", "nvfp4"))}
    jobs = [(wd, b) for wd in heads for b in (1, 5)]
    xs = {b: si.normal_bf16(80 + b, si.TAG_X, b, h, device=DEV) for b in (1, 5)}
    ref = {}
    for wd, b in jobs:
        tok, lg = m.lmhead_argmax(xs[b], heads[wd], with_logits=True)
        ref[wd, b] = (tok.clone(), lg.clone())
    torch.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            outs = []
            for it in range(12):
                wd, b = jobs[(k + it) % len(jobs)]
                outs.append(((wd, b), m.lmhead_argmax(xs[b], heads[wd], with_logits=True, stream=s)))
            s.synchronize()
            for key, (tok, lg) in outs:
                if not (torch.equal(tok, ref[key][0]) and torch.equal(lg, ref[key][1])):
                    errors.append((k, key))
        except Exception as e:  # reported below; a thread's exception is otherwise lost
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
