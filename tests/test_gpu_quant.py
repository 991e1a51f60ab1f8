"""GPU parity of the on-device number encoders, the packed BF16 converter of the
RMSNorms (every f32 pattern) and the weight quantizers against the
oracle, byte for byte: every f32 pattern of the ranges the quantizers feed the
encoders (and a random sample of all 2^32 patterns), special rows (zero,
subnormal, the hand-worked examples), and random matrices with outliers.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import read_table
from parity import DEV, check_quantized, log, mtp

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


def _compare_range(codec, first, count):
    m = mtp()
    out = torch.empty(CHUNK, dtype=torch.int16 if codec == 2 else torch.uint8, device=DEV)
    done = 0
    while done < count:
        n = min(CHUNK, count - done)
        m.mtp_codec_encode_range(codec, first + done, n, out)
        got = out[:n].cpu().numpy()
        want = oracle.encode_range(codec, first + done, n)
        if codec == 2:
            # NaN: the device keeps the sign and the upper payload bits and sets
            # the quiet bit (the oracle returns the canonical quiet NaN)
            got = got.view(np.uint16)
            u = (np.arange(n, dtype=np.uint64) + (first + done)).astype(np.uint32)
            nan = (u & 0x7FFFFFFF) > 0x7F800000
            want = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), want)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (f"codec {codec}: {bad.size} mismatches, first pattern "
                               f"{hex(first + done + int(bad[0]))}: gpu {got[bad[0]]:#x} oracle {want[bad[0]]:#x}")
        done += n


@pytest.mark.parametrize("sign", [0, 0x80000000])
def test_e4m3_encoder_every_pattern_in_range(sign):
    """All f32 with 2^-12 <= |v| < 512 (every E4M3 rounding and saturation
    boundary), both signs, plus zero and the subnormal-f32 floor."""
    log(f"e4m3 range sign={sign:#x}")
    _compare_range(0, sign | 0x39800000, 0x44000000 - 0x39800000)
    _compare_range(0, sign | 0x00000000, 1 << 20)


@pytest.mark.parametrize("sign", [0, 0x80000000])
def test_e2m1_encoder_every_pattern_in_range(sign):
    """All f32 with 2^-3 <= |v| < 16, both signs."""
    log(f"e2m1 range sign={sign:#x}")
    _compare_range(1, sign | 0x3E000000, 0x41800000 - 0x3E000000)


@pytest.mark.parametrize("sign", [0, 0x80000000])
def test_bf16_packed_converter_every_pattern(sign):
    """Every f32 pattern of one sign through the packed f32 -> BF16 converter
    that rounds the RMSNorm outputs (each pattern in the low or the high half
    of a pair), against the oracle's round-to-nearest-even encoder."""
    log(f"bf16 every pattern sign={sign:#x}")
    _compare_range(2, sign, 1 << 31)


def test_encoders_random_patterns_and_specials():
    m = mtp()
    rng = np.random.default_rng(5)
    firsts = rng.integers(0, (1 << 32) - 4096, 2048, dtype=np.uint64)
    specials = [0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F7FFFFF, 0x43E00000, 0x43E80000,
                0x43F00000, 0x40C00000, 0x40BFFFFF, 0x00000001, 0x80000001]
    out = torch.empty(4096, dtype=torch.uint8, device=DEV)
    for codec in (0, 1):
        for f in list(firsts[:64]) + specials:
            n = 4096 if f < (1 << 32) - 4096 else 1
            m.mtp_codec_encode_range(codec, int(f), n, out)
            assert np.array_equal(out[:n].cpu().numpy(), oracle.encode_range(codec, int(f), n)), (codec, hex(int(f)))


def _bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)


def test_fp8_special_rows():
    m = mtp()
    rows = read_table("fp8_row_example.txt")
    golden = [float(eval(r[0])) for r in rows]
    W = torch.zeros((6, 64), dtype=torch.bfloat16)
    W[0, :16] = _bf16(golden)                    # absmax 448: scale 1, codes = hand table
    W[2, 7] = -3.0                               # single nonzero
    W[3] = torch.tensor([0x0001, 0x0040, 0x807F, 0x0002] * 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    W[4] = -0.0
    W[5] = _bf16(list(np.linspace(-1, 1, 64)))
    Wd = W.to(DEV)
    head = m.quantize_head(Wd, "fp8")
    torch.cuda.synchronize()
    check_quantized(head, si.bits(W))
    want = [int(r[1], 16) for r in rows]
    assert head.w[0, :16].cpu().tolist() == want
    assert head.scale[1].item() == 1.0 and head.w[4].cpu().tolist() == [0x80] * 64


def test_nvfp4_golden_example_and_zero():
    m = mtp()
    d = {r[0]: r[1:] for r in read_table("nvfp4_example.txt")}
    row = [float(v) for v in d["row"]]
    W = torch.zeros((3, 256), dtype=torch.bfloat16)
    W[0, :32] = _bf16(row)
    W[2, 3] = -0.0
    head = m.quantize_head(W.to(DEV), "nvfp4")
    torch.cuda.synchronize()
    check_quantized(head, si.bits(W))
    assert head.gscale.item() == 1.0
    assert head.w[0, :16].cpu().tolist() == [int(x, 16) for x in d["packed"]]
    assert head.scale[0, :2].cpu().tolist() == [int(x, 16) for x in d["block_scales"]]
    assert head.w[1].sum().item() == 0 and head.w[2, 1].item() == 0x80


@pytest.mark.parametrize("wdtype,n,k,outl,scale", [
    ("fp8", 1000, 4096, 0.0, 0.02), ("fp8", 333, 5120, 0.01, 1.0), ("fp8", 100, 16, 0.0, 1e-30),
    ("nvfp4", 1000, 4096, 0.01, 0.02), ("nvfp4", 77, 5120, 0.0, 3.0), ("nvfp4", 5, 256, 0.0, 1e-35),
])
def test_quantize_random(wdtype, n, k, outl, scale):
    """Random matrices, including tiny magnitudes (f32 subnormal scale arithmetic)."""
    m = mtp()
    log(f"quantize {wdtype} {n}x{k} scale={scale}")
    W = si.normal_bf16(n + k, si.TAG_LM, n, k, std=scale, outlier_p=outl, device=DEV)
    head = m.quantize_head(W, wdtype)
    torch.cuda.synchronize()
    check_quantized(head, si.bits(W))
