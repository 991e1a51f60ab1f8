"""bench.py's host logic, on the CPU: the one-GPU contract, the algorithmic
byte counts the roofline divides by (recomputed here from the layouts, not
from bench.py), the committed HBM-traffic records, and the counter summary's
copy calibration on a synthetic counter file."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("wd,n,h,b,expect", [
    # BF16: n h 2 weight bytes + b h 2 of x + 4 b of tokens
    (0, 154880, 4096, 1, 154880 * 4096 * 2 + 4096 * 2 + 4),
    # FP8: codes n h + f32 row scales 4 n
    (1, 154880, 4096, 8, 154880 * 4096 + 4 * 154880 + 8 * 4096 * 2 + 8 * 4),
    # NVFP4: codes n h / 2 + E4M3 block scales n h / 16 + the f32 global scale
    (2, 154880, 4096, 1, 154880 * 2048 + 154880 * 256 + 4 + 4096 * 2 + 4),
    (2, 32768, 5120, 8, 32768 * 2560 + 32768 * 320 + 4 + 8 * 5120 * 2 + 8 * 4),
])
def test_lm_head_algorithmic_bytes(wd, n, h, b, expect):
    assert bench.lm_bytes(wd, n, h, b) == expect


def test_headline_byte_counts():
    assert bench.lm_bytes(0, 154880, 4096, 1) == 1268785156
    assert bench.lm_bytes(1, 154880, 4096, 1) == 635016196
    assert bench.lm_bytes(2, 154880, 4096, 1) == 356851720
    # combine: embedding row + target hidden + 3 gammas + fc [h, 2h] + x out, BF16
    assert bench.combine_bytes(1, 4096) == 4096 * 2 * 3 + 3 * 4096 * 2 + 4096 * 8192 * 2


def test_traffic_records_are_consistent():
    """Every committed record's algorithmic bytes match its key, and the counted
    bytes are within 2 % above them (no re-reads)."""
    wds = {"bf16": 0, "fp8": 1, "nvfp4": 2}
    seen = 0
    for line in open(bench.TRAFFIC_FILE):
        f = line.split()
        if not f or f[0] != "traffic":
            continue
        wd, shape, n, b = f[1].split(":")
        V, h = (int(v) for v in shape.split("x"))
        alg = bench.lm_bytes(wds[wd], int(n[1:]), h, int(b[1:]))
        assert int(f[5]) == alg, line
        assert 1.0 <= (int(f[3]) + int(f[4])) / alg < 1.02, line
        assert len(f[2]) == 16
        seen += 1
    assert seen >= 5


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_calibrates_on_the_copy(tmp_path):
    """FETCH_SIZE reading half the copy's bytes doubles every lm_head reading;
    only the workload's own instantiation (format, batch) is averaged."""
    lm = "void mtp::lmhead_argmax_kernel<0, 1, 1, 4, false, 256>(mtp::SweepParams)"
    other = "void mtp::lmhead_argmax_kernel<2, 1, 2, 2, false, 512>(mtp::SweepParams)"
    copy = "__amd_rocclr_copyBuffer"
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(f, "FETCH_SIZE", [(copy, 524288.0), (lm, 600000.0), (other, 1.0), (lm, 620000.0)])
    _counter_csv(w, "WRITE_SIZE", [(copy, 1048576.0), (lm, 16.0), (other, 999.0), (lm, 18.0)])
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-summary", str(f), str(w),
                        "--workload", "bf16_154880x4096_b1"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    rec = [ln.split() for ln in r.stdout.splitlines() if ln.startswith("traffic ")]
    assert len(rec) == 1
    fetch, write = int(rec[0][3]), int(rec[0][4])
    assert fetch == round(610000.0 * 1024 * 2.0)
    assert write == round(17.0 * 1024 * 1.0)
    assert rec[0][1] == "bf16:154880x4096:n154880:b1"
