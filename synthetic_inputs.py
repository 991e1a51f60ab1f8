"""Seeded synthetic inputs for the MTP draft step (shared by tests, bench and smoke).

This module only draws random numbers and shapes them; it holds none of the
draft step's arithmetic. BF16 values are produced by drawing float32 and
converting with torch's float32 -> bfloat16 cast (round to nearest even), so
the stored inputs are plain BF16 bit patterns (numpy uint16).

Every tensor gets its own random stream, keyed by (seed, tag, chunk), so
tensors do not shift one another and large matrices can be drawn in parallel
row chunks. Streams: numpy PCG64 seeded through SeedSequence.

Workloads follow the draft-step shapes the pages speak of (a 154,880 x 4,096
BF16 draft head; glm5next_mtp_head/init.rs draft-head comment) and the
configuration list of this project: weights ~ N(0, 0.02), embeddings and
hidden states ~ N(0, 1), RMSNorm gammas 1 + N(0, 0.1), eps 1e-6; the NVFP4
head adds 1 % outliers scaled x20.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

_ROW_CHUNK = 4096  # rows per independent stream chunk

# tags keep the streams of different tensors apart
TAG_LM = 1
TAG_X = 2
TAG_FC = 3
TAG_EMBED = 4
TAG_GAMMA_E = 5
TAG_GAMMA_H = 6
TAG_GAMMA_F = 7
TAG_TOKENS = 8
TAG_OUTLIER = 9
TAG_HIDDEN = 10


def _rng(seed: int, tag: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag), int(chunk)])))


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(seed: int, tag: int, rows: int, cols: int, std: float = 1.0, mean: float = 0.0,
                outlier_p: float = 0.0, outlier_mult: float = 20.0) -> np.ndarray:
    """BF16 bits [rows, cols] of mean + std * N(0, 1); with probability outlier_p an
    element is multiplied by outlier_mult (Bernoulli mask from its own stream)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    n_chunks = (rows + _ROW_CHUNK - 1) // _ROW_CHUNK

    def work(ci: int) -> None:
        r0 = ci * _ROW_CHUNK
        r1 = min(rows, r0 + _ROW_CHUNK)
        g = _rng(seed, tag, ci)
        v = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        if outlier_p > 0.0:
            m = _rng(seed, tag + 1000 * TAG_OUTLIER, ci).random((r1 - r0, cols), dtype=np.float32) < outlier_p
            v[m] *= np.float32(outlier_mult)
        out[r0:r1] = _to_bf16_bits(v)

    if n_chunks <= 1:
        for ci in range(n_chunks):
            work(ci)
    else:
        with _cf.ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def token_ids(seed: int, b: int, vocab: int) -> np.ndarray:
    return _rng(seed, TAG_TOKENS).integers(0, vocab, size=b, dtype=np.int64).astype(np.int32)


@dataclass
class Workload:
    """One synthetic workload. `kind` is 'step' (combine + lm_head + argmax) or
    'lmhead' (lm_head + argmax on given x)."""
    name: str
    kind: str
    vocab: int
    hidden: int
    batch: int
    wdtype: str = "bf16"            # bf16 | fp8 | nvfp4
    mtp_vocab_size: int = 0
    w_std: float = 0.02
    outlier_p: float = 0.0
    outlier_mult: float = 20.0
    eps: float = 1e-6
    gamma_offset: float = 0.0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # full draft step, tiny: combine -> final norm -> lm_head -> argmax
    "tiny_step": Workload("tiny_step", "step", vocab=4096, hidden=256, batch=1),
    # full draft step at 32,000 x 4,096
    "step_32000x4096": Workload("step_32000x4096", "step", vocab=32000, hidden=4096, batch=1),
    # full draft step at the draft-head shape the pages time (154,880 x 4,096)
    "step_154880x4096": Workload("step_154880x4096", "step", vocab=154880, hidden=4096, batch=1),
    # lm_head + argmax only, BF16, b in {1, 4}
    "bf16_154880x4096_b1": Workload("bf16_154880x4096_b1", "lmhead", 154880, 4096, 1),
    "bf16_154880x4096_b4": Workload("bf16_154880x4096_b4", "lmhead", 154880, 4096, 4),
    # FP8 per-row scale, b in {1, 2, 4, 8}
    **{f"fp8_154880x4096_b{b}": Workload(f"fp8_154880x4096_b{b}", "lmhead", 154880, 4096, b, "fp8")
       for b in (1, 2, 4, 8)},
    # NVFP4 at the draft-head shape
    "nvfp4_154880x4096_b1": Workload("nvfp4_154880x4096_b1", "lmhead", 154880, 4096, 1, "nvfp4"),
    # NVFP4 131,072 x 5,120 with 1 % outliers x20, b in {1, 4, 8}, full and truncated
    **{f"nvfp4_131072x5120_b{b}": Workload(f"nvfp4_131072x5120_b{b}", "lmhead", 131072, 5120, b, "nvfp4",
                                           outlier_p=0.01) for b in (1, 4, 8)},
    **{f"nvfp4_131072x5120_t32768_b{b}": Workload(f"nvfp4_131072x5120_t32768_b{b}", "lmhead", 131072, 5120, b,
                                                  "nvfp4", mtp_vocab_size=32768, outlier_p=0.01)
       for b in (1, 4, 8)},
}


def lm_weight(wl: Workload, seed: int) -> np.ndarray:
    """BF16 lm_head [vocab, hidden] ~ N(0, w_std) (with outliers if configured)."""
    return normal_bf16(seed, TAG_LM, wl.vocab, wl.hidden, std=wl.w_std, outlier_p=wl.outlier_p,
                       outlier_mult=wl.outlier_mult)


def lm_x(wl: Workload, seed: int) -> np.ndarray:
    """BF16 x [batch, hidden] ~ N(0, 1): independent rows."""
    return normal_bf16(seed, TAG_X, wl.batch, wl.hidden)


def step_inputs(wl: Workload, seed: int) -> dict:
    """Inputs of the combine: embedding table [V, h] ~ N(0,1), target hidden [b, h]
    ~ N(0,1), gammas 1 + N(0, 0.1), fc [h, 2h] ~ N(0, w_std), token ids U[0, V)."""
    h = wl.hidden
    return dict(
        embed=normal_bf16(seed, TAG_EMBED, wl.vocab, h),
        hidden=normal_bf16(seed, TAG_HIDDEN, wl.batch, h),
        gamma_e=normal_bf16(seed, TAG_GAMMA_E, 1, h, std=0.1, mean=1.0)[0],
        gamma_h=normal_bf16(seed, TAG_GAMMA_H, 1, h, std=0.1, mean=1.0)[0],
        gamma_f=normal_bf16(seed, TAG_GAMMA_F, 1, h, std=0.1, mean=1.0)[0],
        fc=normal_bf16(seed, TAG_FC, h, 2 * h, std=wl.w_std),
        tokens=token_ids(seed, wl.batch, wl.vocab),
    )
