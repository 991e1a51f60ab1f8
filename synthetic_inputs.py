"""Seeded synthetic inputs for the MTP draft step (shared by tests, bench and smoke).

This module only draws random numbers and shapes them; it holds none of the
draft step's arithmetic. Values are drawn in float32 with torch's seeded
generator on the requested device (Philox on the GPU, so the 1.27 GB heads are
drawn in HBM in milliseconds) and cast to BF16 with torch's float32 -> bfloat16
conversion (round to nearest even). Callers that need the host copy for the
oracle move the tensor to the CPU and view it as uint16 bits (`bits`).

Every tensor gets its own generator, seeded from (seed, tag), so tensors do not
shift one another. The same (seed, tag, shape, device type) gives the same
values on every run of the same torch build.

Workloads follow the draft-step shapes the pages speak of (a 154,880 x 4,096
BF16 draft head; glm5next_mtp_head/init.rs draft-head comment) and this
project's configuration list: weights ~ N(0, 0.02), embeddings and hidden states
~ N(0, 1), RMSNorm gammas 1 + N(0, 0.1), eps 1e-6; the NVFP4 head adds 1 %
outliers scaled x20 (Bernoulli mask).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

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


def _gen(seed: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed((int(seed) * 1_000_003 + int(tag) * 10_007 + 12_345) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal_bf16(seed: int, tag: int, rows: int, cols: int, std: float = 1.0, mean: float = 0.0,
                outlier_p: float = 0.0, outlier_mult: float = 20.0, device="cpu") -> torch.Tensor:
    """BF16 [rows, cols] of mean + std * N(0, 1); with probability outlier_p an
    element is multiplied by outlier_mult."""
    dev = torch.device(device)
    v = torch.randn((rows, cols), generator=_gen(seed, tag, dev), device=dev, dtype=torch.float32)
    v.mul_(std)
    if mean != 0.0:
        v.add_(mean)
    if outlier_p > 0.0:
        m = torch.rand((rows, cols), generator=_gen(seed, tag + 100 * TAG_OUTLIER, dev), device=dev) < outlier_p
        v[m] *= outlier_mult
        del m
    out = v.to(torch.bfloat16)
    del v
    return out


def token_ids(seed: int, b: int, vocab: int) -> np.ndarray:
    g = _gen(seed, TAG_TOKENS, "cpu")
    return torch.randint(0, vocab, (b,), generator=g, dtype=torch.int64).numpy().astype(np.int32)


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a BF16 tensor as uint16 bit patterns (for the oracle)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    """BF16 tensor from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


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


def lm_weight(wl: Workload, seed: int, device="cpu") -> torch.Tensor:
    """BF16 lm_head [vocab, hidden] ~ N(0, w_std) (with outliers if configured)."""
    return normal_bf16(seed, TAG_LM, wl.vocab, wl.hidden, std=wl.w_std, outlier_p=wl.outlier_p,
                       outlier_mult=wl.outlier_mult, device=device)


def lm_x(wl: Workload, seed: int, device="cpu") -> torch.Tensor:
    """BF16 x [batch, hidden] ~ N(0, 1): independent rows."""
    return normal_bf16(seed, TAG_X, wl.batch, wl.hidden, device=device)


def step_inputs(wl: Workload, seed: int, device="cpu") -> dict:
    """Inputs of the combine: embedding table [V, h] ~ N(0,1), target hidden [b, h]
    ~ N(0,1), gammas 1 + N(0, 0.1), fc [h, 2h] ~ N(0, w_std), host token ids U[0, V)."""
    h = wl.hidden
    return dict(
        embed=normal_bf16(seed, TAG_EMBED, wl.vocab, h, device=device),
        hidden=normal_bf16(seed, TAG_HIDDEN, wl.batch, h, device=device),
        gamma_e=normal_bf16(seed, TAG_GAMMA_E, 1, h, std=0.1, mean=1.0, device=device)[0],
        gamma_h=normal_bf16(seed, TAG_GAMMA_H, 1, h, std=0.1, mean=1.0, device=device)[0],
        gamma_f=normal_bf16(seed, TAG_GAMMA_F, 1, h, std=0.1, mean=1.0, device=device)[0],
        fc=normal_bf16(seed, TAG_FC, h, 2 * h, std=wl.w_std, device=device),
        tokens=token_ids(seed, wl.batch, wl.vocab),
    )
