"""Seeded synthetic inputs — the only code the product path and the oracle both use.

This module draws random numbers and casts them to the element type a workload
names; it holds none of the attention arithmetic. Q, K and V are i.i.d.
standard normal (random inputs, as the table in section 1 of
"Attention kernels on a home RTX 5080" uses to measure error), drawn in float32 with
numpy's PCG64 generator from seeds 41, 42 and 43 (41 is the seed of the parity
cases in section "build and reproduction" of "round 21 track b — qsa2"), then
rounded to nearest-even into the workload's dtype.

Workloads are named by what they are, with their sizes (``WORKLOADS``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

SEED_Q, SEED_K, SEED_V = 41, 42, 43


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    dtype: torch.dtype
    causal: bool = False
    window_lo: int = 0
    pos0: int = 0
    mode: int = 0          # 0 exact, 1 INT8-QK / FP8-PV, 2 decode over an INT8-K / E4M3-V cache
    scale: float = field(default=float("nan"))
    window_w: int = 0      # > 0: per-row sliding window, row i sees keys >= pos0 + i - window_w + 1

    def __post_init__(self):
        if math.isnan(self.scale):
            object.__setattr__(self, "scale", 1.0 / math.sqrt(self.D))

    def variant(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def q_shape(self):
        return (self.B, self.Hq, self.Nq, self.D)

    @property
    def kv_shape(self):
        return (self.B, self.Hkv, self.Nk, self.D)

    def visible_pairs(self) -> int:
        """Number of (query row, key) pairs the mask lets through, per head."""
        total = 0
        for i in range(self.Nq):
            hi = self.Nk - 1 if not self.causal else min(self.Nk - 1, self.pos0 + i)
            lo = self.window_lo
            if self.window_w > 0:
                lo = max(lo, self.pos0 + i - self.window_w + 1)
            total += max(0, hi - lo + 1)
        return total

    def flops(self) -> float:
        """4 * D flops per visible (row, key) pair per query head."""
        if not self.causal and self.window_lo == 0 and self.window_w == 0:
            pairs = self.Nq * self.Nk
        else:
            pairs = self.visible_pairs()
        return 4.0 * self.B * self.Hq * pairs * self.D


WORKLOADS = {
    # tiny oracle case: fp32, non-causal (and a causal variant)
    "tiny_fp32_256": Workload("tiny_fp32_256", 1, 2, 2, 256, 256, 64, torch.float32),
    # few-row GQA decode against an f16 KV cache, bottom-right causal
    "gqa_decode_f16_4096": Workload("gqa_decode_f16_4096", 1, 16, 8, 4, 4096, 128,
                                    torch.float16, causal=True, pos0=4092),
    # the same decode against a quantised cache (INT8 K, E4M3 V, per-64-key scales)
    "gqa_decode_kvq_f16_4096": Workload("gqa_decode_kvq_f16_4096", 1, 16, 8, 4, 4096, 128,
                                        torch.float16, causal=True, pos0=4092, mode=2),
    # SDXL-style 1024px self-attention (64x64 latent tokens)
    "sdxl_1024px_bf16": Workload("sdxl_1024px_bf16", 2, 10, 10, 4096, 4096, 64,
                                 torch.bfloat16),
    # video-DiT scale attention, 1 x 40 heads x 32760 tokens x 128
    "video_dit_bf16_32760": Workload("video_dit_bf16_32760", 1, 40, 40, 32760, 32760,
                                     128, torch.bfloat16),
    # the same shape in INT8-QK / FP8-PV mode
    "video_dit_quant_32760": Workload("video_dit_quant_32760", 1, 40, 40, 32760, 32760,
                                      128, torch.bfloat16, mode=1),
}


def normal(shape, seed: int, dtype: torch.dtype) -> torch.Tensor:
    """N(0,1) float32 from PCG64(seed), rounded to nearest-even into dtype (CPU)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    t = torch.from_numpy(x)
    return t if dtype == torch.float32 else t.to(dtype)


def make_qkv(w: Workload, seeds=(SEED_Q, SEED_K, SEED_V)):
    """CPU tensors q [B,Hq,Nq,D], k and v [B,Hkv,Nk,D] in the workload's dtype."""
    return (normal(w.q_shape, seeds[0], w.dtype),
            normal(w.kv_shape, seeds[1], w.dtype),
            normal(w.kv_shape, seeds[2], w.dtype))


def make_kv_codes(w: Workload, seeds=(SEED_K, SEED_V)):
    """A synthetic quantised KV cache of shape w.kv_shape (CPU tensors).

    K codes are int8 samples of a discretised normal (sigma 40, clipped to
    +-127) and V codes float8_e4m3fn casts of normal samples scaled to sigma 100
    (clipped to +-448, stored as uint8 bytes): the spread of codes that blocks of
    N(0,1) data give. Block scales are 4.5/127 and 4.5/448 (about the block
    maximum of N(0,1) data over the code range) times exp(0.1 N(0,1)) per
    64-key block. Returns k_codes int8, k_scales fp32 [B,Hkv,ceil(Nk/64)],
    v_codes uint8, v_scales fp32.
    """
    nblk = (w.Nk + 63) // 64
    sshape = (w.B, w.Hkv, nblk)
    rk = np.random.default_rng(seeds[0])
    kc = np.clip(np.rint(rk.standard_normal(size=w.kv_shape, dtype=np.float32) * 40.0),
                 -127, 127).astype(np.int8)
    ks = (4.5 / 127.0) * np.exp(0.1 * rk.standard_normal(size=sshape)).astype(np.float32)
    rv = np.random.default_rng(seeds[1])
    vf = np.clip(rv.standard_normal(size=w.kv_shape, dtype=np.float32) * 100.0, -448.0, 448.0)
    vc = torch.from_numpy(vf).to(torch.float8_e4m3fn).view(torch.uint8)
    vs = (4.5 / 448.0) * np.exp(0.1 * rv.standard_normal(size=sshape)).astype(np.float32)
    return (torch.from_numpy(kc), torch.from_numpy(ks.astype(np.float32)), vc,
            torch.from_numpy(vs.astype(np.float32)))


def sample_rows(w: Workload, n: int = 256, seed: int = 7) -> np.ndarray:
    """n distinct flat row indices (b*Hq + h)*Nq + i, always holding the first
    row, the last row and rows of the last (partial) 256-row tile."""
    total = w.B * w.Hq * w.Nq
    if n >= total:
        return np.arange(total, dtype=np.int64)
    rng = np.random.default_rng(seed)
    fixed = {0, total - 1, w.Nq - 1}
    tail0 = (w.Nq // 256) * 256
    if tail0 < w.Nq:
        fixed.add(tail0)
        fixed.add((w.Hq - 1) * w.Nq + tail0 + (w.Nq - tail0) // 2)
    rest = rng.choice(total, size=n + len(fixed), replace=False)
    rows = list(sorted(fixed))
    for r in rest:
        if len(rows) >= n:
            break
        if int(r) not in fixed:
            rows.append(int(r))
    return np.array(sorted(rows), dtype=np.int64)
