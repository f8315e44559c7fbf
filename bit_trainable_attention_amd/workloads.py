"""Seeded synthetic workloads for the SageBwd-style INT8 attention path.

This module only draws random inputs and describes the five workload shapes. It
holds none of the method's arithmetic (no normalisation, smoothing, quantisation
or attention), so both the HIP path's tests and the CPU oracle's tests may use it.

Workloads (shapes, dtypes and flags follow the quantised-attention use case of the
SageBwd article, aitrends.kr, paragraphs on QK-norm, K-smoothing, per-block
quantisation and the 325M Llama pretraining run):

  tiny        B1 H2  N256   d64  fp16, non-causal, QK-norm off, K-smoothing on, blk 64
  bf16_d64    B4 H16 N2048  d64  bf16, causal, K += per-(head,channel) bias ~ N(0, var 2),
              dO ~ N(0, var 1e-2), QK-norm on, K-smoothing on, blk 64
  n8192_d128  B2 H16 N8192  d128 fp16, causal, 4 seeded K channels scaled x20 (outliers),
              QK-norm on, K-smoothing on, blk 128
  n32768      B1 H8  N32768 d128 fp16, causal, QK-norm on, K-smoothing on, blk 128
  llama325m   B8 H16 N4096  d64  bf16, causal, QK-norm on, K-smoothing on, blk 64
              (one attention layer of a ~325M Llama-like model, hidden 1024)

Draw recipe: numpy PCG64 with seed 1000 + k (k = 1..5 in the order above); draws
in order Q, K, V, dO (float32 standard normals times the stated std), then the
extras (K bias, outlier channels, and last a per-(head, channel) Q bias for the
Q-smoothing cases, which give any workload q_smooth=True and a q_bias_var); rounding
float32 -> fp16/bf16 is round to nearest even. The same host arrays feed the GPU and
the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # 1-based position in the workload list (seed = 1000 + index)
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp16" | "bf16"
    causal: bool
    qk_norm: bool
    k_smooth: bool
    blk: int
    eps: float = 1e-6
    dO_std: float = 1.0
    k_bias_var: float = 0.0      # variance of the per-(head, channel) bias added to K
    k_outlier_channels: int = 0  # number of K channels scaled by k_outlier_scale
    k_outlier_scale: float = 1.0
    q_smooth: bool = False       # the optional Q-smoothing variant
    q_bias_var: float = 0.0      # variance of the per-(head, channel) bias added to Q (drawn last)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def visible_pairs(self) -> int:
        """(query, key) pairs that enter the softmax, over all heads."""
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * self.H * per_head

    def algorithmic_ops(self) -> int:
        """Seven matmuls, each 2*d ops per visible (query, key) pair."""
        return 14 * self.d * self.visible_pairs()

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, B=1, H=2, N=256, d=64, dtype="fp16", causal=False,
                 qk_norm=False, k_smooth=True, blk=64),
        Workload("bf16_d64", 2, B=4, H=16, N=2048, d=64, dtype="bf16", causal=True,
                 qk_norm=True, k_smooth=True, blk=64, dO_std=0.1, k_bias_var=2.0),
        Workload("n8192_d128", 3, B=2, H=16, N=8192, d=128, dtype="fp16", causal=True,
                 qk_norm=True, k_smooth=True, blk=128, k_outlier_channels=4,
                 k_outlier_scale=20.0),
        Workload("n32768", 4, B=1, H=8, N=32768, d=128, dtype="fp16", causal=True,
                 qk_norm=True, k_smooth=True, blk=128),
        Workload("llama325m", 5, B=8, H=16, N=4096, d=64, dtype="bf16", causal=True,
                 qk_norm=True, k_smooth=True, blk=64),
    ]
}

# The workload the throughput figure is quoted on.
METRIC_WORKLOAD = "n8192_d128"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> 16-bit storage pattern (uint16) of `dtype`, round to nearest even."""
    if dtype == "fp16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f32(b: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit storage pattern (uint16) of `dtype` -> float32 (exact)."""
    if dtype == "fp16":
        return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(b)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw Q, K, V, dO for workload `w` as uint16 bit patterns of w.dtype, shape [B,H,N,d].

    Also returns the extras that were drawn ("k_bias" [H,d] float32, "k_outlier_idx").
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    shape = (w.B, w.H, w.N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32)
    if w.dO_std != 1.0:
        do *= np.float32(w.dO_std)
    out: Dict[str, np.ndarray] = {}
    if w.k_bias_var > 0.0:
        bias = rng.standard_normal((w.H, w.d), dtype=np.float32) * np.float32(np.sqrt(w.k_bias_var))
        k += bias[None, :, None, :]
        out["k_bias"] = bias
    if w.k_outlier_channels > 0:
        idx = np.sort(rng.choice(w.d, size=w.k_outlier_channels, replace=False))
        k[..., idx] *= np.float32(w.k_outlier_scale)
        out["k_outlier_idx"] = idx
    if w.q_bias_var > 0.0:
        qb = rng.standard_normal((w.H, w.d), dtype=np.float32) * np.float32(np.sqrt(w.q_bias_var))
        q += qb[None, :, None, :]
        out["q_bias"] = qb
    out["Q"] = f32_to_bits(q, w.dtype)
    out["K"] = f32_to_bits(k, w.dtype)
    out["V"] = f32_to_bits(v, w.dtype)
    out["dO"] = f32_to_bits(do, w.dtype)
    return out
