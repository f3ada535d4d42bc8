"""Seeded synthetic inputs for the context-parallel attention path.

This module only draws random numbers and casts them; it holds none of the
attention, merge or layout arithmetic, so both the oracle and the HIP path
can take their inputs from it without sharing any of the method.

The five workloads stand in for the pages' own workloads (which need trained
weights and prompts that are not used here):

* a tiny fp32 correctness case;
* FLUX.1-dev joint attention at 512x512 and 1024x1024 (the diffusers
  "Context parallelism" guide benchmarks FLUX.1-dev at 1024x1024 and
  1008x1008); 1024x1024 gives 64*64 = 4096 image tokens plus 512 text tokens;
* a "Ring Anything" case whose sequence length is not divisible by the ring
  degree (the guide's "Ring Anything Attention" section);
* a CogVideoX-style video sequence (the xDiT issue "FLUX with SP" lists a
  CogVideoX 480x720, 9-frame run): 3 latent frames of 30x45 patches plus
  226 text tokens = 4276.

Tensors are laid out [B, S, H, D] (batch, sequence, heads, head dim), the
reading of the (1, 10, 8, 64) example in the diffusers "Attention backends"
page, "Checks" section.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "random_qkv",
           "to_f64"]


@dataclass(frozen=True)
class Workload:
    index: int            # 1..5; also the seed
    name: str
    B: int
    S: int
    H: int
    D: int
    dtype: str            # "f32" or "bf16": the element type handed to the GPU
    qk_gain: float = 1.0  # Q and K draws are multiplied by this before the cast
    outlier_frac: float = 0.0   # fraction of K rows per (b, h) that are scaled
    outlier_gain: float = 1.0
    ring_degree: Optional[int] = None
    ulysses_degree: Optional[int] = None
    ring_anything: bool = False

    @property
    def seed(self) -> int:
        return self.index

    def flops(self, sq: Optional[int] = None, skv: Optional[int] = None,
              heads: Optional[int] = None) -> float:
        """4*B*H*Sq*Skv*D: two contractions (QK^T and PV) of 2 flops per MAC."""
        sq = self.S if sq is None else sq
        skv = self.S if skv is None else skv
        heads = self.H if heads is None else heads
        return 4.0 * self.B * heads * sq * skv * self.D


WORKLOADS = (
    Workload(1, "tiny-f32", B=1, S=256, H=2, D=64, dtype="f32", ring_degree=4),
    # logit std ~3: q.k/sqrt(D) has variance gain^4, so gain = 3**0.5 per operand
    Workload(2, "flux-512", B=1, S=1024 + 512, H=24, D=128, dtype="bf16",
             qk_gain=math.sqrt(3.0), ulysses_degree=2),
    Workload(3, "flux-1024", B=1, S=4096 + 512, H=24, D=128, dtype="bf16",
             qk_gain=math.sqrt(3.0), ring_degree=8),
    Workload(4, "ring-anything-4645", B=1, S=4608 + 37, H=24, D=128,
             dtype="bf16", ring_degree=8, ring_anything=True),
    Workload(5, "video-dit-4276", B=2, S=3 * 30 * 45 + 226, H=30, D=64,
             dtype="bf16", outlier_frac=0.01, outlier_gain=8.0,
             ulysses_degree=2),
)


def workload(key) -> Workload:
    """Look a workload up by index (1..5) or by name."""
    for w in WORKLOADS:
        if key == w.index or key == w.name:
            return w
    raise KeyError(key)


def _cast(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "f32":
        return t.to(torch.float32)
    if dtype == "bf16":
        return t.to(torch.bfloat16)   # round to nearest even
    raise ValueError(dtype)


def make_inputs(key, heads: Optional[int] = None):
    """Draw (q, k, v) for a workload as CPU torch tensors of its dtype.

    Order of draws from numpy's PCG64 with seed = workload index: Q, K, V
    (standard normal, float32, shape [B, S, H, D]); then, for workloads with
    outliers, for each (b, h) in row-major order the round(frac*S) distinct
    sequence positions whose K rows are scaled by ``outlier_gain`` (a power of
    two, so the scaling is exact in bf16); then Q and K are multiplied by
    ``qk_gain``; then the cast.  ``heads`` keeps only the first heads after
    drawing all of them, so a reduced case is a slice of the full one.
    """
    w = workload(key)
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.S, w.H, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.outlier_frac > 0.0:
        n_out = int(round(w.outlier_frac * w.S))
        for b in range(w.B):
            for h in range(w.H):
                rows = rng.choice(w.S, size=n_out, replace=False)
                k[b, rows, h, :] *= np.float32(w.outlier_gain)
    if w.qk_gain != 1.0:
        q *= np.float32(w.qk_gain)
        k *= np.float32(w.qk_gain)
    if heads is not None:
        q, k, v = (a[:, :, :heads, :] for a in (q, k, v))
    return _cast(q, w.dtype), _cast(k, w.dtype), _cast(v, w.dtype)


def random_qkv(seed: int, B: int, Sq: int, Skv: int, H: int, D: int,
               dtype: str = "bf16", gain: float = 1.0):
    """Generic seeded (q, k, v) with Sq query rows and Skv key rows.

    Standard normal float32 draws in the order Q, K, V, Q and K multiplied by
    ``gain``, then cast to ``dtype``.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, D), dtype=np.float32)
    k = rng.standard_normal((B, Skv, H, D), dtype=np.float32)
    v = rng.standard_normal((B, Skv, H, D), dtype=np.float32)
    if gain != 1.0:
        q *= np.float32(gain)
        k *= np.float32(gain)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)


def to_f64(t) -> np.ndarray:
    """Exact upcast of a CPU torch tensor (fp32 or bf16) to a float64 array."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()
