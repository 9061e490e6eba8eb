"""Seeded synthetic inputs for the BitLinear W1.58A8 forward pass.

This module only draws random numbers.  It holds none of the method's
arithmetic (no scales, no rounding to codes, no products): the oracle and the
HIP path both receive the arrays made here and nothing else from this file.

Workloads (shapes are N x K = out x in, following the weight convention
W in R^{d_out x d_in} of "BitNet b1.58 2B4T Guide", section "Ternary Weight
Quantization: absmean Scaling"; M = tokens):

  c1      one 256x256 layer, W ~ N(0, 0.02^2) fp32, X fp32 4x256 ~ N(0,1) with
          channels 7 and 100 scaled x50 in every token, fp32 output.
  c2      batch-1 decode at 2B-class shapes: q,o 2560x2560; k,v 640x2560;
          up 6912x2560 (ReLU^2 on its output); down 2560x6912.  X bf16 ~ N(0,1)
          with 1% of the channels scaled x100.  bf16 output.
  c3      the c2 set as a 30-layer stack, batches 1/8/32/64, X bf16 Student-t
          (nu=3).
  c4      2048-token prefill: 2048 x 2560 -> 6912 (ReLU^2) and
          2048 x 6912 -> 2560.  X bf16 ~ N(0,1) with 0.5% of the channels x100.
  c5      100B-class layer: q,o 8192x8192; k,v 1024x8192; up 28672x8192;
          down 8192x28672.  X bf16 Student-t (nu=3); batches 1, 16, 512.

The outlier channels stand in for the "outlier channels" that the same page
(section "The Limits of Post-Training Quantization") says reach two orders of
magnitude above the median activation.  Real BitNet weights are not used.

Every stream comes from numpy's PCG64 seeded through SeedSequence; each named
matrix and each named input has a child stream of its own so that generating
one array never shifts another.  Order inside an input stream: values first,
then the outlier channel set.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

SIGMA_W = 0.02

# Matrix sets.  Each entry: name -> (N, K, relu2, input group)
SET_2B = {
    "q": (2560, 2560, False, "attn_in"),
    "k": (640, 2560, False, "attn_in"),
    "v": (640, 2560, False, "attn_in"),
    "o": (2560, 2560, False, "o_in"),
    "up": (6912, 2560, True, "up_in"),
    "down": (2560, 6912, False, "down_in"),
}
SET_100B = {
    "q": (8192, 8192, False, "attn_in"),
    "k": (1024, 8192, False, "attn_in"),
    "v": (1024, 8192, False, "attn_in"),
    "o": (8192, 8192, False, "o_in"),
    "up": (28672, 8192, True, "up_in"),
    "down": (8192, 28672, False, "down_in"),
}
SET_PREFILL = {
    "up": (6912, 2560, True, "up_in"),
    "down": (2560, 6912, False, "down_in"),
}
SET_C1 = {"w": (256, 256, False, "x")}

_MATRIX_ORDER = ["w", "q", "k", "v", "o", "up", "down"]
_INPUT_ORDER = ["x", "attn_in", "o_in", "up_in", "down_in"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    matrices: Dict[str, Tuple[int, int, bool, str]]
    batches: Tuple[int, ...]
    x_kind: str              # "normal" or "student_t3"
    x_dtype: str             # "f32" or "bf16"
    y_dtype: str             # "f32" or "bf16"
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    outlier_channels: Optional[Tuple[int, ...]] = None
    layers: int = 1

    def input_k(self, group: str) -> int:
        ks = {k for (_, k, _, g) in self.matrices.values() if g == group}
        assert len(ks) == 1, (group, ks)
        return ks.pop()

    def groups(self) -> List[str]:
        seen: List[str] = []
        for (_, _, _, g) in self.matrices.values():
            if g not in seen:
                seen.append(g)
        return seen


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", 1, SET_C1, (4,), "normal", "f32", "f32",
                   outlier_scale=50.0, outlier_channels=(7, 100)),
    "c2": Workload("c2", 2, SET_2B, (1,), "normal", "bf16", "bf16",
                   outlier_frac=0.01, outlier_scale=100.0),
    "c3": Workload("c3", 3, SET_2B, (1, 8, 32, 64), "student_t3", "bf16", "bf16",
                   layers=30),
    "c4": Workload("c4", 4, SET_PREFILL, (2048,), "normal", "bf16", "bf16",
                   outlier_frac=0.005, outlier_scale=100.0),
    "c5": Workload("c5", 5, SET_100B, (1, 16, 512), "student_t3", "bf16", "bf16"),
}


def _child(seed: int, kind: str, name: str) -> np.random.Generator:
    order = _MATRIX_ORDER if kind == "w" else _INPUT_ORDER
    idx = order.index(name) + (0 if kind == "w" else 100)
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(idx,))
    return np.random.Generator(np.random.PCG64(ss))


def gaussian_weights(seed: int, name: str, n: int, k: int,
                     sigma: float = SIGMA_W) -> np.ndarray:
    """fp32 [n, k] row-major, entries ~ N(0, sigma^2)."""
    rng = _child(seed, "w", name)
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def workload_weights(wl: Workload, name: str) -> np.ndarray:
    n, k, _, _ = wl.matrices[name]
    return gaussian_weights(wl.seed, name, n, k)


def activations_f32(wl: Workload, group: str, m: int) -> np.ndarray:
    """fp32 [m, K] activations of one input group, outliers applied."""
    k = wl.input_k(group)
    rng = _child(wl.seed * 1000 + m, "x", group)
    if wl.x_kind == "normal":
        x = rng.standard_normal((m, k), dtype=np.float32)
    elif wl.x_kind == "student_t3":
        x = rng.standard_t(3.0, size=(m, k)).astype(np.float32)
    else:
        raise ValueError(wl.x_kind)
    if wl.outlier_channels is not None:
        ch = np.array(wl.outlier_channels, dtype=np.int64)
    elif wl.outlier_frac > 0:
        cnt = int(round(wl.outlier_frac * k))
        ch = rng.choice(k, size=cnt, replace=False)
    else:
        ch = np.zeros(0, dtype=np.int64)
    if ch.size:
        x[:, ch] *= np.float32(wl.outlier_scale)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), returned as uint16 bit patterns.

    Input preparation only (the activations are handed over in bf16); uses
    torch's own conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (the low 16 bits are zero)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations(wl: Workload, group: str, m: int) -> Tuple[np.ndarray, str]:
    """Activations in the workload's input dtype.

    Returns (array, dtype): fp32 array for "f32", uint16 bf16 bits for "bf16"."""
    x = activations_f32(wl, group, m)
    if wl.x_dtype == "bf16":
        return to_bf16_bits(x), "bf16"
    return x, "f32"


def random_case(seed: int, m: int, n: int, k: int, x_scale: float = 1.0,
                w_sigma: float = SIGMA_W, x_kind: str = "normal"):
    """Small random (W fp32 [n,k], X fp32 [m,k]) pair for property tests."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    w = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(w_sigma))
    if x_kind == "normal":
        x = rng.standard_normal((m, k), dtype=np.float32) * np.float32(x_scale)
    else:
        x = rng.standard_t(3.0, size=(m, k)).astype(np.float32) * np.float32(x_scale)
    return w, x
