"""Seeded synthetic inputs for the DiT-MLP MXFP6 GEMM workloads.

This module only draws random numbers and rounds them to bfloat16; it holds
none of the MX arithmetic.  The same host tensors feed the HIP library and the
CPU oracle, so neither side ever supplies the other's inputs.

Workloads (the Hedra post "Optimizing Krea 3 on AMD Instinct MI355X with AI
researchers" runs Krea 3's DiT on a 1 MP reference plus a 4 MP output; its
MLP GEMMs in MXFP6 are the subject of the section "We built a faster MXFP6
kernel").  The pages state no matrix shapes; the shapes below are this
library's synthetic stand-ins for one GPU's share of those GEMMs:

=========  ==========================  ===========================================
name       M x K x N                   inputs
=========  ==========================  ===========================================
tiny       256 x 256 x 256             A, W ~ N(0, 1), E2M3 x E2M3, fp32 out
proj       4096 x 3072 x 3072          A ~ N(0, 1), W ~ N(0, 0.02), bf16 out
fc1        20480 x 3072 x 12288        A ~ N(0, 1), W ~ N(0, 0.02), GELU -> E2M3
fc2        20480 x 12288 x 3072        A ~ Student-t(3), 0.1 % of K channels x50
skinny     {8, 16} x 16384 x 13312     A ~ N(0, 1), W ~ N(0, 0.02) as E3M2
sw_fc1     20480 x 3072 x 16384        SwiGLU MLP: stacked gate/up rows (2 x 8192),
                                       A ~ N(0, 1), W ~ N(0, 0.02), SwiGLU -> E2M3
sw_fc2     20480 x 8192 x 3072         A ~ Student-t(3), 0.1 % of K channels x50
=========  ==========================  ===========================================

The SwiGLU MLP uses 8192 = 2/3 * 4 * 3072 hidden features, so its three weight
matrices hold as many parameters as the GELU MLP's two.

Recipe: numpy ``default_rng([workload_index, stream])`` with stream 0 = A,
1 = W, 2 = the outlier-channel choice; draws are float32, then rounded to
bfloat16 (round-to-nearest-even) by torch.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    m: int
    k: int
    n: int
    a_dist: str  # "normal" or "student_t_outliers"
    a_std: float
    w_std: float
    w_fmt: str  # element format of the weights
    out: str  # "f32", "bf16" or "mx" (GELU-tanh then E2M3)
    splits: int = 0  # split-K count, 0 = plain GEMM


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 256, 256, "normal", 1.0, 1.0, "e2m3", "f32"),
    "proj": Workload("proj", 2, 4096, 3072, 3072, "normal", 1.0, 0.02, "e2m3", "bf16"),
    "fc1": Workload("fc1", 3, 20480, 3072, 12288, "normal", 1.0, 0.02, "e2m3", "mx"),
    "fc2": Workload("fc2", 4, 20480, 12288, 3072, "student_t_outliers", 1.0, 0.02, "e2m3", "bf16"),
    "skinny": Workload("skinny", 5, 16, 16384, 13312, "normal", 1.0, 0.02, "e3m2", "bf16", 16),
    "sw_fc1": Workload("sw_fc1", 6, 20480, 3072, 16384, "normal", 1.0, 0.02, "e2m3", "mx"),
    "sw_fc2": Workload("sw_fc2", 7, 20480, 8192, 3072, "student_t_outliers", 1.0, 0.02, "e2m3", "bf16"),
}

T_NU = 3.0
OUTLIER_FRACTION = 0.001
OUTLIER_FACTOR = 50.0


def rng(index: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([index, stream])


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 numpy array -> bfloat16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def outlier_channels(k: int, index: int) -> np.ndarray:
    n_out = int(round(OUTLIER_FRACTION * k))
    return np.sort(rng(index, 2).choice(k, size=n_out, replace=False))


def make_a(w: Workload, m: int | None = None, k: int | None = None) -> torch.Tensor:
    """Activation matrix [m, k] as a bf16 CPU tensor."""
    m = w.m if m is None else m
    k = w.k if k is None else k
    g = rng(w.index, 0)
    if w.a_dist == "normal":
        x = g.standard_normal((m, k), dtype=np.float32) * np.float32(w.a_std)
    elif w.a_dist == "student_t_outliers":
        x = g.standard_t(T_NU, size=(m, k)).astype(np.float32)
        x[:, outlier_channels(k, w.index)] *= np.float32(OUTLIER_FACTOR)
    else:
        raise ValueError(w.a_dist)
    return to_bf16(x)


def make_w(w: Workload, n: int | None = None, k: int | None = None) -> torch.Tensor:
    """Weight matrix [n, k] (PyTorch Linear layout) as a bf16 CPU tensor."""
    n = w.n if n is None else n
    k = w.k if k is None else k
    x = rng(w.index, 1).standard_normal((n, k), dtype=np.float32) * np.float32(w.w_std)
    return to_bf16(x)


def device_normal_bf16(rows: int, cols: int, seed: int, std: float, device) -> torch.Tensor:
    """Seeded N(0, std^2) matrix [rows, cols] drawn on the device, for inputs of
    many GiB that are too large to draw on the host: torch's generator on that
    device seeded with `seed`, fp32 draws in slabs of at most 2^28 values (so
    the fp32 draw never holds more than one slab), each scaled and rounded to
    bf16.  Checks read the rows they sample back from the device."""
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    slab_rows = max(1, (1 << 28) // max(cols, 1))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    for r0 in range(0, rows, slab_rows):
        r1 = min(rows, r0 + slab_rows)
        slab = torch.randn((r1 - r0, cols), generator=gen, dtype=torch.float32, device=device)
        out[r0:r1] = (slab * std).to(torch.bfloat16)
    return out


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 CPU tensor, for the CPU oracle."""
    return t.detach().cpu().to(torch.float64).numpy()


def random_like_workload(seed: int, m: int, k: int, n: int, a_std: float = 1.0, w_std: float = 0.02,
                         t_outliers: bool = False) -> tuple[torch.Tensor, torch.Tensor]:
    """Small seeded (A, W) pair for parity tests at reduced sizes."""
    g = np.random.default_rng([1000 + seed, m, k, n])
    if t_outliers:
        a = g.standard_t(T_NU, size=(m, k)).astype(np.float32)
        n_out = max(1, int(round(OUTLIER_FRACTION * k)))
        a[:, g.choice(k, size=n_out, replace=False)] *= np.float32(OUTLIER_FACTOR)
    else:
        a = g.standard_normal((m, k), dtype=np.float32) * np.float32(a_std)
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(w_std)
    return to_bf16(a), to_bf16(w)
