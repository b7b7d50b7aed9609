"""Input recipes for the benchmarked workloads of the three row reductions.

Shapes follow the QuACK article (无需CUDA代码，给H100加速33%-50%), sections
"NCU 性能分析（Softmax 内核）" (softmax, 16K x 131K fp32) and "内存吞吐量"
(batch 8k-32k, reduction dim 256-262k, fp32 and bf16).  The pages give no
value distributions; the ones here are the library's own stated recipe:
x ~ N(0,1) (cross-entropy logits ~ N(0, sigma=2) in the vocab-like case),
RMSNorm weight ~ U(0.5, 1.5), labels uniform in [0, N), and in the spiky
softmax case each entry independently set to +20 with probability 1 %.
bf16 inputs are the fp32 draw rounded to nearest even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import (SEED, STREAM_DLOSS, STREAM_DY, STREAM_LABELS, STREAM_SPIKES, STREAM_W, STREAM_X,
               labels, normal, spikes_, uniform)

RMSNORM_EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    name: str
    op: str          # "softmax" | "rmsnorm" | "xent" | "xent_grad" | "softmax_bwd" | "rmsnorm_bwd"
    dtype: str       # "f32" | "bf16"
    M: int
    N: int
    sigma: float = 1.0
    spiky: bool = False
    eps: float = RMSNORM_EPS
    extra: dict = field(default_factory=dict)


# The four fixed workloads, smallest first.
SOFTMAX_SMALL = Workload("softmax_f32_256x1024", "softmax", "f32", 256, 1024)
RMSNORM_MAIN = Workload("rmsnorm_bf16_16384x4096", "rmsnorm", "bf16", 16384, 4096)
XENT_VOCAB = Workload("xent_f32_8192x131072", "xent", "f32", 8192, 131072, sigma=2.0)
SOFTMAX_SPIKY = Workload("softmax_f32_16384x131072_spiky", "softmax", "f32", 16384, 131072,
                         spiky=True)
FIXED = [SOFTMAX_SMALL, RMSNORM_MAIN, XENT_VOCAB, SOFTMAX_SPIKY]

# Backward passes (training): the cross-entropy forward fused with its gradient
# on the vocab-like shape above, on a bf16 32K vocabulary and on a bf16 151936-entry
# vocabulary (a row that does not fill a power of two of workgroups; per-row upstream
# gradients dloss ~ U(0.5, 1.5)); the softmax backward from the softmax of
# x ~ N(0, sigma=2) with dy ~ N(0, 1); the RMSNorm backward at the forward's
# shape and a wider fp32 one, x and w as for the forward, dy ~ N(0, 1), rstd from
# the forward.
BACKWARD = [Workload("xentgrad_f32_8192x131072", "xent_grad", "f32", 8192, 131072, sigma=2.0),
            Workload("xentgrad_bf16_16384x32768", "xent_grad", "bf16", 16384, 32768, sigma=2.0),
            Workload("xentgrad_bf16_16384x151936", "xent_grad", "bf16", 16384, 151936,
                     sigma=2.0),
            Workload("softmaxbwd_f32_16384x4096", "softmax_bwd", "f32", 16384, 4096, sigma=2.0),
            Workload("softmaxbwd_bf16_16384x32768", "softmax_bwd", "bf16", 16384, 32768,
                     sigma=2.0),
            Workload("rmsnormbwd_bf16_16384x4096", "rmsnorm_bwd", "bf16", 16384, 4096),
            Workload("rmsnormbwd_f32_16384x16384", "rmsnorm_bwd", "f32", 16384, 16384)]

SWEEP_M = (8192, 16384, 32768)
SWEEP_N = (256, 1024, 4096, 16384, 65536, 262144)


def sweep():
    """All (op, dtype, M, N) points of the 3-op x 2-dtype sweep, x ~ N(0,1)."""
    out = []
    for op in ("softmax", "rmsnorm", "xent"):
        for dtype in ("f32", "bf16"):
            for M in SWEEP_M:
                for N in SWEEP_N:
                    out.append(Workload(f"{op}_{dtype}_{M}x{N}", op, dtype, M, N))
    return out


# The longest rows held on chip (one read, 16 to 256 workgroups per row): 1M, 2M,
# 4M and 8M elements, and 16M for the packed bf16 RMSNorm.
WIDE = [Workload("softmax_f32_1024x1048576", "softmax", "f32", 1024, 1 << 20),
        Workload("rmsnorm_bf16_2048x1048576", "rmsnorm", "bf16", 2048, 1 << 20),
        Workload("softmax_f32_512x2097152", "softmax", "f32", 512, 1 << 21),
        Workload("rmsnorm_bf16_1024x2097152", "rmsnorm", "bf16", 1024, 1 << 21),
        Workload("softmax_f32_256x4194304", "softmax", "f32", 256, 1 << 22),
        Workload("rmsnorm_bf16_512x4194304", "rmsnorm", "bf16", 512, 1 << 22),
        Workload("softmax_f32_128x8388608", "softmax", "f32", 128, 1 << 23),
        Workload("rmsnorm_bf16_256x8388608", "rmsnorm", "bf16", 256, 1 << 23),
        Workload("rmsnorm_f32_256x8388608", "rmsnorm", "f32", 256, 1 << 23),
        Workload("rmsnorm_bf16_128x16777216", "rmsnorm", "bf16", 128, 1 << 24)]

# Rows past the on-chip capacity (read twice): 16M-element fp32 rows and 32M-element
# bf16 rows, the softmax backward's 16M-element fp32 rows and the cross-entropy
# gradient's 16M-element bf16 rows.
LONG = [Workload("softmax_f32_64x16777216", "softmax", "f32", 64, 1 << 24),
        Workload("rmsnorm_bf16_64x33554432", "rmsnorm", "bf16", 64, 1 << 25),
        Workload("softmaxbwd_f32_64x16777216", "softmax_bwd", "f32", 64, 1 << 24, sigma=2.0),
        Workload("xentgrad_bf16_64x16777216", "xent_grad", "bf16", 64, 1 << 24, sigma=2.0)]


# Rows whose length is not a power of two: a 151936-entry vocabulary (softmax) and
# 200000-wide rows (RMSNorm), split into equal shares.
UNEVEN = [Workload("softmax_f32_16384x151936", "softmax", "f32", 16384, 151936),
          Workload("softmax_bf16_16384x151936", "softmax", "bf16", 16384, 151936),
          Workload("rmsnorm_f32_16384x200000", "rmsnorm", "f32", 16384, 200000),
          Workload("rmsnorm_bf16_16384x200000", "rmsnorm", "bf16", 16384, 200000)]


def by_name(name: str) -> Workload:
    for w in FIXED + BACKWARD + WIDE + LONG + UNEVEN + sweep():
        if w.name == name:
            return w
    raise KeyError(name)


def x_rows(w: Workload, *, seed=SEED, rows=None, row0=0, nrows=None, nthreads=0, out=None):
    """The input matrix (or the listed rows of it) for workload ``w``."""
    M = w.M if nrows is None else nrows
    x = normal(M, w.N, sigma=w.sigma, dtype=w.dtype, seed=seed, stream=STREAM_X, rows=rows,
               row0=row0, nthreads=nthreads, out=out)
    if w.spiky:
        spikes_(x, p=0.01, value=20.0, dtype=w.dtype, seed=seed, stream=STREAM_SPIKES, rows=rows,
                row0=row0, nthreads=nthreads)
    return x


def weight(w: Workload, *, seed=SEED) -> np.ndarray:
    """RMSNorm weight[N] ~ U(0.5, 1.5) in the input dtype."""
    return uniform(1, w.N, lo=0.5, hi=1.5, dtype=w.dtype, seed=seed, stream=STREAM_W).reshape(w.N)


def label_rows(w: Workload, *, seed=SEED, rows=None, row0=0, nrows=None) -> np.ndarray:
    """Cross-entropy labels, uniform in [0, N)."""
    M = w.M if nrows is None else nrows
    return labels(M, w.N, seed=seed, stream=STREAM_LABELS, rows=rows, row0=row0)


def dloss_rows(w: Workload, *, seed=SEED, row0=0, nrows=None) -> np.ndarray:
    """Per-row upstream gradient of the loss, U(0.5, 1.5) as float32."""
    M = w.M if nrows is None else nrows
    return uniform(1, M, lo=0.5, hi=1.5, seed=seed, stream=STREAM_DLOSS, row0=row0).reshape(M)


def dy_rows(w: Workload, *, seed=SEED, row0=0, nrows=None) -> np.ndarray:
    """Upstream gradient of a backward pass, N(0, 1) in the input dtype."""
    M = w.M if nrows is None else nrows
    return normal(M, w.N, dtype=w.dtype, seed=seed, stream=STREAM_DY, row0=row0)
