"""Seeded synthetic workloads shaped like the GTR patch grids.

This module only draws random inputs; it holds none of the operator's
arithmetic and is shared by the tests, the benchmark and the smoke check.

The grids stand in for the images of the GTR pages (GTR news write-up,
tokendh.com, sections "Where the speed comes from" and "Resolution scaling";
GTR abstract, arXiv 2609.26590): 640x640 at patch 16 -> 40x40 tokens (1.6K),
768x768 -> 48x48, 2048x2048 -> 128x128 (16.4K).  No dataset is used.

Recipe (one numpy Generator per call set, numpy.random.default_rng(seed)):
  draw z_q, z_k, z_v, z_g ~ N(0, 1) (float32) in that order, each of the
  tensor's full shape [B, heads, H, W, d];
  q = z_q / 8, k = z_k / 8, v = z_v / 8;
  log_alpha = logsigmoid(gate_std * z_g) / 16   (the gate-logit normaliser 16);
  then cast to the call's storage dtype (fp16 round-to-nearest-even, or fp32).
Both the GPU path and the oracle read exactly these stored values.
"""

from dataclasses import dataclass, field
from typing import List

import numpy as np

SCAN_NAMES = {0: "L2R", 1: "R2L", 2: "T2B", 3: "B2T", 4: "ROTATE_BATCH"}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    H: int
    W: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str                 # "fp16" or "fp32"
    gate_std: float
    seeds: List[int] = field(default_factory=list)
    dirs: List[int] = field(default_factory=list)   # one call per (seed, dir) pair

    @property
    def T(self):
        return self.H * self.W

    @property
    def calls(self):
        return list(zip(self.seeds, self.dirs))


# The five synthetic configurations the operator is specified on.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 16, 16, 64, 64, 64, "fp32", 1.0, [0], [0]),
    "gtr1.6k": Workload("gtr1.6k", 1, 12, 40, 40, 64, 64, 64, "fp16", 1.0,
                        [1, 1, 1, 1], [0, 1, 2, 3]),
    "img768": Workload("img768", 1, 16, 48, 48, 64, 64, 64, "fp16", 1.0,
                       [200 + i for i in range(12)], [i % 4 for i in range(12)]),
    "hires16.4k": Workload("hires16.4k", 1, 12, 128, 128, 64, 64, 64, "fp16", 2.0,
                           [3, 3, 3, 3], [0, 1, 2, 3]),
    "batched": Workload("batched", 32, 16, 64, 64, 128, 64, 64, "fp16", 1.0, [4], [4]),
}


def _logsigmoid(y):
    # log(sigmoid(y)) = -log(1 + exp(-y)), evaluated without overflow
    return -np.logaddexp(np.zeros((), dtype=y.dtype), -y)


def make_inputs(B, heads, H, W, d_k, d_v, dtype="fp16", gate_std=1.0, seed=0):
    """Return (q, k, v, log_alpha) as numpy arrays of the storage dtype."""
    rng = np.random.default_rng(seed)
    shp_k = (B, heads, H, W, d_k)
    shp_v = (B, heads, H, W, d_v)
    npd = np.float16 if dtype == "fp16" else np.float32
    q = (rng.standard_normal(shp_k, dtype=np.float32) * np.float32(0.125)).astype(npd)
    k = (rng.standard_normal(shp_k, dtype=np.float32) * np.float32(0.125)).astype(npd)
    v = (rng.standard_normal(shp_v, dtype=np.float32) * np.float32(0.125)).astype(npd)
    zg = rng.standard_normal(shp_k, dtype=np.float32)
    la = (_logsigmoid(zg * np.float32(gate_std)) / np.float32(16.0)).astype(npd)
    return q, k, v, la


def workload_inputs(wl: Workload, seed: int, B=None, heads=None):
    """Inputs of one call of a named workload (B / heads may be overridden)."""
    return make_inputs(B or wl.B, heads or wl.heads, wl.H, wl.W, wl.d_k, wl.d_v,
                       wl.dtype, wl.gate_std, seed)


# Spatial SwiGLU step on the same grids.  The hidden width is 8/3 of the model
# width (the usual SwiGLU ratio): 768 = 12 heads x 64 -> 2048 channels at
# 16.4K; 1024 = 16 x 64 -> 2736 (8/3 x 1024 rounded up to a multiple of 16)
# at 768x768.
@dataclass(frozen=True)
class SwigluWorkload:
    name: str
    B: int
    H: int
    W: int
    C: int
    seed: int

    @property
    def T(self):
        return self.H * self.W


SWIGLU_WORKLOADS = {
    "swiglu_hires16.4k": SwigluWorkload("swiglu_hires16.4k", 1, 128, 128, 2048, 5),
    "swiglu_img768": SwigluWorkload("swiglu_img768", 1, 48, 48, 2736, 6),
}


def make_swiglu_inputs(B, H, W, C, seed=0, bias=True, packed=False):
    """Return (gate, value, weight, bias) as float16 numpy arrays.

    Recipe: numpy.random.default_rng(seed); gate and value ~ N(0, 1) drawn in
    that order, [B, H, W, C] each (the pre-activations of two linear
    projections of normalised tokens); weight [C, 3, 3] and bias [C] ~
    U(-1/3, 1/3), the default initialisation bound 1/sqrt(fan_in) of a 3x3
    depthwise layer (fan_in = 9).  With packed=True gate and value are
    returned as two views into one [B, H, W, 2C] array (gate first), the
    layout of a single fused up-projection.
    """
    rng = np.random.default_rng(seed)
    shp = (B, H, W, C)
    g = rng.standard_normal(shp, dtype=np.float32).astype(np.float16)
    v = rng.standard_normal(shp, dtype=np.float32).astype(np.float16)
    w = rng.uniform(-1.0 / 3.0, 1.0 / 3.0, (C, 3, 3)).astype(np.float16)
    b = rng.uniform(-1.0 / 3.0, 1.0 / 3.0, C).astype(np.float16) if bias else None
    if packed:
        both = np.concatenate([g, v], axis=-1)
        g, v = both[..., :C], both[..., C:]
    return g, v, w, b


# SAGA-style non-causal gated linear attention on the same token counts.
@dataclass(frozen=True)
class SagaWorkload:
    name: str
    B: int
    heads: int
    N: int
    d_k: int
    d_v: int
    seed: int


SAGA_WORKLOADS = {
    "saga_hires16.4k": SagaWorkload("saga_hires16.4k", 1, 12, 128 * 128, 64, 64, 7),
    "saga_batched": SagaWorkload("saga_batched", 32, 16, 64 * 64, 128, 64, 8),
}


def make_saga_inputs(B, heads, N, d_k, d_v, seed=0):
    """Return (q, k, v, a, b) as float16 numpy arrays.

    Recipe: numpy.random.default_rng(seed) draws z_q, z_k, z_v, z_a, z_b
    ~ N(0, 1) (float32) in that order; q, k, v = z / 8 as for the attention
    workloads; the gates a = sigmoid(z_a) [B, heads, N, d_k] and
    b = sigmoid(z_b) [B, heads, N, d_v], values in (0, 1).
    """
    rng = np.random.default_rng(seed)
    sk, sv = (B, heads, N, d_k), (B, heads, N, d_v)
    q = (rng.standard_normal(sk, dtype=np.float32) * np.float32(0.125)).astype(np.float16)
    k = (rng.standard_normal(sk, dtype=np.float32) * np.float32(0.125)).astype(np.float16)
    v = (rng.standard_normal(sv, dtype=np.float32) * np.float32(0.125)).astype(np.float16)
    za = rng.standard_normal(sk, dtype=np.float32)
    zb = rng.standard_normal(sv, dtype=np.float32)
    a = (np.float32(1.0) / (np.float32(1.0) + np.exp(-za))).astype(np.float16)
    b = (np.float32(1.0) / (np.float32(1.0) + np.exp(-zb))).astype(np.float16)
    return q, k, v, a, b


def make_bwd_inputs(B, heads, H, W, d_v, d_k=64, seed=0):
    """Return (d_out, d_final_state, initial_state) for the backward pass.

    Recipe: numpy.random.default_rng(seed) draws d_out ~ N(0, 1) as float16
    [B, heads, H, W, d_v], then d_final_state and initial_state ~ N(0, 1) / 8
    as float32 [B, heads, d_k, d_v], in that order.
    """
    rng = np.random.default_rng(seed)
    do = rng.standard_normal((B, heads, H, W, d_v), dtype=np.float32).astype(np.float16)
    dfin = (rng.standard_normal((B, heads, d_k, d_v), dtype=np.float32) * np.float32(0.125))
    init = (rng.standard_normal((B, heads, d_k, d_v), dtype=np.float32) * np.float32(0.125))
    return do, dfin, init
