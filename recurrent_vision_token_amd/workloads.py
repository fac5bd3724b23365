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
