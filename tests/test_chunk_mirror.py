"""The chunkwise decomposition (numpy mirror of the kernels) equals the oracle."""

import numpy as np
import pytest

from oracle import gla_forward
from recurrent_vision_token_amd.workloads import make_inputs
from tests.chunk_mirror import mirror_forward


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("H,W,C,m,d", [
    (7, 9, 16, 1, 0),     # ragged tail chunk, one chunk per span
    (7, 9, 32, 2, 1),
    (5, 13, 64, 3, 2),    # T < 2 chunks
    (9, 16, 16, 4, 3),
    (1, 1, 16, 1, 0),
    (12, 12, 48, 2, 4),   # rotate per batch element
])
def test_mirror_equals_oracle_fp64(H, W, C, m, d):
    rng = np.random.default_rng(H * 100 + W)
    B = 4 if d == 4 else 1
    q = rng.standard_normal((B, 2, H, W, 5))
    k = rng.standard_normal((B, 2, H, W, 5))
    v = rng.standard_normal((B, 2, H, W, 3))
    la = -0.3 * rng.random((B, 2, H, W, 5))
    o_ref, s_ref = gla_forward(q, k, v, la, d)
    o, s = mirror_forward(q, k, v, la, d, C=C, m=m)
    assert rel(o, o_ref) < 1e-12
    assert rel(s, s_ref) < 1e-12


def test_mirror_fp16_rounding_within_tolerance():
    # the 16-bit operand roundings of the kernels stay well inside the fp16
    # acceptance bound (relative Frobenius 5e-3, max abs 2e-2 * max|ref|)
    q, k, v, la = make_inputs(1, 2, 24, 24, 64, 64, "fp16", 2.0, seed=5)
    o_ref, s_ref = gla_forward(q, k, v, la, 2)
    o, s = mirror_forward(q, k, v, la, 2, C=64, m=2, fp16=True)
    assert rel(o, o_ref) < 1e-3
    assert np.abs(o - o_ref).max() < 2e-3 * np.abs(o_ref).max()
    assert rel(s, s_ref) < 1e-3
