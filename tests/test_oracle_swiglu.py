"""Pins for the Spatial SwiGLU oracle, each independent of the oracle's own code.

The pages give no numeric example of this step, so the oracle is pinned by a
hand-worked example (tests/golden/swiglu_hand_2x3.json), pure-Python brute
force with explicit bounds checks, two library routines that fix the
convolution convention (torch's grouped conv2d and scipy's correlate2d, both
in float64), the zero-padding boundary in closed form (interior 9, edge 6,
corner 4 taps), the impulse response (which shows the tap orientation),
closed forms of SiLU and scipy's expit, and linearity.  Together they catch a
flipped kernel (convolution instead of correlation), transposed grid axes,
a missing or doubled pad, the gate and value branches swapped, the bias placed
inside the gate, and SiLU replaced by the bare sigmoid.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch

from oracle import depthwise_conv3x3, silu, spatial_swiglu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B, H, W, C, bias=True):
    g = rng.standard_normal((B, H, W, C))
    v = rng.standard_normal((B, H, W, C))
    w = rng.uniform(-1, 1, (C, 3, 3))
    b = rng.uniform(-1, 1, C) if bias else None
    return g, v, w, b


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "swiglu_hand_2x3.json")) as f:
        fx = json.load(f)
    value = np.array(fx["value"], dtype=np.float64)[None, :, :, None]
    weight = np.array(fx["weight"], dtype=np.float64)[None]
    bias = np.array([fx["bias"]])
    sign = np.array(fx["gate_sign"], dtype=np.float64)
    gate = sign * np.log(np.array(fx["gate_log_arg"], dtype=np.float64))
    conv = depthwise_conv3x3(value, weight, bias)[0, :, :, 0]
    assert np.array_equal(conv, np.array(fx["conv_plus_bias"]))
    h = spatial_swiglu(gate[None, :, :, None], value, weight, bias)[0, :, :, 0]
    want = gate * np.array(fx["sigmoid_of_gate"]) * np.array(fx["conv_plus_bias"])
    np.testing.assert_allclose(h, want, rtol=1e-14, atol=0)


def test_brute_force_loops():
    rng = np.random.default_rng(11)
    B, H, W, C = 2, 3, 4, 3
    g, v, w, b = rand_case(rng, B, H, W, C)
    got = spatial_swiglu(g, v, w, b)
    for bi in range(B):
        for y in range(H):
            for x in range(W):
                for c in range(C):
                    acc = b[c]
                    for dy in (-1, 0, 1):
                        for dx in (-1, 0, 1):
                            yy, xx = y + dy, x + dx
                            if 0 <= yy < H and 0 <= xx < W:
                                acc += w[c, dy + 1, dx + 1] * v[bi, yy, xx, c]
                    gg = g[bi, y, x, c]
                    want = gg / (1.0 + math.exp(-gg)) * acc
                    assert abs(got[bi, y, x, c] - want) <= 1e-13 * (1 + abs(want))


def test_matches_torch_grouped_conv2d():
    # torch's depthwise layer (groups = channels, padding 1) in float64 on the CPU
    rng = np.random.default_rng(12)
    B, H, W, C = 2, 7, 5, 6
    g, v, w, b = rand_case(rng, B, H, W, C)
    vt = torch.from_numpy(v).permute(0, 3, 1, 2)            # NCHW
    ref = torch.nn.functional.conv2d(vt, torch.from_numpy(w)[:, None], torch.from_numpy(b),
                                     padding=1, groups=C)
    ref = ref.permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(depthwise_conv3x3(v, w, b), ref, rtol=1e-13, atol=1e-13)
    want = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * ref
    np.testing.assert_allclose(spatial_swiglu(g, v, w, b), want, rtol=1e-13, atol=1e-13)


def test_matches_scipy_correlate2d_per_channel():
    rng = np.random.default_rng(13)
    H, W, C = 6, 9, 4
    _, v, w, _ = rand_case(rng, 1, H, W, C, bias=False)
    got = depthwise_conv3x3(v, w)
    for c in range(C):
        ref = scipy.signal.correlate2d(v[0, :, :, c], w[c], mode="same", boundary="fill")
        np.testing.assert_allclose(got[0, :, :, c], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("H,W", [(1, 1), (1, 5), (4, 1), (2, 2), (5, 7)])
def test_zero_padding_tap_counts(H, W):
    # all-ones value and kernel: each output counts the in-grid neighbours
    v = np.ones((1, H, W, 1))
    w = np.ones((1, 3, 3))
    got = depthwise_conv3x3(v, w)[0, :, :, 0]
    rows = np.array([min(y + 1, H - 1) - max(y - 1, 0) + 1 for y in range(H)])
    cols = np.array([min(x + 1, W - 1) - max(x - 1, 0) + 1 for x in range(W)])
    assert np.array_equal(got, np.outer(rows, cols).astype(np.float64))
    if H >= 3 and W >= 3:
        assert got[1, 1] == 9 and got[0, 1] == 6 and got[0, 0] == 4


def test_impulse_response_shows_tap_orientation():
    # a unit impulse at (y0, x0) lands tap (i, j) at output (y0 - i + 1, x0 - j + 1)
    H, W = 5, 5
    v = np.zeros((1, H, W, 1))
    v[0, 2, 2, 0] = 1.0
    w = np.arange(1.0, 10.0).reshape(1, 3, 3)
    got = depthwise_conv3x3(v, w)[0, :, :, 0]
    for i in range(3):
        for j in range(3):
            assert got[2 - i + 1, 2 - j + 1] == w[0, i, j]
    assert np.count_nonzero(got) == 9


def test_identity_kernel_and_bias_only():
    rng = np.random.default_rng(14)
    g, v, _, b = rand_case(rng, 1, 4, 6, 5)
    ident = np.zeros((5, 3, 3))
    ident[:, 1, 1] = 1.0
    np.testing.assert_allclose(spatial_swiglu(g, v, ident), silu(g) * v, rtol=1e-15)
    np.testing.assert_allclose(spatial_swiglu(g, np.zeros_like(v), ident, b), silu(g) * b,
                               rtol=1e-15)


def test_channels_are_independent_and_batch_split():
    rng = np.random.default_rng(15)
    g, v, w, b = rand_case(rng, 3, 4, 5, 6)
    full = spatial_swiglu(g, v, w, b)
    for c in range(6):
        one = spatial_swiglu(g[..., c:c + 1], v[..., c:c + 1], w[c:c + 1], b[c:c + 1])
        np.testing.assert_allclose(full[..., c:c + 1], one, rtol=1e-15)
    for bi in range(3):
        np.testing.assert_allclose(full[bi:bi + 1], spatial_swiglu(g[bi:bi + 1], v[bi:bi + 1],
                                                                   w, b), rtol=1e-15)


def test_linear_in_value():
    rng = np.random.default_rng(16)
    g, v1, w, _ = rand_case(rng, 1, 5, 4, 3, bias=False)
    v2 = rng.standard_normal(v1.shape)
    lhs = spatial_swiglu(g, 2.5 * v1 - 0.75 * v2, w)
    rhs = 2.5 * spatial_swiglu(g, v1, w) - 0.75 * spatial_swiglu(g, v2, w)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_silu_closed_forms_and_tails():
    ln3, ln7 = math.log(3.0), math.log(7.0)
    got = silu(np.array([0.0, ln3, -ln3, ln7, -ln7]))
    want = np.array([0.0, 0.75 * ln3, -0.25 * ln3, 0.875 * ln7, -0.125 * ln7])
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        tails = silu(np.array([-800.0, -40.0, 40.0, 800.0]))
    assert tails[0] == 0.0 and tails[3] == 800.0
    assert abs(tails[1] - (-40.0 * math.exp(-40.0))) <= 1e-12 * 40.0 * math.exp(-40.0)
    assert tails[2] == 40.0 * (1.0 / (1.0 + math.exp(-40.0)))


def test_silu_matches_scipy_expit():
    x = np.linspace(-30.0, 30.0, 4001)
    np.testing.assert_allclose(silu(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-300)


def test_gate_and_value_are_not_interchangeable():
    # the conv acts on the value branch only: swapping the branches changes the result
    rng = np.random.default_rng(17)
    g, v, w, b = rand_case(rng, 1, 4, 4, 2)
    assert not np.allclose(spatial_swiglu(g, v, w, b), spatial_swiglu(v, g, w, b))
    # and a kernel that is not a pure centre tap mixes neighbours, unlike plain SwiGLU
    assert not np.allclose(spatial_swiglu(g, v, w), silu(g) * v * w[:, 1, 1])
