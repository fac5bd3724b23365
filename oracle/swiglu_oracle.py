"""CPU oracle for the Spatial SwiGLU token-mixing step.

TEST INFRASTRUCTURE ONLY.  Like gla_oracle.py, this is the plain, slow,
obviously correct reference the GPU path is checked against.  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product path never calls it and shares no code with it.

What it computes (float64 throughout):

  * SwiGLU is a gated linear unit: one linear branch passed through SiLU
    (the gate) multiplies another linear branch (the value) element by
    element.  The Spatial SwiGLU of GTR puts a 3x3 depthwise convolution into
    the value branch, so that every patch sees its eight grid neighbours
    directly; each channel is filtered on its own with its own 3x3 kernel
    (GTR news write-up, tokendh.com, section "The flaw of one-way scanning and
    GTR's fix", the Spatial SwiGLU and depthwise-convolution notes; GTR
    abstract, arXiv 2609.26590: "spatially enhanced SwiGLU blocks").
  * With the two branch pre-activations G = x W_gate and V = x W_value laid out
    on the patch grid, the fused step is

        h[b, y, x, c] = silu(G[b, y, x, c]) * ( bias[c]
                        + sum_{i, j in 0..2} w[c, i, j] * V[b, y+i-1, x+j-1, c] )

    with silu(g) = g / (1 + exp(-g)).  The projections themselves (x W_gate,
    x W_value and the output projection) are dense matrix products and are
    not part of this step.

Readings where the pages are silent (each listed with its reason in the
design notes of the repository):
  * zero padding of one patch on every side, stride 1, so the output grid is
    the input grid ("same" size);
  * the kernel is applied as a cross-correlation (tap w[c, i, j] weighs the
    neighbour at row offset i-1 and column offset j-1), the convention of
    deep-learning convolution layers;
  * the convolution carries an optional per-channel bias, added before the
    gate multiplies; no activation follows the convolution;
  * the conv acts on the value branch only; the gate branch is SiLU of its
    projection, unfiltered.

Tensors use the channels-last grid layout [B][H][W][C] (a token's channels
are contiguous), the layout the projections produce.
"""

import numpy as np


def silu(g):
    """SiLU (swish with unit slope), g * sigmoid(g), in float64.

    Written as g * e^g / (1 + e^g) for negative g and g / (1 + e^-g) otherwise,
    so that no exponential overflows.
    """
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))                       # in (0, 1]
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig


def depthwise_conv3x3(value, weight, bias=None):
    """3x3 depthwise convolution of a channels-last grid, float64.

    value: [B, H, W, C]; weight: [C, 3, 3] (a [C, 1, 3, 3] layer weight may be
    passed as is); bias: [C] or None.  Zero padding of one patch, stride 1;
    tap (i, j) weighs the neighbour at offset (i - 1, j - 1).  Each output is
    the sum of the nine taps, done as nine shifted copies of the zero-padded
    grid, one per tap.
    """
    v = np.asarray(value, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64).reshape(-1, 3, 3)
    B, H, W, C = v.shape
    if w.shape[0] != C:
        raise ValueError("weight has %d channels, value has %d" % (w.shape[0], C))
    padded = np.zeros((B, H + 2, W + 2, C), dtype=np.float64)
    padded[:, 1:H + 1, 1:W + 1, :] = v
    acc = np.zeros((B, H, W, C), dtype=np.float64)
    for i in range(3):
        for j in range(3):
            # output (y, x) reads padded (y + i, x + j) = value (y + i - 1, x + j - 1)
            acc += w[:, i, j] * padded[:, i:i + H, j:j + W, :]
    if bias is not None:
        acc += np.asarray(bias, dtype=np.float64).reshape(C)
    return acc


def spatial_swiglu(gate, value, weight, bias=None):
    """Fused Spatial SwiGLU step: silu(gate) * (depthwise_conv3x3(value) + bias).

    gate, value: [B, H, W, C] (any float dtype; taken exactly, computed in
    float64); weight: [C, 3, 3]; bias: [C] or None.  Returns float64
    [B, H, W, C].
    """
    g = np.asarray(gate, dtype=np.float64)
    if g.shape != np.shape(value):
        raise ValueError("gate and value shapes differ")
    return silu(g) * depthwise_conv3x3(value, weight, bias)
