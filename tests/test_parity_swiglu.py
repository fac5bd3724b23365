"""GPU parity of the Spatial SwiGLU kernel against the CPU oracle.

Every case calls the HIP kernel through the C ABI (gla_spatial_swiglu) and
compares it element by element with the float64 oracle on the same float16
inputs.  Besides the float16 bar used for the attention path (relative
Frobenius error <= 5e-3, max |error| <= 2e-2 max |ref|), each element must
meet a bound derived from the kernel's arithmetic:

  * each tap is an exact fp16 x fp16 product added in float32: nine rounded
    additions, at most 9 * 2^-24 * A with A = |bias| + sum |w v|;
  * silu in float32 (scaled argument, hardware exp2 and reciprocal, each
    within an ulp or two): relative error below (|g| + 8) * 2^-24;
  * the final float16 round to nearest even: 2^-11 relative, 2^-25 absolute
    for subnormals.

The test allows |got - ref| <= 2^-11 |ref| + 2^-20 (|silu g| A + (1 + |g|) |ref|)
+ 2^-24, a margin of 2x or more on each term.
"""

import numpy as np
import pytest
import torch

from oracle import depthwise_conv3x3, silu, spatial_swiglu as oracle_swiglu
from recurrent_vision_token_amd import GlaError, spatial_swiglu
from recurrent_vision_token_amd.workloads import SWIGLU_WORKLOADS, make_swiglu_inputs

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def to_dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def run(g, v, w, b, packed_from=None):
    """Upload, call the kernel, return float64 output on the host."""
    if packed_from is not None:
        both = to_dev(packed_from)
        C = g.shape[-1]
        gt, vt = both[..., :C], both[..., C:]
    else:
        gt, vt = to_dev(g), to_dev(v)
    out = spatial_swiglu(gt, vt, to_dev(w), to_dev(b))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(got, g, v, w, b, label=""):
    ref = oracle_swiglu(g, v, w, b)
    g64 = g.astype(np.float64)
    a = depthwise_conv3x3(np.abs(v.astype(np.float64)), np.abs(w.astype(np.float64)),
                          None if b is None else np.abs(b.astype(np.float64)))
    bound = (2.0 ** -11 * np.abs(ref) + 2.0 ** -20 * (np.abs(silu(g64)) * a +
                                                      (1 + np.abs(g64)) * np.abs(ref))
             + 2.0 ** -24)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), label
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), "%s: |err| %.3g > bound %.3g at %s (ref %.6g)" % (
        label, err[worst], bound[worst], worst, ref[worst])
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 5e-3 and err.max() <= 2e-2 * np.abs(ref).max(), label
    return rel


@pytest.mark.parametrize("B,H,W,C", [
    (1, 16, 32, 64),        # exactly one tile
    (2, 37, 45, 136),       # ragged rows, columns and channels, two images
    (1, 70, 33, 72),        # more rows than one tile, a 1-column tail tile
    (3, 9, 100, 200),       # short grid, several column tiles
    (1, 64, 64, 8),         # one channel group
])
def test_parity_shapes(B, H, W, C):
    g, v, w, b = make_swiglu_inputs(B, H, W, C, seed=100 + H)
    print("swiglu case", B, H, W, C, flush=True)
    check(run(g, v, w, b), g, v, w, b, "%dx%dx%dx%d" % (B, H, W, C))


@pytest.mark.parametrize("H,W", [(1, 1), (1, 70), (70, 1), (2, 2), (3, 31)])
def test_degenerate_grids(H, W):
    g, v, w, b = make_swiglu_inputs(2, H, W, 24, seed=7 + H + W)
    print("swiglu degenerate", H, W, flush=True)
    check(run(g, v, w, b), g, v, w, b, "%dx%d" % (H, W))


def test_without_bias():
    g, v, w, _ = make_swiglu_inputs(1, 20, 40, 128, seed=21, bias=False)
    check(run(g, v, w, None), g, v, w, None, "no bias")


def test_fused_projection_halves():
    # gate and value as the two halves of one [B, H, W, 2C] tensor (ld = 2C)
    B, H, W, C = 2, 24, 35, 96
    g, v, w, b = make_swiglu_inputs(B, H, W, C, seed=22, packed=True)
    both = np.concatenate([g, v], axis=-1)
    check(run(g, v, w, b, packed_from=both), np.ascontiguousarray(g), np.ascontiguousarray(v),
          w, b, "packed")


def test_gate_tails_and_impulse():
    # gate values across the whole float16 activation range, value an impulse
    # grid: checks the silu tails (no NaN, signed zeros) and the tap orientation
    B, H, W, C = 1, 12, 40, 64
    rng = np.random.default_rng(23)
    g = rng.uniform(-90, 90, (B, H, W, C)).astype(np.float16)
    v = np.zeros((B, H, W, C), np.float16)
    v[0, 5, 17, :] = 1.0
    v[0, 0, 0, :] = -2.0
    v[0, H - 1, W - 1, :] = 3.0
    w = rng.uniform(-1, 1, (C, 3, 3)).astype(np.float16)
    b = np.zeros(C, np.float16)
    check(run(g, v, w, b), g, v, w, b, "tails")


def test_output_stays_in_bounds_and_is_deterministic():
    B, H, W, C = 1, 19, 21, 40
    g, v, w, b = make_swiglu_inputs(B, H, W, C, seed=24)
    n = B * H * W * C
    canary = torch.full((n + 4096,), 7.0, dtype=torch.float16, device=dev())
    out = canary[2048:2048 + n].view(B, H, W, C)
    gt, vt, wt, bt = to_dev(g), to_dev(v), to_dev(w), to_dev(b)
    spatial_swiglu(gt, vt, wt, bt, out=out)
    first = out.clone()
    spatial_swiglu(gt, vt, wt, bt, out=out)
    torch.cuda.synchronize()
    c = canary.cpu().numpy()
    assert np.all(c[:2048] == 7.0) and np.all(c[2048 + n:] == 7.0)
    assert torch.equal(first, out)
    check(out.cpu().numpy().astype(np.float64), g, v, w, b, "canary")


def test_binding_rejects_bad_tensors():
    g = torch.zeros((1, 4, 4, 12), dtype=torch.float16, device=dev())
    w = torch.zeros((12, 3, 3), dtype=torch.float16, device=dev())
    with pytest.raises(GlaError):
        spatial_swiglu(g, g.clone(), w)                  # C = 12 is not a multiple of 8
    g8 = torch.zeros((1, 4, 4, 16), dtype=torch.float16, device=dev())
    w8 = torch.zeros((16, 3, 3), dtype=torch.float16, device=dev())
    with pytest.raises(ValueError):
        spatial_swiglu(g8.float(), g8.float(), w8.float())
    with pytest.raises(ValueError):
        spatial_swiglu(g8, g8.transpose(1, 2), w8)       # not a dense token layout


@pytest.mark.parametrize("name", sorted(SWIGLU_WORKLOADS))
def test_full_size_workloads(name):
    wl = SWIGLU_WORKLOADS[name]
    g, v, w, b = make_swiglu_inputs(wl.B, wl.H, wl.W, wl.C, seed=wl.seed)
    print("swiglu workload", name, flush=True)
    rel = check(run(g, v, w, b), g, v, w, b, name)
    print("%s rel %.3g" % (name, rel), flush=True)
