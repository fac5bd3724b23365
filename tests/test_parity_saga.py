"""GPU parity of the SAGA-style gated linear attention against the CPU oracle.

Every case calls the HIP kernels through the C ABI (gla_saga_fwd) and compares
out and the gated key-value map kv with the float64 oracle on the same float16
inputs: the float16 bar of the attention path (relative Frobenius error
<= 5e-3, max |error| <= 2e-2 max |ref|) and, element by element, a bound
derived from the kernels' arithmetic:

  * k * alpha and v * beta are rounded to float16 (2^-11 relative each, or
    2^-25 absolute in the subnormal range) and their products summed in
    float32 over at most N = 16K tokens (below 2^-10 relative to the sum of
    magnitudes): |dKV| <= 2^-9 (|K A|^T |V B|) + 2^-24 (sum |K A| + sum |V B|);
  * the map is read as float16 after a power-of-two scaling per MFMA operand
    (16 value columns x 32 key dims): at most 2^-12 of the operand's largest
    |KV| entry, bounded here by 2^-11 max |KV|;
  * O = Q KV is summed in float32 and rounded to float16 (2^-11 relative).

  |dO| <= 2^-11 |O| + |Q| (bound on |dKV| + 2^-11 max|KV|) + 2^-24
"""

import numpy as np
import pytest
import torch

from oracle import saga_forward
from recurrent_vision_token_amd import GlaError, saga_fwd
from recurrent_vision_token_amd.workloads import SAGA_WORKLOADS, make_saga_inputs

pytestmark = pytest.mark.gpu


def run(q, k, v, a, b, want_kv=True):
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v, a, b)]
    out, kv = saga_fwd(*t, want_kv=want_kv)
    torch.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64),
            None if kv is None else kv.cpu().numpy().astype(np.float64))


def check(got_out, got_kv, q, k, v, a, b, label=""):
    ref_out, ref_kv = saga_forward(q, k, v, a, b)
    f = lambda x: np.abs(x.astype(np.float64))
    mag = np.matmul(np.swapaxes(f(k) * f(a), -1, -2), f(v) * f(b))       # |K A|^T |V B|
    # a product rounded into the float16 subnormal range is off by up to 2^-25
    # absolute: add 2^-24 (sum_t |k a|_ti + sum_t |v b|_tj)
    sub = 2.0 ** -24 * ((f(k) * f(a)).sum(axis=-2)[..., :, None] +
                        (f(v) * f(b)).sum(axis=-2)[..., None, :])
    kv_bound = 2.0 ** -9 * mag + sub
    kv_max = np.abs(ref_kv).max(axis=(-2, -1), keepdims=True)
    if got_kv is not None:
        err = np.abs(got_kv - ref_kv)
        bound = kv_bound
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), "%s kv: %.3g > %.3g at %s" % (label, err[worst], bound[worst],
                                                                    worst)
    bound = (2.0 ** -11 * np.abs(ref_out) +
             np.matmul(f(q), kv_bound + 2.0 ** -11 * kv_max) + 2.0 ** -24)
    err = np.abs(got_out - ref_out)
    assert np.all(np.isfinite(got_out)), label
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), "%s out: %.3g > %.3g at %s (ref %.4g)" % (
        label, err[worst], bound[worst], worst, ref_out[worst])
    rel = np.linalg.norm(got_out - ref_out) / np.linalg.norm(ref_out)
    assert rel <= 5e-3 and err.max() <= 2e-2 * np.abs(ref_out).max(), (label, rel)
    if got_kv is not None:
        relk = np.linalg.norm(got_kv - ref_kv) / np.linalg.norm(ref_kv)
        assert relk <= 5e-3, (label, relk)
    return rel


@pytest.mark.parametrize("B,heads,N,dk,dv", [
    (1, 2, 64, 64, 64),          # one chunk, one output block
    (2, 3, 1000, 64, 64),        # ragged chunk and output tails, several spans
    (1, 4, 4099, 64, 128),
    (1, 3, 777, 128, 64),
    (2, 2, 300, 128, 128),
    (1, 1, 1, 64, 64),           # a single token
    (1, 1, 17, 128, 128),
])
def test_parity_shapes(B, heads, N, dk, dv):
    q, k, v, a, b = make_saga_inputs(B, heads, N, dk, dv, seed=N + dk)
    print("saga case", B, heads, N, dk, dv, flush=True)
    out, kv = run(q, k, v, a, b)
    check(out, kv, q, k, v, a, b, "%dx%dx%d %d/%d" % (B, heads, N, dk, dv))


def test_without_kv_output_and_deterministic():
    q, k, v, a, b = make_saga_inputs(1, 3, 2500, 64, 64, seed=41)
    o1, kv = run(q, k, v, a, b, want_kv=False)
    assert kv is None
    o2, _ = run(q, k, v, a, b, want_kv=False)
    assert np.array_equal(o1, o2)
    check(o1, None, q, k, v, a, b, "no kv")


def test_large_and_tiny_maps_keep_their_precision():
    # the per-column power-of-two scaling keeps a map far outside float16's
    # comfortable range exact to float16 precision, in both directions
    for scale in (64.0, 1.0 / 4096.0):
        q, k, v, a, b = make_saga_inputs(1, 2, 3000, 64, 64, seed=42)
        v = (v.astype(np.float32) * np.float32(scale)).astype(np.float16)
        out, kv = run(q, k, v, a, b)
        check(out, kv, q, k, v, a, b, "scale %g" % scale)


def test_gate_zero_and_one():
    q, k, v, _, _ = make_saga_inputs(1, 2, 500, 64, 64, seed=43)
    ones_k, ones_v = np.ones_like(k), np.ones_like(v)
    out, kv = run(q, k, v, ones_k, ones_v)
    check(out, kv, q, k, v, ones_k, ones_v, "ungated")
    zero_a = np.zeros_like(k)
    out0, kv0 = run(q, k, v, zero_a, ones_v)
    assert np.all(out0 == 0) and np.all(kv0 == 0)


def test_binding_rejects_bad_tensors():
    dev = torch.device("cuda:0")
    x = torch.zeros((1, 2, 8, 64), dtype=torch.float16, device=dev)
    y = torch.zeros((1, 2, 8, 32), dtype=torch.float16, device=dev)
    with pytest.raises(GlaError):
        saga_fwd(x, x, y, x, y)                  # d_v = 32 is not built
    with pytest.raises(ValueError):
        saga_fwd(x, x, x, x, x[..., :32])        # beta shape differs from v


@pytest.mark.parametrize("name", sorted(SAGA_WORKLOADS))
def test_full_size_workloads(name):
    wl = SAGA_WORKLOADS[name]
    q, k, v, a, b = make_saga_inputs(wl.B, wl.heads, wl.N, wl.d_k, wl.d_v, seed=wl.seed)
    print("saga workload", name, flush=True)
    if wl.B * wl.heads > 64:
        # check a sample of (b, h) sequences at full length against the oracle
        out, kv = run(q, k, v, a, b)
        rng = np.random.default_rng(0)
        for bh in rng.choice(wl.B * wl.heads, 12, replace=False):
            bi, h = divmod(int(bh), wl.heads)
            sl = (slice(bi, bi + 1), slice(h, h + 1))
            check(out[sl], kv[sl], q[sl], k[sl], v[sl], a[sl], b[sl], "%s bh %d" % (name, bh))
    else:
        out, kv = run(q, k, v, a, b)
        rel = check(out, kv, q, k, v, a, b, name)
        print("%s rel %.3g" % (name, rel), flush=True)
