"""Pins for the SAGA oracle, each independent of the oracle's own code.

The pages print no numeric example, so the oracle is pinned by a hand-worked
example (tests/golden/saga_hand_2tok.json), the explicit per-token gated maps
G_i * (k_i^T v_i) summed in a Python loop (the form the factorisation
replaces), the ungated special case against the quadratic (Q K^T) V order,
a single token in closed form, token-permutation invariance (the form is
non-causal), and linearity / scaling.  Together they catch a gate applied to
the wrong operand, a transposed map, a dropped gate, a causal mask slipped in,
and swapped key / value dims.
"""

import json
import os

import numpy as np

from oracle import saga_forward, saga_kv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(rng, B, nh, N, dk, dv):
    q = rng.standard_normal((B, nh, N, dk))
    k = rng.standard_normal((B, nh, N, dk))
    v = rng.standard_normal((B, nh, N, dv))
    a = rng.uniform(0, 1, (B, nh, N, dk))
    b = rng.uniform(0, 1, (B, nh, N, dv))
    return q, k, v, a, b


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "saga_hand_2tok.json")) as f:
        fx = json.load(f)
    t = {n: np.array(fx[n], dtype=np.float64)[None, None] for n in ("q", "k", "v", "alpha", "beta")}
    out, kv = saga_forward(t["q"], t["k"], t["v"], t["alpha"], t["beta"])
    assert np.array_equal(kv[0, 0], np.array(fx["kv"]))
    assert np.array_equal(out[0, 0], np.array(fx["out"]))


def test_explicit_gated_maps_loop():
    # the KVGate form before factorisation: G_i = alpha_i^T beta_i times k_i^T v_i
    rng = np.random.default_rng(31)
    B, nh, N, dk, dv = 2, 3, 7, 5, 4
    q, k, v, a, b = rand(rng, B, nh, N, dk, dv)
    out, kv = saga_forward(q, k, v, a, b)
    for bi in range(B):
        for h in range(nh):
            m = np.zeros((dk, dv))
            for i in range(N):
                gate = np.outer(a[bi, h, i], b[bi, h, i])
                m += gate * np.outer(k[bi, h, i], v[bi, h, i])
            np.testing.assert_allclose(kv[bi, h], m, rtol=1e-13, atol=1e-13)
            for t in range(N):
                o = np.array([sum(q[bi, h, t, r] * m[r, c] for r in range(dk)) for c in range(dv)])
                np.testing.assert_allclose(out[bi, h, t], o, rtol=1e-12, atol=1e-12)


def test_ungated_is_quadratic_order_linear_attention():
    rng = np.random.default_rng(32)
    q, k, v, _, _ = rand(rng, 1, 2, 9, 6, 3)
    ones_k, ones_v = np.ones_like(k), np.ones_like(v)
    out, _ = saga_forward(q, k, v, ones_k, ones_v)
    quad = np.matmul(np.matmul(q, np.swapaxes(k, -1, -2)), v)      # (Q K^T) V, all pairs
    np.testing.assert_allclose(out, quad, rtol=1e-12, atol=1e-12)


def test_single_token_closed_form():
    rng = np.random.default_rng(33)
    q, k, v, a, b = rand(rng, 1, 1, 1, 4, 3)
    out, _ = saga_forward(q, k, v, a, b)
    want = np.dot(q[0, 0, 0], k[0, 0, 0] * a[0, 0, 0]) * (v[0, 0, 0] * b[0, 0, 0])
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=1e-14)


def test_non_causal_permutation_invariance():
    rng = np.random.default_rng(34)
    q, k, v, a, b = rand(rng, 1, 2, 11, 4, 5)
    perm = rng.permutation(11)
    out, kv = saga_forward(q, k, v, a, b)
    # permuting the key/value tokens leaves every output unchanged
    out2, kv2 = saga_forward(q, k[:, :, perm], v[:, :, perm], a[:, :, perm], b[:, :, perm])
    np.testing.assert_allclose(kv2, kv, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-12)
    # and the first token's output depends on the last token (no causal mask)
    v3 = v.copy()
    v3[:, :, -1] += 1.0
    out3, _ = saga_forward(q, k, v3, a, b)
    assert not np.allclose(out3[:, :, 0], out[:, :, 0])


def test_linearity_and_gate_scaling():
    rng = np.random.default_rng(35)
    q, k, v, a, b = rand(rng, 2, 1, 6, 3, 4)
    v2 = rng.standard_normal(v.shape)
    o1, _ = saga_forward(q, k, v, a, b)
    o2, _ = saga_forward(q, k, v2, a, b)
    o12, _ = saga_forward(q, k, 2.0 * v - 0.5 * v2, a, b)
    np.testing.assert_allclose(o12, 2.0 * o1 - 0.5 * o2, rtol=1e-12, atol=1e-12)
    os_, _ = saga_forward(q, k, v, 0.5 * a, 4.0 * b)
    np.testing.assert_allclose(os_, 2.0 * o1, rtol=1e-13, atol=1e-13)
    # gates on the key side act per key dim: a gate that zeroes key dim 0 equals
    # dropping that dim from q and k
    a0 = a.copy()
    a0[..., 0] = 0.0
    oz, _ = saga_forward(q, k, v, a0, b)
    od, _ = saga_forward(q[..., 1:], k[..., 1:], v, a[..., 1:], b)
    np.testing.assert_allclose(oz, od, rtol=1e-12, atol=1e-12)


def test_kv_shape_and_batches_independent():
    rng = np.random.default_rng(36)
    q, k, v, a, b = rand(rng, 3, 2, 5, 4, 6)
    out, kv = saga_forward(q, k, v, a, b)
    assert kv.shape == (3, 2, 4, 6) and out.shape == (3, 2, 5, 6)
    o1, _ = saga_forward(q[1:2, 1:2], k[1:2, 1:2], v[1:2, 1:2], a[1:2, 1:2], b[1:2, 1:2])
    np.testing.assert_allclose(out[1:2, 1:2], o1, rtol=1e-14)
    np.testing.assert_allclose(saga_kv(k, v, a, b), kv, rtol=0)
