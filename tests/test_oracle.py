"""Pins for the CPU oracle, each independent of the oracle's own code.

The pages print no numeric example of the operator, so the oracle is pinned
by: a hand-derived worked example and hand-listed scan orders (tests/golden),
the brute-force quadratic form of the recurrence on tiny inputs, closed forms
(alpha = 1 linear attention, alpha -> 0, a first-order IIR filter from scipy
for d_k = 1), direction / grid invariants, linearity, state consistency,
composition across a split of the scan, and causality.  Together they catch a
dropped term, a sign flip in the gate, decay applied after the add instead of
before, exclusive instead of inclusive outputs, decay on the value side, a
wrong scan order, and transposed operands.  The initial-state input is pinned
by the brute-force form with the state's own decay written out and by
linearity; the gate activation by closed forms, the logsigmoid identity,
its tails and scipy's independent log_expit.
"""

import json
import os

import numpy as np
import pytest
import scipy.signal

from oracle import gla_forward, scan_order

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return np.linalg.norm(a - b) / den


def rand_inputs(rng, B, nh, H, W, dk, dv, gate_scale=0.5):
    q = rng.standard_normal((B, nh, H, W, dk))
    k = rng.standard_normal((B, nh, H, W, dk))
    v = rng.standard_normal((B, nh, H, W, dv))
    la = -gate_scale * rng.random((B, nh, H, W, dk))
    return q, k, v, la


# ---------------------------------------------------------------- golden pins

def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_1x3.json")))
    q = np.array(g["q"]).reshape(1, 1, 1, 3, 2)
    k = np.array(g["k"]).reshape(1, 1, 1, 3, 2)
    v = np.array(g["v"]).reshape(1, 1, 1, 3, 1)
    la = np.log(np.array(g["alpha"])).reshape(1, 1, 1, 3, 2)
    for name, d in (("L2R", 0), ("R2L", 1)):
        out, fin = gla_forward(q, k, v, la, d)
        exp = g["expected"][name]
        np.testing.assert_allclose(out.reshape(3, 1), exp["out"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(fin.reshape(2, 1), exp["final_state"], rtol=0, atol=1e-14)


def test_scan_orders_hand_listed():
    g = json.load(open(os.path.join(GOLDEN, "scan_orders_2x3.json")))
    for d, order in g["orders"].items():
        assert scan_order(g["H"], g["W"], int(d)).tolist() == order


@pytest.mark.parametrize("H,W", [(1, 1), (1, 5), (4, 1), (3, 7), (6, 6)])
def test_scan_order_is_permutation(H, W):
    for d in range(4):
        p = scan_order(H, W, d)
        assert sorted(p.tolist()) == list(range(H * W))


# ------------------------------------------------------------ brute force pin

def brute_force(q, k, v, la, d):
    """o_t = sum_{s<=t} sum_i q_t[i] exp(sum_{r=s+1..t} la_r[i]) k_s[i] v_s (scan order)."""
    B, nh, H, W, dk = q.shape
    dv = v.shape[-1]
    T = H * W
    perm = scan_order(H, W, d)
    out = np.zeros((B, nh, T, dv))
    fin = np.zeros((B, nh, dk, dv))
    for b in range(B):
        for h in range(nh):
            Q = q[b, h].reshape(T, dk)[perm]
            K = k[b, h].reshape(T, dk)[perm]
            V = v[b, h].reshape(T, dv)[perm]
            L = la[b, h].reshape(T, dk)[perm]
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    for i in range(dk):
                        dec = np.exp(sum(L[r, i] for r in range(s + 1, t + 1)))
                        acc += Q[t, i] * dec * K[s, i] * V[s]
                out[b, h, perm[t]] = acc
            for i in range(dk):
                for s in range(T):
                    dec = np.exp(sum(L[r, i] for r in range(s + 1, T)))
                    fin[b, h, i] += dec * K[s, i] * V[s]
    return out.reshape(B, nh, H, W, dv), fin


@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_brute_force(d):
    rng = np.random.default_rng(10 + d)
    q, k, v, la = rand_inputs(rng, 1, 2, 3, 4, 3, 2)
    out, fin = gla_forward(q, k, v, la, d)
    bo, bf = brute_force(q, k, v, la, d)
    assert rel(out, bo) < TOL
    assert rel(fin, bf) < TOL


def test_rotate_batch_matches_per_element_direction():
    rng = np.random.default_rng(3)
    q, k, v, la = rand_inputs(rng, 5, 2, 3, 4, 3, 2)
    out, fin = gla_forward(q, k, v, la, 4)
    for b in range(5):
        bo, bf = brute_force(q[b:b + 1], k[b:b + 1], v[b:b + 1], la[b:b + 1], b % 4)
        assert rel(out[b:b + 1], bo) < TOL
        assert rel(fin[b:b + 1], bf) < TOL


# ----------------------------------------------------------------- closed forms

@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_alpha_one_is_causal_linear_attention(d):
    rng = np.random.default_rng(20 + d)
    q, k, v, _ = rand_inputs(rng, 2, 3, 5, 6, 4, 3)
    la = np.zeros_like(q)
    out, fin = gla_forward(q, k, v, la, d)
    perm = scan_order(5, 6, d)
    for b in range(2):
        for h in range(3):
            Q = q[b, h].reshape(30, 4)[perm]
            K = k[b, h].reshape(30, 4)[perm]
            V = v[b, h].reshape(30, 3)[perm]
            ref = np.tril(Q @ K.T) @ V
            got = out[b, h].reshape(30, 3)[perm]
            assert rel(got, ref) < TOL
            assert rel(fin[b, h], K.T @ V) < TOL


def test_dk1_constant_gate_is_first_order_filter():
    # with d_k = 1 and a constant gate a, each state column is the IIR filter
    # S_t = a S_{t-1} + k_t v_t, which scipy.signal.lfilter evaluates directly
    rng = np.random.default_rng(7)
    H, W, dv = 4, 9, 5
    a = 0.83
    q, k, v, _ = rand_inputs(rng, 1, 1, H, W, 1, dv)
    la = np.full_like(q, np.log(a))
    out, fin = gla_forward(q, k, v, la, 2)
    perm = scan_order(H, W, 2)
    K = k[0, 0].reshape(-1)[perm]
    V = v[0, 0].reshape(-1, dv)[perm]
    Q = q[0, 0].reshape(-1)[perm]
    S = scipy.signal.lfilter([1.0], [1.0, -a], K[:, None] * V, axis=0)
    ref = Q[:, None] * S
    assert rel(out[0, 0].reshape(-1, dv)[perm], ref) < TOL
    assert rel(fin[0, 0, 0], S[-1]) < TOL


def test_alpha_zero_limit():
    rng = np.random.default_rng(8)
    q, k, v, _ = rand_inputs(rng, 1, 2, 3, 5, 4, 3)
    la = np.full_like(q, -np.inf)
    out, fin = gla_forward(q, k, v, la, 1)
    ref = np.einsum("bhxyi,bhxyi->bhxy", q, k)[..., None] * v
    assert rel(out, ref) < TOL
    last = scan_order(3, 5, 1)[-1]
    r, c = divmod(int(last), 5)
    assert rel(fin, k[:, :, r, c, :, None] * v[:, :, r, c, None, :]) < TOL


# ------------------------------------------------------------------ invariants

def test_direction_invariants():
    rng = np.random.default_rng(11)
    q, k, v, la = rand_inputs(rng, 2, 2, 4, 6, 3, 2)
    fw = lambda x: x[:, :, :, ::-1, :]  # noqa: E731
    fh = lambda x: x[:, :, ::-1, :, :]  # noqa: E731
    tr = lambda x: np.swapaxes(x, 2, 3)  # noqa: E731

    o1, s1 = gla_forward(q, k, v, la, 1)
    o0, s0 = gla_forward(fw(q), fw(k), fw(v), fw(la), 0)
    assert rel(o1, fw(o0)) < TOL and rel(s1, s0) < TOL

    o3, s3 = gla_forward(q, k, v, la, 3)
    o2, s2 = gla_forward(fh(q), fh(k), fh(v), fh(la), 2)
    assert rel(o3, fh(o2)) < TOL and rel(s3, s2) < TOL

    o2, s2 = gla_forward(q, k, v, la, 2)
    o0, s0 = gla_forward(tr(q), tr(k), tr(v), tr(la), 0)
    assert rel(o2, tr(o0)) < TOL and rel(s2, s0) < TOL


def test_degenerate_grids():
    rng = np.random.default_rng(12)
    # H x 1: a single column
    q, k, v, la = rand_inputs(rng, 1, 2, 6, 1, 3, 2)
    o0, s0 = gla_forward(q, k, v, la, 0)
    for d in (1, 2):
        o, s = gla_forward(q, k, v, la, d)
        assert rel(o, o0) < TOL and rel(s, s0) < TOL
    # 1 x W: a single row
    q, k, v, la = rand_inputs(rng, 1, 2, 1, 6, 3, 2)
    o0, s0 = gla_forward(q, k, v, la, 0)
    for d in (2, 3):
        o, s = gla_forward(q, k, v, la, d)
        assert rel(o, o0) < TOL and rel(s, s0) < TOL
    # 1 x 1: o = (q . k) v
    q, k, v, la = rand_inputs(rng, 1, 1, 1, 1, 4, 3)
    for d in range(4):
        o, s = gla_forward(q, k, v, la, d)
        assert rel(o[0, 0, 0, 0], np.dot(q[0, 0, 0, 0], k[0, 0, 0, 0]) * v[0, 0, 0, 0]) < TOL
        assert rel(s[0, 0], np.outer(k[0, 0, 0, 0], v[0, 0, 0, 0])) < TOL


def test_linearity():
    rng = np.random.default_rng(13)
    q, k, v, la = rand_inputs(rng, 1, 2, 3, 4, 3, 2)
    v2 = rng.standard_normal(v.shape)
    oa, sa = gla_forward(q, k, v, la, 2)
    ob, sb = gla_forward(q, k, v2, la, 2)
    oc, sc = gla_forward(q, k, v + v2, la, 2)
    assert rel(oc, oa + ob) < TOL and rel(sc, sa + sb) < TOL
    od, _ = gla_forward(2.5 * q, k, v, la, 2)
    assert rel(od, 2.5 * oa) < TOL


@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_final_state_consistency(d):
    rng = np.random.default_rng(14 + d)
    q, k, v, la = rand_inputs(rng, 2, 2, 3, 5, 4, 3)
    out, fin = gla_forward(q, k, v, la, d)
    last = scan_order(3, 5, d)[-1]
    r, c = divmod(int(last), 5)
    ref = np.einsum("bhi,bhij->bhj", q[:, :, r, c], fin)
    assert rel(out[:, :, r, c], ref) < TOL


def test_composition_across_a_split():
    # the state after the first rows, fed as the initial state of the rest,
    # reproduces the full left->right run (the chunk hand-off of the pages)
    rng = np.random.default_rng(15)
    q, k, v, la = rand_inputs(rng, 1, 2, 6, 5, 3, 2)
    full_o, full_s = gla_forward(q, k, v, la, 0)
    o1, s1 = gla_forward(q[:, :, :2], k[:, :, :2], v[:, :, :2], la[:, :, :2], 0)
    o2, s2 = gla_forward(q[:, :, 2:], k[:, :, 2:], v[:, :, 2:], la[:, :, 2:], 0, initial_state=s1)
    assert rel(np.concatenate([o1, o2], axis=2), full_o) < TOL
    assert rel(s2, full_s) < TOL


@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_causality(d):
    rng = np.random.default_rng(16 + d)
    H, W = 4, 5
    q, k, v, la = rand_inputs(rng, 1, 2, H, W, 3, 2)
    perm = scan_order(H, W, d)
    t0 = 9
    later = perm[t0 + 1:]
    q2, k2, v2, la2 = (x.copy() for x in (q, k, v, la))
    for x in (q2, k2, v2, la2):
        flat = x.reshape(1, 2, H * W, -1)
        flat[:, :, later] += rng.standard_normal(flat[:, :, later].shape)
    o_a, _ = gla_forward(q, k, v, la, d)
    o_b, _ = gla_forward(q2, k2, v2, la2, d)
    early = perm[:t0 + 1]
    fa = o_a.reshape(1, 2, H * W, -1)[:, :, early]
    fb = o_b.reshape(1, 2, H * W, -1)[:, :, early]
    assert np.array_equal(fa, fb)


# ------------------------------------------------- initial state, gate logits

@pytest.mark.parametrize("d", [0, 2, 3])
def test_brute_force_with_initial_state(d):
    # o_t = q_t (diag(prod_{r<=t} alpha_r) S0 + sum_{s<=t} ...): the initial
    # state is decayed by every step up to and including t, written out by hand
    rng = np.random.default_rng(40 + d)
    q, k, v, la = rand_inputs(rng, 1, 2, 3, 4, 3, 2)
    s0 = rng.standard_normal((1, 2, 3, 2))
    out, fin = gla_forward(q, k, v, la, d, initial_state=s0)
    bo, bf = brute_force(q, k, v, la, d)
    H, W, T = 3, 4, 12
    perm = scan_order(H, W, d)
    for h in range(2):
        Q = q[0, h].reshape(T, 3)[perm]
        L = la[0, h].reshape(T, 3)[perm]
        for t in range(T):
            extra = np.zeros(2)
            for i in range(3):
                extra += Q[t, i] * np.exp(sum(L[r, i] for r in range(t + 1))) * s0[0, h, i]
            bo.reshape(1, 2, T, 2)[0, h, perm[t]] += extra
        for i in range(3):
            bf[0, h, i] += np.exp(sum(L[r, i] for r in range(T))) * s0[0, h, i]
    assert rel(out, bo) < TOL
    assert rel(fin, bf) < TOL


def test_initial_state_enters_linearly():
    # the outputs are affine in the initial state: doubling it doubles the
    # difference from the zero-state run
    rng = np.random.default_rng(44)
    q, k, v, la = rand_inputs(rng, 2, 2, 4, 3, 4, 3)
    s0 = rng.standard_normal((2, 2, 4, 3))
    o0, f0 = gla_forward(q, k, v, la, 1)
    o1, f1 = gla_forward(q, k, v, la, 1, initial_state=s0)
    o2, f2 = gla_forward(q, k, v, la, 1, initial_state=2 * s0)
    assert rel(o2 - o0, 2 * (o1 - o0)) < TOL
    assert rel(f2 - f0, 2 * (f1 - f0)) < TOL


def test_gate_activation_closed_forms():
    from oracle import log_alpha_from_logits as act
    ln2 = np.log(2.0)
    assert abs(act(0.0, 1.0) + ln2) < 1e-15
    assert abs(act(0.0, 16.0) + ln2 / 16) < 1e-16
    # sigmoid(ln 3) = 3/4
    assert abs(act(np.log(3.0), 2.0) - np.log(0.75) / 2) < 1e-15
    # logsigmoid(z) - logsigmoid(-z) = z for any z
    z = np.linspace(-40, 40, 161)
    assert np.max(np.abs(act(z, 1.0) - act(-z, 1.0) - z)) < 1e-12
    # tails: -log(1 + e^-z) ~ -e^-z for large z, ~ z for very negative z
    assert abs(act(40.0, 1.0) + np.exp(-40.0)) < 1e-30
    assert abs(act(-800.0, 1.0) + 800.0) < 1e-12
    # alpha = sigmoid(z)^(1/tau), checked against a direct evaluation
    zz = np.linspace(-8, 8, 33)
    assert np.max(np.abs(np.exp(16.0 * act(zz, 16.0)) - 1.0 / (1.0 + np.exp(-zz)))) < 1e-15
    for bad in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            act(0.0, bad)


def test_gate_activation_matches_scipy():
    from scipy.special import log_expit
    from oracle import log_alpha_from_logits as act
    z = np.random.default_rng(45).standard_normal(1000) * 6
    assert np.max(np.abs(act(z, 16.0) - log_expit(z) / 16.0)) < 1e-15
