"""Pins for the backward oracle (gla_backward), each independent of its code.

The gradients are pinned by central finite differences of the pinned forward
oracle (every coordinate of a tiny case, all four directions and the batch
rotation, with an initial state and a final-state gradient), by torch's
float64 autograd through the closed quadratic form of the recurrence (a
different formulation: cumulative log-decays and an explicit causal sum), by
the closed-form gradients of causal linear attention when alpha = 1, and by
the identity dlog_alpha_t = sum_{s >= t} (q_s * dq_s - k_s * dk_s) plus the
final-state term, a second derivation of the gate gradient.  Together they
catch a dropped term, a decay applied one step off, the final-state or
initial-state gradient missing, and a wrong scan order in the reverse sweep.
"""

import numpy as np
import pytest
import torch

from oracle import gla_backward, gla_forward, scan_order


def rand_case(rng, B, nh, H, W, dk, dv, gate=0.4):
    q = rng.standard_normal((B, nh, H, W, dk))
    k = rng.standard_normal((B, nh, H, W, dk))
    v = rng.standard_normal((B, nh, H, W, dv))
    la = -gate * rng.uniform(0.05, 1.0, (B, nh, H, W, dk))
    do = rng.standard_normal((B, nh, H, W, dv))
    init = rng.standard_normal((B, nh, dk, dv))
    dfin = rng.standard_normal((B, nh, dk, dv))
    return q, k, v, la, do, init, dfin


def loss(q, k, v, la, do, d, init, dfin):
    out, fin = gla_forward(q, k, v, la, d, initial_state=init)
    return float(np.sum(do * out) + np.sum(dfin * fin))


@pytest.mark.parametrize("d", [0, 1, 2, 3, 4])
def test_finite_differences_every_coordinate(d):
    rng = np.random.default_rng(60 + d)
    B = 2 if d == 4 else 1
    q, k, v, la, do, init, dfin = rand_case(rng, B, 1, 2, 3, 3, 2)
    grads = gla_backward(q, k, v, la, do, d, d_final_state=dfin, initial_state=init, segment=4)
    args = [q, k, v, la, init]
    eps = 1e-6
    for which, g in zip((0, 1, 2, 3, 4), (grads[0], grads[1], grads[2], grads[3], grads[4])):
        x = args[which]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            lp = loss(ap[0], ap[1], ap[2], ap[3], do, d, ap[4], dfin)
            lm = loss(am[0], am[1], am[2], am[3], do, d, am[4], dfin)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg="input %d" % which)


def test_torch_autograd_of_the_quadratic_form():
    # o_t = sum_{s<=t} (q_t * exp(b_t - b_s)) . k_s v_s + (q_t * exp(b_t)) S0 and
    # final = exp(b_T) S0 + sum_s exp(b_T - b_s) k_s v_s, b the cumulative
    # log-decay in scan order; autograd differentiates it on its own
    rng = np.random.default_rng(70)
    B, nh, H, W, dk, dv = 1, 2, 3, 5, 4, 3
    q, k, v, la, do, init, dfin = rand_case(rng, B, nh, H, W, dk, dv)
    for d in range(4):
        perm = scan_order(H, W, d)
        T = H * W
        tq, tk, tv, tla, tinit = (torch.tensor(x.reshape(B, nh, T, -1)[:, :, perm] if x.ndim == 5
                                               else x, dtype=torch.float64, requires_grad=True)
                                  for x in (q, k, v, la, init))
        b = torch.cumsum(tla, dim=2)                                   # [B, nh, T, dk]
        dec = torch.exp(b[:, :, :, None, :] - b[:, :, None, :, :])    # [.., t, s, dk]
        mask = torch.tril(torch.ones(T, T, dtype=torch.float64))[:, :, None]
        scores = torch.einsum("bhti,bhtsi,bhsi->bhts", tq, dec * mask, tk)
        out = torch.einsum("bhts,bhsj->bhtj", scores, tv) + \
            torch.einsum("bhti,bhij->bhtj", tq * torch.exp(b), tinit)
        fin = torch.exp(b[:, :, -1, :])[..., None] * tinit + \
            torch.einsum("bhsi,bhsj->bhij", tk * torch.exp(b[:, :, -1:, :] - b), tv)
        L = (out * torch.tensor(do.reshape(B, nh, T, dv)[:, :, perm])).sum() + \
            (fin * torch.tensor(dfin)).sum()
        L.backward()
        g = gla_backward(q, k, v, la, do, d, d_final_state=dfin, initial_state=init, segment=4)
        for got, t in zip(g[:4], (tq, tk, tv, tla)):
            ref = np.zeros(got.reshape(B, nh, T, -1).shape)
            ref[:, :, perm] = t.grad.numpy()
            np.testing.assert_allclose(got.reshape(ref.shape), ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g[4], tinit.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_alpha_one_is_causal_linear_attention():
    rng = np.random.default_rng(71)
    B, nh, H, W, dk, dv = 1, 1, 4, 4, 5, 3
    q, k, v, la, do, init, dfin = rand_case(rng, B, nh, H, W, dk, dv)
    la = np.zeros_like(la)
    g = gla_backward(q, k, v, la, do, 0, d_final_state=dfin, initial_state=init)
    T = H * W
    Q, K, V, dO = (x.reshape(T, -1) for x in (q[0, 0], k[0, 0], v[0, 0], do[0, 0]))
    M = np.tril(np.ones((T, T)))
    S0, dSf = init[0, 0], dfin[0, 0]
    np.testing.assert_allclose(g[0].reshape(T, dk), (dO @ V.T * M) @ K + dO @ S0.T, rtol=1e-11)
    np.testing.assert_allclose(g[1].reshape(T, dk), (V @ dO.T * M.T) @ Q + V @ dSf.T, rtol=1e-11)
    np.testing.assert_allclose(g[2].reshape(T, dv), (K @ Q.T * M.T) @ dO + K @ dSf, rtol=1e-11)
    np.testing.assert_allclose(g[4][0, 0], Q.T @ dO + dSf, rtol=1e-11)


@pytest.mark.parametrize("d", [0, 2, 3])
def test_gate_gradient_suffix_sum_identity(d):
    rng = np.random.default_rng(72 + d)
    B, nh, H, W, dk, dv = 2, 2, 5, 7, 4, 3
    q, k, v, la, do, init, dfin = rand_case(rng, B, nh, H, W, dk, dv)
    dq, dk_, _, dla, _ = gla_backward(q, k, v, la, do, d, d_final_state=dfin, initial_state=init,
                                      segment=8)
    _, fin = gla_forward(q, k, v, la, d, initial_state=init)
    T = H * W
    perm = scan_order(H, W, d)
    x = (q * dq - k * dk_).reshape(B, nh, T, dk)[:, :, perm]
    suffix = np.cumsum(x[:, :, ::-1], axis=2)[:, :, ::-1]
    suffix = suffix + np.einsum("bhij,bhij->bhi", dfin, fin)[:, :, None, :]
    np.testing.assert_allclose(dla.reshape(B, nh, T, dk)[:, :, perm], suffix, rtol=1e-10,
                               atol=1e-12)


def test_segment_length_does_not_matter():
    rng = np.random.default_rng(73)
    args = rand_case(rng, 1, 2, 6, 11, 4, 4)
    q, k, v, la, do, init, dfin = args
    a = gla_backward(q, k, v, la, do, 1, d_final_state=dfin, initial_state=init, segment=64)
    b = gla_backward(q, k, v, la, do, 1, d_final_state=dfin, initial_state=init, segment=5)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)
