"""CPU oracle for gated linear attention with key-only decay over a patch grid.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
reference that the GPU path is checked against.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never calls it and shares no code with it.

What it computes (float64 throughout, token by token):

  * A running d_k x d_v "memory summary" S is carried from token to token; each
    token reads it once and updates it once, so the cost is linear in the
    token count (GTR news write-up, tokendh.com, section "What linear attention
    saves": the running summary replacing pairwise comparison).
  * A learnable forget gate decides how much of the summary survives each step
    (same section: the GLA forget gate).  The gate acts on the key side only;
    the value-side decay is the constant 1 (same section: key-only decay).
    With alpha_t = exp(log_alpha_t) in (0, 1]^{d_k} the step is

        S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,        o_t = q_t S_t

    i.e. the past is decayed before the current token is added, and the output
    of token t includes token t itself.
  * A token only sees tokens earlier in scan order; each call scans the H x W
    grid in one of four directions, left->right, right->left, top->bottom,
    bottom->top (GTR news write-up, section "The flaw of one-way scanning and
    GTR's fix"; GTR abstract, arXiv 2609.26590: alternating spatial scan
    directions).  The state is carried across row / column ends: one sequence
    of H*W steps per (batch, head).

Readings where the pages are silent (each listed with its reason in the
design notes of the repository):
  * right->left flips the column index only (rows still top to bottom);
    top->bottom is column-major with columns left to right; bottom->top flips
    the row index of top->bottom (columns still left to right).
  * scan_dir 4 ("rotate") gives batch element b the direction b mod 4.
  * no 1/sqrt(d_k) scaling, no normaliser, zero initial state unless one is
    given.

Inputs and outputs use the grid layout [B][heads][H][W][d]; outputs are
written back in grid order, not scan order.
"""

import numpy as np

SCAN_L2R = 0
SCAN_R2L = 1
SCAN_T2B = 2
SCAN_B2T = 3
SCAN_ROTATE_BATCH = 4


def scan_order(H, W, scan_dir):
    """Return perm with perm[t] = row-major grid index visited at scan step t.

    Direction definitions follow the four scan directions of the GTR news
    write-up (section on one-way scanning and GTR's fix), read as in the module
    docstring.
    """
    H = int(H)
    W = int(W)
    rows = np.arange(H, dtype=np.int64)
    cols = np.arange(W, dtype=np.int64)
    if scan_dir == SCAN_L2R:
        r, c = np.meshgrid(rows, cols, indexing="ij")          # row-major walk
    elif scan_dir == SCAN_R2L:
        r, c = np.meshgrid(rows, cols[::-1], indexing="ij")    # each row right to left
    elif scan_dir == SCAN_T2B:
        c, r = np.meshgrid(cols, rows, indexing="ij")          # column-major walk
    elif scan_dir == SCAN_B2T:
        c, r = np.meshgrid(cols, rows[::-1], indexing="ij")    # each column bottom to top
    else:
        raise ValueError("scan_dir must be 0..3 here, got %r" % (scan_dir,))
    return (r * W + c).reshape(-1)


def batch_directions(B, scan_dir):
    """Direction used by each batch element (scan_dir 4 rotates b -> b mod 4)."""
    if scan_dir == SCAN_ROTATE_BATCH:
        return [b % 4 for b in range(B)]
    if scan_dir not in (0, 1, 2, 3):
        raise ValueError("scan_dir must be 0..4, got %r" % (scan_dir,))
    return [scan_dir] * B


def log_alpha_from_logits(z, tau):
    """Forget-gate activation: log alpha = logsigmoid(z) / tau, in float64.

    The pages describe a learnable forget gate on the key side (GTR news
    write-up, section "What linear attention saves"); its activation is read
    as the usual gated-linear-attention one, alpha = sigmoid(z)^(1/tau), which
    is also how the synthetic workloads draw their gates (logsigmoid of a
    normal draw, divided by 16).  logsigmoid(z) = -log(1 + exp(-z)) is
    evaluated as min(z, 0) - log1p(exp(-|z|)), which never overflows.
    """
    tau = float(tau)
    if not (tau > 0.0 and np.isfinite(tau)):
        raise ValueError("tau must be positive and finite")
    z = np.asarray(z, dtype=np.float64)
    return (np.minimum(z, 0.0) - np.log1p(np.exp(-np.abs(z)))) / tau


def gla_forward(q, k, v, log_alpha, scan_dir, initial_state=None):
    """Token-by-token recurrence in float64.

    q, k, log_alpha: [B, heads, H, W, d_k]; v: [B, heads, H, W, d_v]
    initial_state:   optional [B, heads, d_k, d_v] (zero if None)
    returns (out [B, heads, H, W, d_v], final_state [B, heads, d_k, d_v]),
    both float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    la = np.asarray(log_alpha, dtype=np.float64)
    B, nh, H, W, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or la.shape != q.shape or v.shape[:-1] != q.shape[:-1]:
        raise ValueError("shape mismatch among q, k, v, log_alpha")
    T = H * W
    qf = q.reshape(B, nh, T, dk)
    kf = k.reshape(B, nh, T, dk)
    vf = v.reshape(B, nh, T, dv)
    af = np.exp(la.reshape(B, nh, T, dk))      # alpha_t = exp(log alpha_t)

    out = np.zeros((B, nh, T, dv), dtype=np.float64)
    final = np.zeros((B, nh, dk, dv), dtype=np.float64)
    if initial_state is not None:
        init = np.asarray(initial_state, dtype=np.float64)
        if init.shape != (B, nh, dk, dv):
            raise ValueError("initial_state must be [B, heads, d_k, d_v]")
    else:
        init = np.zeros((B, nh, dk, dv), dtype=np.float64)

    dirs = batch_directions(B, scan_dir)
    for d in sorted(set(dirs)):
        bs = np.array([b for b in range(B) if dirs[b] == d], dtype=np.int64)
        perm = scan_order(H, W, d)
        S = init[bs].copy()                                  # [nb, heads, dk, dv]
        for t in range(T):
            p = perm[t]
            a_t = af[bs, :, p, :]                            # [nb, heads, dk]
            k_t = kf[bs, :, p, :]
            v_t = vf[bs, :, p, :]
            # decay the past on the key side, then add the current token
            S = a_t[..., :, None] * S + k_t[..., :, None] * v_t[..., None, :]
            # the output of token t reads the state that already holds token t
            out[bs, :, p, :] = np.einsum("...i,...ij->...j", qf[bs, :, p, :], S)
        final[bs] = S
    return out.reshape(B, nh, H, W, dv), final


def gla_backward(q, k, v, log_alpha, d_out, scan_dir, d_final_state=None, initial_state=None,
                 segment=64):
    """Gradients of the recurrence, float64, by reverse mode token by token.

    For L = sum(d_out * out) + sum(d_final_state * final_state), with out and
    final_state those of gla_forward, returns
    (dq, dk, dv, dlog_alpha, d_initial_state): the first four shaped like
    their inputs, d_initial_state [B, heads, d_k, d_v] (the gradient with
    respect to the state before the first scan step, whether or not one was
    given).

    The adjoint of the state, G_t = dL/dS_t, runs backwards along the scan:
    G_t gathers q_t^T d_out_t and what flows back from S_{t+1} through the
    decay, G_t = q_t^T d_out_t + diag(alpha_{t+1}) G_{t+1}, starting from
    d_final_state.  Differentiating S_t = diag(alpha_t) S_{t-1} + k_t^T v_t
    and o_t = q_t S_t then gives
        dq_t = S_t d_out_t^T,  dk_t = G_t v_t^T,  dv_t = k_t G_t,
        dlog_alpha_t[i] = alpha_t[i] * sum_j G_t[i, j] S_{t-1}[i, j],
    and dL/dS_{-1} = diag(alpha_0) G_0.  The forward states are recomputed per
    segment of `segment` steps from states saved at segment starts.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    la = np.asarray(log_alpha, dtype=np.float64)
    do = np.asarray(d_out, dtype=np.float64)
    B, nh, H, W, dk = q.shape
    dv = v.shape[-1]
    if (k.shape != q.shape or la.shape != q.shape or v.shape[:-1] != q.shape[:-1]
            or do.shape != v.shape):
        raise ValueError("shape mismatch among q, k, v, log_alpha, d_out")
    T = H * W
    qf = q.reshape(B, nh, T, dk)
    kf = k.reshape(B, nh, T, dk)
    vf = v.reshape(B, nh, T, dv)
    dof = do.reshape(B, nh, T, dv)
    af = np.exp(la.reshape(B, nh, T, dk))
    init = (np.zeros((B, nh, dk, dv)) if initial_state is None
            else np.asarray(initial_state, dtype=np.float64))
    dfin = (np.zeros((B, nh, dk, dv)) if d_final_state is None
            else np.asarray(d_final_state, dtype=np.float64))
    if init.shape != (B, nh, dk, dv) or dfin.shape != (B, nh, dk, dv):
        raise ValueError("states must be [B, heads, d_k, d_v]")

    dq = np.zeros_like(qf)
    dkk = np.zeros_like(kf)
    dvv = np.zeros_like(vf)
    dla = np.zeros_like(qf)
    dinit = np.zeros((B, nh, dk, dv))
    dirs = batch_directions(B, scan_dir)
    for d in sorted(set(dirs)):
        bs = np.array([b for b in range(B) if dirs[b] == d], dtype=np.int64)
        perm = scan_order(H, W, d)
        starts = list(range(0, T, segment))
        # forward: the state before each segment
        saved = []
        S = init[bs].copy()
        for t in range(T):
            if t % segment == 0:
                saved.append(S.copy())
            p = perm[t]
            S = af[bs, :, p, :][..., :, None] * S + \
                kf[bs, :, p, :][..., :, None] * vf[bs, :, p, :][..., None, :]
        # backward, segment by segment from the end
        G = dfin[bs].copy()
        for m in range(len(starts) - 1, -1, -1):
            t0, t1 = starts[m], min(T, starts[m] + segment)
            states = [saved[m]]                      # states[i] = S_{t0 + i - 1}
            for t in range(t0, t1):
                p = perm[t]
                states.append(af[bs, :, p, :][..., :, None] * states[-1] +
                              kf[bs, :, p, :][..., :, None] * vf[bs, :, p, :][..., None, :])
            for t in range(t1 - 1, t0 - 1, -1):
                p = perm[t]
                S_t, S_prev = states[t - t0 + 1], states[t - t0]
                a_t = af[bs, :, p, :]
                G = G + qf[bs, :, p, :][..., :, None] * dof[bs, :, p, :][..., None, :]
                dq[bs, :, p, :] = np.einsum("...ij,...j->...i", S_t, dof[bs, :, p, :])
                dkk[bs, :, p, :] = np.einsum("...ij,...j->...i", G, vf[bs, :, p, :])
                dvv[bs, :, p, :] = np.einsum("...i,...ij->...j", kf[bs, :, p, :], G)
                dla[bs, :, p, :] = a_t * np.einsum("...ij,...ij->...i", G, S_prev)
                G = a_t[..., :, None] * G
        dinit[bs] = G
    return (dq.reshape(q.shape), dkk.reshape(k.shape), dvv.reshape(v.shape),
            dla.reshape(q.shape), dinit)
