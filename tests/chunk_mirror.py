"""numpy mirror of the chunkwise decomposition the HIP kernels use.

Not the oracle and not the product: a CPU model of the kernels' algebra
(spans of chunks, per-chunk cumulative log-decay, 16-token sub-block anchors,
span summaries, the span-boundary scan, and the inter-chunk term), so that the
decomposition itself can be checked against the token recurrence in float64
without a GPU.  With ``fp16=True`` it rounds the operands to binary16 at the
points where the kernels store 16-bit tiles, which estimates the rounding error
the GPU path should show.

The chunkwise form follows the pages' description of the operator: fixed-size
chunks computed in parallel inside, a boundary state handed from chunk to chunk,
and chunk summaries computed for all chunks at once with only the boundary
hand-off done in order (GTR news write-up, tokendh.com, section "Where the
speed comes from").  The factoring of the rank-1 decay mask into row and column
scalings is the Hadamard-product identity of the SAGA summary (gist.science,
Methodology section B).
"""

import numpy as np

SUB = 16


def _scan_order(H, W, d):
    # independent restatement of the four grid walks (row-major cell index)
    idx = np.arange(H * W).reshape(H, W)
    if d == 0:
        return idx.reshape(-1)
    if d == 1:
        return idx[:, ::-1].reshape(-1)
    if d == 2:
        return idx.T.reshape(-1)
    if d == 3:
        return idx[::-1, :].T.reshape(-1)
    raise ValueError(d)


def _r16(x, on):
    return x.astype(np.float16).astype(np.float64) if on else x


def _chunk_tiles(x, c0, C, T):
    """Rows [c0, c0+C) of a [N, T, d] array, zero-padded past T."""
    n = min(C, T - c0)
    out = np.zeros((x.shape[0], C, x.shape[2]))
    out[:, :n] = x[:, c0:c0 + n]
    return out


def span_summary(K, V, LA, s, m, C, T, fp16=False):
    """(G, L) of span s: L is the state reached from zero over the span."""
    N, _, dk = K.shape
    dv = V.shape[2]
    G = np.ones((N, dk))
    L = np.zeros((N, dk, dv))
    n_chunks = -(-T // C)
    for c in range(s * m, min((s + 1) * m, n_chunks)):
        k = _chunk_tiles(K, c * C, C, T)
        v = _chunk_tiles(V, c * C, C, T)
        la = _chunk_tiles(LA, c * C, C, T)
        b = np.cumsum(la, axis=1)
        blast = b[:, -1, :]
        kl = _r16(k * np.exp(blast[:, None, :] - b), fp16)
        L = np.exp(blast)[:, :, None] * L + np.einsum("nti,ntj->nij", kl, v)
        G = G * np.exp(blast)
    return G, L


def chunk_output(Q, K, V, LA, c, C, T, S, fp16=False, split_state=True):
    """Outputs of chunk c given its entry state S; returns (O, S_next)."""
    q = _chunk_tiles(Q, c * C, C, T)
    k = _chunk_tiles(K, c * C, C, T)
    v = _chunk_tiles(V, c * C, C, T)
    la = _chunk_tiles(LA, c * C, C, T)
    N = q.shape[0]
    nsb = C // SUB
    # cumulative decay inside each 16-token sub-block, and sub-block totals
    cs = np.cumsum(la.reshape(N, nsb, SUB, -1), axis=2)          # [N, nsb, 16, dk]
    D = cs[:, :, -1, :]                                          # [N, nsb, dk]
    Bst = np.concatenate([np.zeros_like(D[:, :1]), np.cumsum(D, axis=1)[:, :-1]], axis=1)
    blast = D.sum(axis=1)                                        # [N, dk]
    ql = _r16((q.reshape(N, nsb, SUB, -1) * np.exp(cs)), fp16)
    kd = _r16((k.reshape(N, nsb, SUB, -1) * np.exp(-cs)), fp16)
    vv = v.reshape(N, nsb, SUB, -1)
    A = np.zeros((N, nsb, SUB, nsb, SUB))
    tri = np.tril(np.ones((SUB, SUB)))
    for I in range(nsb):
        for J in range(I + 1):
            if J == I:
                a = np.einsum("nti,nsi->nts", ql[:, I], kd[:, J]) * tri
            else:
                f = np.exp(Bst[:, I] - Bst[:, J])                 # <= 1 per key dim
                kf = _r16(kd[:, J] * f[:, None, :], fp16)
                a = np.einsum("nti,nsi->nts", ql[:, I], kf)
            A[:, I, :, J, :] = a
    A = _r16(A, fp16).reshape(N, C, C)
    # entry state as the 16-bit operand (optionally a hi + lo pair)
    if fp16 and split_state:
        s_hi = _r16(S, True)
        s_lo = _r16(S - s_hi, True)
        s_op = s_hi + s_lo
    else:
        s_op = _r16(S, fp16)
    qinter = _r16(ql * np.exp(Bst)[:, :, None, :], fp16).reshape(N, C, -1)
    O = A @ v + qinter @ s_op
    kl = _r16(kd * np.exp(blast[:, None, None, :] - Bst[:, :, None, :]), fp16).reshape(N, C, -1)
    S_next = np.exp(blast)[:, :, None] * S + np.einsum("nti,ntj->nij", kl, v)
    return O, S_next


def mirror_forward(q, k, v, log_alpha, scan_dir, C=64, m=4, fp16=False, split_state=True):
    """Full chunkwise forward: span summaries -> span scan -> per-span outputs."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    la = np.asarray(log_alpha, dtype=np.float64)
    B, nh, H, W, dk = q.shape
    dv = v.shape[-1]
    T = H * W
    assert C % SUB == 0
    out = np.zeros((B, nh, T, dv))
    fin = np.zeros((B, nh, dk, dv))
    for b in range(B):
        d = b % 4 if scan_dir == 4 else scan_dir
        perm = _scan_order(H, W, d)
        Q = q[b].reshape(nh, T, dk)[:, perm]
        K = k[b].reshape(nh, T, dk)[:, perm]
        V = v[b].reshape(nh, T, dv)[:, perm]
        LA = la[b].reshape(nh, T, dk)[:, perm]
        n_chunks = -(-T // C)
        n_spans = -(-n_chunks // m)
        # all span summaries (parallel on the GPU), then the boundary scan
        aggs = [span_summary(K, V, LA, s, m, C, T, fp16) for s in range(n_spans)]
        S = np.zeros((nh, dk, dv))
        entry = []
        for G, L in aggs:
            entry.append(S)
            S = G[:, :, None] * S + L
        fin[b] = S
        # per-span outputs seeded with the span's entry state
        Ob = np.zeros((nh, n_chunks * C, dv))
        for s in range(n_spans):
            St = entry[s]
            for c in range(s * m, min((s + 1) * m, n_chunks)):
                O, St = chunk_output(Q, K, V, LA, c, C, T, St, fp16, split_state)
                Ob[:, c * C:(c + 1) * C] = O
        out[b][:, perm] = Ob[:, :T]
    return out.reshape(B, nh, H, W, dv), fin
