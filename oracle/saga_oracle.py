"""CPU oracle for SAGA-style non-causal gated linear attention.

TEST INFRASTRUCTURE ONLY.  Like gla_oracle.py, this is the plain, slow,
obviously correct reference that the GPU path is checked against.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; the
product path never calls it and shares no code with it.

What it computes (float64):

  * Linear attention builds one d_k x d_v key-value map from the per-token
    maps k_i^T v_i and reads it with every query (SAGA summary, gist.science,
    background of the technical summary: attention reordered from (QK^T)V to
    Q(K^T V)).
  * SAGA's KVGate scales each token's map k_i^T v_i element by element with an
    input-dependent gate matrix G_i before the maps are summed (same summary,
    Methodology section A).
  * With G_i the outer product alpha_i^T beta_i, the identity
    (u^T v) * (x^T y) = (u * x)^T (v * y) moves the gate onto the keys and the
    values, so the map is never formed per token:

        KV = sum_i G_i * (k_i^T v_i) = (K * A)^T (V * B),      O = Q KV

    (same summary, Methodology section B), A = [alpha_i] [N, d_k] and
    B = [beta_i] [N, d_v] the gate vectors of the N tokens.

Readings where the pages are silent (listed with their reasons in the design
notes of the repository):
  * the op takes the gates as inputs (how they are produced is upstream), and
    any feature map on Q and K is applied upstream too;
  * no normaliser and no scale: O = Q KV exactly as printed;
  * every token attends to every token of its (batch, head) sequence (the
    form is non-causal; there is no scan order).

Tensors use [B][heads][N][d] (N tokens, d_k for q, k, a; d_v for v, b, out).
"""

import numpy as np


def saga_kv(k, v, a, b):
    """Gated key-value map KV = (K * A)^T (V * B) per (batch, head), float64.

    k, a: [B, heads, N, d_k]; v, b: [B, heads, N, d_v].  Returns
    [B, heads, d_k, d_v].
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if k.shape != a.shape or v.shape != b.shape or k.shape[:3] != v.shape[:3]:
        raise ValueError("shape mismatch among k, v, a, b")
    ka = k * a
    vb = v * b
    return np.matmul(np.swapaxes(ka, -1, -2), vb)


def saga_forward(q, k, v, a, b):
    """Non-causal gated linear attention O = Q [(K * A)^T (V * B)], float64.

    Returns (out [B, heads, N, d_v], kv [B, heads, d_k, d_v]).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = saga_kv(k, v, a, b)
    if q.shape != np.shape(k):
        raise ValueError("q and k shapes differ")
    return np.matmul(q, kv), kv
