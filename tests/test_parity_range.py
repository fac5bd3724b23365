"""GPU parity under strong forgetting and large keys on every float16 path.

A 32-token step whose decay would push a scaled float16 operand out of range
(a 16-token decay below -10 in log2 in some key dim, or queries / keys of
magnitude 32 and above) is computed exactly, token by token in float32, on
every float16 forward path: the automatic choice, forced two and three
passes, and the single pass.  The cases follow the strong-forgetting regime
of a learnable forget gate (GTR news write-up, tokendh.com, section "What
linear attention saves"): log-alpha of -2 per step, gate logits of -30 with
the fused activation, alpha -> 0 (log-alpha -1e4), decay concentrated in a
few key dims and rows, and keys scaled to 40.  Each is held to the float16
bar against the oracle, for every supported head size.
"""

import numpy as np
import pytest

from oracle import gla_forward, log_alpha_from_logits
from recurrent_vision_token_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu

FP16_REL, FP16_MAX = 5e-3, 2e-2
CASES = ["la_minus2", "logits_minus30", "alpha_to_zero", "mixed", "big_keys"]


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def dev(*xs):
    torch = _torch()
    return [torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0") for x in xs]


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(got, ref, what):
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err <= FP16_REL and mx <= FP16_MAX, "%s: rel %.3g max %.3g" % (what, err, mx)


def case_inputs(case, B, heads, H, W, dk, dv, seed):
    """(q, k, v, gate, gate_mode, log_alpha for the oracle)."""
    q, k, v, la = make_inputs(B, heads, H, W, dk, dv, "fp16", 1.0, seed=seed)
    if case == "logits_minus30":
        z = np.full(q.shape, -30.0, dtype=np.float16)
        return q, k, v, z, "logits", log_alpha_from_logits(z, 16.0)
    if case == "la_minus2":
        gl = np.full(q.shape, -2.0, dtype=np.float16)
    elif case == "alpha_to_zero":
        gl = np.full(q.shape, -1.0e4, dtype=np.float16)
    elif case == "mixed":
        # strong decay in a few key dims of some rows only
        gl = la.copy()
        gl[:, :, ::3, :, 5] = -3.0
        gl[:, :, H // 2, :, 40:44] = -60.0
    else:
        # ordinary decay, keys of one in five rows scaled to magnitude ~40
        gl = la
        k = k.copy()
        k[:, :, ::5] = (k[:, :, ::5].astype(np.float32) * 320.0).astype(np.float16)
    return q, k, v, gl, "log_alpha", gl


def run(q, k, v, gate, gate_mode, init, d, mode):
    from recurrent_vision_token_amd import gla_chunk_fwd_ex, set_forward_mode
    torch = _torch()
    tq, tk, tv, tg, ti = dev(q, k, v, gate, init)
    try:
        set_forward_mode(mode)
        out, fs = gla_chunk_fwd_ex(tq, tk, tv, tg, d, gate_mode=gate_mode, tau=16.0,
                                   initial_state=ti)
        torch.cuda.synchronize()
    finally:
        set_forward_mode("auto")
    return host(out), host(fs)


@pytest.mark.parametrize("mode", ["auto", "three_pass", "two_pass", "single_pass"])
@pytest.mark.parametrize("case", CASES)
def test_strong_forgetting_d64(case, mode):
    # 40x40: two-pass spans of two chunks (several steps each), three-pass
    # spans of one; both directions of the row / column scans
    print("range: %s %s" % (case, mode), flush=True)
    B, heads, H, W = 1, 2, 40, 40
    q, k, v, gate, gm, ref_la = case_inputs(case, B, heads, H, W, 64, 64, seed=41)
    init = (np.random.default_rng(42).standard_normal((B, heads, 64, 64)) * 0.25).astype(np.float32)
    for d in (1, 2):
        o, s = run(q, k, v, gate, gm, init, d, mode)
        ro, rs = gla_forward(q, k, v, ref_la, d, initial_state=init)
        check(o, ro, "%s %s dir %d out" % (case, mode, d))
        check(s, rs, "%s %s dir %d final_state" % (case, mode, d))


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("case", CASES)
def test_strong_forgetting_wide_heads(case, dk, dv):
    print("range: %s d_k=%d d_v=%d" % (case, dk, dv), flush=True)
    B, heads, H, W = 1, 2, 21, 29
    q, k, v, gate, gm, ref_la = case_inputs(case, B, heads, H, W, dk, dv, seed=43)
    init = (np.random.default_rng(44).standard_normal((B, heads, dk, dv)) * 0.25).astype(np.float32)
    o, s = run(q, k, v, gate, gm, init, 3, "auto")
    ro, rs = gla_forward(q, k, v, ref_la, 3, initial_state=init)
    check(o, ro, "%s %dx%d out" % (case, dk, dv))
    check(s, rs, "%s %dx%d final_state" % (case, dk, dv))


def test_ragged_exact_step_writes_every_valid_row():
    # a ragged last step taken exactly: every output row is written (the
    # buffer starts as NaN) and right
    print("range: ragged exact step", flush=True)
    torch = _torch()
    from recurrent_vision_token_amd import gla_chunk_fwd
    B, heads, H, W = 1, 1, 3, 13           # 39 tokens: one full step and 7 rows
    q, k, v, _ = make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, seed=45)
    gl = np.full(q.shape, -2.0, dtype=np.float16)
    tq, tk, tv, tg = dev(q, k, v, gl)
    out = torch.full((B, heads, H, W, 64), float("nan"), dtype=torch.float16, device="cuda:0")
    gla_chunk_fwd(tq, tk, tv, tg, 0, out=out)
    torch.cuda.synchronize()
    ro, _ = gla_forward(q, k, v, gl, 0)
    check(host(out), ro, "ragged exact out")
