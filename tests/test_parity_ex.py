"""GPU parity of the extended entry point (initial state, fused gate
activation) through the C ABI, against the CPU oracle.

Same acceptance as the plain entry: relative Frobenius error <= 5e-3 and
max |err| <= 2e-2 * max |ref| for out and final_state.  The oracle applies
the gate activation in float64 to the same float16 logits the kernels read.
"""

import numpy as np
import pytest

from oracle import gla_forward, log_alpha_from_logits
from recurrent_vision_token_amd.workloads import WORKLOADS, make_inputs, workload_inputs

from .test_parity import check

pytestmark = pytest.mark.gpu

TAU = 16.0


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def logits_like(la, rng, std=1.0):
    # gate logits in float16 with the workloads' spread
    return (rng.standard_normal(la.shape) * std).astype(np.float16)


def run_ex(q, k, v, gate, d, gate_mode, init=None, inplace=False):
    torch = _torch()
    from recurrent_vision_token_amd import gla_chunk_fwd_ex
    dev = torch.device("cuda:0")
    tq, tk, tv, tg = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v, gate))
    ti = None if init is None else torch.from_numpy(np.ascontiguousarray(init, dtype=np.float32)).to(dev)
    out, fs = gla_chunk_fwd_ex(tq, tk, tv, tg, d, gate_mode=gate_mode, tau=TAU, initial_state=ti,
                               final_state=ti if inplace else None)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), fs.cpu().numpy().astype(np.float64)


def parity_ex(q, k, v, gate, d, gate_mode, init=None, what="", inplace=False):
    la = log_alpha_from_logits(gate, TAU) if gate_mode == "logits" else gate
    o, s = run_ex(q, k, v, gate, d, gate_mode, init, inplace)
    init32 = None if init is None else np.asarray(init, dtype=np.float32)
    ro, rs = gla_forward(q, k, v, la, d, initial_state=init32)
    check(o, ro, True, what + " out")
    check(s, rs, True, what + " final_state")
    return o, s


def rand_state(rng, B, heads, dk, dv, scale=0.5):
    return (rng.standard_normal((B, heads, dk, dv)) * scale).astype(np.float32)


@pytest.mark.parametrize("d", [0, 1, 2, 3])
@pytest.mark.parametrize("H,W", [(7, 9), (37, 53)])
def test_initial_state(H, W, d):
    rng = np.random.default_rng(H * W + d)
    q, k, v, la = make_inputs(1, 3, H, W, 64, 64, "fp16", 1.0, seed=H + 3 * W + d)
    parity_ex(q, k, v, la, d, "log_alpha", rand_state(rng, 1, 3, 64, 64), "init %dx%d" % (H, W))


def test_initial_state_4_byte_aligned():
    # the entry promises 4-byte alignment for the initial state; the
    # three-pass scan reads it there: a state one float into a buffer
    torch = _torch()
    from recurrent_vision_token_amd import _lib, gla_chunk_fwd_ex
    rng = np.random.default_rng(5)
    q, k, v, la = make_inputs(1, 3, 40, 40, 64, 64, "fp16", 1.0, seed=17)
    init = rand_state(rng, 1, 3, 64, 64)
    dev = torch.device("cuda:0")
    buf = torch.zeros(1 + init.size, dtype=torch.float32, device=dev)
    ti = buf[1:].view(init.shape)
    ti.copy_(torch.from_numpy(init).to(dev))
    assert ti.data_ptr() % 16 == 4
    tq, tk, tv, tg = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v, la))
    try:
        _lib.set_forward_mode("three_pass")
        assert _lib.plan_forward("fp16", 1, 3, 40, 40, 64, 64)[2] == 3
        out, fs = gla_chunk_fwd_ex(tq, tk, tv, tg, 1, gate_mode="log_alpha", tau=TAU, initial_state=ti)
        torch.cuda.synchronize()
    finally:
        _lib.set_forward_mode("auto")
    ro, rs = gla_forward(q, k, v, la, 1, initial_state=init)
    check(out.float().cpu().numpy().astype(np.float64), ro, True, "4-byte aligned init out")
    check(fs.cpu().numpy().astype(np.float64), rs, True, "4-byte aligned init final_state")


@pytest.mark.parametrize("d", [0, 1, 2, 3])
@pytest.mark.parametrize("H,W", [(1, 1), (7, 9), (37, 53), (129, 7)])
def test_fused_gate(H, W, d):
    rng = np.random.default_rng(7 * H + W + d)
    q, k, v, la = make_inputs(1, 2, H, W, 64, 64, "fp16", 1.0, seed=2 * H + W + d)
    parity_ex(q, k, v, logits_like(la, rng), d, "logits", None, "gate %dx%d" % (H, W))


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (128, 128)])
def test_both_head_dims(dk, dv):
    rng = np.random.default_rng(dk + dv)
    q, k, v, la = make_inputs(2, 2, 24, 21, dk, dv, "fp16", 1.0, seed=dk * 3 + dv)
    parity_ex(q, k, v, logits_like(la, rng, 2.0), 4, "logits", rand_state(rng, 2, 2, dk, dv),
              "dk%d dv%d" % (dk, dv))


def test_many_sequences_single_span():
    # batch*heads fills the chip: one span per sequence, the initial state is
    # read by the output kernel directly
    rng = np.random.default_rng(8)
    q, k, v, la = make_inputs(32, 16, 16, 16, 64, 64, "fp16", 1.0, seed=88)
    parity_ex(q, k, v, logits_like(la, rng), 4, "logits", rand_state(rng, 32, 16, 64, 64),
              "512 sequences")


def test_gate_at_the_domain_edge():
    # z = -10 everywhere: alpha = sigmoid(-10)^(1/16), 16-step decay about -10
    q, k, v, la = make_inputs(1, 2, 20, 20, 64, 64, "fp16", 1.0, seed=12)
    z = np.full_like(la, np.float16(-10.0))
    parity_ex(q, k, v, z, 1, "logits", None, "z=-10")
    z = np.full_like(la, np.float16(30.0))          # alpha ~ 1
    parity_ex(q, k, v, z, 2, "logits", None, "z=+30")


def test_hires_workload_fused_gate():
    wl = WORKLOADS["hires16.4k"]
    seed, d = wl.calls[1]
    q, k, v, la = workload_inputs(wl, seed)
    rng = np.random.default_rng(5)
    parity_ex(q, k, v, logits_like(la, rng, wl.gate_std), d, "logits",
              rand_state(rng, 1, 12, 64, 64), "16.4K fused gate + initial state")


@pytest.mark.parametrize("d", [0, 2])
def test_resume_across_calls(d):
    # a scan cut into two calls, the second seeded with the first's final
    # state, matches the uncut call: rows (L->R) or columns (T->B) split
    torch = _torch()
    H, W = 48, 40
    q, k, v, la = make_inputs(1, 4, H, W, 64, 64, "fp16", 1.0, seed=31 + d)
    o_full, s_full = run_ex(q, k, v, la, d, "log_alpha")
    if d == 0:
        cut = 17
        parts = [(slice(0, cut), slice(None)), (slice(cut, H), slice(None))]
    else:
        cut = 13
        parts = [(slice(None), slice(0, cut)), (slice(None), slice(cut, W))]
    state = None
    outs = []
    for rs, cs in parts:
        sub = [np.ascontiguousarray(x[:, :, rs, cs]) for x in (q, k, v, la)]
        o, state = run_ex(*sub, d, "log_alpha", init=state)
        outs.append(o)
    o_cut = np.concatenate(outs, axis=2 if d == 0 else 3)
    check(o_cut, o_full, True, "resumed out")
    check(state, s_full, True, "resumed state")
    del torch


def test_state_updated_in_place():
    rng = np.random.default_rng(9)
    q, k, v, la = make_inputs(1, 3, 40, 40, 64, 64, "fp16", 1.0, seed=19)
    init = rand_state(rng, 1, 3, 64, 64)
    parity_ex(q, k, v, la, 3, "log_alpha", init, "in place", inplace=True)


def test_fused_matches_host_activation():
    # the fused activation and log_alpha computed on the host (rounded to
    # float16 the same way) give the same outputs to within rounding
    rng = np.random.default_rng(10)
    q, k, v, la = make_inputs(1, 4, 32, 32, 64, 64, "fp16", 1.0, seed=20)
    z = logits_like(la, rng, 2.0)
    la16 = log_alpha_from_logits(z, TAU).astype(np.float16)
    o1, s1 = run_ex(q, k, v, z, 0, "logits")
    o2, s2 = run_ex(q, k, v, la16, 0, "log_alpha")
    check(o1, o2, True, "fused vs host out")
    check(s1, s2, True, "fused vs host state")
