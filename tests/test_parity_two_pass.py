"""GPU parity of the two-pass forward path against the oracle, and of the two
forward paths against each other.

The two-pass path (span summaries, then output workgroups that fold the
earlier spans' summaries into their own entry state, with no scan kernel) is
the automatic choice for short float16 sequences with d_k = d_v = 64;
gla_set_forward_mode forces either path.  Every case here is held to the
float16 bar against the oracle; calls of both paths share one workspace on
one stream, and a captured graph is replayed, with every result checked.
"""

import numpy as np
import pytest

from oracle import gla_forward, log_alpha_from_logits
from recurrent_vision_token_amd.workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

FP16_REL, FP16_MAX = 5e-3, 2e-2


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


class forward_mode:
    """Force a forward path for the block, then go back to automatic."""

    def __init__(self, mode):
        self.mode = mode

    def __enter__(self):
        from recurrent_vision_token_amd import set_forward_mode
        set_forward_mode(self.mode)

    def __exit__(self, *exc):
        from recurrent_vision_token_amd import set_forward_mode
        set_forward_mode("auto")


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


def plan(B, heads, H, W):
    from recurrent_vision_token_amd._lib import plan_spans
    return plan_spans("fp16", B, heads, H, W, 64, 64)


def fwd(inputs, d, **kw):
    from recurrent_vision_token_amd import gla_chunk_fwd
    out, fs = gla_chunk_fwd(*dev(*inputs), d, **kw)
    _torch().cuda.synchronize()
    return host(out), host(fs)


def test_automatic_choice():
    print("two pass: plan", flush=True)
    n16 = (1600 + 63) // 64
    # short sequences: spans of at most 4 chunks, 2..16 of them
    sc, ns = plan(1, 12, 40, 40)
    assert (sc, ns) == (2, 13), (sc, ns)
    sc, ns = plan(1, 16, 48, 48)
    assert (sc, ns) == (3, 12), (sc, ns)
    # forced three passes: the three-pass plan (one chunk per span here)
    with forward_mode("three_pass"):
        assert plan(1, 12, 40, 40) == (1, n16)
    # long sequences stay on three passes unless forced
    assert plan(1, 12, 128, 128)[0] == 4
    with forward_mode("two_pass"):
        sc, ns = plan(1, 12, 128, 128)
        assert (sc, ns) == (16, 16), (sc, ns)
        # forced with many sequences: no residency condition
        assert plan(64, 16, 40, 40) == (2, 13)
    # automatically, sequences that fill the device alone are not split
    assert plan(64, 16, 40, 40) == (25, 1)
    # one chunk: no split on either path
    assert plan(1, 12, 8, 8) == (1, 1)


@pytest.mark.parametrize("d", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("H,W", [(21, 29), (40, 40), (9, 113)])
def test_two_pass_against_oracle(H, W, d):
    B = 4 if d == 4 else 1
    print("two pass: %dx%d dir %d" % (H, W, d), flush=True)
    x = make_inputs(B, 3, H, W, 64, 64, "fp16", 1.0, seed=7 * H + W + d)
    with forward_mode("two_pass"):
        o, s = fwd(x, d)
    ro, rs = gla_forward(*x, d)
    check(o, ro, "out")
    check(s, rs, "final_state")


@pytest.mark.parametrize("name", ["gtr1.6k", "img768"])
def test_workloads_both_paths(name):
    wl = WORKLOADS[name]
    print("two pass: workload %s" % name, flush=True)
    for seed, d in list(zip(wl.seeds, wl.dirs))[:4]:
        x = workload_inputs(wl, seed)
        ro, rs = gla_forward(*x, d)
        got = {}
        for mode in ("two_pass", "three_pass"):
            with forward_mode(mode):
                got[mode] = fwd(x, d)
            check(got[mode][0], ro, "%s %s dir %d out" % (name, mode, d))
            check(got[mode][1], rs, "%s %s dir %d final_state" % (name, mode, d))


@pytest.mark.parametrize("H,W", [(64, 64), (32, 128), (16, 63)])
def test_forced_long_spans(H, W):
    # up to 16 spans of up to 4 chunks; exactly 16 spans for the first two
    print("two pass: forced %dx%d" % (H, W), flush=True)
    x = make_inputs(1, 2, H, W, 64, 64, "fp16", 2.0, seed=H * W)
    with forward_mode("two_pass"):
        sc, ns = plan(1, 2, H, W)
        assert 2 <= ns <= 16
        o, s = fwd(x, 2)
    ro, rs = gla_forward(*x, 2)
    check(o, ro, "out")
    check(s, rs, "final_state")


def test_extended_entry():
    # fused gate activation and an initial state on the two-pass path
    from recurrent_vision_token_amd import gla_chunk_fwd_ex
    print("two pass: extended entry", flush=True)
    torch = _torch()
    rng = np.random.default_rng(11)
    q, k, v, _ = make_inputs(2, 3, 33, 27, 64, 64, "fp16", 1.0, seed=12)
    z = (rng.standard_normal(q.shape) * 2.0).astype(np.float16)
    init = (rng.standard_normal((2, 3, 64, 64)) * 0.5).astype(np.float32)
    la = log_alpha_from_logits(z, 16.0)
    for d in (1, 3):
        with forward_mode("two_pass"):
            tq, tk, tv, tz, ti = dev(q, k, v, z, init)
            out, fs = gla_chunk_fwd_ex(tq, tk, tv, tz, d, gate_mode="logits", tau=16.0,
                                       initial_state=ti)
            torch.cuda.synchronize()
        ro, rs = gla_forward(q, k, v, la, d, initial_state=init)
        check(host(out), ro, "ex out dir %d" % d)
        check(host(fs), rs, "ex final_state dir %d" % d)


def test_many_calls_and_both_paths_on_one_stream():
    # many calls in a row, of two shapes, mixed with three-pass calls on the
    # same workspace; every two-pass result equals that call's own result on a
    # fresh workspace
    from recurrent_vision_token_amd import gla_chunk_fwd, release_workspaces
    torch = _torch()
    print("two pass: many calls", flush=True)
    shapes = [(1, 12, 40, 40, 1), (2, 5, 23, 31, 2)]
    inputs = [dev(*make_inputs(B, h, H, W, 64, 64, "fp16", 1.0, seed=s)) for B, h, H, W, s in shapes]
    ref = []
    for i, x in enumerate(inputs):
        release_workspaces()
        with forward_mode("two_pass"):
            o, s = gla_chunk_fwd(*x, i)
        torch.cuda.synchronize()
        ref.append((o.clone(), s.clone()))
    B, h, H, W, s = shapes[0]
    ro, rs = gla_forward(*make_inputs(B, h, H, W, 64, 64, "fp16", 1.0, seed=s), 0)
    check(host(ref[0][0]), ro, "reference out")
    check(host(ref[0][1]), rs, "reference final_state")
    outs = []
    for n in range(24):
        i = (n // 3) % 2
        mode = "three_pass" if n % 5 == 4 else "two_pass"
        with forward_mode(mode):
            o, s = gla_chunk_fwd(*inputs[i], i)
        outs.append((n, i, mode, o, s))
    torch.cuda.synchronize()
    for n, i, mode, o, s in outs:
        if mode == "two_pass":
            assert torch.equal(o, ref[i][0]) and torch.equal(s, ref[i][1]), (n, i)
        else:
            check(host(o), host(ref[i][0]).astype(np.float64), "three-pass call %d" % n)


def test_graph_replay():
    torch = _torch()
    from recurrent_vision_token_amd import gla_chunk_fwd
    print("two pass: graph replay", flush=True)
    x = dev(*make_inputs(1, 12, 40, 40, 64, 64, "fp16", 1.0, seed=31))
    with forward_mode("two_pass"):
        o_ref, s_ref = gla_chunk_fwd(*x, 3)
        torch.cuda.synchronize()
        o_ref, s_ref = o_ref.clone(), s_ref.clone()
        stream = torch.cuda.Stream()
        out = torch.empty_like(o_ref)
        fs = torch.empty_like(s_ref)
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            gla_chunk_fwd(*x, 3, out=out, final_state=fs, stream=stream.cuda_stream)  # warm-up
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            gla_chunk_fwd(*x, 3, out=out, final_state=fs, stream=stream.cuda_stream)
        for rep in range(4):
            out.zero_()
            fs.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, o_ref) and torch.equal(fs, s_ref), rep
            o2, _ = gla_chunk_fwd(*x, 0)                   # eager work between replays
            torch.cuda.synchronize()


def test_forced_mode_where_two_passes_do_not_apply():
    # forcing two passes leaves other head dims, float32 and single-chunk
    # sequences on their usual paths, with the same results
    from recurrent_vision_token_amd._lib import plan_forward
    print("two pass: forced mode elsewhere", flush=True)
    with forward_mode("two_pass"):
        assert plan_forward("fp16", 1, 12, 40, 40, 64, 64)[2] == 2
        assert plan_forward("fp16", 1, 12, 40, 40, 128, 64)[2] == 3
        assert plan_forward("fp32", 1, 12, 40, 40, 64, 64)[2] == 3
        assert plan_forward("fp16", 1, 12, 8, 8, 64, 64)[2] == 1
        x = make_inputs(1, 2, 24, 21, 128, 64, "fp16", 1.0, seed=77)
        o, s = fwd(x, 3)
    ro, rs = gla_forward(*x, 3)
    check(o, ro, "d_k 128 out")
    check(s, rs, "d_k 128 final_state")



def test_forced_two_pass_more_workgroups_than_the_device_holds():
    # 8 x 16 sequences of 13 spans: 1664 output workgroups, several rounds on
    # the device (the path has no waits between workgroups); three sampled
    # sequences against the oracle
    print("two pass: many sequences", flush=True)
    B, heads, H, W = 8, 16, 40, 40
    x = make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, seed=91)
    with forward_mode("two_pass"):
        assert plan(B, heads, H, W) == (2, 13)
        o, s = fwd(x, 4)
    for b, h in ((0, 0), (3, 7), (7, 15)):
        xs = [t[b:b + 1, h:h + 1] for t in x]
        ro, rs = gla_forward(*xs, b % 4)
        check(o[b:b + 1, h:h + 1], ro, "out b%d h%d" % (b, h))
        check(s[b:b + 1, h:h + 1], rs, "final_state b%d h%d" % (b, h))


def test_in_place_state_update_with_more_workgroups_than_the_device_holds():
    # final_state == initial_state: every two-pass output workgroup reads the
    # initial state while the last span's workgroup writes the final state, so
    # an in-place call takes three passes even when two are forced; checked on
    # 1664 output workgroups' worth of sequences, sampled against the oracle
    from recurrent_vision_token_amd import gla_chunk_fwd_ex
    print("two pass: in-place state, many sequences", flush=True)
    torch = _torch()
    B, heads, H, W = 8, 16, 40, 40
    x = make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, seed=93)
    init = (np.random.default_rng(94).standard_normal((B, heads, 64, 64)) * 0.5).astype(np.float32)
    with forward_mode("two_pass"):
        assert plan(B, heads, H, W) == (2, 13)
        tq, tk, tv, tl, ts = dev(*x, init)
        out, fs = gla_chunk_fwd_ex(tq, tk, tv, tl, 4, initial_state=ts, final_state=ts)
        torch.cuda.synchronize()
    assert fs.data_ptr() == ts.data_ptr()
    o, s = host(out), host(ts)
    for b, h in ((0, 0), (2, 5), (5, 9), (7, 15)):
        xs = [t[b:b + 1, h:h + 1] for t in x]
        ro, rs = gla_forward(*xs, b % 4, initial_state=init[b:b + 1, h:h + 1])
        check(o[b:b + 1, h:h + 1], ro, "in-place out b%d h%d" % (b, h))
        check(s[b:b + 1, h:h + 1], rs, "in-place final_state b%d h%d" % (b, h))
