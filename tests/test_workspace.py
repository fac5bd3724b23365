"""GPU tests of the workspace the library keeps per (device, stream).

Every kernel of the library is deterministic (fixed summation orders), so a
call's results are compared bit for bit with the same call made on a freshly
allocated workspace (after gla_release_workspaces): reuse across calls of
different sizes, growth, interleaving on two streams and release must not
change a single bit.  One small case per entry point is also held to the
float16 bar against the oracle, so the reference calls are themselves right.
"""

import numpy as np
import pytest

from oracle import gla_backward, gla_forward, saga_forward
from recurrent_vision_token_amd.workloads import make_bwd_inputs, make_inputs, make_saga_inputs

pytestmark = pytest.mark.gpu

FP16_REL, FP16_MAX = 5e-3, 2e-2


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def dev_tensors(*xs):
    torch = _torch()
    dev = torch.device("cuda:0")
    return [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in xs]


def host(*ts):
    return [None if t is None else t.float().cpu().numpy().astype(np.float64) for t in ts]


def close(got, ref, what):
    err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err <= FP16_REL and mx <= FP16_MAX, "%s: rel %.3g max %.3g" % (what, err, mx)


# forward cases: (B, heads, H, W, seed); the first two split into many spans
FWD = [(1, 4, 64, 64, 11), (1, 2, 16, 24, 12), (2, 3, 48, 40, 13)]


def fwd_call(case, d, stream=None):
    from recurrent_vision_token_amd import gla_chunk_fwd
    B, heads, H, W, seed = case
    q, k, v, la = dev_tensors(*make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, seed=seed))
    return gla_chunk_fwd(q, k, v, la, d, stream=stream)


def test_forward_reuse_across_sizes_is_bitwise_stable():
    torch = _torch()
    from recurrent_vision_token_amd import release_workspaces
    print("workspace: forward reuse", flush=True)
    release_workspaces()
    fresh = []
    for c in FWD:                                   # each on a freshly allocated workspace
        o, s = fwd_call(c, 1)
        torch.cuda.synchronize()
        fresh.append(host(o, s))
        release_workspaces()
    # big, small, medium, big again: the buffer grows once and is reused
    order = [0, 1, 2, 0, 1]
    got = []
    for i in order:
        o, s = fwd_call(FWD[i], 1)
        got.append((i, o, s))
    torch.cuda.synchronize()
    for i, o, s in got:
        ho, hs = host(o, s)
        assert np.array_equal(ho, fresh[i][0]) and np.array_equal(hs, fresh[i][1]), FWD[i]
    # the small case is right, not only stable
    B, heads, H, W, seed = FWD[1]
    ro, rs = gla_forward(*make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, seed=seed), 1)
    close(fresh[1][0], ro, "out")
    close(fresh[1][1], rs, "final_state")


def test_two_streams_interleaved():
    torch = _torch()
    from recurrent_vision_token_amd import gla_chunk_fwd
    print("workspace: two streams", flush=True)
    cases = [FWD[0], FWD[2]]
    inputs = [dev_tensors(*make_inputs(B, h, H, W, 64, 64, "fp16", 1.0, seed=s))
              for (B, h, H, W, s) in cases]
    torch.cuda.synchronize()
    ref = []
    for (q, k, v, la) in inputs:
        o, s = gla_chunk_fwd(q, k, v, la, 2)
        torch.cuda.synchronize()
        ref.append(host(o, s))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(4):                            # both streams busy at once
        for j, st in enumerate(streams):
            q, k, v, la = inputs[(j + rep) % 2]
            with torch.cuda.stream(st):
                o, s = gla_chunk_fwd(q, k, v, la, 2, stream=st.cuda_stream)
            outs.append(((j + rep) % 2, o, s))
    torch.cuda.synchronize()
    for i, o, s in outs:
        ho, hs = host(o, s)
        assert np.array_equal(ho, ref[i][0]) and np.array_equal(hs, ref[i][1]), i


@pytest.mark.parametrize("mode", ["auto", "single_pass"])
def test_two_host_threads_on_one_stream(mode):
    # the workspace cache's lock is held from a call's lookup until its last
    # launch, so two threads' calls on one stream never interleave their
    # launches on the stream's buffers; sizes differ, so the buffers are
    # regrown and reused while the other thread's work is queued
    import threading

    torch = _torch()
    from recurrent_vision_token_amd import gla_chunk_fwd, set_forward_mode
    print("workspace: two threads, one stream, %s" % mode, flush=True)
    cases = [FWD[0], FWD[1]]
    inputs = [dev_tensors(*make_inputs(B, h, H, W, 64, 64, "fp16", 1.0, seed=s))
              for (B, h, H, W, s) in cases]
    try:
        set_forward_mode(mode)
        ref = []
        for (q, k, v, la) in inputs:
            o, s = gla_chunk_fwd(q, k, v, la, 3)
            torch.cuda.synchronize()
            ref.append(host(o, s))
        st = torch.cuda.Stream()
        results = [[], []]
        errors = []

        def worker(j):
            try:
                q, k, v, la = inputs[j]
                with torch.cuda.stream(st):
                    for _ in range(24):
                        results[j].append(gla_chunk_fwd(q, k, v, la, 3, stream=st.cuda_stream))
            except Exception as e:  # reported below, in the test's thread
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
    finally:
        set_forward_mode("auto")
    assert not errors, errors
    for j in range(2):
        assert len(results[j]) == 24
        for o, s in results[j]:
            ho, hs = host(o, s)
            assert np.array_equal(ho, ref[j][0]) and np.array_equal(hs, ref[j][1]), cases[j]


def test_backward_and_saga_reuse():
    torch = _torch()
    from recurrent_vision_token_amd import gla_chunk_bwd, release_workspaces, saga_fwd
    print("workspace: backward and SAGA reuse", flush=True)

    def bwd(B, heads, H, W, seed):
        q, k, v, la = make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, seed=seed)
        do, dfin, init = make_bwd_inputs(B, heads, H, W, 64, seed=seed + 1)
        t = dev_tensors(q, k, v, la, do, dfin, init)
        g = gla_chunk_bwd(*t[:5], 3, d_final_state=t[5], initial_state=t[6],
                          want_d_initial_state=True)
        return g, (q, k, v, la, do, dfin, init)

    def saga(B, heads, N, seed):
        t = dev_tensors(*make_saga_inputs(B, heads, N, 64, 64, seed=seed))
        return saga_fwd(*t, want_kv=True)

    big_b, small_b = (1, 3, 40, 48, 21), (1, 2, 9, 13, 22)
    big_s, small_s = (2, 3, 3000, 23), (1, 2, 300, 24)
    release_workspaces()
    g_small, args = bwd(*small_b)
    torch.cuda.synchronize()
    ref_b = host(*g_small)
    s_small = saga(*small_s)
    torch.cuda.synchronize()
    ref_s = host(*s_small)
    release_workspaces()
    bwd(*big_b)
    saga(*big_s)
    g2, _ = bwd(*small_b)
    s2 = saga(*small_s)
    torch.cuda.synchronize()
    for a, b in zip(host(*g2), ref_b):
        assert np.array_equal(a, b)
    for a, b in zip(host(*s2), ref_s):
        assert np.array_equal(a, b)
    # and the references are right
    q, k, v, la, do, dfin, init = args
    want = gla_backward(q, k, v, la, do, 3, d_final_state=dfin, initial_state=init)
    for got, ref, name in zip(ref_b, want, ("dq", "dk", "dv", "dla", "d_init")):
        close(got, ref, name)
    ro, rkv = saga_forward(*make_saga_inputs(small_s[0], small_s[1], small_s[2], 64, 64,
                                             seed=small_s[3]))
    close(ref_s[0], ro, "saga out")
    close(ref_s[1], rkv, "saga kv")


def test_release_then_call_again():
    torch = _torch()
    from recurrent_vision_token_amd import release_workspaces
    print("workspace: release", flush=True)
    o1, s1 = fwd_call(FWD[2], 0)
    torch.cuda.synchronize()
    a = host(o1, s1)
    release_workspaces()
    release_workspaces()                             # nothing held: a no-op
    o2, s2 = fwd_call(FWD[2], 0)
    torch.cuda.synchronize()
    b = host(o2, s2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
