"""Calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Under stream capture the library takes each call's workspace as a
stream-ordered allocation of the graph.  Every replay is checked bit for bit
against the eager call on the same inputs (the kernels are deterministic),
with eager work and synchronisations between the replays.
"""

import numpy as np
import pytest

from recurrent_vision_token_amd.workloads import make_bwd_inputs, make_inputs, make_saga_inputs

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def dev_tensors(*xs):
    torch = _torch()
    return [torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0") for x in xs]


def replay_and_compare(run, outs_of):
    """run(stream_handle) enqueues the calls and returns their output tensors."""
    torch = _torch()
    eager = [t.clone() for t in run(torch.cuda.current_stream().cuda_stream)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        captured = run(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in captured:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(captured, eager):
            assert torch.equal(a, b), "replay %d differs from the eager call" % rep
        torch.randn(1 << 16, device="cuda:0").sum().item()   # eager work between replays
    del g


def test_forward_graph_replay():
    from recurrent_vision_token_amd import gla_chunk_fwd
    print("graph: forward", flush=True)
    t = dev_tensors(*make_inputs(1, 4, 48, 40, 64, 64, "fp16", 1.0, seed=31))

    def run(stream):
        outs = []
        for d in range(4):
            o, f = gla_chunk_fwd(*t, d, stream=stream)
            outs += [o, f]
        return outs
    replay_and_compare(run, None)


def test_backward_and_saga_graph_replay():
    from recurrent_vision_token_amd import gla_chunk_bwd, saga_fwd
    print("graph: backward and SAGA", flush=True)
    q, k, v, la = make_inputs(1, 3, 24, 40, 64, 64, "fp16", 1.0, seed=32)
    do, dfin, init = make_bwd_inputs(1, 3, 24, 40, 64, seed=33)
    tb = dev_tensors(q, k, v, la, do, dfin, init)
    ts = dev_tensors(*make_saga_inputs(2, 3, 2000, 64, 64, seed=34))

    def run(stream):
        g = gla_chunk_bwd(*tb[:5], 1, d_final_state=tb[5], initial_state=tb[6],
                          want_d_initial_state=True, stream=stream)
        o, kv = saga_fwd(*ts, want_kv=True, stream=stream)
        return list(g) + [o, kv]
    replay_and_compare(run, None)
