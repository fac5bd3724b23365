"""GPU parity of the chunkwise backward pass against the CPU oracle.

Every case calls gla_chunk_bwd through the C ABI on float16 inputs and
compares dq, dk, dv, dlog_alpha and d_initial_state with the float64 oracle
(gla_backward) on the same values, to the float16 bar of the forward pass:
relative Frobenius error <= 5e-3 and max |error| <= 2e-2 max |ref| for each.
"""

import numpy as np
import pytest
import torch

from oracle import gla_backward
from recurrent_vision_token_amd import GlaError, gla_chunk_bwd
from recurrent_vision_token_amd.workloads import WORKLOADS, make_bwd_inputs, make_inputs

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dlog_alpha", "d_initial_state")


def dev():
    return torch.device("cuda:0")


def run(q, k, v, la, do, d, dfin=None, init=None):
    t = [torch.from_numpy(x).to(dev()) for x in (q, k, v, la, do)]
    f = None if dfin is None else torch.from_numpy(dfin).to(dev())
    s0 = None if init is None else torch.from_numpy(init).to(dev())
    out = gla_chunk_bwd(t[0], t[1], t[2], t[3], t[4], d, d_final_state=f, initial_state=s0,
                        want_d_initial_state=True)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy().astype(np.float64) for x in out]


def check(got, ref, label, tol=5e-3, mtol=2e-2):
    for name, a, b in zip(NAMES, got, ref):
        rel = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)
        mx = np.abs(a - b).max() / max(np.abs(b).max(), 1e-30)
        assert np.all(np.isfinite(a)), (label, name)
        assert rel <= tol and mx <= mtol, "%s %s: rel %.3g max %.3g" % (label, name, rel, mx)


def case(B, heads, H, W, d, seed, gate_std=1.0, states=True, dk=64, dv=64):
    q, k, v, la = make_inputs(B, heads, H, W, dk, dv, "fp16", gate_std, seed)
    do, dfin, init = make_bwd_inputs(B, heads, H, W, dv, d_k=dk, seed=seed + 1)
    if not states:
        dfin = init = None
    print("bwd case", B, heads, H, W, d, seed, flush=True)
    got = run(q, k, v, la, do, d, dfin, init)
    ref = gla_backward(q, k, v, la, do, d, d_final_state=dfin, initial_state=init)
    check(got, ref, "%dx%d %dx%d dir %d" % (B, heads, H, W, d))


@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_odd_grids_all_directions(d):
    case(1, 2, 13, 11, d, seed=300 + d)


@pytest.mark.parametrize("H,W", [(1, 1), (1, 37), (29, 1), (7, 9), (8, 8), (16, 24)])
def test_grid_shapes(H, W):
    case(1, 2, H, W, 0, seed=310 + H * W)


def test_without_states_and_rotation():
    case(4, 2, 12, 10, 4, seed=320, states=False)
    case(4, 2, 12, 10, 4, seed=321)


def test_strong_decay():
    case(1, 3, 20, 20, 2, seed=330, gate_std=2.0)


def test_deterministic():
    q, k, v, la = make_inputs(1, 2, 17, 19, 64, 64, "fp16", 1.0, 340)
    do, dfin, init = make_bwd_inputs(1, 2, 17, 19, 64, seed=341)
    a = run(q, k, v, la, do, 1, dfin, init)
    b = run(q, k, v, la, do, 1, dfin, init)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_binding_rejects_unbuilt_dims():
    x = torch.zeros((1, 1, 4, 4, 96), dtype=torch.float16, device=dev())
    with pytest.raises(GlaError):
        gla_chunk_bwd(x, x, x, x, x.clone(), 0)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("d", [0, 3, 4])
def test_head_dims(dk, dv, d):
    # wider heads run as 64 x 64 blocks whose gradients add up
    B = 4 if d == 4 else 1
    case(B, 2, 21, 19, d, seed=370 + dk + dv + d, dk=dk, dv=dv)


def test_batched_shape_sampled():
    # the batched configuration (32 x 16 sequences of 64 x 64 tokens,
    # d_k = 128, d_v = 64, directions rotating over the batch): the whole
    # call on the GPU, a sample of sequences against the oracle
    wl = WORKLOADS["batched"]
    B, heads, H, W = wl.B, wl.heads, wl.H, wl.W
    q, k, v, la = make_inputs(B, heads, H, W, wl.d_k, wl.d_v, "fp16", wl.gate_std, 380)
    do, dfin, init = make_bwd_inputs(B, heads, H, W, wl.d_v, d_k=wl.d_k, seed=381)
    print("bwd batched shape", flush=True)
    got = run(q, k, v, la, do, 4, dfin, init)
    for x in got:
        assert np.all(np.isfinite(x))
    rng = np.random.default_rng(382)
    for bh in rng.choice(B * heads, 3, replace=False):
        b, h = divmod(int(bh), heads)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = gla_backward(q[sl], k[sl], v[sl], la[sl], do[sl], b % 4, d_final_state=dfin[sl],
                           initial_state=init[sl])
        check([x[sl] for x in got], ref, "batched b %d h %d" % (b, h))


def test_full_size_16k():
    wl = WORKLOADS["hires16.4k"]
    q, k, v, la = make_inputs(1, wl.heads, wl.H, wl.W, 64, 64, "fp16", wl.gate_std, 3)
    do, dfin, init = make_bwd_inputs(1, wl.heads, wl.H, wl.W, 64, seed=350)
    for d in (0, 1, 2, 3):
        print("bwd 16.4K dir", d, flush=True)
        got = run(q, k, v, la, do, d, dfin, init)
        ref = gla_backward(q, k, v, la, do, d, d_final_state=dfin, initial_state=init)
        check(got, ref, "16.4K dir %d" % d)


def test_many_spans_per_summary_workgroup():
    # 8 x 16 sequences of 64 chunks: 8192 spans of one chunk, so every
    # workgroup of the summaries kernel streams sixteen spans (crossing
    # sequence boundaries) on a 256-CU device; the rotation gives every
    # sequence group its own direction.  A sample of sequences is held to the
    # oracle, and the whole output to finiteness.
    B, heads, H, W = 8, 16, 64, 64
    q, k, v, la = make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, 360)
    do, dfin, init = make_bwd_inputs(B, heads, H, W, 64, seed=361)
    print("bwd many spans", flush=True)
    got = run(q, k, v, la, do, 4, dfin, init)
    for x in got:
        assert np.all(np.isfinite(x))
    rng = np.random.default_rng(362)
    for bh in rng.choice(B * heads, 3, replace=False):
        b, h = divmod(int(bh), heads)
        sl = (slice(b, b + 1), slice(h, h + 1))
        # batch element b scans in direction b % 4
        ref = gla_backward(q[sl], k[sl], v[sl], la[sl], do[sl], b % 4, d_final_state=dfin[sl],
                           initial_state=init[sl])
        check([x[sl] for x in got], ref, "many spans b %d h %d" % (b, h))


def test_uneven_chunks_per_persistent_workgroup():
    # 2 x 5 sequences of 63 x 65 tokens: 64 chunks each (the last one
    # ragged), 640 in all, against the chunk kernel's 512 persistent
    # workgroups on a 256-CU device: the first 128 workgroups take a second
    # chunk (sequences 8 and 9), the others stop after one, so the refill of
    # a next chunk is taken on some workgroups and skipped on others
    B, heads, H, W = 2, 5, 63, 65
    q, k, v, la = make_inputs(B, heads, H, W, 64, 64, "fp16", 1.0, 390)
    do, dfin, init = make_bwd_inputs(B, heads, H, W, 64, seed=391)
    print("bwd uneven persistent", flush=True)
    got = run(q, k, v, la, do, 4, dfin, init)
    for x in got:
        assert np.all(np.isfinite(x))
    for bh in (0, 4, 8, 9):
        b, h = divmod(bh, heads)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = gla_backward(q[sl], k[sl], v[sl], la[sl], do[sl], b % 4, d_final_state=dfin[sl],
                           initial_state=init[sl])
        check([x[sl] for x in got], ref, "uneven b %d h %d" % (b, h))


@pytest.mark.parametrize("pairs", ["1", "0"])
def test_chunk_pairs_and_single_chunks(pairs, monkeypatch):
    # The chunk kernel takes pairs of chunks (the second entering with the
    # first one's next state, the scans giving the forward state per pair)
    # when every persistent workgroup has many chunks, else single chunks;
    # GLA_BWD_PAIRS forces either.  Odd chunk counts leave a pair of one
    # chunk at each sequence's end; wide heads run the accumulating variants;
    # the rotation mixes directions within a call.
    monkeypatch.setenv("GLA_BWD_PAIRS", pairs)
    case(1, 2, 13, 11, 1, seed=400)                 # 3 chunks: one pair and a ragged one
    case(1, 2, 1, 37, 0, seed=401)                  # a single chunk
    case(2, 3, 16, 24, 4, seed=402)                 # 6 chunks, rotation, 6 sequences
    case(4, 2, 21, 19, 4, seed=403, dk=128, dv=64)  # 7 chunks, dv accumulated over key blocks
    case(1, 2, 21, 19, 2, seed=404, dk=64, dv=128)  # dq, dk, dlog-alpha accumulated
    case(1, 3, 20, 20, 3, seed=405, gate_std=2.0)   # strong decay
