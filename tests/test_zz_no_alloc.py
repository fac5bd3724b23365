"""gla_chunk_fwd_noalloc (span states in the library's fixed device array, no
allocation in the call) against gla_chunk_fwd on the same inputs.

Both entries take the same work split here, so their results must agree bit
for bit; the float16 bar against each other is checked as well.  Calls run
one after another on one stream with shrinking sizes, so each later call
finds the array holding an earlier, larger call's states.
"""

import numpy as np
import pytest

from recurrent_vision_token_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu

FP16_REL, FP16_MAX = 5e-3, 2e-2


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _inputs(B, heads, H, W, seed, d_k=64, d_v=64):
    torch = _torch()
    arrs = make_inputs(B, heads, H, W, d_k, d_v, "fp16", 1.0, seed)
    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0") for a in arrs]


def _check(got, ref, what):
    got = got.double().cpu().numpy()
    ref = ref.double().cpu().numpy()
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err <= FP16_REL and mx <= FP16_MAX, "%s: rel %.3g max %.3g" % (what, err, mx)


def _both(B, heads, H, W, scan_dir, seed, d_k=64, d_v=64, exact=True):
    """Run both entries on one input; compare (bit for bit when exact)."""
    torch = _torch()
    from recurrent_vision_token_amd import _lib

    q, k, v, la = _inputs(B, heads, H, W, seed, d_k, d_v)
    ref_out, ref_fs = _lib.gla_chunk_fwd(q, k, v, la, scan_dir)
    out = torch.full_like(ref_out, float("nan"))
    fs = torch.full_like(ref_fs, float("nan"))
    _lib.gla_chunk_fwd_noalloc(q, k, v, la, scan_dir, out, fs)
    torch.cuda.synchronize()
    what = "B=%d heads=%d %dx%d dir %d" % (B, heads, H, W, scan_dir)
    _check(out, ref_out, what + " out")
    _check(fs, ref_fs, what + " final_state")
    if exact:
        assert torch.equal(out, ref_out), what + ": out differs from gla_chunk_fwd"
        assert torch.equal(fs, ref_fs), what + ": final_state differs from gla_chunk_fwd"


def _uses_scratch(B, heads, H, W, d_k=64, d_v=64):
    # float32 gate products with float16 span states on the three-pass path,
    # float32 summaries and gate products on the two-pass path
    from recurrent_vision_token_amd import _lib
    _, n_spans, kernels = _lib.plan_forward("fp16", B, heads, H, W, d_k, d_v)
    per_span = d_k * 4 + d_k * d_v * 2 if kernels == 3 else (d_k * d_v + d_k) * 4
    return n_spans > 1, B * heads * n_spans * per_span


def test_calls_in_a_row_shrinking():
    from recurrent_vision_token_amd import _lib
    _lib.set_forward_mode("auto")
    cases = [(1, 12, 128, 128, 0, 3),    # three passes, many spans
             (1, 12, 40, 40, 2, 1),      # two passes
             (1, 4, 21, 29, 1, 11),      # two passes, fewer spans
             (2, 3, 9, 113, 4, 12)]      # batch rotation of directions
    for B, heads, H, W, d, seed in cases:
        split, nbytes = _uses_scratch(B, heads, H, W)
        assert split and nbytes <= _lib.NOALLOC_SCRATCH_BYTES, (B, heads, H, W, nbytes)
        print("noalloc case", B, heads, H, W, d, flush=True)
        _both(B, heads, H, W, d, seed)


def test_unsplit_and_wide_heads():
    from recurrent_vision_token_amd import _lib
    _lib.set_forward_mode("auto")
    for B, heads, H, W, dk, dv in [(1, 2, 7, 9, 64, 64), (1, 12, 40, 40, 128, 64),
                                   (1, 6, 33, 31, 64, 128), (1, 4, 48, 48, 128, 128)]:
        print("noalloc case", B, heads, H, W, dk, dv, flush=True)
        _both(B, heads, H, W, 0, 21, dk, dv)


def test_single_pass_mode_takes_the_automatic_split():
    from recurrent_vision_token_amd import _lib
    try:
        _lib.set_forward_mode("single_pass")
        q, k, v, la = _inputs(1, 12, 40, 40, 5)
        torch = _torch()
        out = torch.empty_like(v)
        fs = torch.empty((1, 12, 64, 64), dtype=torch.float32, device="cuda:0")
        _lib.gla_chunk_fwd_noalloc(q, k, v, la, 3, out, fs)
        _lib.set_forward_mode("auto")
        ref_out, ref_fs = _lib.gla_chunk_fwd(q, k, v, la, 3)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(fs, ref_fs)
    finally:
        _lib.set_forward_mode("auto")


def test_forced_split_beyond_the_scratch_is_rejected():
    torch = _torch()
    from recurrent_vision_token_amd import _lib
    B, heads, H, W = 1, 160, 32, 32
    q, k, v, la = _inputs(B, heads, H, W, 8)
    out = torch.full_like(v, float("nan"))
    try:
        _lib.set_forward_mode("two_pass")
        span_chunks, n_spans, kernels = _lib.plan_forward("fp16", B, heads, H, W, 64, 64)
        assert kernels == 2                 # two passes: float32 summaries only
        assert B * heads * n_spans * (64 * 64 + 64) * 4 > _lib.NOALLOC_SCRATCH_BYTES
        with pytest.raises(_lib.GlaError) as e:
            _lib.gla_chunk_fwd_noalloc(q, k, v, la, 0, out)
        assert e.value.status == -8
        torch.cuda.synchronize()
        assert torch.isnan(out).all()                 # nothing was enqueued
    finally:
        _lib.set_forward_mode("auto")
    _both(B, heads, H, W, 0, 8)                       # the automatic split fits


def test_automatic_splits_fit_the_scratch():
    # an automatic split has at most one span per resident output workgroup:
    # a single long sequence takes them all, for every supported head size
    from recurrent_vision_token_amd import _lib
    _lib.set_forward_mode("auto")
    for dk, dv in [(64, 64), (64, 128), (128, 64), (128, 128)]:
        for B, heads, H, W in [(1, 1, 1024, 1024), (1, 3, 512, 512), (1, 12, 128, 128)]:
            split, nbytes = _uses_scratch(B, heads, H, W, dk, dv)
            assert nbytes <= _lib.NOALLOC_SCRATCH_BYTES, (dk, dv, B, heads, H, W, nbytes)
