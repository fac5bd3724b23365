"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest
import torch

from recurrent_vision_token_amd import _lib

# A call that passes validation enqueues kernels on the placeholder pointers
# below; such "accepted" checks only run where no device could execute them.
NO_DEVICE = torch.cuda.device_count() == 0
accepted = pytest.mark.skipif(not NO_DEVICE, reason="would launch on placeholder pointers")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")

# plausible-looking device addresses; validation never dereferences them
P = [0x7F0000000000 + i * (1 << 32) for i in range(8)]
Q, K, V, LA, OUT, FS = P[0], P[1], P[2], P[3], P[4], P[5]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_\w+)\s*\(", text)))


def call(dtype="fp16", q=Q, k=K, v=V, la=LA, scan_dir=0, B=1, heads=2, H=8, W=8, d_k=64,
         d_v=64, chunk=64, out=OUT, fs=FS):
    """dtype "fp16" / "fp32" selects gla_chunk_fwd / gla_chunk_fwd_f32, "noalloc"
    the float16 entry without allocation."""
    if dtype == "noalloc":
        return _lib.raw_call_noalloc(q, k, v, la, scan_dir, B, heads, H, W, d_k, d_v, chunk, out,
                                     fs, None)
    return _lib.raw_call(dtype, q, k, v, la, scan_dir, B, heads, H, W, d_k, d_v, chunk, out, fs,
                         None)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_release_with_nothing_held_makes_no_hip_call():
    # no workspace exists in a process that made no accepted call on a device
    assert _lib.load().gla_release_workspaces() == 0


def test_status_strings_and_version():
    for code in range(-8, 1):
        s = _lib.status_str(code)
        assert s and s != "unknown status"
    assert _lib.status_str(-99) == "unknown status"
    assert _lib.load().gla_version() >= 100


@pytest.mark.parametrize("dtype", ["fp16", "fp32", "noalloc"])
def test_argument_errors(dtype):
    assert call(dtype, scan_dir=5) == -5
    assert call(dtype, scan_dir=-1) == -5
    for kw in ("q", "k", "v", "la", "out"):
        assert call(dtype, **{kw: None}) == -1, kw
    for kw in ("B", "heads", "H", "W"):
        assert call(dtype, **{kw: 0}) == -2, kw
    assert call(dtype, H=1 << 16, W=1 << 16) == -2          # T beyond 2^30
    # one sequence's rows of one tensor reach 2 GiB (32-bit byte offsets)
    dk = 128
    w = 1024 if dtype == "fp32" else 2048      # rows of 512 (fp32) or 256 bytes
    assert call(dtype, B=1, heads=1, H=4096, W=w, d_k=dk) == -2
    if NO_DEVICE:
        assert call(dtype, B=1, heads=1, H=4096, W=w - 1, d_k=dk) != -2
    assert call(dtype, chunk=32) == -3
    assert call(dtype, d_k=96) == -3
    assert call(dtype, d_v=32) == -3
    assert call(dtype, q=Q + 8) == -4
    assert call(dtype, out=OUT + 2) == -4
    assert call(dtype, fs=FS + 2) == -4
    assert call(dtype, out=Q) == -6                          # out aliases q
    assert call(dtype, out=V + 64) == -6                     # out overlaps v
    assert call(dtype, fs=OUT + 1024) == -6                  # final_state inside out


def test_noalloc_entry_is_float16_only_and_checks_first():
    # the scratch lookup is a HIP call; every argument check comes before it
    assert call("noalloc", d_k=96) == -3
    assert call("noalloc", out=K) == -6
    assert _lib.NOALLOC_SCRATCH_BYTES == 32 << 20
    text = open(HEADER).read()
    assert re.search(r"#define GLA_NOALLOC_SCRATCH_BYTES \(32u << 20\)", text)


def test_binding_checks_caller_outputs():
    # caller-supplied outputs are checked for shape, dtype, layout and device
    # before any pointer reaches the library (host-only helpers)
    dev = torch.device("cpu")
    good = torch.empty(2, 3, 4, 5, 8, dtype=torch.float16)
    _lib._check_out(good, "out", (2, 3, 4, 5, 8), torch.float16, dev)
    bad = [good.float(),                                      # dtype
           good[..., :4],                                     # shape
           torch.empty(2, 3, 4, 8, 5, dtype=torch.float16).transpose(3, 4),  # not contiguous
           torch.empty(2, 3, 4, 5, 8, dtype=torch.float16, device="meta"),   # device
           None]
    for t in bad:
        with pytest.raises(ValueError):
            _lib._check_out(t, "out", (2, 3, 4, 5, 8), torch.float16, dev)
    out, fs = _lib._outputs(2, 3, 4, 5, 64, 8, torch.float16, dev, good, None, False)
    assert out is good and fs is None
    with pytest.raises(ValueError, match="final_state"):
        _lib._outputs(2, 3, 4, 5, 64, 8, torch.float16, dev, good,
                      torch.empty(2, 3, 64, 8, dtype=torch.float16), True)
    with pytest.raises(ValueError, match="out"):
        _lib._outputs(2, 3, 4, 5, 64, 8, torch.float16, dev, good[:1], None, True)


def call_ex(gate_mode=1, tau=16.0, init=None, fs=FS, out=OUT, **kw):
    a = dict(q=Q, k=K, v=V, la=LA, scan_dir=0, B=1, heads=2, H=8, W=8, d_k=64, d_v=64, chunk=64)
    a.update(kw)
    return _lib.raw_call_ex(a["q"], a["k"], a["v"], a["la"], gate_mode, tau, init, a["scan_dir"],
                            a["B"], a["heads"], a["H"], a["W"], a["d_k"], a["d_v"], a["chunk"],
                            out, fs, None)


def test_extended_entry_argument_errors():
    ns = 2 * 64 * 64 * 4                                     # bytes of one state tensor
    init = P[6]
    assert call_ex(gate_mode=2) == -3                        # unknown gate mode, checked first
    assert call_ex(gate_mode=-1, scan_dir=9) == -3
    for bad in (0.0, -1.0, float("inf"), float("nan"), 1e-45):
        assert call_ex(gate_mode=1, tau=bad) == -2, bad
    if NO_DEVICE:
        assert call_ex(gate_mode=0, tau=0.0) not in (-2, -3)  # tau ignored for log_alpha
    assert call_ex(init=init + 2) == -4                      # misaligned initial state
    assert call_ex(init=OUT + 64) == -6                      # initial state inside out
    if NO_DEVICE:
        assert call_ex(init=init, fs=init) not in (-6,)       # in-place state update allowed
    assert call_ex(init=init, fs=init + ns // 2) == -6       # partial overlap rejected
    assert call_ex(init=init, fs=init - ns + 4) == -6
    if NO_DEVICE:
        assert call_ex(init=Q) not in (-6,)                   # may share memory with inputs
    assert call_ex(q=None) == -1
    assert call_ex(scan_dir=7) == -5
    assert call_ex(chunk=32) == -3


def test_unbuilt_head_dims_are_rejected():
    for dtype in ("fp16", "fp32", "noalloc"):
        for dk, dv in ((96, 64), (256, 64), (64, 256), (32, 32)):
            assert call(dtype, d_k=dk, d_v=dv) == -3, (dtype, dk, dv)
    assert call("fp32", d_k=96, scan_dir=9) == -5            # direction checked first


def test_kernel_event_hook_validation():
    lib = _lib.load()
    assert _lib.set_kernel_events([]) == 0
    assert _lib.set_kernel_events([1, 2, 3, 4]) == -2
    assert _lib.set_kernel_events([1, 2, None, 4, 5, 6]) == -1
    assert lib.gla_set_kernel_events(None, 6) == -1
    assert _lib.set_kernel_events([]) == 0


def test_plan_spans_argument_errors():
    import ctypes
    lib = _lib.load()
    a, b = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.gla_plan_spans(0, 1, 12, 128, 128, 64, 64, 64, None, ctypes.byref(b)) == -1
    assert lib.gla_plan_spans(0, 1, 12, 128, 128, 64, 64, 32, ctypes.byref(a), ctypes.byref(b)) == -3
    assert lib.gla_plan_spans(1, 1, 12, 128, 128, 96, 64, 64, ctypes.byref(a), ctypes.byref(b)) == -3
    assert lib.gla_plan_spans(0, 0, 12, 128, 128, 64, 64, 64, ctypes.byref(a), ctypes.byref(b)) == -2


def test_plan_forward_argument_errors():
    import ctypes
    lib = _lib.load()
    a, b, c = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    assert lib.gla_plan_forward(0, 1, 12, 128, 128, 64, 64, 64, ctypes.byref(a), ctypes.byref(b),
                                None) == -1
    assert lib.gla_plan_forward(0, 1, 12, 128, 128, 64, 64, 32, ctypes.byref(a), ctypes.byref(b),
                                ctypes.byref(c)) == -3
    assert lib.gla_plan_forward(0, 1, 0, 128, 128, 64, 64, 64, ctypes.byref(a), ctypes.byref(b),
                                ctypes.byref(c)) == -2


def test_forward_mode_setter():
    # a host-only setting: no HIP call, so this runs without a device
    lib = _lib.load()
    for bad in (-1, 4, 99):
        assert lib.gla_set_forward_mode(bad) == -2
    for mode in ("three_pass", "two_pass", "single_pass", "auto"):
        _lib.set_forward_mode(mode)
    with pytest.raises(ValueError):
        _lib.set_forward_mode("single")
    assert lib.gla_set_forward_mode(0) == 0


def call_sw(gate=P[0], value=P[1], ld=None, weight=P[2], bias=P[3], B=1, H=16, W=16, C=64,
            out=P[4]):
    return _lib.raw_call_swiglu(gate, value, C if ld is None else ld, weight, bias, B, H, W, C,
                                out, None)


def test_spatial_swiglu_argument_errors():
    for kw in ("gate", "value", "weight", "out"):
        assert call_sw(**{kw: None}) == -1, kw
    for kw in ("B", "H", "W", "C"):
        assert call_sw(**{kw: 0}) == -2, kw
    assert call_sw(C=64, ld=56) == -2                         # ld_in < C
    assert call_sw(C=60) == -3                                # C not a multiple of 8
    assert call_sw(C=64, ld=68) == -3                         # ld_in not a multiple of 8
    # one image's rows reach 2 GiB (32-bit byte offsets)
    assert call_sw(H=1024, W=1024, C=1024) == -2
    assert call_sw(gate=P[0] + 8) == -4
    assert call_sw(value=P[1] + 2) == -4
    assert call_sw(weight=P[2] + 4) == -4
    assert call_sw(bias=P[3] + 8) == -4
    assert call_sw(out=P[4] + 8) == -4
    assert call_sw(out=P[0]) == -6                            # out aliases gate
    assert call_sw(out=P[1] + 16 * 16 * 64) == -6             # out overlaps value's tail
    assert call_sw(out=P[2] - 16) == -6                       # out runs into the weights
    assert call_sw(out=P[3] - 16 * 16 * 128 + 16) == -6       # out runs into the bias
    if NO_DEVICE:
        assert call_sw(bias=None) not in (-1, -2, -3, -4, -6)  # bias is optional
        assert call_sw(value=P[0] + 128, ld=128) not in (-2, -3, -4, -6)  # fused halves
        assert call_sw(H=1024, W=1023, C=1024) not in (-2,)


def call_saga(q=P[0], k=P[1], v=P[2], a=P[3], b=P[4], B=1, heads=2, N=300, d_k=64, d_v=64,
              out=P[5], kv=P[6]):
    return _lib.raw_call_saga(q, k, v, a, b, B, heads, N, d_k, d_v, out, kv, None)


def test_saga_argument_errors():
    for kw in ("q", "k", "v", "a", "b", "out"):
        assert call_saga(**{kw: None}) == -1, kw
    for kw in ("B", "heads", "N", "d_k", "d_v"):
        assert call_saga(**{kw: 0}) == -2, kw
    assert call_saga(d_k=96) == -3
    assert call_saga(d_v=32) == -3
    assert call_saga(N=1 << 24, d_k=64, d_v=64) == -2       # a sequence's rows reach 2 GiB
    assert call_saga(q=P[0] + 8) == -4
    assert call_saga(out=P[5] + 2) == -4
    assert call_saga(kv=P[6] + 4) == -4
    assert call_saga(out=P[0]) == -6                         # out aliases q
    assert call_saga(out=P[4] + 64) == -6                    # out overlaps beta
    assert call_saga(kv=P[5] + 1024) == -6                   # kv inside out
    assert call_saga(kv=P[1]) == -6                          # kv aliases k
    if NO_DEVICE:
        assert call_saga(kv=None) not in (-1, -2, -3, -4, -6)  # kv is optional
        assert call_saga(N=(1 << 24) - 1) not in (-2,)
