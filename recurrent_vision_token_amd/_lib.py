"""ctypes binding of libgla.so (argument marshalling only).

Every step of the forward pass runs in the HIP kernels behind the C ABI of
include/gla.h; this module only checks tensors, allocates outputs with torch,
and passes raw device pointers and the current HIP stream.  There is no CPU
fallback: when the library is missing or no GPU is present, calls raise.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# GLA_LIBRARY names another build of the same library (the host-sanitizer
# build, libgla_san.so); by default the in-tree libgla.so
LIB_PATH = os.environ.get("GLA_LIBRARY") or os.path.join(PKG, "libgla.so")

GLA_OK = 0
STATUS = {
    0: "GLA_OK", -1: "GLA_ERR_NULL", -2: "GLA_ERR_SHAPE", -3: "GLA_ERR_UNSUPPORTED",
    -4: "GLA_ERR_ALIGN", -5: "GLA_ERR_SCAN_DIR", -6: "GLA_ERR_ALIAS", -7: "GLA_ERR_HIP",
    -8: "GLA_ERR_SCRATCH",
}
# size of the fixed device array of gla_chunk_fwd_noalloc (GLA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20
EXPORTED = ("gla_chunk_bwd", "gla_chunk_fwd", "gla_chunk_fwd_ex", "gla_chunk_fwd_f32",
            "gla_chunk_fwd_noalloc",
            "gla_plan_forward", "gla_plan_spans", "gla_release_workspaces",
            "gla_saga_fwd", "gla_set_forward_mode", "gla_set_kernel_events",
            "gla_spatial_swiglu", "gla_status_str", "gla_version")
FORWARD_MODES = {"auto": 0, "three_pass": 1, "two_pass": 2, "single_pass": 3}
GATE_MODES = {"log_alpha": 0, "logits": 1}

_lib = None


class GlaError(RuntimeError):
    def __init__(self, status, text):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, text))
        self.status = status


def load():
    """Load libgla.so (built in-tree by recurrent_vision_token_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("%s is not built; run python recurrent_vision_token_amd/build.py "
                           "(hipcc for gfx950)" % LIB_PATH)
    # torch first: it brings its own HIP runtime under the same soname as the
    # system one libgla.so names, and a process gets one of them, the first
    # loaded.  Loading the library first would put torch on a runtime it was
    # not built against (torch.cuda then reports no device).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    sig = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, vp]
    for name in ("gla_chunk_fwd", "gla_chunk_fwd_f32", "gla_chunk_fwd_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = sig
        fn.restype = ctypes.c_int
    lib.gla_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, i, ctypes.c_float, vp] + sig[4:]
    lib.gla_chunk_fwd_ex.restype = ctypes.c_int
    lib.gla_spatial_swiglu.argtypes = [vp, vp, i, vp, vp, i, i, i, i, vp, vp]
    lib.gla_saga_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp]
    lib.gla_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                  vp, vp, vp, vp, vp, vp]
    lib.gla_chunk_bwd.restype = ctypes.c_int
    lib.gla_saga_fwd.restype = ctypes.c_int
    lib.gla_spatial_swiglu.restype = ctypes.c_int
    lib.gla_status_str.argtypes = [ctypes.c_int]
    lib.gla_status_str.restype = ctypes.c_char_p
    lib.gla_plan_spans.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.gla_plan_spans.restype = ctypes.c_int
    lib.gla_plan_forward.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i),
                                     ctypes.POINTER(i)]
    lib.gla_plan_forward.restype = ctypes.c_int
    lib.gla_set_kernel_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.gla_set_kernel_events.restype = ctypes.c_int
    lib.gla_version.argtypes = []
    lib.gla_version.restype = ctypes.c_int
    lib.gla_release_workspaces.argtypes = []
    lib.gla_release_workspaces.restype = ctypes.c_int
    lib.gla_set_forward_mode.argtypes = [ctypes.c_int]
    lib.gla_set_forward_mode.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status):
    return load().gla_status_str(int(status)).decode()


def raw_call(dtype, q, k, v, la, scan_dir, B, heads, H, W, d_k, d_v, chunk, out, final_state,
             stream):
    """Call the C entry point with integer pointers; returns the status code."""
    lib = load()
    fn = lib.gla_chunk_fwd if dtype == "fp16" else lib.gla_chunk_fwd_f32
    return fn(q, k, v, la, scan_dir, B, heads, H, W, d_k, d_v, chunk, out, final_state, stream)


def raw_call_noalloc(q, k, v, la, scan_dir, B, heads, H, W, d_k, d_v, chunk, out, final_state,
                     stream):
    """Call gla_chunk_fwd_noalloc with integer pointers; returns the status code."""
    return load().gla_chunk_fwd_noalloc(q, k, v, la, scan_dir, B, heads, H, W, d_k, d_v, chunk,
                                        out, final_state, stream)


def raw_call_ex(q, k, v, gate, gate_mode, tau, initial_state, scan_dir, B, heads, H, W, d_k,
                d_v, chunk, out, final_state, stream):
    """Call gla_chunk_fwd_ex with integer pointers; returns the status code."""
    return load().gla_chunk_fwd_ex(q, k, v, gate, gate_mode, tau, initial_state, scan_dir, B,
                                   heads, H, W, d_k, d_v, chunk, out, final_state, stream)


def _check(q, k, v, log_alpha):
    import torch

    tens = (q, k, v, log_alpha)
    if not all(isinstance(t, torch.Tensor) and t.is_cuda for t in tens):
        raise ValueError("q, k, v, log_alpha must be device tensors")
    dt = q.dtype
    if dt not in (torch.float16, torch.float32) or any(t.dtype != dt for t in tens):
        raise ValueError("q, k, v, log_alpha must all be float16 or all float32")
    if q.dim() != 5:
        raise ValueError("expected [B, heads, H, W, d] tensors")
    B, heads, H, W, d_k = q.shape
    d_v = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or tuple(v.shape[:4]) != (B, heads, H, W):
        raise ValueError("shape mismatch among q, k, v, log_alpha")
    if not all(t.is_contiguous() for t in tens):
        raise ValueError("tensors must be contiguous")
    return B, heads, H, W, d_k, d_v


def _check_out(t, name, shape, dtype, dev):
    """Raise ValueError unless a caller-supplied output tensor fits the call."""
    import torch

    if (not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape)
            or not t.is_contiguous() or t.device != dev):
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s"
                         % (name, str(dtype).replace("torch.", ""), list(shape), dev))


def _outputs(B, heads, H, W, d_k, d_v, dt, dev, out, final_state, want_final_state):
    """Check or allocate the forward outputs (out, final_state)."""
    import torch

    if out is None:
        out = torch.empty((B, heads, H, W, d_v), dtype=dt, device=dev)
    else:
        _check_out(out, "out", (B, heads, H, W, d_v), dt, dev)
    if final_state is None:
        if want_final_state:
            final_state = torch.empty((B, heads, d_k, d_v), dtype=torch.float32, device=dev)
    else:
        _check_out(final_state, "final_state", (B, heads, d_k, d_v), torch.float32, dev)
    return out, final_state


def gla_chunk_fwd(q, k, v, log_alpha, scan_dir, chunk=64, out=None, final_state=None,
                  want_final_state=True, stream=None):
    """Chunkwise GLA forward on device tensors.

    q, k, log_alpha: [B, heads, H, W, d_k]; v: [B, heads, H, W, d_v]; all float16
    (or all float32), contiguous, on one HIP device.  Returns (out, final_state);
    final_state is float32 [B, heads, d_k, d_v] or None.
    """
    import torch

    B, heads, H, W, d_k, d_v = _check(q, k, v, log_alpha)
    dt = q.dtype
    dev = q.device
    out, final_state = _outputs(B, heads, H, W, d_k, d_v, dt, dev, out, final_state,
                                want_final_state)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    fs_ptr = final_state.data_ptr() if final_state is not None else None
    rc = raw_call("fp16" if dt == torch.float16 else "fp32", q.data_ptr(), k.data_ptr(),
                  v.data_ptr(), log_alpha.data_ptr(), int(scan_dir), B, heads, H, W, d_k, d_v,
                  int(chunk), out.data_ptr(), fs_ptr, stream)
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return out, final_state


def gla_chunk_fwd_noalloc(q, k, v, log_alpha, scan_dir, out, final_state=None, chunk=64,
                          stream=None):
    """Float16 forward through gla_chunk_fwd_noalloc (no device allocation in
    the call): the caller passes out (float16 [B, heads, H, W, d_v]) and
    optionally final_state (float32 [B, heads, d_k, d_v]).  Same results as
    gla_chunk_fwd; returns (out, final_state)."""
    import torch

    B, heads, H, W, d_k, d_v = _check(q, k, v, log_alpha)
    if q.dtype != torch.float16:
        raise ValueError("gla_chunk_fwd_noalloc takes float16 tensors")
    dev = q.device
    _check_out(out, "out", (B, heads, H, W, d_v), torch.float16, dev)
    if final_state is not None:
        _check_out(final_state, "final_state", (B, heads, d_k, d_v), torch.float32, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    fs_ptr = final_state.data_ptr() if final_state is not None else None
    rc = raw_call_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(),
                          int(scan_dir), B, heads, H, W, d_k, d_v, int(chunk), out.data_ptr(),
                          fs_ptr, stream)
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return out, final_state


def gla_chunk_fwd_ex(q, k, v, gate, scan_dir, gate_mode="log_alpha", tau=16.0,
                     initial_state=None, chunk=64, out=None, final_state=None,
                     want_final_state=True, stream=None):
    """Extended float16 forward: optional initial state and fused gate activation.

    gate holds log_alpha (gate_mode "log_alpha") or the gate logits z
    (gate_mode "logits", log_alpha = logsigmoid(z) / tau); same shape and
    dtype as q.  initial_state: float32 [B, heads, d_k, d_v] or None; it may be
    passed as final_state too, to update the state in place.
    """
    import torch

    B, heads, H, W, d_k, d_v = _check(q, k, v, gate)
    if q.dtype != torch.float16:
        raise ValueError("gla_chunk_fwd_ex takes float16 tensors")
    if gate_mode not in GATE_MODES:
        raise ValueError("gate_mode must be one of %s" % sorted(GATE_MODES))
    dev = q.device
    init_ptr = None
    if initial_state is not None:
        if (initial_state.dtype != torch.float32 or not initial_state.is_contiguous() or
                tuple(initial_state.shape) != (B, heads, d_k, d_v) or initial_state.device != dev):
            raise ValueError("initial_state must be contiguous float32 [B, heads, d_k, d_v] "
                             "on the tensors' device")
        init_ptr = initial_state.data_ptr()
    out, final_state = _outputs(B, heads, H, W, d_k, d_v, q.dtype, dev, out, final_state,
                                want_final_state)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    fs_ptr = final_state.data_ptr() if final_state is not None else None
    rc = raw_call_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), gate.data_ptr(),
                     GATE_MODES[gate_mode], float(tau), init_ptr, int(scan_dir), B, heads, H, W,
                     d_k, d_v, int(chunk), out.data_ptr(), fs_ptr, stream)
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return out, final_state


def raw_call_swiglu(gate, value, ld_in, weight, bias, B, H, W, C, out, stream):
    """Call gla_spatial_swiglu with integer pointers; returns the status code."""
    return load().gla_spatial_swiglu(gate, value, ld_in, weight, bias, B, H, W, C, out, stream)


def spatial_swiglu(gate, value, weight, bias=None, out=None, stream=None):
    """Spatial SwiGLU step: silu(gate) * (3x3 depthwise conv of value + bias).

    gate, value: float16 device tensors [B, H, W, C] with unit channel stride
    and equal, dense token strides (ld >= C elements between tokens: C for
    separate tensors, 2C for the two halves of one [B, H, W, 2C] projection).
    weight: float16 [C, 3, 3] or [C, 1, 3, 3]; bias: float16 [C] or None.
    Returns out, float16 [B, H, W, C] contiguous.
    """
    import torch

    tens = [gate, value, weight] + ([bias] if bias is not None else [])
    if not all(isinstance(t, torch.Tensor) and t.is_cuda for t in tens):
        raise ValueError("gate, value, weight, bias must be device tensors")
    if any(t.dtype != torch.float16 for t in tens):
        raise ValueError("spatial_swiglu takes float16 tensors")
    if gate.dim() != 4 or value.shape != gate.shape:
        raise ValueError("gate and value must be [B, H, W, C] of one shape")
    B, H, W, C = gate.shape
    ld = gate.stride(2)
    dense = (ld, W * ld, H * W * ld)
    for t in (gate, value):
        if t.stride(3) != 1 or (t.stride(2), t.stride(1), t.stride(0)) != dense:
            raise ValueError("gate and value need unit channel stride and equal dense token "
                             "strides")
    if weight.numel() != C * 9 or not weight.is_contiguous():
        raise ValueError("weight must be contiguous [C, 3, 3]")
    if bias is not None and (bias.numel() != C or not bias.is_contiguous()):
        raise ValueError("bias must be contiguous [C]")
    if out is None:
        out = torch.empty((B, H, W, C), dtype=torch.float16, device=gate.device)
    else:
        _check_out(out, "out", (B, H, W, C), torch.float16, gate.device)
    if stream is None:
        stream = torch.cuda.current_stream(gate.device).cuda_stream
    rc = raw_call_swiglu(gate.data_ptr(), value.data_ptr(), ld, weight.data_ptr(),
                         bias.data_ptr() if bias is not None else None, B, H, W, C,
                         out.data_ptr(), stream)
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return out


def raw_call_bwd(q, k, v, la, d_out, d_final, init, scan_dir, B, heads, H, W, d_k, d_v, chunk,
                 dq, dk, dv, dla, d_init, stream):
    """Call gla_chunk_bwd with integer pointers; returns the status code."""
    return load().gla_chunk_bwd(q, k, v, la, d_out, d_final, init, scan_dir, B, heads, H, W, d_k,
                                d_v, chunk, dq, dk, dv, dla, d_init, stream)


def gla_chunk_bwd(q, k, v, log_alpha, d_out, scan_dir, d_final_state=None, initial_state=None,
                  want_d_initial_state=False, chunk=64, stream=None):
    """Chunkwise backward pass (float16, d_k and d_v in {64, 128}).

    Gradients of sum(d_out * out) + sum(d_final_state * final_state) for the
    forward call gla_chunk_fwd / gla_chunk_fwd_ex(q, k, v, log_alpha, scan_dir,
    initial_state=...).  Returns (dq, dk, dv, dlog_alpha, d_initial_state):
    float16 tensors shaped like q, k, v, log_alpha, and the float32 gradient of
    the state before the first step when want_d_initial_state, else None.
    """
    import torch

    B, heads, H, W, d_k, d_v = _check(q, k, v, log_alpha)
    if q.dtype != torch.float16:
        raise ValueError("gla_chunk_bwd takes float16 tensors")
    if (not isinstance(d_out, torch.Tensor) or d_out.dtype != torch.float16 or d_out.shape != v.shape
            or not d_out.is_contiguous() or d_out.device != q.device):
        raise ValueError("d_out must be a contiguous float16 tensor shaped like v")
    dev = q.device
    for name, st in (("d_final_state", d_final_state), ("initial_state", initial_state)):
        if st is not None and (st.dtype != torch.float32 or not st.is_contiguous() or
                               tuple(st.shape) != (B, heads, d_k, d_v) or st.device != dev):
            raise ValueError("%s must be contiguous float32 [B, heads, d_k, d_v]" % name)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dla = torch.empty_like(log_alpha)
    d_init = (torch.empty((B, heads, d_k, d_v), dtype=torch.float32, device=dev)
              if want_d_initial_state else None)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda t: t.data_ptr() if t is not None else None
    rc = raw_call_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_alpha.data_ptr(),
                      d_out.data_ptr(), ptr(d_final_state), ptr(initial_state), int(scan_dir), B,
                      heads, H, W, d_k, d_v, int(chunk), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      dla.data_ptr(), ptr(d_init), stream)
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return dq, dk, dv, dla, d_init


def raw_call_saga(q, k, v, alpha, beta, B, heads, N, d_k, d_v, out, kv, stream):
    """Call gla_saga_fwd with integer pointers; returns the status code."""
    return load().gla_saga_fwd(q, k, v, alpha, beta, B, heads, N, d_k, d_v, out, kv, stream)


def saga_fwd(q, k, v, alpha, beta, out=None, kv=None, want_kv=False, stream=None):
    """SAGA-style non-causal gated linear attention O = Q [(K * A)^T (V * B)].

    q, k, alpha: float16 [B, heads, N, d_k]; v, beta: float16 [B, heads, N, d_v];
    contiguous, on one device.  Returns (out float16 [B, heads, N, d_v], kv),
    kv the float32 gated key-value maps [B, heads, d_k, d_v] when want_kv (or a
    kv tensor is passed), else None.
    """
    import torch

    tens = (q, k, v, alpha, beta)
    if not all(isinstance(t, torch.Tensor) and t.is_cuda for t in tens):
        raise ValueError("q, k, v, alpha, beta must be device tensors")
    if any(t.dtype != torch.float16 for t in tens):
        raise ValueError("saga_fwd takes float16 tensors")
    if q.dim() != 4:
        raise ValueError("expected [B, heads, N, d] tensors")
    B, heads, N, d_k = q.shape
    d_v = v.shape[-1]
    if (k.shape != q.shape or alpha.shape != q.shape or tuple(v.shape[:3]) != (B, heads, N)
            or beta.shape != v.shape):
        raise ValueError("shape mismatch among q, k, v, alpha, beta")
    if not all(t.is_contiguous() for t in tens):
        raise ValueError("tensors must be contiguous")
    dev = q.device
    if out is None:
        out = torch.empty((B, heads, N, d_v), dtype=torch.float16, device=dev)
    else:
        _check_out(out, "out", (B, heads, N, d_v), torch.float16, dev)
    if kv is None:
        if want_kv:
            kv = torch.empty((B, heads, d_k, d_v), dtype=torch.float32, device=dev)
    else:
        _check_out(kv, "kv", (B, heads, d_k, d_v), torch.float32, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = raw_call_saga(q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), beta.data_ptr(),
                       B, heads, N, d_k, d_v, out.data_ptr(),
                       kv.data_ptr() if kv is not None else None, stream)
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return out, kv


def release_workspaces():
    """Free the workspace buffers the library keeps per (device, stream)
    (waits for the work of every device that holds one)."""
    rc = load().gla_release_workspaces()
    if rc != 0:
        raise GlaError(rc, status_str(rc))


def set_forward_mode(mode):
    """Choose the float16 forward path for later calls, process-wide: "auto",
    "three_pass", "two_pass" or "single_pass" (see gla_set_forward_mode)."""
    if mode not in FORWARD_MODES:
        raise ValueError("mode must be one of %s" % sorted(FORWARD_MODES))
    rc = load().gla_set_forward_mode(FORWARD_MODES[mode])
    if rc != 0:
        raise GlaError(rc, status_str(rc))


def set_kernel_events(handles):
    """Arm the measurement hook with six hipEvent_t handles (ints), or clear it."""
    lib = load()
    if not handles:
        return lib.gla_set_kernel_events(None, 0)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    return lib.gla_set_kernel_events(arr, len(handles))


def plan_forward(dtype, B, heads, H, W, d_k, d_v, chunk=64):
    """(span_chunks, n_spans, kernels) the forward call would use on the current
    device; kernels is 1 (no split), 2 (two-pass path) or 3 (three passes)."""
    a, b, c = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    rc = load().gla_plan_forward(1 if dtype == "fp32" else 0, B, heads, H, W, d_k, d_v, chunk,
                                 ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return a.value, b.value, c.value


def plan_spans(dtype, B, heads, H, W, d_k, d_v, chunk=64):
    """(span_chunks, n_spans) the forward call would use on the current device."""
    a, b = ctypes.c_int(0), ctypes.c_int(0)
    rc = load().gla_plan_spans(1 if dtype == "fp32" else 0, B, heads, H, W, d_k, d_v, chunk,
                               ctypes.byref(a), ctypes.byref(b))
    if rc != GLA_OK:
        raise GlaError(rc, status_str(rc))
    return a.value, b.value
