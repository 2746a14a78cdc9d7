"""Python binding of libgdn, the frame-wise Gated DeltaNet recurrence on MI355X (gfx950).

Argument marshalling only: every step of the recurrence runs in the HIP kernels of
``libgdn.so`` (built from ``csrc/``), reached through the C ABI declared in
``include/libgdn.h``. PyTorch supplies device memory and the current HIP stream. There is no
CPU fallback: if the shared library is missing or fails to load, every call raises.

Recurrence (gen-hub.ru, "NVIDIA SANA-WM: минутное 720p видео с одной видеокарты", section
"Архитектура: четыре нетривиальных решения"), per (b, h), c = 1/sqrt(D*S) by default:
    R = V_f - gamma_f (c K_f) M;  M <- gamma_f M + beta_f (c K_f)^T R;  O_f = Q_f M.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["GdnError", "Problem", "load", "library_path", "workspace_size", "forward_framewise",
           "forward_framewise_save", "saved_size", "step_frame", "step_frame_noalloc",
           "prepare_step_frame", "prepare_temporal_conv",
           "backward_framewise", "check_timeout",
           "abi_version", "set_trace", "read_trace", "KERNEL_NAMES", "SCHEDULES", "GDN_F32",
           "GDN_BF16"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16, GDN_FP8_E4M3 = 0, 1, 2
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
          4: "GDN_ERR_STRIDE", 5: "GDN_ERR_ALIGN", 6: "GDN_ERR_ALIAS", 7: "GDN_ERR_WORKSPACE",
          8: "GDN_ERR_HIP", 9: "GDN_ERR_TIMEOUT"}
KERNEL_NAMES = {0: "products", 1: "combine", 2: "scan", 3: "step_partial", 4: "step_reduce",
                5: "fused_reset", 6: "fused", 7: "scan_bwd", 8: "bwd", 9: "scan_states",
                10: "tconv", 11: "attn", 12: "step_output", 13: "bwd_qdo", 14: "step_fused",
                15: "attn_combine"}
SCHEDULES = {"auto": 0, "staged": 1, "fused": 2}


class GdnError(RuntimeError):
    def __init__(self, code, message):
        self.code = code
        self.name = STATUS.get(code, "GDN_ERR_%d" % code)
        super().__init__("%s: %s" % (self.name, message))


class Problem(ctypes.Structure):
    """Mirror of gdn_problem (include/libgdn.h)."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
                ("frames", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("use_delta", ctypes.c_int32), ("key_scale", ctypes.c_float),
                ("qkv_stride_b", ctypes.c_int64), ("qkv_stride_h", ctypes.c_int64),
                ("qkv_stride_t", ctypes.c_int64), ("o_stride_b", ctypes.c_int64),
                ("o_stride_h", ctypes.c_int64), ("o_stride_t", ctypes.c_int64),
                ("schedule", ctypes.c_int32)]


class TconvProblem(ctypes.Structure):
    """gdn_tconv_problem of include/libgdn.h."""
    _fields_ = [("batch", ctypes.c_int32), ("frames", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("channels", ctypes.c_int32), ("block_frames", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("x_stride_b", ctypes.c_int64), ("x_stride_t", ctypes.c_int64),
                ("x_stride_s", ctypes.c_int64),
                ("y_stride_b", ctypes.c_int64), ("y_stride_t", ctypes.c_int64),
                ("y_stride_s", ctypes.c_int64)]


class AttnProblem(ctypes.Structure):
    """gdn_attn_problem of include/libgdn.h."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("q_frames", ctypes.c_int32),
                ("kv_frames", ctypes.c_int32), ("q_frame0", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
                ("q_stride_t", ctypes.c_int64),
                ("kv_stride_b", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64),
                ("kv_stride_t", ctypes.c_int64),
                ("o_stride_b", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
                ("o_stride_t", ctypes.c_int64)]


class TraceEntry(ctypes.Structure):
    """Mirror of gdn_trace_entry (include/libgdn.h)."""
    _fields_ = [("kernel", ctypes.c_int32), ("stream", ctypes.c_int32), ("units", ctypes.c_int64)]


_lock = threading.Lock()
_lib = None
_vp = ctypes.c_void_p


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdn.so (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise ImportError("libgdn.so is not built at %s; run __graft_entry__.build()"
                                  % _LIB_PATH)
            # torch ships its own HIP runtime (same soname). Loading torch first makes
            # libgdn.so bind to that copy, so streams and pointers from torch are valid here;
            # loading libgdn.so first would map a second runtime into the process.
            import torch  # noqa: F401
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.POINTER(Problem)
            lib.gdn_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn_workspace_size.restype = ctypes.c_int
            for fn in (lib.gdn_forward_framewise, lib.gdn_step_frame):
                fn.argtypes = [P] + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]
                fn.restype = ctypes.c_int
            lib.gdn_tconv_forward.argtypes = [ctypes.POINTER(TconvProblem)] + [_vp] * 7
            lib.gdn_tconv_forward.restype = ctypes.c_int
            lib.gdn_attention_framecausal.argtypes = [ctypes.POINTER(AttnProblem)] + [_vp] * 5
            lib.gdn_attention_framecausal.restype = ctypes.c_int
            lib.gdn_attention_workspace_size.argtypes = [ctypes.POINTER(AttnProblem),
                                                         ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn_attention_workspace_size.restype = ctypes.c_int
            lib.gdn_attention_framecausal_ws.argtypes = ([ctypes.POINTER(AttnProblem)] + [_vp] * 5
                                                         + [ctypes.c_size_t, _vp])
            lib.gdn_attention_framecausal_ws.restype = ctypes.c_int
            lib.gdn_forward_framewise_fp8.argtypes = [P] + [_vp] * 11 + [_vp, ctypes.c_size_t, _vp]
            lib.gdn_forward_framewise_fp8.restype = ctypes.c_int
            lib.gdn_backward_framewise.argtypes = [P] + [_vp] * 14 + [_vp, ctypes.c_size_t, _vp]
            lib.gdn_backward_framewise.restype = ctypes.c_int
            lib.gdn_saved_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn_saved_size.restype = ctypes.c_int
            lib.gdn_forward_framewise_save.argtypes = ([P] + [_vp] * 8 + [_vp, ctypes.c_size_t]
                                                       + [_vp, ctypes.c_size_t, _vp])
            lib.gdn_forward_framewise_save.restype = ctypes.c_int
            lib.gdn_backward_framewise_saved.argtypes = ([P] + [_vp] * 5 + [_vp, ctypes.c_size_t]
                                                         + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp])
            lib.gdn_backward_framewise_saved.restype = ctypes.c_int
            lib.gdn_step_frame_noalloc.argtypes = [P] + [_vp] * 8 + [_vp]
            lib.gdn_step_frame_noalloc.restype = ctypes.c_int
            lib.gdn_check_timeout.argtypes = [P, ctypes.c_int, _vp, _vp]
            lib.gdn_check_timeout.restype = ctypes.c_int
            lib.gdn_status_string.argtypes = [ctypes.c_int]
            lib.gdn_status_string.restype = ctypes.c_char_p
            lib.gdn_last_error_message.restype = ctypes.c_char_p
            lib.gdn_abi_version.restype = ctypes.c_int
            lib.gdn_set_trace.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
            lib.gdn_set_trace.restype = ctypes.c_int
            lib.gdn_trace_read.argtypes = [ctypes.POINTER(TraceEntry), ctypes.c_int]
            lib.gdn_trace_read.restype = ctypes.c_int
            _lib = lib
    return _lib


def abi_version() -> int:
    return int(load().gdn_abi_version())


def set_trace(handles):
    """Arm the launch trace of later calls on this host thread with hipEvent_t handles (ints,
    an even number: a start and an end event per launch), or disarm it (None / empty)."""
    global _trace_arr
    if not handles:
        _trace_arr = None
        _check(load().gdn_set_trace(None, 0))
        return
    if len(handles) % 2:
        raise GdnError(2, "trace events come in pairs")
    _trace_arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(load().gdn_set_trace(_trace_arr, len(handles) // 2))


_trace_arr = None


def read_trace():
    """Launches of the last call on this thread while the trace was armed:
    list of (kernel name, stream index, units)."""
    lib = load()
    n = lib.gdn_trace_read(None, 0)
    arr = (TraceEntry * max(n, 1))()
    n = lib.gdn_trace_read(arr, n)
    return [(KERNEL_NAMES.get(e.kernel, str(e.kernel)), e.stream, e.units) for e in arr[:n]]


def _check(code):
    if code != 0:
        raise GdnError(code, load().gdn_last_error_message().decode(errors="replace"))


def workspace_size(p: Problem, mode) -> int:
    """mode: 0 / False forward, 1 / True step, 2 backward, 3 backward from saved states."""
    n = ctypes.c_size_t(0)
    _check(load().gdn_workspace_size(ctypes.byref(p), int(mode), ctypes.byref(n)))
    return int(n.value)


def check_timeout(p: Problem, mode, workspace, stream=None):
    """Raise GdnError(GDN_ERR_TIMEOUT) if the last call that used `workspace` (problem p, the
    workspace mode of gdn_workspace_size) gave up a bounded wait of the fused schedule (its
    outputs after that wait are NaN). Synchronises the stream first; a no-op for schedules
    without waits."""
    _check(load().gdn_check_timeout(ctypes.byref(p), int(mode), _ptr(workspace), _stream(stream)))


def _after(p, mode, ws, own_ws, stream, check):
    """check None: check the time-out flag when the binding allocated the workspace itself (no
    one else can read it) and the stream is not being captured into a graph."""
    import torch
    if check is None:
        check = own_ws and not torch.cuda.is_current_stream_capturing()
    if check:
        check_timeout(p, mode, ws, stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return GDN_FP8_E4M3
    raise GdnError(3, "Q/K/V must be bfloat16, float32, or E4M3 codes (uint8 / float8_e4m3fn), "
                      "got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _problem(q, o, F, use_delta, key_scale, schedule=0):
    B, H, T, D = q.shape
    if T % F:
        raise GdnError(2, "token count %d is not a whole number of frames (F=%d)" % (T, F))
    if q.stride(3) != 1 or o.stride(3) != 1:
        raise GdnError(4, "the head dimension must be contiguous")
    return Problem(B, H, D, T // F, F, _dtype_code(q), int(bool(use_delta)),
                   0.0 if key_scale is None else float(key_scale),
                   q.stride(0), q.stride(1), q.stride(2), o.stride(0), o.stride(1), o.stride(2),
                   _schedule_code(schedule))


def _schedule_code(schedule):
    if isinstance(schedule, int):
        return schedule
    if schedule not in SCHEDULES:
        raise GdnError(2, "schedule must be one of %s, got %r" % (sorted(SCHEDULES), schedule))
    return SCHEDULES[schedule]


def _check_f32(name, t, shape):
    """Gates and states cross the ABI as contiguous fp32 arrays."""
    import torch
    if t is None:
        return
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise GdnError(4, "%s must be a contiguous float32 tensor of shape %s (got %s %s%s)"
                       % (name, tuple(shape), t.dtype, tuple(t.shape),
                          "" if t.is_contiguous() else ", non-contiguous"))


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(p, step_mode, workspace, device):
    import torch
    need = workspace_size(p, step_mode)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def forward_framewise(q, k, v, gamma, beta, state=None, *, use_delta=True, key_scale=None,
                      out=None, state_out=None, return_state=True, workspace=None, stream=None,
                      schedule="auto", check_timeout=None):
    """All frames: q, k, v [B, H, F*S, D] (D contiguous, any other strides, same strides for
    all three); gamma, beta fp32 [B, H, F]; state fp32 [B, H, D, D] or None (zero).
    schedule: "auto", "staged" (products, scan, outputs as three passes) or "fused" (one pass;
    bf16 with D = 64 or 128).
    check_timeout: after the call, synchronise and raise GdnError(GDN_ERR_TIMEOUT) if a bounded
    wait of the fused schedule gave up (its later outputs are NaN); None (default) checks only
    when the binding allocated the workspace itself and the stream is not being captured. The
    other forward and backward calls take the same argument.
    Returns (o, state_out); o has q's shape and dtype, state_out is None when
    return_state is False."""
    import torch
    B, H, T, D = q.shape
    F = gamma.shape[2]
    if k.stride() != q.stride() or v.stride() != q.stride() or k.shape != q.shape \
            or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdnError(4, "q, k and v must share shape, dtype and strides")
    if out is None:
        out = torch.empty((B, H, T, D), dtype=q.dtype, device=q.device)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _check_f32("gamma", gamma, (B, H, F))
    _check_f32("beta", beta, (B, H, F))
    _check_f32("state", state, (B, H, D, D))
    _check_f32("state_out", state_out, (B, H, D, D))
    p = _problem(q, out, F, use_delta, key_scale, schedule)
    ws, nbytes = _workspace(p, False, workspace, q.device)
    _check(load().gdn_forward_framewise(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                        _ptr(beta), _ptr(state), _ptr(out), _ptr(state_out),
                                        _ptr(ws), nbytes, _stream(stream)))
    _after(p, 0, ws, workspace is None, stream, check_timeout)
    return out, state_out


def saved_size(p) -> int:
    """Bytes of the buffer forward_framewise_save keeps for backward_framewise (saved=...)."""
    n = ctypes.c_size_t(0)
    _check(load().gdn_saved_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def forward_framewise_save(q, k, v, gamma, beta, state=None, *, use_delta=True, key_scale=None,
                           out=None, state_out=None, return_state=True, saved=None,
                           workspace=None, stream=None, check_timeout=None):
    """forward_framewise on the fused schedule (bf16, D = 64 or 128) that also keeps what the
    backward needs (the frames' key-key products and every state), so that
    backward_framewise(..., saved=saved) skips recomputing the forward.
    Returns (o, state_out, saved); saved is a uint8 device tensor of saved_size bytes."""
    import torch
    B, H, T, D = q.shape
    F = gamma.shape[2]
    if k.stride() != q.stride() or v.stride() != q.stride() or k.shape != q.shape \
            or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdnError(4, "q, k and v must share shape, dtype and strides")
    if out is None:
        out = torch.empty((B, H, T, D), dtype=q.dtype, device=q.device)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _check_f32("gamma", gamma, (B, H, F))
    _check_f32("beta", beta, (B, H, F))
    _check_f32("state", state, (B, H, D, D))
    _check_f32("state_out", state_out, (B, H, D, D))
    p = _problem(q, out, F, use_delta, key_scale, "fused")
    if saved is None:
        saved = torch.empty(saved_size(p), dtype=torch.uint8, device=q.device)
    ws, nbytes = _workspace(p, False, workspace, q.device)
    _check(load().gdn_forward_framewise_save(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(state),
        _ptr(out), _ptr(state_out), _ptr(saved), saved.numel() * saved.element_size(), _ptr(ws),
        nbytes, _stream(stream)))
    _after(p, 0, ws, workspace is None, stream, check_timeout)
    return out, state_out, saved


def forward_framewise_fp8(q, k, v, q_scale, k_scale, v_scale, gamma, beta, state=None, *,
                          use_delta=True, key_scale=None, out=None, state_out=None,
                          return_state=True, workspace=None, stream=None, schedule="auto",
                          check_timeout=None):
    """All frames from E4M3 inputs: q, k, v [B, H, F*S, D] of OCP FP8 E4M3 codes (torch.uint8
    or torch.float8_e4m3fn, D contiguous, same strides); q_scale, k_scale, v_scale, gamma, beta
    fp32 [B, H, F]; an element's value is its frame's scale times the code's value.
    Returns (o, state_out) with o bf16 [B, H, F*S, D]."""
    import torch
    B, H, T, D = q.shape
    F = gamma.shape[2]
    if k.stride() != q.stride() or v.stride() != q.stride() or k.shape != q.shape \
            or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdnError(4, "q, k and v must share shape, dtype and strides")
    if _dtype_code(q) != GDN_FP8_E4M3:
        raise GdnError(3, "forward_framewise_fp8 takes E4M3 codes (uint8 or float8_e4m3fn)")
    if out is None:
        out = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16:
        raise GdnError(3, "the output of the E4M3 forward is bfloat16")
    if state_out is None and return_state:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale),
                    ("gamma", gamma), ("beta", beta)):
        _check_f32(name, t, (B, H, F))
    _check_f32("state", state, (B, H, D, D))
    _check_f32("state_out", state_out, (B, H, D, D))
    p = _problem(q, out, F, use_delta, key_scale, schedule)
    ws, nbytes = _workspace(p, False, workspace, q.device)
    _check(load().gdn_forward_framewise_fp8(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
        _ptr(gamma), _ptr(beta), _ptr(state), _ptr(out), _ptr(state_out), _ptr(ws), nbytes,
        _stream(stream)))
    _after(p, 0, ws, workspace is None, stream, check_timeout)
    return out, state_out


def temporal_conv(x, weight, bias=None, cache=None, *, block_frames, out=None, cache_out=None,
                  return_cache=True, stream=None):
    """Block-causal temporal convolution (gdn_tconv_forward). x [B, T, S, C] (bf16 or fp32,
    channels contiguous); weight fp32 [C, 3] (taps on frames t-1, t, t+1); bias fp32 [C] or
    None; cache [B, S, C] (x's dtype, contiguous): the previous block's last frame, or None for
    the first block. Returns (y, cache_out); cache_out (x[:, -1]) may be `cache` itself."""
    import torch
    B, T, S, C = x.shape
    if out is None:
        out = torch.empty((B, T, S, C), dtype=x.dtype, device=x.device)
    if cache_out is None and return_cache:
        cache_out = torch.empty((B, S, C), dtype=x.dtype, device=x.device)
    if x.stride(3) != 1 or out.stride(3) != 1:
        raise GdnError(4, "the channel dimension must be contiguous")
    for name, t in (("cache", cache), ("cache_out", cache_out)):
        if t is not None and (t.dtype != x.dtype or tuple(t.shape) != (B, S, C) or not t.is_contiguous()):
            raise GdnError(4, "%s must be a contiguous %s tensor of shape %s" % (name, x.dtype, (B, S, C)))
    _check_f32("weight", weight, (C, 3))
    _check_f32("bias", bias, (C,))
    code = _dtype_code(x)
    p = TconvProblem(B, T, S, C, int(block_frames), code, x.stride(0), x.stride(1), x.stride(2),
                     out.stride(0), out.stride(1), out.stride(2))
    _check(load().gdn_tconv_forward(ctypes.byref(p), _ptr(x), _ptr(weight), _ptr(bias), _ptr(cache),
                                    _ptr(out), _ptr(cache_out), _stream(stream)))
    return out, cache_out


def prepare_temporal_conv(x, weight, bias=None, cache=None, *, block_frames, out, cache_out=None,
                          stream=None):
    """temporal_conv with every argument checked and marshalled once: returns a function of no
    arguments that enqueues the same gdn_tconv_forward call again (same buffers; their contents
    may change between calls) and raises GdnError if it fails. For streaming loops that convolve
    one block per call from the cache (cache_out may be cache)."""
    B, T, S, C = x.shape
    if x.stride(3) != 1 or out.stride(3) != 1:
        raise GdnError(4, "the channel dimension must be contiguous")
    for name, t in (("cache", cache), ("cache_out", cache_out)):
        if t is not None and (t.dtype != x.dtype or tuple(t.shape) != (B, S, C) or not t.is_contiguous()):
            raise GdnError(4, "%s must be a contiguous %s tensor of shape %s" % (name, x.dtype, (B, S, C)))
    _check_f32("weight", weight, (C, 3))
    _check_f32("bias", bias, (C,))
    p = TconvProblem(B, T, S, C, int(block_frames), _dtype_code(x), x.stride(0), x.stride(1),
                     x.stride(2), out.stride(0), out.stride(1), out.stride(2))
    fn = load().gdn_tconv_forward
    args = (ctypes.byref(p), _ptr(x), _ptr(weight), _ptr(bias), _ptr(cache), _ptr(out),
            _ptr(cache_out), _stream(stream))
    keep = (p, x, weight, bias, cache, out, cache_out)   # alive while the call is

    def call():
        code = fn(*args)
        if code:
            _check(code)
        return keep[5], keep[6]
    return call


def attention_problem(q, k, out, tokens_per_frame, q_frame0=0, scale=None):
    """The gdn_attn_problem of an attention call on these tensors (o's strides from `out`)."""
    B, H, Tq, D = q.shape
    S = int(tokens_per_frame)
    return AttnProblem(B, H, D, S, Tq // S, k.shape[2] // S, int(q_frame0), GDN_BF16,
                       0.0 if scale is None else float(scale), *q.stride()[:3], *k.stride()[:3],
                       *out.stride()[:3])


def attention_workspace_size(p: AttnProblem) -> int:
    """Bytes of workspace that attention_framecausal(..., workspace=) may use for problem p
    (0: the call would not split its keys)."""
    n = ctypes.c_size_t(0)
    _check(load().gdn_attention_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def attention_framecausal(q, k, v, *, tokens_per_frame, q_frame0=0, scale=None, out=None,
                          workspace=None, stream=None):
    """Frame-causal softmax attention (gdn_attention_framecausal). q [B, H, Tq, D], k, v
    [B, H, Tk, D] (bf16, D contiguous, k and v with the same strides); q's rows are frames
    q_frame0 .. q_frame0 + Tq/S - 1, k's and v's frames 0 .. Tk/S - 1. Returns o like q.
    workspace: a uint8 device tensor of attention_workspace_size bytes lets a single-frame
    call split its keys over more workgroups (gdn_attention_framecausal_ws); "auto" allocates
    one when the call would use it."""
    import torch
    B, H, Tq, D = q.shape
    Tk = k.shape[2]
    S = int(tokens_per_frame)
    if Tq % S or Tk % S:
        raise GdnError(2, "token counts must be whole frames of %d tokens" % S)
    if k.stride() != v.stride() or k.shape != v.shape:
        raise GdnError(4, "k and v must share shape and strides")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise GdnError(3, "attention takes bfloat16 q, k, v")
    if out is None:
        out = torch.empty((B, H, Tq, D), dtype=torch.bfloat16, device=q.device)
    if q.stride(3) != 1 or k.stride(3) != 1 or out.stride(3) != 1:
        raise GdnError(4, "the head dimension must be contiguous")
    p = AttnProblem(B, H, D, S, Tq // S, Tk // S, int(q_frame0), GDN_BF16,
                    0.0 if scale is None else float(scale), *q.stride()[:3], *k.stride()[:3],
                    *out.stride()[:3])
    if workspace is None:
        _check(load().gdn_attention_framecausal(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(out), _stream(stream)))
        return out
    if isinstance(workspace, str):
        if workspace != "auto":
            raise GdnError(2, "workspace must be a tensor, None or \"auto\"")
        n = attention_workspace_size(p)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check(load().gdn_attention_framecausal_ws(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(out), _ptr(workspace), workspace.numel(),
                                               _stream(stream)))
    return out


def step_frame(q, k, v, gamma, beta, state, commit=True, *, use_delta=True, key_scale=None,
               out=None, state_out=None, workspace=None, stream=None, schedule="auto",
               check_timeout=None):
    """One frame: q, k, v [B, H, S, D]; gamma, beta fp32 [B, H]; state fp32 [B, H, D, D].
    schedule: "staged" keeps the bf16 step's three launches; "auto" / "fused" run them as one
    where the shape and device allow. check_timeout as in forward_framewise.
    Returns (o, new_state) when commit, else (o, None). state_out may be `state` itself."""
    import torch
    B, H, S, D = q.shape
    if k.stride() != q.stride() or v.stride() != q.stride() or k.shape != q.shape \
            or v.shape != q.shape:
        raise GdnError(4, "q, k and v must share shape and strides")
    if out is None:
        out = torch.empty((B, H, S, D), dtype=q.dtype, device=q.device)
    if commit and state_out is None:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    if not commit:
        state_out = None
    _check_f32("gamma", gamma, (B, H))
    _check_f32("beta", beta, (B, H))
    _check_f32("state", state, (B, H, D, D))
    _check_f32("state_out", state_out, (B, H, D, D))
    p = _problem(q, out, 1, use_delta, key_scale, schedule)
    ws, nbytes = _workspace(p, True, workspace, q.device)
    _check(load().gdn_step_frame(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                 _ptr(beta), _ptr(state), _ptr(out), _ptr(state_out), _ptr(ws),
                                 nbytes, _stream(stream)))
    _after(p, 1, ws, workspace is None, stream, check_timeout)
    return out, state_out


def prepare_step_frame(q, k, v, gamma, beta, state, commit=True, *, use_delta=True,
                       key_scale=None, out=None, state_out=None, workspace=None, stream=None,
                       schedule="auto"):
    """step_frame with every argument checked and marshalled once: returns a function of no
    arguments that enqueues the same gdn_step_frame call again (on the same buffers, whose
    contents may change between calls) and raises GdnError if it fails. For loops that issue
    many steps from the host (a streaming server), where the per-call checks of step_frame
    would cost more host time than the step takes on the GPU."""
    import torch
    B, H, S, D = q.shape
    if k.stride() != q.stride() or v.stride() != q.stride() or k.shape != q.shape \
            or v.shape != q.shape:
        raise GdnError(4, "q, k and v must share shape and strides")
    if out is None:
        out = torch.empty((B, H, S, D), dtype=q.dtype, device=q.device)
    if commit and state_out is None:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    if not commit:
        state_out = None
    _check_f32("gamma", gamma, (B, H))
    _check_f32("beta", beta, (B, H))
    _check_f32("state", state, (B, H, D, D))
    _check_f32("state_out", state_out, (B, H, D, D))
    p = _problem(q, out, 1, use_delta, key_scale, schedule)
    ws, nbytes = _workspace(p, True, workspace, q.device)
    fn = load().gdn_step_frame
    args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(state),
            _ptr(out), _ptr(state_out), _ptr(ws), nbytes, _stream(stream))
    keep = (p, q, k, v, gamma, beta, state, out, state_out, ws)   # alive while the call is

    def call():
        code = fn(*args)
        if code:
            _check(code)
        return keep[7], keep[8]
    return call


def step_frame_noalloc(q, k, v, gamma, beta, state, commit=True, *, use_delta=True,
                       key_scale=None, out=None, state_out=None, stream=None, schedule="auto"):
    """step_frame through gdn_step_frame_noalloc: the workspace is the library's own static
    device scratch (no workspace argument, nothing allocated by the library; calls on one GPU
    share it and must not overlap). out and state_out, when not given, are allocated here by
    torch; pass them for a call that allocates nothing at all."""
    import torch
    B, H, S, D = q.shape
    if k.stride() != q.stride() or v.stride() != q.stride() or k.shape != q.shape \
            or v.shape != q.shape:
        raise GdnError(4, "q, k and v must share shape and strides")
    if out is None:
        out = torch.empty((B, H, S, D), dtype=q.dtype, device=q.device)
    if commit and state_out is None:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    if not commit:
        state_out = None
    _check_f32("gamma", gamma, (B, H))
    _check_f32("beta", beta, (B, H))
    _check_f32("state", state, (B, H, D, D))
    _check_f32("state_out", state_out, (B, H, D, D))
    p = _problem(q, out, 1, use_delta, key_scale, schedule)
    _check(load().gdn_step_frame_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                         _ptr(beta), _ptr(state), _ptr(out), _ptr(state_out),
                                         _stream(stream)))
    return out, state_out


def backward_framewise(q, k, v, gamma, beta, d_o, state=None, d_state_out=None, *,
                       use_delta=True, key_scale=None, dq=None, dk=None, dv=None,
                       return_state_grad=True, saved=None, workspace=None, stream=None,
                       schedule="auto", check_timeout=None):
    """Gradients of forward_framewise. q, k, v [B, H, F*S, D] (bf16, D = 64 or 128, same
    strides); d_o: dL/dO with o's shape (any strides with D contiguous); gamma, beta fp32
    [B, H, F]; state, d_state_out fp32 [B, H, D, D] or None. With saved (from
    forward_framewise_save on the same inputs) the forward states are not recomputed and state
    is not read. schedule: "fused" runs the reverse chain inside the pass over Q and dO
    (ticket-ordered), "staged" as a separate scan, "auto" picks by problem size.
    Returns (dq, dk, dv, dgamma, dbeta, d_state_in); d_state_in is None when
    return_state_grad is False."""
    import torch
    B, H, T, D = q.shape
    F = gamma.shape[2]
    if k.stride() != q.stride() or v.stride() != q.stride() or k.shape != q.shape \
            or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype \
            or d_o.shape != q.shape or d_o.dtype != q.dtype:
        raise GdnError(4, "q, k and v must share shape, dtype and strides; d_o must match their "
                          "shape and dtype")
    if d_o.stride(3) != 1:
        raise GdnError(4, "the head dimension of d_o must be contiguous")

    def like_q(t):
        if t is not None:
            return t
        return torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)

    dq, dk, dv = like_q(dq), like_q(dk), like_q(dv)
    dg = torch.empty((B, H, F), dtype=torch.float32, device=q.device)
    db = torch.empty((B, H, F), dtype=torch.float32, device=q.device)
    dsi = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device) \
        if return_state_grad else None
    _check_f32("gamma", gamma, (B, H, F))
    _check_f32("beta", beta, (B, H, F))
    _check_f32("state", state, (B, H, D, D))
    _check_f32("d_state_out", d_state_out, (B, H, D, D))
    p = _problem(q, d_o, F, use_delta, key_scale, schedule)
    if saved is not None:
        ws, nbytes = _workspace(p, 3, workspace, q.device)
        _check(load().gdn_backward_framewise_saved(
            ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(saved),
            saved.numel() * saved.element_size(), _ptr(d_o), _ptr(d_state_out), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(dg), _ptr(db), _ptr(dsi), _ptr(ws), nbytes, _stream(stream)))
        _after(p, 3, ws, workspace is None, stream, check_timeout)
        return dq, dk, dv, dg, db, dsi
    ws, nbytes = _workspace(p, 2, workspace, q.device)
    _check(load().gdn_backward_framewise(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(state),
        _ptr(d_o), _ptr(d_state_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db),
        _ptr(dsi), _ptr(ws), nbytes, _stream(stream)))
    _after(p, 2, ws, workspace is None, stream, check_timeout)
    return dq, dk, dv, dg, db, dsi
