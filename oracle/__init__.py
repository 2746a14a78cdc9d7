"""Python access to the fp64 CPU oracle of the frame-wise Gated DeltaNet recurrence.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package. The GPU library never imports it and shares no code
with it. The arithmetic lives in ``gdn_oracle.c``; this module only builds that file with gcc,
loads it with ctypes and passes fp64 numpy arrays to it.

The recurrence (gen-hub.ru, "NVIDIA SANA-WM: минутное 720p видео с одной видеокарты", section
"Архитектура: четыре нетривиальных решения"): per head a D x D state M; for each frame f the
keys are scaled by c = 1/sqrt(D*S), the residual R = V_f - gamma_f * (c K_f) M is formed, the
state becomes gamma_f M + beta_f (c K_f)^T R, and the frame's output is O_f = Q_f M.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_ubyte)


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    lib.gdn_oracle_forward.argtypes = ([ctypes.c_int] * 6 + [ctypes.c_double] + [_dp] * 8
                                       + [ctypes.c_int])
    lib.gdn_oracle_forward.restype = ctypes.c_int
    lib.gdn_oracle_step.argtypes = ([ctypes.c_int] * 5 + [ctypes.c_double] + [_dp] * 8
                                    + [ctypes.c_int])
    lib.gdn_oracle_step.restype = ctypes.c_int
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    if hasattr(lib, "gdn_oracle_forward_fp8"):
        lib.gdn_oracle_e4m3.argtypes = [ctypes.c_uint]
        lib.gdn_oracle_e4m3.restype = ctypes.c_double
        lib.gdn_oracle_forward_fp8.argtypes = ([ctypes.c_int] * 6 + [ctypes.c_double] + [_u8p] * 3
                                               + [_dp] * 8 + [ctypes.c_int])
        lib.gdn_oracle_forward_fp8.restype = ctypes.c_int
    if hasattr(lib, "gdn_oracle_backward"):
        lib.gdn_oracle_backward.argtypes = ([ctypes.c_int] * 6 + [ctypes.c_double] + [_dp] * 14
                                            + [ctypes.c_int])
        lib.gdn_oracle_backward.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(_LIB)
    return _lib


def load_variant(src_text: str, workdir: str):
    """Compile a modified copy of the oracle source (used by the mutation tests to check
    that the pins catch planted mistakes) and return its bound library."""
    src = os.path.join(workdir, "variant.c")
    out = os.path.join(workdir, "libvariant.so")
    with open(src, "w") as fh:
        fh.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c99", src, "-o",
                           out, "-lm"])
    return _bind(out)


def source_text() -> str:
    with open(_SRC) as fh:
        return fh.read()


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def forward(q, k, v, gamma, beta, state_in=None, *, use_delta=True, key_scale=None,
            nthreads=0, lib=None):
    """All frames. q, k, v: [B, H, F*S, D]; gamma, beta: [B, H, F]; state_in: [B, H, D, D].

    Returns (o [B, H, F*S, D], state_out [B, H, D, D]) as fp64 arrays.
    lib="numpy" runs the frame-streaming numpy variant (oracle/stream.py) instead of the C code.
    """
    if isinstance(lib, str) and lib == "numpy":
        from . import stream
        return stream.forward(q, k, v, gamma, beta, state_in, use_delta=use_delta,
                              key_scale=key_scale)
    q, k, v, gamma, beta = map(_f64, (q, k, v, gamma, beta))
    B, H, T, D = q.shape
    F = gamma.shape[2]
    assert T % F == 0, "token count must be a whole number of frames"
    S = T // F
    assert k.shape == q.shape and v.shape == q.shape and beta.shape == gamma.shape
    st = None if state_in is None else _f64(state_in)
    o = np.empty_like(q)
    so = np.empty((B, H, D, D), dtype=np.float64)
    c = 0.0 if key_scale is None else float(key_scale)   # 0 selects the oracle's default
    rc = (lib or _load()).gdn_oracle_forward(B, H, D, S, F, int(bool(use_delta)), c, _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(gamma), _ptr(beta), _ptr(st), _ptr(o),
                                    _ptr(so), int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_forward failed with code %d" % rc)
    return o, so


def e4m3_value(code: int, lib=None) -> float:
    """Value of one OCP FP8 E4M3 code (0..255)."""
    return float((lib or _load()).gdn_oracle_e4m3(int(code)))


def forward_fp8(q8, k8, v8, q_scale, k_scale, v_scale, gamma, beta, state_in=None, *,
                use_delta=True, key_scale=None, nthreads=0, lib=None):
    """All frames from 8-bit inputs. q8, k8, v8: uint8 OCP FP8 E4M3 codes [B, H, F*S, D];
    q_scale, k_scale, v_scale, gamma, beta: [B, H, F]; element value = scale[b, h, f] * E4M3(code).

    Returns (o [B, H, F*S, D], state_out [B, H, D, D]) as fp64 arrays.
    """
    q8, k8, v8 = (np.ascontiguousarray(x, dtype=np.uint8) for x in (q8, k8, v8))
    q_scale, k_scale, v_scale, gamma, beta = map(_f64, (q_scale, k_scale, v_scale, gamma, beta))
    B, H, T, D = q8.shape
    F = gamma.shape[2]
    assert T % F == 0, "token count must be a whole number of frames"
    S = T // F
    assert k8.shape == q8.shape and v8.shape == q8.shape
    assert q_scale.shape == gamma.shape and k_scale.shape == gamma.shape and v_scale.shape == gamma.shape
    st = None if state_in is None else _f64(state_in)
    o = np.empty(q8.shape, dtype=np.float64)
    so = np.empty((B, H, D, D), dtype=np.float64)
    c = 0.0 if key_scale is None else float(key_scale)
    u8 = lambda a: a.ctypes.data_as(_u8p)
    rc = (lib or _load()).gdn_oracle_forward_fp8(
        B, H, D, S, F, int(bool(use_delta)), c, u8(q8), u8(k8), u8(v8), _ptr(q_scale),
        _ptr(k_scale), _ptr(v_scale), _ptr(gamma), _ptr(beta), _ptr(st), _ptr(o), _ptr(so),
        int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_forward_fp8 failed with code %d" % rc)
    return o, so


def step(q, k, v, gamma, beta, state_in, *, commit=True, use_delta=True, key_scale=None,
         nthreads=0, lib=None):
    """One frame. q, k, v: [B, H, S, D]; gamma, beta: [B, H]; state_in: [B, H, D, D].

    Returns (o, state_out); state_out is None when commit is False.
    """
    if isinstance(lib, str) and lib == "numpy":
        from . import stream
        o, so = stream.forward(q, k, v, np.asarray(gamma)[..., None], np.asarray(beta)[..., None],
                               np.asarray(state_in, np.float64), use_delta=use_delta,
                               key_scale=key_scale)
        return o, (so if commit else None)
    q, k, v, gamma, beta, st = map(_f64, (q, k, v, gamma, beta, state_in))
    B, H, S, D = q.shape
    o = np.empty_like(q)
    so = np.empty((B, H, D, D), dtype=np.float64) if commit else None
    c = 0.0 if key_scale is None else float(key_scale)   # 0 selects the oracle's default
    rc = (lib or _load()).gdn_oracle_step(B, H, D, S, int(bool(use_delta)), c, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(gamma), _ptr(beta), _ptr(st), _ptr(o), _ptr(so),
                                 int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_step failed with code %d" % rc)
    return o, so


def backward(q, k, v, gamma, beta, state_in, d_o, d_state_out=None, *, use_delta=True,
             key_scale=None, nthreads=0, lib=None):
    """Gradients of the forward for upstream gradients d_o = dL/dO [B, H, F*S, D] and
    d_state_out = dL/dstate_out [B, H, D, D] (None: zero).

    Returns (dq, dk, dv [B, H, F*S, D], dgamma, dbeta [B, H, F], d_state_in [B, H, D, D]) as
    fp64 arrays; d_state_in is the gradient with respect to state_in (a zero initial state when
    state_in is None).
    """
    q, k, v, gamma, beta, d_o = map(_f64, (q, k, v, gamma, beta, d_o))
    B, H, T, D = q.shape
    F = gamma.shape[2]
    assert T % F == 0, "token count must be a whole number of frames"
    S = T // F
    st = None if state_in is None else _f64(state_in)
    dso = None if d_state_out is None else _f64(d_state_out)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    dg, db = np.empty_like(gamma), np.empty_like(gamma)
    dsi = np.empty((B, H, D, D), dtype=np.float64)
    c = 0.0 if key_scale is None else float(key_scale)
    rc = (lib or _load()).gdn_oracle_backward(
        B, H, D, S, F, int(bool(use_delta)), c, _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
        _ptr(beta), _ptr(st), _ptr(d_o), _ptr(dso), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
        _ptr(db), _ptr(dsi), int(nthreads))
    if rc != 0:
        raise RuntimeError("gdn_oracle_backward failed with code %d" % rc)
    return dq, dk, dv, dg, db, dsi
