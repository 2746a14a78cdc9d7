"""Shared helpers of the GPU tests: seeded inputs in both precisions and the parity measure."""
from __future__ import annotations

import numpy as np

import gdn_synth

TOL = {"f32": 1e-4, "bf16": 1e-2}   # max|d| / max|ref|, fp32 state in both cases


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU values"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def random_qkv(rng, shape, dtype, relu=False):
    """fp32 values already representable in `dtype` (bf16 rounding done on the host)."""
    out = []
    for i in range(3):
        x = rng.standard_normal(shape).astype(np.float32)
        if relu and i < 2:
            x = np.maximum(x, 0)
        if dtype == "bf16":
            x = gdn_synth.bf16_bits_to_f32(gdn_synth.f32_to_bf16_bits(x))
        out.append(x)
    return out


def to_dev(x, dtype, dev, layout="head"):
    """[B, H, T, D] fp32 numpy -> torch tensor of `dtype` with the given storage layout."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    if layout == "token":
        t = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    return t.to(dev)


def to_np(t):
    return t.float().cpu().numpy()


class HostFrames:
    """Host-side inputs of one (b, h) slice of a workload, frame by frame, generated ahead of
    use by a thread pool (numpy releases the GIL in the hashing and table lookups).

    Calling it with f returns (q_f, k_f, v_f, gamma_f, beta_f): [S, D] fp32 values (rounded
    through bf16 for bf16 workloads) and fp32 gates; pass_of(f) selects the pass for frame f.
    """

    def __init__(self, w, b, h, count, pass_of=None, frame_of=None, workers=8, ahead=48):
        from concurrent.futures import ThreadPoolExecutor
        self.w, self.b, self.h = w, b, h
        self.pass_of = pass_of or (lambda f: 0)
        self.frame_of = frame_of or (lambda f: f)
        self.pool = ThreadPoolExecutor(workers)
        self.ahead = ahead
        self.count = count
        self.fut = {}

    def _make(self, i):
        w, b, h = self.w, self.b, self.h
        f, p = self.frame_of(i), self.pass_of(i)
        out = []
        for tid in (gdn_synth.TID_Q, gdn_synth.TID_K, gdn_synth.TID_V):
            relu = w.relu_qk and tid != gdn_synth.TID_V
            z = gdn_synth.normal_slice(w.seed, tid, b, h, f, w.S, w.D, p, relu)
            if w.dtype == "bf16":
                z = gdn_synth.bf16_bits_to_f32(gdn_synth.f32_to_bf16_bits(z))
            out.append(z)
        g, bt = gdn_synth.gates_cpu(w, heads=[h], frames=[f], pass_=p)
        return out[0], out[1], out[2], float(g[b, 0, 0]), float(bt[b, 0, 0])

    def __call__(self, i):
        for j in range(i, min(self.count, i + self.ahead)):
            if j not in self.fut:
                self.fut[j] = self.pool.submit(self._make, j)
        return self.fut.pop(i).result()

    def close(self):
        for fu in self.fut.values():
            fu.cancel()
        self.pool.shutdown(wait=True)


class HipEvents:
    """Timing-enabled hipEvent_t handles through the HIP runtime that torch already loaded."""

    def __init__(self):
        import ctypes
        import torch  # noqa: F401  (loads the runtime)
        self.ct = ctypes
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self):
        e = self.ct.c_void_p()
        assert self.rt.hipEventCreate(self.ct.byref(e)) == 0
        self.made.append(e.value)
        return e.value

    def ms(self, a, b):
        assert self.rt.hipEventSynchronize(b) == 0
        out = self.ct.c_float()
        assert self.rt.hipEventElapsedTime(self.ct.byref(out), a, b) == 0
        return float(out.value)

    def close(self):
        for e in self.made:
            self.rt.hipEventDestroy(e)
        self.made = []
