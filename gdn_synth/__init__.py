"""Seeded synthetic inputs for the frame-wise GDN workloads.

This module feeds both sides of every comparison: the fp64 CPU oracle (numpy, on the host) and
the GPU library (torch tensors on the device). It holds none of the recurrence's arithmetic,
only random-number generation, the workload table and bf16 bit conversions.

Generator (counter-based, so any (tensor, b, h, f, pass) slice can be made on its own):

* ``hash32`` is the 32-bit integer hash "lowbias32" published by C. Wellons ("Prospecting for
  Hash Functions", 2018): x ^= x>>16; x *= 0x7feb352d; x ^= x>>15; x *= 0x846ca68b; x ^= x>>16,
  all modulo 2**32.
* A slice key chains the hash over (seed, tensor id, b, h, f, pass).
* Element e of a slice (e = s*D + d) draws the word w = hash32(hash32(e) ^ key).
* Normal values: NT[w >> 8], where NT[n] = Phi^-1((n + 0.5) / 2**24) is the fp64 normal
  quantile rounded to fp32 (scipy.special.ndtri), i.e. an exact-quantile N(0, 1) with 2**24
  levels. bf16 tensors take round-to-nearest-even of that fp32 value.
* Uniform gates: lo + (hi - lo) * ((w >> 8) + 0.5) / 2**24 in fp64, rounded to fp32.
* E4M3 workloads (8-bit Q, K, V with one scale per (tensor, b, h, f)): the frame's fp32 normal
  values x get the power-of-two scale s = 2**(E - 8), E the binary exponent of max|x| (max|x| =
  m 2**E with m in [0.5, 1)), so that |x| / s < 256 stays inside E4M3's finite range (448);
  x / s is then exact, and the codes are torch's round-to-nearest-even conversion to
  float8_e4m3fn. Both the scale and the division are exact, so host and device codes agree.

The host path uses numpy uint32 arithmetic; the device path uses torch int64 arithmetic whose
intermediates stay below 2**49, so both are exact and produce identical bits.

Workloads: frame-wise GDN at the shapes of the pages' video workloads (SANA-WM: 961 latent
frames for a 60 s 720p clip, gen-hub.ru article, architecture section; SANA-Streaming at
1280x704, jefxiong.cn digest item 1). These synthetic Gaussian inputs stand in for the model's
activations; no dataset or weights are involved.
"""
from __future__ import annotations

import dataclasses
import threading

import numpy as np

M32 = 0xFFFFFFFF
NLEVELS_BITS = 24

TID_Q, TID_K, TID_V, TID_GAMMA, TID_BETA, TID_STATE = 1, 2, 3, 4, 5, 6


# --------------------------------------------------------------------------- host (numpy)
def hash32(x):
    """lowbias32 on numpy uint32 (array or scalar); wraps modulo 2**32."""
    x = np.asarray(x, dtype=np.uint32)
    with np.errstate(over="ignore"):
        x = x ^ (x >> np.uint32(16))
        x = x * np.uint32(0x7FEB352D)
        x = x ^ (x >> np.uint32(15))
        x = x * np.uint32(0x846CA68B)
        x = x ^ (x >> np.uint32(16))
    return x


def slice_key(seed, tid, b, h, f, pass_=0) -> int:
    x = int(hash32(np.uint32((seed ^ 0x9E3779B9) & M32)))
    for part in (tid, b, h, f, pass_):
        x = int(hash32(np.uint32((x ^ int(part)) & M32)))
    return x


_table_lock = threading.Lock()
_table = None


def normal_table() -> np.ndarray:
    """NT[n] = Phi^-1((n + 0.5) / 2**24) rounded to fp32 (2**24 entries, cached)."""
    global _table
    with _table_lock:
        if _table is None:
            from scipy.special import ndtri
            n = np.arange(1 << NLEVELS_BITS, dtype=np.float64)
            _table = ndtri((n + 0.5) / float(1 << NLEVELS_BITS)).astype(np.float32)
    return _table


_elem_hash_cache = {}


def _elem_hash(n: int) -> np.ndarray:
    h = _elem_hash_cache.get(n)
    if h is None:
        h = hash32(np.arange(n, dtype=np.uint32))
        if n <= (1 << 22):
            _elem_hash_cache[n] = h
    return h


def words(seed, tid, b, h, f, n, pass_=0) -> np.ndarray:
    """The n uint32 words of slice (tid, b, h, f, pass)."""
    key = np.uint32(slice_key(seed, tid, b, h, f, pass_))
    return hash32(_elem_hash(n) ^ key)


def normal_slice(seed, tid, b, h, f, S, D, pass_=0, relu=False) -> np.ndarray:
    """fp32 [S, D] normal values of one (tensor, b, h, f, pass) slice."""
    w = words(seed, tid, b, h, f, S * D, pass_)
    z = normal_table()[(w >> np.uint32(32 - NLEVELS_BITS)).astype(np.int64)]
    if relu:
        z = np.maximum(z, np.float32(0.0))
    return z.reshape(S, D)


def uniform_value(seed, tid, b, h, f, lo, hi, pass_=0) -> np.float32:
    w = int(words(seed, tid, b, h, f, 1, pass_)[0])
    u = ((w >> (32 - NLEVELS_BITS)) + 0.5) / float(1 << NLEVELS_BITS)
    return np.float32(lo + (hi - lo) * u)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    D: int
    S: int
    F: int                      # frames (forward) or frames streamed (step mode)
    dtype: str                  # "f32" or "bf16" for Q, K, V, O; "fp8": E4M3 Q, K, V, bf16 O
    use_delta: bool
    gamma: tuple                # (lo, hi) of U(lo, hi); lo == hi means a constant
    beta: tuple
    relu_qk: bool = False       # ReLU applied to Q and K by the generator
    passes: int = 1             # step mode: denoising passes per frame
    step_mode: bool = False

    @property
    def tokens(self) -> int:
        return self.B * self.F * self.S

    def elem_bytes(self) -> int:
        """Bytes per element of Q, K and V."""
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", 0, 1, 2, 16, 16, 8, "f32", True, (0.9, 1.0), (0.0, 1.0)),
        Workload("block_causal_bf16", 1, 1, 16, 64, 1560, 21, "bf16", False, (1.0, 1.0),
                 (1.0, 1.0), relu_qk=True),
        Workload("gdn_880x81_bf16", 2, 2, 16, 128, 880, 81, "bf16", True, (0.85, 1.0),
                 (0.1, 0.9)),
        Workload("gdn_720p_60s_bf16", 3, 1, 16, 128, 3520, 961, "bf16", True, (0.9, 1.0),
                 (0.1, 0.9)),
        Workload("stream_720p_bf16", 4, 1, 16, 128, 3520, 240, "bf16", True, (0.9, 1.0),
                 (0.1, 0.9), passes=4, step_mode=True),
        Workload("gdn_720p_60s_fp8", 5, 1, 16, 128, 3520, 961, "fp8", True, (0.9, 1.0),
                 (0.1, 0.9)),
    ]
}
WORKLOAD_ORDER = ["tiny_f32", "block_causal_bf16", "gdn_880x81_bf16", "gdn_720p_60s_bf16",
                  "stream_720p_bf16", "gdn_720p_60s_fp8"]


def gates_cpu(w: Workload, heads=None, frames=None, pass_=0):
    """gamma, beta as fp32 [B, len(heads), len(frames)] for the selected heads and frames."""
    heads = range(w.H) if heads is None else list(heads)
    frames = range(w.F) if frames is None else list(frames)
    g = np.empty((w.B, len(heads), len(frames)), np.float32)
    bt = np.empty_like(g)
    for b in range(w.B):
        for hi, h in enumerate(heads):
            for fi, f in enumerate(frames):
                g[b, hi, fi] = (np.float32(w.gamma[0]) if w.gamma[0] == w.gamma[1] else
                                uniform_value(w.seed, TID_GAMMA, b, h, f, *w.gamma, pass_))
                bt[b, hi, fi] = (np.float32(w.beta[0]) if w.beta[0] == w.beta[1] else
                                 uniform_value(w.seed, TID_BETA, b, h, f, *w.beta, pass_))
    return g, bt


def qkv_cpu(w: Workload, heads=None, frames=None, pass_=0):
    """Q, K, V for the selected heads/frames: [B, nh, nf*S, D] as fp32 values
    (already rounded through bf16 for bf16 workloads) plus the raw storage arrays
    (fp32, or uint16 bf16 bits)."""
    heads = range(w.H) if heads is None else list(heads)
    frames = range(w.F) if frames is None else list(frames)
    out_vals, out_raw = [], []
    for tid in (TID_Q, TID_K, TID_V):
        relu = w.relu_qk and tid in (TID_Q, TID_K)
        raw = np.empty((w.B, len(heads), len(frames) * w.S, w.D),
                       np.float32 if w.dtype == "f32" else np.uint16)
        for b in range(w.B):
            for hi, h in enumerate(heads):
                for fi, f in enumerate(frames):
                    z = normal_slice(w.seed, tid, b, h, f, w.S, w.D, pass_, relu)
                    raw[b, hi, fi * w.S:(fi + 1) * w.S] = (z if w.dtype == "f32"
                                                           else f32_to_bf16_bits(z))
        vals = raw if w.dtype == "f32" else bf16_bits_to_f32(raw)
        out_vals.append(vals)
        out_raw.append(raw)
    return out_vals, out_raw


@dataclasses.dataclass(frozen=True)
class TconvWorkload:
    """Block-causal temporal convolution at the GDN block's width: x [B, T, S, C] ~ N(0, 1),
    taps [C, 3] ~ N(0, 1/3), bias [C] ~ N(0, 0.1^2) (synthetic weights)."""
    name: str
    seed: int
    B: int
    T: int
    S: int
    C: int
    block_frames: int
    dtype: str


TCONV_WORKLOADS = {
    w.name: w for w in [
        # the 720p 60 s video at the width H*D = 16*128 of the GDN block, one block per latent
        # frame (frame-wise generation)
        TconvWorkload("tconv_720p_60s_bf16", 6, 1, 961, 3520, 2048, 1, "bf16"),
    ]
}
TID_TCONV_X, TID_TCONV_W = 7, 8


def tconv_weights(w: TconvWorkload):
    """taps [C, 3] and bias [C], fp32, from the counter-based normal generator."""
    z = normal_slice(w.seed, TID_TCONV_W, 0, 0, 0, 4, w.C)   # [4, C]
    taps = (z[:3].T / np.sqrt(3.0)).astype(np.float32)
    bias = (0.1 * z[3]).astype(np.float32)
    return np.ascontiguousarray(taps), bias


def tconv_x_cpu(w: TconvWorkload, frames=None, batches=None):
    """x values [nb, nf, S, C] fp32 (bf16-rounded for bf16) for the selected frames."""
    frames = range(w.T) if frames is None else list(frames)
    batches = range(w.B) if batches is None else list(batches)
    out = np.empty((len(batches), len(frames), w.S, w.C), np.float32)
    for bi, b in enumerate(batches):
        for fi, f in enumerate(frames):
            z = normal_slice(w.seed, TID_TCONV_X, b, 0, f, w.S, w.C)
            out[bi, fi] = z if w.dtype == "f32" else bf16_bits_to_f32(f32_to_bf16_bits(z))
    return out


def e4m3_codes(x, S, D):
    """Quantise frames of fp32 values to E4M3 with one power-of-two scale per frame.

    x: torch float32 [nf*S, D] (host or device). Returns (codes uint8 [nf*S, D], scales
    float32 [nf]) on x's device."""
    import torch
    nf = x.shape[0] // S
    xf = x.reshape(nf, S * D)
    _, e = torch.frexp(xf.abs().amax(dim=1))
    e = e.to(torch.int32)
    # 2**(E - 8) and its inverse built from their bit patterns (exact, no libm)
    scale = ((e - 8 + 127) << 23).view(torch.float32)
    inv = ((8 - e + 127) << 23).view(torch.float32)
    codes = (xf * inv[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(nf * S, D), scale


def qkv_fp8_cpu(w: Workload, heads=None, frames=None, pass_=0):
    """E4M3 Q, K, V for the selected heads/frames: codes uint8 [B, nh, nf*S, D] and scales
    float32 [B, nh, nf], for each of Q, K, V (lists of three)."""
    import torch
    heads = range(w.H) if heads is None else list(heads)
    frames = range(w.F) if frames is None else list(frames)
    codes, scales = [], []
    for tid in (TID_Q, TID_K, TID_V):
        c = np.empty((w.B, len(heads), len(frames) * w.S, w.D), np.uint8)
        sc = np.empty((w.B, len(heads), len(frames)), np.float32)
        for b in range(w.B):
            for hi, h in enumerate(heads):
                for fi, f in enumerate(frames):
                    z = torch.from_numpy(normal_slice(w.seed, tid, b, h, f, w.S, w.D, pass_))
                    cc, ss = e4m3_codes(z, w.S, w.D)
                    c[b, hi, fi * w.S:(fi + 1) * w.S] = cc.numpy()
                    sc[b, hi, fi] = ss.numpy()[0]
        codes.append(c)
        scales.append(sc)
    return codes, scales


# --------------------------------------------------------------------------- device (torch)
class TorchGen:
    """Device-side twin of the host generator (torch int64 arithmetic, exact)."""

    def __init__(self, device):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.table = torch.from_numpy(normal_table()).to(self.device)
        self._eh = {}

    @staticmethod
    def _mul32(x, c):
        lo, hi = c & 0xFFFF, c >> 16
        return (x * lo + (((x * hi) & 0xFFFF) << 16)) & M32

    def hash32(self, x):
        x = x ^ (x >> 16)
        x = self._mul32(x, 0x7FEB352D)
        x = x ^ (x >> 15)
        x = self._mul32(x, 0x846CA68B)
        return x ^ (x >> 16)

    def elem_hash(self, n):
        t = self._eh.get(n)
        if t is None:
            t = self.hash32(self.torch.arange(n, dtype=self.torch.int64, device=self.device))
            self._eh[n] = t
        return t

    def fill_normal(self, dst, seed, tid, b, h, f0, S, D, pass_=0, relu=False, chunk=32):
        """Write frames f0 .. f0 + nf - 1 of slice (tid, b, h) into dst, a [nf*S, D] view
        (any strides) of dtype float32 or bfloat16."""
        torch = self.torch
        nf = dst.shape[0] // S
        eh = self.elem_hash(S * D)
        for c0 in range(0, nf, chunk):
            c1 = min(nf, c0 + chunk)
            keys = torch.tensor([slice_key(seed, tid, b, h, f0 + f, pass_) for f in range(c0, c1)],
                                dtype=torch.int64, device=self.device)
            w = self.hash32(eh[None, :] ^ keys[:, None])
            z = self.table[w >> (32 - NLEVELS_BITS)]
            if relu:
                z = torch.clamp_min(z, 0.0)
            dst[c0 * S:c1 * S].copy_(z.view((c1 - c0) * S, D).to(dst.dtype))
            del w, z


    def fill_e4m3(self, codes, scales, seed, tid, b, h, f0, S, D, pass_=0, chunk=32):
        """Write E4M3 codes of frames f0 .. f0 + nf - 1 of slice (tid, b, h) into codes, a
        [nf*S, D] uint8 view, and their scales into scales, a [nf] float32 view."""
        torch = self.torch
        nf = codes.shape[0] // S
        eh = self.elem_hash(S * D)
        for c0 in range(0, nf, chunk):
            c1 = min(nf, c0 + chunk)
            keys = torch.tensor([slice_key(seed, tid, b, h, f0 + f, pass_) for f in range(c0, c1)],
                                dtype=torch.int64, device=self.device)
            wd = self.hash32(eh[None, :] ^ keys[:, None])
            z = self.table[wd >> (32 - NLEVELS_BITS)].view((c1 - c0) * S, D)
            cc, ss = e4m3_codes(z, S, D)
            codes[c0 * S:c1 * S].copy_(cc)
            scales[c0:c1].copy_(ss)
            del wd, z, cc, ss


def tconv_x_torch(w: TconvWorkload, device, gen=None):
    """x [B, T, S, C] on the device (the same values as tconv_x_cpu)."""
    import torch
    gen = gen or TorchGen(device)
    x = torch.empty((w.B, w.T, w.S, w.C), dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                    device=device)
    for b in range(w.B):
        gen.fill_normal(x[b].view(w.T * w.S, w.C), w.seed, TID_TCONV_X, b, 0, 0, w.S, w.C)
    return x


def gates_torch(w: Workload, device, pass_=0):
    """gamma, beta [B, H, F] fp32 on the device (made on the host: they are tiny)."""
    import torch
    g, bt = gates_cpu(w, pass_=pass_)
    return torch.from_numpy(g).to(device), torch.from_numpy(bt).to(device)


def qkv_fp8_torch(w: Workload, device, layout="head", frames=None, pass_=0, gen=None):
    """E4M3 Q, K, V on the device: ([q, k, v] uint8 codes [B, H, T, D] (layout as qkv_torch),
    [q_scale, k_scale, v_scale] float32 [B, H, nf])."""
    import torch
    f0, nf = (0, w.F) if frames is None else frames
    gen = gen or TorchGen(device)
    T = nf * w.S
    codes, scales = [], []
    for tid in (TID_Q, TID_K, TID_V):
        if layout == "head":
            x = torch.empty((w.B, w.H, T, w.D), dtype=torch.uint8, device=device)
        else:
            x = torch.empty((w.B, T, w.H, w.D), dtype=torch.uint8, device=device).permute(0, 2, 1, 3)
        sc = torch.empty((w.B, w.H, nf), dtype=torch.float32, device=device)
        for b in range(w.B):
            for h in range(w.H):
                gen.fill_e4m3(x[b, h], sc[b, h], w.seed, tid, b, h, f0, w.S, w.D, pass_)
        codes.append(x)
        scales.append(sc)
    return codes, scales


def qkv_torch(w: Workload, device, layout="head", frames=None, pass_=0, gen=None):
    """Allocate and fill Q, K, V on the device.

    layout "head": [B, H, T, D] contiguous; layout "token": storage [B, T, H, D] returned as a
    [B, H, T, D] view (token-major). T = nf * S for frames f0 .. f0 + nf - 1.
    """
    import torch
    f0, nf = (0, w.F) if frames is None else frames
    gen = gen or TorchGen(device)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    T = nf * w.S
    out = []
    for tid in (TID_Q, TID_K, TID_V):
        if layout == "head":
            x = torch.empty((w.B, w.H, T, w.D), dtype=dt, device=device)
        else:
            x = torch.empty((w.B, T, w.H, w.D), dtype=dt, device=device).permute(0, 2, 1, 3)
        relu = w.relu_qk and tid in (TID_Q, TID_K)
        for b in range(w.B):
            for h in range(w.H):
                gen.fill_normal(x[b, h], w.seed, tid, b, h, f0, w.S, w.D, pass_, relu)
        out.append(x)
    return out
