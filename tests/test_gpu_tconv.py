"""Block-causal temporal convolution on the GPU (gdn_tconv_forward through the C ABI) against
the oracle (oracle/tconv.py).

Tolerance: max|d| / max|ref| <= 1e-2 for bf16 (output rounding), 1e-5 for fp32.
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import gdn_synth  # noqa: E402
from gpu_util import rel_err  # noqa: E402
from oracle import tconv  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"bf16": 1e-2, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rounded(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make(B, T, S, C, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rounded(rng.standard_normal((B, T, S, C)), dtype)
    cache = rounded(rng.standard_normal((B, S, C)), dtype)
    w = (rng.standard_normal((C, 3)) / np.sqrt(3)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return x, cache, w, bias


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


CASES = [
    # B, T, S, C, block_frames, dtype, cache, bias, layout
    (2, 6, 5, 16, 2, "bf16", True, True, "btsc"),
    (1, 37, 3, 64, 1, "f32", False, True, "btsc"),     # several 16-frame chunks, ragged
    (1, 40, 7, 24, 5, "bf16", True, False, "btsc"),
    (2, 17, 4, 32, 17, "f32", True, True, "bstc"),      # one block; frames not outermost
    (1, 3, 2, 8, 3, "bf16", False, False, "btsc"),
    (1, 48, 6, 2048, 3, "bf16", True, True, "bstc"),    # the GDN block's width
    (2, 1, 7, 64, 1, "bf16", True, True, "btsc"),       # one frame (the streaming call)
    (1, 1, 5, 24, 1, "f32", False, False, "bstc"),      # one frame, no cache: positions ragged
    (3, 1, 3, 2048, 1, "bf16", True, False, "bstc"),
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_tconv_matches_oracle(case):
    B, T, S, C, tb, dtype, with_cache, with_bias, layout = case
    say("tconv", case)
    x, cache, w, bias = make(B, T, S, C, dtype, zlib.crc32(repr(case).encode()) & 0xFFFF)
    xd = x.to(DEV) if layout == "btsc" else x.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    cd = cache.to(DEV) if with_cache else None
    wd = torch.from_numpy(w).to(DEV)
    bd = torch.from_numpy(bias).to(DEV) if with_bias else None
    y, c_out = gdn.temporal_conv(xd, wd, bd, cd, block_frames=tb)
    torch.cuda.synchronize()
    ry, rc = tconv.tconv_sequence(f64(x), w, bias if with_bias else None, tb,
                                  f64(cache) if with_cache else None)
    e = rel_err(f64(y), ry)
    say("  y err %.2e" % e)
    assert e <= TOL[dtype]
    assert np.array_equal(f64(c_out), rc), "cache_out must be the last frame, bit for bit"


def test_tconv_streaming_in_place_cache():
    """Block by block from the previous call's cache, cache updated in place; equals the whole
    sequence in one call bit for bit, and the oracle's streaming form."""
    B, T, S, C, tb = 1, 12, 5, 64, 3
    x, cache, w, bias = make(B, T, S, C, "bf16", 7)
    xd, wd, bd = x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(bias).to(DEV)
    whole, _ = gdn.temporal_conv(xd, wd, bd, cache.to(DEV), block_frames=tb)
    c = cache.to(DEV).clone()
    parts = []
    for i in range(T // tb):
        y, _ = gdn.temporal_conv(xd[:, i * tb:(i + 1) * tb], wd, bd, c, block_frames=tb, cache_out=c)
        parts.append(y)
    torch.cuda.synchronize()
    streamed = torch.cat(parts, dim=1)
    assert torch.equal(streamed, whole)
    assert torch.equal(c, xd[:, -1])
    ry, _ = tconv.tconv_stream(f64(x), w, bias, tb, f64(cache))
    assert rel_err(f64(streamed), ry) <= TOL["bf16"]


def test_tconv_one_frame_stream_in_place_cache():
    """One frame per call (the streaming step), cache updated in place: equals the whole sequence
    in one call bit for bit."""
    B, T, S, C = 2, 6, 9, 64
    x, cache, w, bias = make(B, T, S, C, "bf16", 11)
    xd, wd, bd = x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(bias).to(DEV)
    whole, _ = gdn.temporal_conv(xd, wd, bd, cache.to(DEV), block_frames=1)
    c = cache.to(DEV).clone()
    parts = []
    for t in range(T):
        y, _ = gdn.temporal_conv(xd[:, t:t + 1], wd, bd, c, block_frames=1, cache_out=c)
        parts.append(y)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=1), whole)
    assert torch.equal(c, xd[:, -1])


def test_tconv_prepared_calls_stream_like_the_binding():
    """prepare_temporal_conv per frame (arguments marshalled once), cache updated in place:
    the frames equal the whole sequence in one call bit for bit."""
    B, T, S, C = 1, 5, 12, 128
    x, cache, w, bias = make(B, T, S, C, "bf16", 21)
    xd, wd, bd = x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(bias).to(DEV)
    whole, _ = gdn.temporal_conv(xd, wd, bd, cache.to(DEV), block_frames=1)
    c = cache.to(DEV).clone()
    outs = [torch.empty_like(xd[:, :1]) for _ in range(T)]
    calls = [gdn.prepare_temporal_conv(xd[:, t:t + 1], wd, bd, c, block_frames=1, out=outs[t], cache_out=c)
             for t in range(T)]
    for t in range(T):
        y, cc = calls[t]()
        assert y is outs[t] and cc is c
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), whole)
    assert torch.equal(c, xd[:, -1])


def test_tconv_deterministic():
    x, cache, w, bias = make(1, 33, 4, 128, "bf16", 9)
    args = (x.to(DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(bias).to(DEV), cache.to(DEV))
    y1, _ = gdn.temporal_conv(*args, block_frames=1)
    y2, _ = gdn.temporal_conv(*args, block_frames=1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_tconv_720p_full_launch():
    """The whole 961-frame video at the GDN width, as bench.py times it; oracle on sampled frames
    (each from its left neighbour: one block per frame) and the cache_out."""
    w = gdn_synth.TCONV_WORKLOADS["tconv_720p_60s_bf16"]
    say("tconv 720p: generating the input on the device")
    x = gdn_synth.tconv_x_torch(w, DEV)
    taps, bias = gdn_synth.tconv_weights(w)
    y, c_out = gdn.temporal_conv(x, torch.from_numpy(taps).to(DEV), torch.from_numpy(bias).to(DEV),
                                 block_frames=w.block_frames)
    torch.cuda.synchronize()
    for t in (0, 1, 480, w.T - 1):
        frames = [t] if t == 0 else [t - 1, t]
        xs = gdn_synth.tconv_x_cpu(w, frames=frames).astype(np.float64)
        cache = None if t == 0 else xs[:, 0]
        ry, _ = tconv.tconv_sequence(xs[:, -1:], taps, bias, 1, cache)
        e = rel_err(f64(y[:, t:t + 1]), ry)
        say("  frame %d err %.2e" % (t, e))
        assert e <= TOL["bf16"]
    last = gdn_synth.tconv_x_cpu(w, frames=[w.T - 1])
    assert np.array_equal(f64(c_out), last[:, 0].astype(np.float64))
