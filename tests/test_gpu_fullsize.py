"""Full-size workloads on the GPU, in the launch configuration bench.py times, checked against
the oracle on sampled heads and frames (early frames through the C oracle, every frame of one
head through the frame-streaming oracle variant).

Tolerance: max|d| / max|ref| <= 1e-2 (bf16 inputs, fp32 state), per compared slice.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import gdn_synth  # noqa: E402
import oracle  # noqa: E402
from gpu_util import TOL, HostFrames, rel_err, to_np  # noqa: E402
from oracle import stream  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_gdn_720p_60s_full_launch():
    w = gdn_synth.WORKLOADS["gdn_720p_60s_bf16"]
    S = w.S
    say("720p 60 s workload: generating inputs on the device")
    q, k, v = gdn_synth.qkv_torch(w, DEV)
    g, b = gdn_synth.gates_torch(w, DEV)
    o, st = gdn.forward_framewise(q, k, v, g, b)
    o2, st2 = gdn.forward_framewise(q, k, v, g, b)
    torch.cuda.synchronize()
    del q, k, v
    say("  forward done; checking properties")
    assert torch.isfinite(st).all()
    assert torch.equal(o, o2) and torch.equal(st, st2), "not bitwise reproducible"
    del o2
    for h in range(w.H):
        assert torch.isfinite(o[0, h]).all(), "non-finite output in head %d" % h

    say("  C oracle: head 12, frames 0-3")
    (qc, kc, vc), _ = gdn_synth.qkv_cpu(w, heads=[12], frames=range(4))
    gc, bc = gdn_synth.gates_cpu(w, heads=[12], frames=range(4))
    ro, _ = oracle.forward(qc, kc, vc, gc, bc)
    e = rel_err(to_np(o[:, 12:13, :4 * S]), ro)
    say("  frames 0-3 err %.3e" % e)
    assert e <= TOL["bf16"]

    say("  streaming oracle: head 5, all %d frames" % w.F)
    keep = {0, 1, 480, w.F - 1}
    src = HostFrames(w, 0, 5, w.F)
    try:
        outs, M = stream.forward_frames(src, w.F, w.D, S, keep=keep)
    finally:
        src.close()
    for f in sorted(keep):
        e = rel_err(to_np(o[0, 5, f * S:(f + 1) * S]), outs[f])
        say("  frame %d err %.3e" % (f, e))
        assert e <= TOL["bf16"]
    e = rel_err(to_np(st[0, 5]), M)
    say("  final state err %.3e" % e)
    assert e <= TOL["bf16"]


def test_stream_720p_full_protocol():
    w = gdn_synth.WORKLOADS["stream_720p_bf16"]
    S, P = w.S, w.passes
    say("streaming workload: %d frames x %d passes, generating inputs" % (w.F, P))
    gen = gdn_synth.TorchGen(DEV)
    passes = []
    for p in range(P):
        q, k, v = gdn_synth.qkv_torch(w, DEV, pass_=p, gen=gen)
        g, b = gdn_synth.gates_torch(w, DEV, pass_=p)
        passes.append((q, k, v, g.permute(2, 0, 1).contiguous(), b.permute(2, 0, 1).contiguous()))
    state = torch.zeros((w.B, w.H, w.D, w.D), dtype=torch.float32, device=DEV)
    keep = {0, 1, w.F - 1}
    kept_o, kept_s = {}, {}
    for f in range(w.F):
        sl = slice(f * S, (f + 1) * S)
        for p in range(P):
            q, k, v, g, b = passes[p]
            last = p == P - 1
            o, _ = gdn.step_frame(q[:, :, sl], k[:, :, sl], v[:, :, sl], g[f], b[f], state,
                                  commit=last, state_out=state if last else None)
            if f in keep:
                kept_o[(f, p)] = o.clone()
        if f in keep:
            kept_s[f] = state.clone()
    torch.cuda.synchronize()
    say("  GPU protocol done")
    assert torch.isfinite(state).all()

    heads = [3, 14]
    say("  C oracle: heads %s, frames 0-1, every pass" % heads)
    M = np.zeros((w.B, len(heads), w.D, w.D))
    for f in (0, 1):
        for p in range(P):
            (qc, kc, vc), _ = gdn_synth.qkv_cpu(w, heads=heads, frames=[f], pass_=p)
            gc, bc = gdn_synth.gates_cpu(w, heads=heads, frames=[f], pass_=p)
            ro, rs = oracle.step(qc, kc, vc, gc[..., 0], bc[..., 0], M, commit=(p == P - 1))
            e = rel_err(to_np(kept_o[(f, p)][:, heads]), ro)
            assert e <= TOL["bf16"], "frame %d pass %d err %.3e" % (f, p, e)
        M = rs
        e = rel_err(to_np(kept_s[f][:, heads]), M)
        say("  frame %d committed state err %.3e" % (f, e))
        assert e <= TOL["bf16"]

    say("  streaming oracle: head 3, all %d frames x %d passes" % (w.F, P))
    src = HostFrames(w, 0, 3, w.F * P, pass_of=lambda i: i % P, frame_of=lambda i: i // P)
    try:
        M = np.zeros((w.D, w.D))
        for f in range(w.F):
            for p in range(P):
                outs, Mn = stream.forward_frames(lambda _f, i=f * P + p: src(i), 1, w.D, S,
                                                 state_in=M)
                if f == w.F - 1:
                    e = rel_err(to_np(kept_o[(f, p)][0, 3]), outs[0])
                    say("  last frame pass %d err %.3e" % (p, e))
                    assert e <= TOL["bf16"]
            M = Mn  # the last pass commits
    finally:
        src.close()
    e = rel_err(to_np(kept_s[w.F - 1][0, 3]), M)
    say("  final committed state err %.3e" % e)
    assert e <= TOL["bf16"]
