"""Full-size workloads on the GPU, in the launch configuration bench.py times, checked against
the oracle on every head: each head's final state and its outputs at sampled frames (the
frame-streaming oracle variant over the whole sequence), plus the first frames of one head
through the C oracle from host-generated inputs.

The full-sequence comparisons take the inputs the device generated (gdn_synth's torch
generator, bit-identical to its host generator: test_generator_device_matches_host), copied to
the host per head; no value comes from the library.

Tolerance: max|d| / max|ref| <= 1e-2 (bf16 inputs, fp32 state), per compared slice.
"""
import os
import sys
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import gdn_synth  # noqa: E402
import oracle  # noqa: E402
from gpu_util import TOL, rel_err, to_np  # noqa: E402
from oracle import stream  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# oracle heads in flight (host threads, BLAS single-threaded in each), within the host's share
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_bits(t):
    """bf16 device tensor -> uint16 numpy array of its bits (host copy)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(bits):
    return gdn_synth.bf16_bits_to_f32(bits)


def run_heads(jobs, work):
    """Run work(*job) for each job on a thread pool; at most WORKERS jobs hold their inputs at
    once. Returns the results in job order.

    BLAS is limited to one thread once, around the whole pool: its threaded kernels are not
    reentrant, and a limit entered and left per worker would let one worker's exit restore the
    threaded mode while others are inside a product."""
    from threadpoolctl import threadpool_limits
    gate = threading.Semaphore(WORKERS)

    def one(job):
        try:
            return work(*job())
        finally:
            gate.release()

    futs = []
    with threadpool_limits(1), ThreadPoolExecutor(WORKERS) as pool:
        for job in jobs:
            gate.acquire()
            futs.append(pool.submit(one, job))
        return [f.result() for f in futs]


@pytest.mark.timeout(1200)
def test_gdn_720p_60s_full_launch():
    w = gdn_synth.WORKLOADS["gdn_720p_60s_bf16"]
    S, F, D = w.S, w.F, w.D
    say("720p 60 s workload: generating inputs on the device")
    q, k, v = gdn_synth.qkv_torch(w, DEV)
    g, b = gdn_synth.gates_torch(w, DEV)
    o, st = gdn.forward_framewise(q, k, v, g, b)
    o2, st2 = gdn.forward_framewise(q, k, v, g, b)
    torch.cuda.synchronize()
    say("  forward done; checking properties")
    assert torch.isfinite(st).all()
    assert torch.equal(o, o2) and torch.equal(st, st2), "not bitwise reproducible"
    del o2, st2
    for h in range(w.H):
        assert torch.isfinite(o[0, h]).all(), "non-finite output in head %d" % h

    say("  C oracle: head 12, frames 0-3, from host-generated inputs")
    (qc, kc, vc), _ = gdn_synth.qkv_cpu(w, heads=[12], frames=range(4))
    gc, bc = gdn_synth.gates_cpu(w, heads=[12], frames=range(4))
    ro, _ = oracle.forward(qc, kc, vc, gc, bc)
    e = rel_err(to_np(o[:, 12:13, :4 * S]), ro)
    say("  frames 0-3 err %.3e" % e)
    assert e <= TOL["bf16"]

    keep = (0, 1, 480, F - 1)
    gh, bh = gdn_synth.gates_cpu(w)
    say("  streaming oracle: every head, all %d frames; outputs at frames %s" % (F, keep))

    def job(h):
        def fetch():
            kb, vb = host_bits(k[0, h]), host_bits(v[0, h])
            qk = {f: f32(host_bits(q[0, h, f * S:(f + 1) * S])) for f in keep}
            return h, kb, vb, qk
        return fetch

    def work(h, kb, vb, qk):
        def src(f):
            kf = f32(kb[f * S:(f + 1) * S])
            return qk.get(f, kf), kf, f32(vb[f * S:(f + 1) * S]), gh[0, h, f], bh[0, h, f]
        return stream.forward_frames(src, F, D, S, keep=set(keep))

    res = run_heads([job(h) for h in range(w.H)], work)
    worst_o = worst_s = 0.0
    for h, (outs, M) in enumerate(res):
        for f in keep:
            e = rel_err(to_np(o[0, h, f * S:(f + 1) * S]), outs[f])
            worst_o = max(worst_o, e)
            assert e <= TOL["bf16"], "head %d frame %d err %.3e" % (h, f, e)
        e = rel_err(to_np(st[0, h]), M)
        worst_s = max(worst_s, e)
        assert e <= TOL["bf16"], "head %d final state err %.3e" % (h, e)
    say("  all %d heads: worst output err %.3e, worst final state err %.3e" % (w.H, worst_o, worst_s))


@pytest.mark.timeout(1200)
def test_stream_720p_full_protocol():
    w = gdn_synth.WORKLOADS["stream_720p_bf16"]
    S, P, D, F = w.S, w.passes, w.D, w.F
    say("streaming workload: %d frames x %d passes, generating inputs" % (F, P))
    gen = gdn_synth.TorchGen(DEV)
    passes = []
    for p in range(P):
        q, k, v = gdn_synth.qkv_torch(w, DEV, pass_=p, gen=gen)
        g, b = gdn_synth.gates_torch(w, DEV, pass_=p)
        passes.append((q, k, v, g.permute(2, 0, 1).contiguous(), b.permute(2, 0, 1).contiguous()))
    state = torch.zeros((w.B, w.H, D, D), dtype=torch.float32, device=DEV)
    keep = {0, 1, F - 1}
    kept_o, kept_s = {}, {}
    for f in range(F):
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
    say("  C oracle: heads %s, frames 0-1, every pass, from host-generated inputs" % heads)
    M = np.zeros((w.B, len(heads), D, D))
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

    gates = [gdn_synth.gates_cpu(w, pass_=p) for p in range(P)]
    say("  streaming oracle: every head, all %d frames x %d passes" % (F, P))

    def job(h):
        def fetch():
            kb = [host_bits(passes[p][1][0, h]) for p in range(P)]
            vb = [host_bits(passes[p][2][0, h]) for p in range(P)]
            ql = [f32(host_bits(passes[p][0][0, h, (F - 1) * S:])) for p in range(P)]
            return h, kb, vb, ql
        return fetch

    def work(h, kb, vb, ql):
        M = np.zeros((D, D))
        last_o = []
        for f in range(F):
            sl = slice(f * S, (f + 1) * S)
            for p in range(P):
                kf, vf = f32(kb[p][sl]), f32(vb[p][sl])
                qf = ql[p] if f == F - 1 else kf
                gf, bf = gates[p][0][0, h, f], gates[p][1][0, h, f]
                outs, Mn = stream.forward_frames(lambda _f: (qf, kf, vf, gf, bf), 1, D, S,
                                                 state_in=M, keep={0} if f == F - 1 else set())
                if f == F - 1:
                    last_o.append(outs[0])
            M = Mn   # the last pass commits
        return last_o, M

    res = run_heads([job(h) for h in range(w.H)], work)
    worst_o = worst_s = 0.0
    for h, (last_o, M) in enumerate(res):
        for p in range(P):
            e = rel_err(to_np(kept_o[(F - 1, p)][0, h]), last_o[p])
            worst_o = max(worst_o, e)
            assert e <= TOL["bf16"], "head %d last frame pass %d err %.3e" % (h, p, e)
        e = rel_err(to_np(kept_s[F - 1][0, h]), M)
        worst_s = max(worst_s, e)
        assert e <= TOL["bf16"], "head %d final committed state err %.3e" % (h, e)
    say("  all %d heads: worst last-frame output err %.3e, worst final state err %.3e"
        % (w.H, worst_o, worst_s))
