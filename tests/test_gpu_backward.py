"""Backward (gradients) on the GPU, through the C ABI, against the fp64 backward oracle.

Tolerance: max|d| / max|ref| <= 1e-2 per gradient (bf16 data; the forward states and the state
gradients enter the per-frame products rounded to bf16).
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import gdn_synth  # noqa: E402
import oracle  # noqa: E402
from gpu_util import TOL, rel_err, random_qkv, to_dev, to_np  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ["dq", "dk", "dv", "dgamma", "dbeta", "dstate_in"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_round(x):
    return gdn_synth.bf16_bits_to_f32(gdn_synth.f32_to_bf16_bits(np.asarray(x, np.float32)))


def run_case(B, H, D, S, F, delta, with_state, with_dm, layout, seed, schedule="auto"):
    rng = np.random.default_rng(seed)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    d_o = bf16_round(rng.standard_normal((B, H, F * S, D)))
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32) if with_state else None
    dm = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32) if with_dm else None
    dev = [to_dev(x, "bf16", DEV, layout) for x in (q, k, v)]
    ddo = to_dev(d_o, "bf16", DEV, layout)
    tg, tb = torch.from_numpy(g).to(DEV), torch.from_numpy(b).to(DEV)
    ts0 = None if s0 is None else torch.from_numpy(s0).to(DEV)
    tdm = None if dm is None else torch.from_numpy(dm).to(DEV)
    got = gdn.backward_framewise(*dev, tg, tb, ddo, ts0, tdm, use_delta=delta, schedule=schedule)
    torch.cuda.synchronize()
    ref = oracle.backward(q, k, v, g, b, s0, d_o, dm, use_delta=delta)
    return got, ref


CASES = [
    # B, H, D, S, F, delta, initial state, dstate_out, layout
    (1, 2, 128, 200, 5, True, True, True, "head"),
    (1, 1, 64, 64, 7, True, False, False, "head"),
    (2, 2, 64, 130, 4, True, True, True, "token"),
    (1, 2, 128, 96, 6, False, True, True, "head"),
    (1, 3, 64, 33, 3, False, False, True, "head"),
    (1, 1, 128, 1, 9, True, True, True, "head"),      # one token per frame
    (1, 2, 128, 300, 1, True, True, False, "head"),   # one frame
    (1, 16, 128, 3520, 2, True, True, True, "head"),  # the 720p frame size
]


@pytest.mark.parametrize("schedule", ["staged", "fused"])
@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_backward_matches_oracle(case, schedule):
    """Both schedules of the reverse chain: a separate scan (staged) and the ticket-ordered chain
    inside the pass over Q and dO (fused)."""
    say("backward", schedule, case)
    got, ref = run_case(*case, seed=zlib.crc32(repr(case).encode()), schedule=schedule)
    errs = {}
    for name, x, r in zip(NAMES, got, ref):
        errs[name] = rel_err(to_np(x), r)
    say("  " + " ".join("%s %.2e" % kv for kv in errs.items()))
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_in_place_state_gradient_and_determinism():
    B, H, D, S, F = 1, 2, 128, 70, 5
    rng = np.random.default_rng(31)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    d_o = bf16_round(rng.standard_normal((B, H, F * S, D)))
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    dm = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV),
                                                          to_dev(d_o, "bf16", DEV)]
    tdm = torch.from_numpy(dm).to(DEV)
    r1 = gdn.backward_framewise(*args, None, tdm.clone())
    r2 = gdn.backward_framewise(*args, None, tdm.clone())
    # in place: the state gradient overwrites dstate_out
    lib = gdn.load()
    import ctypes
    p = gdn._problem(args[0], args[5], F, True, None)
    ws, nb = gdn._workspace(p, 2, None, args[0].device)
    outs = [torch.empty_like(args[0]) for _ in range(3)]
    dg = torch.empty((B, H, F), dtype=torch.float32, device=DEV)
    db = torch.empty((B, H, F), dtype=torch.float32, device=DEV)
    inplace = tdm.clone()
    code = lib.gdn_backward_framewise(
        ctypes.byref(p), *[ctypes.c_void_p(t.data_ptr()) for t in args[:5]], None,
        ctypes.c_void_p(args[5].data_ptr()), ctypes.c_void_p(inplace.data_ptr()),
        *[ctypes.c_void_p(t.data_ptr()) for t in outs], ctypes.c_void_p(dg.data_ptr()),
        ctypes.c_void_p(db.data_ptr()), ctypes.c_void_p(inplace.data_ptr()),
        ctypes.c_void_p(ws.data_ptr()), nb, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert code == 0
    for a, c in zip(r1, r2):
        assert torch.equal(a, c), "backward is not bitwise repeatable"
    assert torch.equal(inplace, r1[5])
    for a, c in zip(outs, r1[:3]):
        assert torch.equal(a, c)


def test_backward_880x81_sampled_heads():
    w = gdn_synth.WORKLOADS["gdn_880x81_bf16"]
    say("backward on the 880x81 workload, oracle on head 7 of batch 1")
    q, k, v = gdn_synth.qkv_torch(w, DEV)
    g, b = gdn_synth.gates_torch(w, DEV)
    gen = np.random.default_rng(41)
    d_o_np = bf16_round(gen.standard_normal((w.B, w.H, w.F * w.S, w.D)).astype(np.float32))
    d_o = torch.from_numpy(d_o_np).to(torch.bfloat16).to(DEV)
    got = gdn.backward_framewise(q, k, v, g, b, d_o)
    torch.cuda.synchronize()
    heads = [7]
    (qc, kc, vc), _ = gdn_synth.qkv_cpu(w, heads=heads)
    gc, bc = gdn_synth.gates_cpu(w, heads=heads)
    ref = oracle.backward(qc[1:2], kc[1:2], vc[1:2], gc[1:2], bc[1:2], None,
                          d_o_np[1:2, heads])
    errs = {}
    for name, x, r in zip(NAMES, got, ref):
        errs[name] = rel_err(to_np(x[1:2, heads]), r)
    say("  " + " ".join("%s %.2e" % kv for kv in errs.items()))
    assert max(errs.values()) <= TOL["bf16"], errs


SAVED_CASES = [
    # B, H, D, S, F, delta, initial state, dstate_out, layout
    (1, 2, 128, 200, 5, True, True, True, "head"),
    (2, 2, 64, 130, 4, True, True, True, "token"),
    (1, 2, 128, 96, 6, False, True, False, "head"),
    (1, 1, 128, 1, 9, True, False, True, "head"),     # one token per frame
    (1, 16, 128, 3520, 2, True, True, True, "head"),  # the 720p frame size
]


@pytest.mark.parametrize("schedule", ["staged", "fused"])
@pytest.mark.parametrize("case", SAVED_CASES, ids=["-".join(map(str, c)) for c in SAVED_CASES])
def test_backward_from_saved_forward(case, schedule):
    """forward_framewise_save gives the fused forward's outputs bitwise and keeps the states (slot
    0 = the initial state and slot F = the final state, transposed, bitwise); the backward from
    that buffer (either schedule of the reverse chain) matches the oracle and the recomputing
    backward."""
    say("backward from saved", schedule, case)
    B, H, D, S, F, delta, with_state, with_dm, layout = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + 1)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    d_o = bf16_round(rng.standard_normal((B, H, F * S, D)))
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32) if with_state else None
    dm = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32) if with_dm else None
    dev = [to_dev(x, "bf16", DEV, layout) for x in (q, k, v)]
    ddo = to_dev(d_o, "bf16", DEV, layout)
    tg, tb = torch.from_numpy(g).to(DEV), torch.from_numpy(b).to(DEV)
    ts0 = None if s0 is None else torch.from_numpy(s0).to(DEV)
    tdm = None if dm is None else torch.from_numpy(dm).to(DEV)
    o_f, st_f = gdn.forward_framewise(*dev, tg, tb, ts0, use_delta=delta, schedule="fused")
    o_s, st_s, saved = gdn.forward_framewise_save(*dev, tg, tb, ts0, use_delta=delta)
    got = gdn.backward_framewise(*dev, tg, tb, ddo, None, tdm, use_delta=delta, saved=saved, schedule=schedule)
    rec = gdn.backward_framewise(*dev, tg, tb, ddo, ts0, tdm, use_delta=delta, schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_s) and torch.equal(st_f, st_s)
    p = gdn.Problem(B, H, D, S, F, gdn.GDN_BF16, int(delta), 0.0, 0, 0, D, 0, 0, D)
    nst = B * H * (F + 1) * D * D
    states = saved[saved.numel() - 4 * nst:].view(torch.float32).view(B, H, F + 1, D, D)
    assert saved.numel() == gdn.saved_size(p)
    init = ts0 if ts0 is not None else torch.zeros((B, H, D, D), device=DEV)
    assert torch.equal(states[:, :, 0], init.transpose(2, 3))
    assert torch.equal(states[:, :, F], st_s.transpose(2, 3))
    ref = oracle.backward(q, k, v, g, b, s0, d_o, dm, use_delta=delta)
    errs = {n: rel_err(to_np(x), r) for n, x, r in zip(NAMES, got, ref)}
    agree = {n: rel_err(to_np(x), to_np(y)) for n, x, y in zip(NAMES, got, rec)}
    say("  oracle " + " ".join("%s %.2e" % kv for kv in errs.items()))
    say("  vs recomputing " + " ".join("%s %.2e" % kv for kv in agree.items()))
    assert max(errs.values()) <= TOL["bf16"], errs
    assert max(agree.values()) <= TOL["bf16"], agree
    if schedule == "fused":
        # the chained recompute runs the same fused forward (without outputs), so the two
        # backwards see the same states and agree bit for bit
        for n, x, y in zip(NAMES, got, rec):
            assert torch.equal(x, y), n


def test_backward_chain_deterministic_and_in_place():
    """The chained schedule: bitwise repeatable, and the state gradient may overwrite dstate_out."""
    B, H, D, S, F = 1, 3, 128, 150, 6
    rng = np.random.default_rng(53)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    d_o = bf16_round(rng.standard_normal((B, H, F * S, D)))
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    dm = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV),
                                                          to_dev(d_o, "bf16", DEV)]
    tdm = torch.from_numpy(dm).to(DEV)
    r1 = gdn.backward_framewise(*args, None, tdm.clone(), schedule="fused")
    r2 = gdn.backward_framewise(*args, None, tdm.clone(), schedule="fused")
    inplace = tdm.clone()
    r3 = gdn.backward_framewise(*args, None, inplace, schedule="fused", return_state_grad=False)
    torch.cuda.synchronize()
    for a, c in zip(r1, r2):
        assert torch.equal(a, c), "chained backward is not bitwise repeatable"
    for a, c in zip(r1[:5], r3[:5]):
        assert torch.equal(a, c)


def test_backward_chain_time_out_path(monkeypatch):
    """The chained schedule's bounded waits, forced from the host: with GDN_FUSED_SPIN_LIMIT=0
    every step after the first gives up at once, continues with NaN and still ends; the time-out
    flag at byte 4 of the workspace is set.
    From saved states only the reverse chain waits: the gradients that depend on G (dK, dV,
    dgamma, dbeta of every frame but the last, dstate_in) are NaN, dQ is finite.
    Recomputing, the fused forward that rebuilds the states times out as well: every state
    after frame 0 is NaN, so dQ is NaN past frame 0 (frame 0's state comes from the initial
    state without a wait) and so is the last frame's dK (it reads the state before it).
    Without the override the same calls are finite and the flag is clear."""
    B, H, D, S, F = 1, 2, 64, 64, 4
    rng = np.random.default_rng(59)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    d_o = bf16_round(rng.standard_normal((B, H, F * S, D)))
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV),
                                                          to_dev(d_o, "bf16", DEV)]
    p = gdn._problem(args[0], args[5], F, True, None, "fused")
    ws2 = torch.zeros(gdn.workspace_size(p, 2), dtype=torch.uint8, device=DEV)
    ws3 = torch.zeros(gdn.workspace_size(p, 3), dtype=torch.uint8, device=DEV)
    _, _, saved = gdn.forward_framewise_save(*args[:5])
    torch.cuda.synchronize()

    def flag(ws):
        return int(ws[4:8].view(torch.int32).item())

    monkeypatch.setenv("GDN_FUSED_SPIN_LIMIT", "0")
    bad_s = gdn.backward_framewise(*args, saved=saved, schedule="fused", workspace=ws3)
    torch.cuda.synchronize()
    flag_s = flag(ws3)
    bad_r = gdn.backward_framewise(*args, schedule="fused", workspace=ws2)
    torch.cuda.synchronize()
    flag_r = flag(ws2)
    for mode, ws in ((3, ws3), (2, ws2)):
        with pytest.raises(gdn.GdnError) as ei:   # the C ABI reports the flag
            gdn.check_timeout(p, mode, ws)
        assert ei.value.code == 9
    with pytest.raises(gdn.GdnError) as ei:       # the binding checks its own workspace
        gdn.backward_framewise(*args, saved=saved, schedule="fused")
    assert ei.value.code == 9
    monkeypatch.delenv("GDN_FUSED_SPIN_LIMIT")
    good = gdn.backward_framewise(*args, schedule="fused", workspace=ws2)
    torch.cuda.synchronize()
    assert flag_s == 1 and flag_r == 1
    assert flag(ws2) == 0
    gdn.check_timeout(p, 2, ws2)
    last, early = slice((F - 1) * S, F * S), slice(0, (F - 1) * S)
    for dq, dk, dv, dg, db, dsi in (bad_s, bad_r):
        assert torch.isfinite(dv[:, :, last].float()).all()   # G of the last frame needs no wait
        assert torch.isnan(dk[:, :, early].float()).all() and torch.isnan(dv[:, :, early].float()).all()
        assert torch.isnan(dg[:, :, :F - 1]).all() and torch.isnan(db[:, :, :F - 1]).all()
        assert torch.isnan(dsi).all()
    assert torch.isfinite(bad_s[1][:, :, last].float()).all()   # saved M_{F-2} is finite
    assert torch.isnan(bad_r[1][:, :, last].float()).all()      # recomputed M_{F-2} is NaN
    assert torch.isfinite(bad_s[0].float()).all()
    assert torch.isfinite(bad_r[0][:, :, :S].float()).all()
    assert torch.isnan(bad_r[0][:, :, S:].float()).all()
    for t in good:
        assert torch.isfinite(t.float()).all()
