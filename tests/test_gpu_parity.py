"""GPU path (through the C ABI) against the CPU oracle, element by element.

Tolerance: max|d| / max|ref| <= 1e-4 for fp32 inputs, <= 1e-2 for bf16 inputs (fp32 state).
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import gdn_synth  # noqa: E402
import oracle  # noqa: E402
from gpu_util import TOL, HipEvents, rel_err, random_qkv, to_dev, to_np  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# --------------------------------------------------------------------------- generator
def test_generator_device_matches_host():
    w = gdn_synth.WORKLOADS["gdn_720p_60s_bf16"]
    gen = gdn_synth.TorchGen(DEV)
    dst = torch.empty((2 * w.S, w.D), dtype=torch.bfloat16, device=DEV)
    gen.fill_normal(dst, w.seed, gdn_synth.TID_K, 0, 5, 100, w.S, w.D)
    host = np.concatenate([gdn_synth.f32_to_bf16_bits(
        gdn_synth.normal_slice(w.seed, gdn_synth.TID_K, 0, 5, f, w.S, w.D)) for f in (100, 101)])
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, host)


# --------------------------------------------------------------------------- workloads
def run_workload_forward(w, layout="head", schedule="auto"):
    q, k, v = gdn_synth.qkv_torch(w, DEV, layout=layout)
    g, b = gdn_synth.gates_torch(w, DEV)
    o, st = gdn.forward_framewise(q, k, v, g, b, use_delta=w.use_delta, schedule=schedule)
    torch.cuda.synchronize()
    return o, st


@pytest.mark.parametrize("layout", ["head", "token"])
def test_tiny_f32_full(layout):
    w = gdn_synth.WORKLOADS["tiny_f32"]
    say("tiny_f32 layout", layout)
    o, st = run_workload_forward(w, layout)
    (qc, kc, vc), _ = gdn_synth.qkv_cpu(w)
    gc, bc = gdn_synth.gates_cpu(w)
    ro, rs = oracle.forward(qc, kc, vc, gc, bc)
    assert rel_err(to_np(o), ro) <= TOL["f32"]
    assert rel_err(to_np(st), rs) <= TOL["f32"]


@pytest.mark.parametrize("schedule", ["staged", "fused"])
def test_block_causal_bf16_full(schedule):
    w = gdn_synth.WORKLOADS["block_causal_bf16"]
    say("block_causal_bf16 full", schedule)
    o, st = run_workload_forward(w, schedule=schedule)
    (qc, kc, vc), _ = gdn_synth.qkv_cpu(w)
    gc, bc = gdn_synth.gates_cpu(w)
    ro, rs = oracle.forward(qc, kc, vc, gc, bc, use_delta=False)
    e1, e2 = rel_err(to_np(o), ro), rel_err(to_np(st), rs)
    say("  O err %.3e state err %.3e" % (e1, e2))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


@pytest.mark.parametrize("schedule", ["staged", "fused"])
def test_gdn_880x81_bf16_sampled_heads(schedule):
    w = gdn_synth.WORKLOADS["gdn_880x81_bf16"]
    say("gdn_880x81_bf16 full launch, oracle on heads 0 and 15,", schedule)
    o, st = run_workload_forward(w, schedule=schedule)
    heads = [0, 15]
    (qc, kc, vc), _ = gdn_synth.qkv_cpu(w, heads=heads)
    gc, bc = gdn_synth.gates_cpu(w, heads=heads)
    ro, rs = oracle.forward(qc, kc, vc, gc, bc)
    e1 = rel_err(to_np(o[:, heads]), ro)
    e2 = rel_err(to_np(st[:, heads]), rs)
    say("  O err %.3e state err %.3e" % (e1, e2))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


# --------------------------------------------------------------------------- shape sweep
SWEEP = [
    # B, H, D, S, F, dtype, delta, layout
    (1, 1, 16, 1, 1, "f32", True, "head"),
    (1, 2, 16, 17, 3, "f32", True, "token"),
    (2, 1, 32, 100, 2, "f32", True, "head"),
    (1, 3, 64, 65, 3, "f32", False, "head"),
    (1, 1, 128, 33, 2, "f32", True, "head"),
    (1, 1, 16, 5, 4, "bf16", True, "head"),
    (1, 2, 32, 64, 3, "bf16", True, "token"),
    (2, 3, 64, 130, 4, "bf16", True, "head"),
    (1, 2, 64, 77, 5, "bf16", False, "token"),
    (1, 2, 128, 1, 6, "bf16", True, "head"),
    (1, 9, 128, 200, 3, "bf16", True, "head"),
    (1, 2, 128, 1000, 2, "bf16", False, "head"),
]


@pytest.mark.parametrize("case", SWEEP, ids=["-".join(map(str, c)) for c in SWEEP])
def test_forward_sweep(case):
    B, H, D, S, F, dt, delta, layout = case
    say("forward sweep", case)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q, k, v = random_qkv(rng, (B, H, F * S, D), dt)
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    o, st = gdn.forward_framewise(to_dev(q, dt, DEV, layout), to_dev(k, dt, DEV, layout),
                                  to_dev(v, dt, DEV, layout), torch.from_numpy(g).to(DEV),
                                  torch.from_numpy(b).to(DEV), torch.from_numpy(s0).to(DEV),
                                  use_delta=delta)
    torch.cuda.synchronize()
    ro, rs = oracle.forward(q, k, v, g, b, s0, use_delta=delta)
    e1, e2 = rel_err(to_np(o), ro), rel_err(to_np(st), rs)
    say("  O err %.3e state err %.3e" % (e1, e2))
    assert e1 <= TOL[dt] and e2 <= TOL[dt]


# --------------------------------------------------------------------------- schedules
# The fused single-pass forward (bf16, D = 64 / 128) against the oracle and against the staged
# schedule (same products; the state step sums in another order, so states agree to fp32
# rounding and outputs to bf16 rounding).
FUSED = [
    # B, H, D, S, F, delta, initial state, layout
    (1, 2, 128, 200, 10, True, True, "head"),
    (2, 3, 64, 130, 7, True, False, "token"),
    (1, 1, 128, 1, 5, True, True, "head"),        # one token per frame
    (1, 2, 128, 96, 9, False, True, "head"),
    (1, 4, 64, 77, 12, False, False, "head"),
    (1, 3, 128, 64, 60, True, True, "head"),      # a long chain of frames
    (1, 16, 128, 3520, 3, True, True, "head"),    # the 720p frame size
]


@pytest.mark.parametrize("case", FUSED, ids=["-".join(map(str, c)) for c in FUSED])
def test_fused_forward(case):
    B, H, D, S, F, delta, with_state, layout = case
    say("fused forward", case)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32) if with_state else None
    args = [to_dev(x, "bf16", DEV, layout) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                                  torch.from_numpy(b).to(DEV)]
    ds = None if s0 is None else torch.from_numpy(s0).to(DEV)
    o1, st1 = gdn.forward_framewise(*args, ds, use_delta=delta, schedule="fused")
    o2, st2 = gdn.forward_framewise(*args, ds, use_delta=delta, schedule="staged")
    torch.cuda.synchronize()
    ro, rs = oracle.forward(q, k, v, g, b, s0, use_delta=delta)
    e1, e2 = rel_err(to_np(o1), ro), rel_err(to_np(st1), rs)
    d1, d2 = rel_err(to_np(o1), to_np(o2)), rel_err(to_np(st1), to_np(st2))
    say("  O err %.3e state err %.3e; vs staged O %.3e state %.3e" % (e1, e2, d1, d2))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]
    assert d2 <= 1e-5 and d1 <= 1e-2


GATE_CASES = [
    # name, gamma, beta
    ("gamma 0: every frame forgets the state", 0.0, None),
    ("beta 0: pure decay of the initial state", None, 0.0),
    ("gamma 1, beta 1", 1.0, 1.0),
]


@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0].split(":")[0] for c in GATE_CASES])
def test_fused_gate_extremes(case):
    """Extreme gate values through both schedules: gamma = 0 (M_f built from frame f alone),
    beta = 0 (M_f = gamma^f M_0, outputs Q M_f), gamma = beta = 1."""
    name, gv, bv = case
    B, H, D, S, F = 1, 2, 128, 70, 6
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = (np.full((B, H, F), gv) if gv is not None else rng.uniform(0.85, 1.0, (B, H, F))).astype(np.float32)
    b = (np.full((B, H, F), bv) if bv is not None else rng.uniform(0.1, 0.9, (B, H, F))).astype(np.float32)
    s0 = (0.3 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    ro, rs = oracle.forward(q, k, v, g, b, s0)
    for sched in ("fused", "staged"):
        o, st = gdn.forward_framewise(*args, torch.from_numpy(s0).to(DEV), schedule=sched)
        torch.cuda.synchronize()
        e1, e2 = rel_err(to_np(o), ro), rel_err(to_np(st), rs)
        say("  %s %s: O err %.3e state err %.3e" % (name, sched, e1, e2))
        assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_fused_many_short_chains():
    """1024 (b, h) chains of 3 frames each: tickets spread every chain's frames far apart."""
    B, H, D, S, F = 4, 256, 64, 24, 3
    rng = np.random.default_rng(21)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    o, st = gdn.forward_framewise(*args, schedule="fused")
    torch.cuda.synchronize()
    ro, rs = oracle.forward(q, k, v, g, b)
    e1, e2 = rel_err(to_np(o), ro), rel_err(to_np(st), rs)
    say("  O err %.3e state err %.3e" % (e1, e2))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_fused_nan_stays_in_its_head():
    """A NaN in one head's initial state reaches every output of that head and nothing else."""
    B, H, D, S, F = 1, 3, 64, 40, 4
    rng = np.random.default_rng(22)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    s0[0, 1, :, :] = np.nan
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    o, st = gdn.forward_framewise(*args, torch.from_numpy(s0).to(DEV), schedule="fused")
    torch.cuda.synchronize()
    o = to_np(o)
    assert np.isnan(o[0, 1]).all() and np.isnan(to_np(st)[0, 1]).all()
    s_ok = s0.copy()
    s_ok[0, 1] = 0.0
    ro, rs = oracle.forward(q, k, v, g, b, s_ok)
    for h in (0, 2):
        assert rel_err(o[0, h], ro[0, h]) <= TOL["bf16"]
        assert rel_err(to_np(st)[0, h], rs[0, h]) <= TOL["bf16"]


def test_fused_in_place_state_and_determinism():
    rng = np.random.default_rng(11)
    B, H, D, S, F = 1, 2, 128, 50, 9
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    ds = torch.from_numpy(s0).to(DEV)
    o_ref, s_ref = gdn.forward_framewise(*args, ds.clone(), schedule="fused")
    o, s = gdn.forward_framewise(*args, ds, state_out=ds, schedule="fused")
    torch.cuda.synchronize()
    assert s.data_ptr() == ds.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(ds, s_ref)


def test_launch_trace():
    rng = np.random.default_rng(12)
    B, H, D, S, F = 1, 2, 128, 64, 10
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    ev = HipEvents()
    handles = [ev.new() for _ in range(2 * 8)]
    try:
        gdn.set_trace(handles)
        gdn.forward_framewise(*args, schedule="staged")
        staged = gdn.read_trace()
        gdn.forward_framewise(*args, schedule="fused")
        fused = gdn.read_trace()
        gdn.set_trace(None)
        torch.cuda.synchronize()
        assert [k_ for k_, _, _ in staged] == ["products", "scan", "products"]
        assert [u for _, _, u in staged] == [B * H * F] * 3
        assert [k_ for k_, _, _ in fused] == ["fused_reset", "fused"]
        assert fused[1][2] == B * H * F
        for i in range(len(fused)):
            assert ev.ms(handles[2 * i], handles[2 * i + 1]) >= 0.0
    finally:
        gdn.set_trace(None)
        ev.close()


STEP_SWEEP = [
    (1, 2, 16, 16, "f32", True),
    (1, 1, 32, 70, "f32", False),
    (1, 2, 128, 300, "f32", True),
    (2, 2, 16, 9, "bf16", True),
    (1, 3, 64, 257, "bf16", True),
    (1, 2, 64, 100, "bf16", False),
    (1, 4, 128, 700, "bf16", True),
]


@pytest.mark.parametrize("case", STEP_SWEEP, ids=["-".join(map(str, c)) for c in STEP_SWEEP])
def test_step_sweep(case):
    B, H, D, S, dt, delta = case
    say("step sweep", case)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q, k, v = random_qkv(rng, (B, H, S, D), dt)
    g = rng.uniform(0.85, 1.0, (B, H)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H)).astype(np.float32)
    s0 = (0.3 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    dq, dk, dv = (to_dev(x, dt, DEV) for x in (q, k, v))
    dg, db, ds = (torch.from_numpy(x).to(DEV) for x in (g, b, s0))
    o, st = gdn.step_frame(dq, dk, dv, dg, db, ds, commit=True, use_delta=delta)
    o2, none = gdn.step_frame(dq, dk, dv, dg, db, ds, commit=False, use_delta=delta)
    torch.cuda.synchronize()
    assert none is None
    ro, rs = oracle.step(q, k, v, g, b, s0, use_delta=delta)
    e1, e2 = rel_err(to_np(o), ro), rel_err(to_np(st), rs)
    say("  O err %.3e state err %.3e" % (e1, e2))
    assert e1 <= TOL[dt] and e2 <= TOL[dt]
    assert torch.equal(o, o2), "uncommitted pass must give the same output"
    assert np.array_equal(to_np(ds), s0), "state_in must not change"


# column-block step (bf16, D = 64 / 128): single token, many heads (one split per block), ragged
# splits and chunks, no delta term, token-major storage ([B, T, H, D] viewed as [B, H, T, D]),
# the streaming shape
STEP_COLS = [
    (1, 3, 128, 700, True, "head"),
    (2, 2, 64, 257, True, "head"),
    (1, 2, 128, 1, True, "head"),
    (2, 40, 64, 100, True, "head"),
    (1, 2, 128, 333, False, "head"),
    (2, 3, 128, 500, True, "token"),
    (1, 4, 64, 130, False, "token"),
    (1, 16, 128, 3520, True, "head"),
]


@pytest.mark.parametrize("case", STEP_COLS, ids=["-".join(map(str, c)) for c in STEP_COLS])
def test_step_column_blocks(case):
    """The column-block step kernels against the oracle; a second call is bitwise identical."""
    say("step, column blocks", case)
    B, H, D, S, delta, layout = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q, k, v = random_qkv(rng, (B, H, S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H)).astype(np.float32)
    s0 = (0.3 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    dev = [to_dev(x, "bf16", DEV, layout) for x in (q, k, v)] + [torch.from_numpy(x).to(DEV) for x in (g, b, s0)]
    o1, s1 = gdn.step_frame(*dev, use_delta=delta)
    o2, s2 = gdn.step_frame(*dev, use_delta=delta)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ro, rs = oracle.step(q, k, v, g, b, s0, use_delta=delta)
    e1, e2 = rel_err(to_np(o1), ro), rel_err(to_np(s1), rs)
    say("  O err %.3e state err %.3e" % (e1, e2))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_step_launch_trace():
    """bf16 with D = 128 runs the column-block step kernels; fp32 the whole-state ones and the
    forward's output kernel."""
    ev = HipEvents()
    handles = [ev.new() for _ in range(2 * 4)]
    try:
        kinds = {}
        for dt in ("bf16", "f32"):
            rng = np.random.default_rng(3)
            q, k, v = random_qkv(rng, (1, 2, 100, 128), dt)
            args = [to_dev(x, dt, DEV) for x in (q, k, v)] + [
                torch.full((1, 2), 0.9, device=DEV), torch.full((1, 2), 0.5, device=DEV),
                torch.zeros((1, 2, 128, 128), device=DEV)]
            gdn.set_trace(handles)
            gdn.step_frame(*args)
            kinds[dt] = [k_ for k_, _, _ in gdn.read_trace()]
            gdn.set_trace(None)
        torch.cuda.synchronize()
        assert kinds["bf16"] == ["step_partial", "step_reduce", "step_output"]
        assert kinds["f32"] == ["step_partial", "step_reduce", "products"]
    finally:
        gdn.set_trace(None)
        ev.close()


def test_step_in_place_commit():
    rng = np.random.default_rng(5)
    B, H, D, S = 1, 2, 64, 96
    q, k, v = random_qkv(rng, (B, H, S, D), "bf16")
    g = rng.uniform(0.9, 1.0, (B, H)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H)).astype(np.float32)
    s0 = (0.3 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    ds = torch.from_numpy(s0).to(DEV)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    o_ref, s_ref = gdn.step_frame(*args, ds.clone())
    o, s = gdn.step_frame(*args, ds, state_out=ds)
    torch.cuda.synchronize()
    assert s.data_ptr() == ds.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(ds, s_ref)


def test_step_chain_equals_forward_and_oracle():
    rng = np.random.default_rng(6)
    B, H, D, S, F = 1, 3, 128, 120, 5
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    dq, dk, dv = (to_dev(x, "bf16", DEV) for x in (q, k, v))
    dg, db = torch.from_numpy(g).to(DEV), torch.from_numpy(b).to(DEV)
    of, sf = gdn.forward_framewise(dq, dk, dv, dg, db)
    state = torch.zeros((B, H, D, D), dtype=torch.float32, device=DEV)
    outs = []
    for f in range(F):
        sl = slice(f * S, (f + 1) * S)
        o, state = gdn.step_frame(dq[:, :, sl], dk[:, :, sl], dv[:, :, sl],
                                  dg[:, :, f].contiguous(), db[:, :, f].contiguous(), state)
        outs.append(o)
    torch.cuda.synchronize()
    os_ = torch.cat(outs, dim=2)
    ro, rs = oracle.forward(q, k, v, g, b)
    assert rel_err(to_np(os_), ro) <= TOL["bf16"]
    assert rel_err(to_np(state), rs) <= TOL["bf16"]
    assert rel_err(to_np(of), to_np(os_)) <= TOL["bf16"]
    assert rel_err(to_np(sf), to_np(state)) <= TOL["bf16"]


def test_determinism_bitwise():
    rng = np.random.default_rng(8)
    B, H, D, S, F = 1, 4, 128, 333, 4
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    o1, s1 = gdn.forward_framewise(*args)
    o2, s2 = gdn.forward_framewise(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_fused_wait_timeout_path(monkeypatch):
    """The bounded wait's time-out path, forced from the host: with GDN_FUSED_SPIN_LIMIT=0 every
    frame after the first gives up at once, so frame 0 is exact, every later output and the
    final state are NaN, and the workspace's time-out flag is set; the default clears it."""
    B, H, D, S, F = 1, 2, 128, 64, 5
    rng = np.random.default_rng(23)
    q, k, v = random_qkv(rng, (B, H, F * S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    args = [to_dev(x, "bf16", DEV) for x in (q, k, v)] + [torch.from_numpy(g).to(DEV),
                                                          torch.from_numpy(b).to(DEV)]
    p = gdn.Problem(B, H, D, S, F, gdn.GDN_BF16, 1, 0.0, H * F * S * D, F * S * D, D,
                    H * F * S * D, F * S * D, D, gdn.SCHEDULES["fused"])
    ws = torch.zeros(gdn.workspace_size(p, False), dtype=torch.uint8, device=DEV)
    ro, _ = oracle.forward(q, k, v, g, b)
    monkeypatch.setenv("GDN_FUSED_SPIN_LIMIT", "0")
    o, st = gdn.forward_framewise(*args, workspace=ws, schedule="fused")
    torch.cuda.synchronize()
    flag = int(ws[4:8].view(torch.int32).item())
    with pytest.raises(gdn.GdnError) as ei:      # the C ABI reports the flag
        gdn.check_timeout(p, 0, ws)
    assert ei.value.code == 9
    with pytest.raises(gdn.GdnError) as ei:      # the binding checks its own workspace
        gdn.forward_framewise(*args, schedule="fused")
    assert ei.value.code == 9
    o = to_np(o)
    assert flag == 1
    assert rel_err(o[:, :, :S], ro[:, :, :S]) <= TOL["bf16"]
    assert np.isnan(o[:, :, S:]).all() and np.isnan(to_np(st)).all()
    monkeypatch.delenv("GDN_FUSED_SPIN_LIMIT")
    o, st = gdn.forward_framewise(*args, workspace=ws, schedule="fused")
    torch.cuda.synchronize()
    assert int(ws[4:8].view(torch.int32).item()) == 0
    gdn.check_timeout(p, 0, ws)
    gdn.forward_framewise(*args, schedule="fused", check_timeout=True)
    assert rel_err(to_np(o), ro) <= TOL["bf16"]
