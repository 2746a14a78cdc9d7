"""The one-launch step (bf16, D = 64 / 128, B*H a multiple of 8): every head's workgroups meet
inside the launch on one XCD instead of crossing two launch boundaries. Its phases keep the
arithmetic and summation order of the three-launch path (schedule "staged"), so both must agree
bit for bit; the oracle checks them too.

Also: a workspace that starts as random bytes (the per-head epochs make each launch's meeting
flags new), repeated calls, the time-out path (GDN_FUSED_SPIN_LIMIT=0: every meeting gives up
at once, NaN results, the time-out word read and cleared by gdn_check_timeout), and capture
into a HIP graph replayed several times.
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from gpu_util import TOL, HipEvents, random_qkv, rel_err, to_dev, to_np  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(case):
    B, H, D, S, delta, layout = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q, k, v = random_qkv(rng, (B, H, S, D), "bf16")
    g = rng.uniform(0.85, 1.0, (B, H)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H)).astype(np.float32)
    s0 = (0.3 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    dev = [to_dev(x, "bf16", DEV, layout) for x in (q, k, v)] + [torch.from_numpy(x).to(DEV) for x in (g, b, s0)]
    return (q, k, v, g, b, s0), dev


def kinds_of(fn):
    ev = HipEvents()
    handles = [ev.new() for _ in range(2 * 4)]
    try:
        gdn.set_trace(handles)
        out = fn()
        kinds = [k_ for k_, _, _ in gdn.read_trace()]
    finally:
        gdn.set_trace(None)
        torch.cuda.synchronize()
        ev.close()
    return kinds, out


# B, H, D, S, delta, layout: the streaming shape (16 workgroups per head, 2 heads per XCD);
# D = 64 (one workgroup per split); token-major storage with ragged splits and chunks; one token;
# no delta term with 3 heads per XCD; 128 heads of one workgroup each
CASES = [
    (1, 16, 128, 3520, True, "head"),
    (1, 8, 64, 1000, True, "head"),
    (2, 8, 128, 777, True, "token"),
    (1, 8, 128, 1, True, "head"),
    (1, 24, 128, 500, False, "head"),
    (2, 64, 64, 64, True, "head"),
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_one_launch_equals_three_launches(case):
    say("one-launch step", case)
    B, H, D, S, delta, layout = case
    host, dev = inputs(case)
    q, k, v, g, b, s = dev
    k1, (o1, s1) = kinds_of(lambda: gdn.step_frame(q, k, v, g, b, s, use_delta=delta))
    k3, (o3, s3) = kinds_of(lambda: gdn.step_frame(q, k, v, g, b, s, use_delta=delta, schedule="staged"))
    assert k1 == ["step_fused"], k1
    assert k3 == ["step_partial", "step_reduce", "step_output"], k3
    assert torch.equal(o1, o3), "outputs differ from the three-launch path"
    assert torch.equal(s1, s3), "states differ from the three-launch path"
    # not committing: the same output, no state written
    o2, none = gdn.step_frame(q, k, v, g, b, s, commit=False, use_delta=delta)
    # committing in place
    si = s.clone()
    o4, s4 = gdn.step_frame(q, k, v, g, b, si, state_out=si, use_delta=delta)
    torch.cuda.synchronize()
    assert none is None and torch.equal(o2, o1)
    assert s4.data_ptr() == si.data_ptr() and torch.equal(si, s1) and torch.equal(o4, o1)
    # against the oracle (two heads at the larger shapes)
    heads = list(range(H)) if B * H * S <= 16 * 1000 else [0, H - 1]
    qh, kh, vh, gh, bh, s0 = host
    sel = (slice(None), heads)
    ro, rs = oracle.step(qh[sel], kh[sel], vh[sel], gh[sel], bh[sel], s0[sel], use_delta=delta)
    e1, e2 = rel_err(to_np(o1[sel]), ro), rel_err(to_np(s1[sel]), rs)
    say("  heads %s: O err %.3e state err %.3e" % (heads, e1, e2))
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_one_launch_random_workspace_and_repeats():
    """The meeting flags and epochs live in the caller's workspace: random initial bytes and
    repeated calls on the same workspace give the same results as the three launches."""
    case = (1, 16, 128, 700, True, "head")
    _, (q, k, v, g, b, s) = inputs(case)
    ref_o, ref_s = gdn.step_frame(q, k, v, g, b, s, schedule="staged")
    p = gdn._problem(q, ref_o, 1, True, None)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1234)
    ws = torch.randint(0, 256, (gdn.workspace_size(p, True),), dtype=torch.uint8, device=DEV,
                       generator=gen)
    # the time-out word must not read as set by chance
    ws[:8] = 0
    for rep in range(4):
        o, st = gdn.step_frame(q, k, v, g, b, s, workspace=ws, check_timeout=True)
        assert torch.equal(o, ref_o) and torch.equal(st, ref_s), "call %d differs" % rep


def test_one_launch_time_out(monkeypatch):
    """GDN_FUSED_SPIN_LIMIT=0: every meeting gives up at once; state and outputs are NaN and
    gdn_check_timeout reports it once (it clears the word)."""
    case = (1, 8, 128, 300, True, "head")
    _, (q, k, v, g, b, s) = inputs(case)
    ref_o, ref_s = gdn.step_frame(q, k, v, g, b, s)
    p = gdn._problem(q, ref_o, 1, True, None)
    ws = torch.zeros(gdn.workspace_size(p, True), dtype=torch.uint8, device=DEV)
    monkeypatch.setenv("GDN_FUSED_SPIN_LIMIT", "0")
    o, st = gdn.step_frame(q, k, v, g, b, s, workspace=ws, check_timeout=False)
    with pytest.raises(gdn.GdnError) as ei:
        gdn.check_timeout(p, 1, ws)
    assert ei.value.code == 9
    assert torch.isnan(st).all() and torch.isnan(o.float()).all()
    monkeypatch.delenv("GDN_FUSED_SPIN_LIMIT")
    gdn.check_timeout(p, 1, ws)   # cleared by the read above
    o, st = gdn.step_frame(q, k, v, g, b, s, workspace=ws, check_timeout=True)
    assert torch.equal(o, ref_o) and torch.equal(st, ref_s)


def test_one_launch_graph_replay():
    """Captured into a graph: each replay reads the epochs the previous one advanced, so the
    replays meet afresh; eager work (clearing the outputs) between replays."""
    case = (1, 16, 128, 900, True, "head")
    _, (q, k, v, g, b, s) = inputs(case)
    ref_o, ref_s = gdn.step_frame(q, k, v, g, b, s)
    p = gdn._problem(q, ref_o, 1, True, None)
    ws = torch.empty(gdn.workspace_size(p, True), dtype=torch.uint8, device=DEV)
    o, st = torch.empty_like(ref_o), torch.empty_like(ref_s)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gdn.step_frame(q, k, v, g, b, s, out=o, state_out=st, workspace=ws, check_timeout=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.step_frame(q, k, v, g, b, s, out=o, state_out=st, workspace=ws, check_timeout=False)
    for rep in range(4):
        o.zero_()
        st.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(st, ref_s), "replay %d differs" % rep
    gdn.check_timeout(p, 1, ws)


def test_prepared_step_call_equals_step_frame():
    """prepare_step_frame marshals the arguments once; calling it again after the inputs change
    in place gives what step_frame gives on the new contents."""
    case = (1, 8, 128, 500, True, "head")
    _, (q, k, v, g, b, s) = inputs(case)
    o = torch.empty_like(q)
    so = torch.empty_like(s)
    call = gdn.prepare_step_frame(q, k, v, g, b, s, out=o, state_out=so)
    for rep in range(3):
        ref_o, ref_s = gdn.step_frame(q, k, v, g, b, s)
        out, st = call()
        torch.cuda.synchronize()
        assert out is o and st is so
        assert torch.equal(o, ref_o) and torch.equal(so, ref_s), "call %d differs" % rep
        q.mul_(0.5)   # new contents, same buffers
    with pytest.raises(gdn.GdnError):
        gdn.prepare_step_frame(q, k[:, :, :10], v, g, b, s)
