"""gdn_step_frame_noalloc (the step without a workspace argument, for callers that cannot
allocate) through the C ABI, against gdn_step_frame with a workspace of its own on the same
inputs: two calls in a row on the library's shared scratch, the second smaller, then the
whole-state fp32 kernels; each output is also checked against the oracle.

Bar: the two entry points run the same kernels on the same inputs, so their outputs and
states must agree bit for bit; against the oracle max|d| / max|ref| <= 1e-2 (bf16) or 1e-4
(fp32).
"""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import oracle  # noqa: E402
from gpu_util import TOL, random_qkv, rel_err, to_dev, to_np  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CALLS = [
    # B, H, D, S, dtype, commit, heads checked against the oracle
    (1, 16, 128, 3520, "bf16", True, [0, 13]),   # the streaming shape (8.5 MiB of scratch)
    (1, 3, 64, 300, "bf16", False, [1]),          # smaller, right after on the same scratch
    (2, 2, 16, 40, "f32", True, [0, 1]),          # the whole-state kernels
]


def test_noalloc_step_matches_step_frame():
    lib = gdn.load()
    rng = np.random.default_rng(71)
    for B, H, D, S, dtype, commit, heads in CALLS:
        say("noalloc step", (B, H, D, S, dtype, commit))
        q, k, v = random_qkv(rng, (B, H, S, D), dtype)
        g = rng.uniform(0.85, 1.0, (B, H)).astype(np.float32)
        b = rng.uniform(0.1, 0.9, (B, H)).astype(np.float32)
        m = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
        qd, kd, vd = (to_dev(x, dtype, DEV) for x in (q, k, v))
        gd, bd, md = (torch.from_numpy(x).to(DEV) for x in (g, b, m))
        # the existing entry point with its own workspace
        ref_o, ref_s = gdn.step_frame(qd, kd, vd, gd, bd, md, commit=commit)
        # the new one through the C ABI; every buffer allocated before the call
        o = torch.full_like(ref_o, float("nan"))
        s = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device=DEV) if commit else None
        p = gdn._problem(qd, o, 1, True, None)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        code = lib.gdn_step_frame_noalloc(ctypes.byref(p), gdn._ptr(qd), gdn._ptr(kd), gdn._ptr(vd),
                                          gdn._ptr(gd), gdn._ptr(bd), gdn._ptr(md), gdn._ptr(o),
                                          gdn._ptr(s), st)
        assert code == 0, lib.gdn_last_error_message()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), "output differs from gdn_step_frame"
        if commit:
            assert torch.equal(s, ref_s), "state differs from gdn_step_frame"
        ro, rs = oracle.step(q[:, heads], k[:, heads], v[:, heads], g[:, heads], b[:, heads],
                             m[:, heads].astype(np.float64), commit=commit)
        e = rel_err(to_np(o[:, heads]), ro)
        say("  oracle err o %.2e" % e)
        assert e <= TOL[dtype]
        if commit:
            e = rel_err(to_np(s[:, heads]), rs)
            say("  oracle err state %.2e" % e)
            assert e <= TOL[dtype]


def test_noalloc_step_rejects_problems_beyond_the_scratch():
    # 512 heads of D = 128 at 3520 tokens need 48 MiB of step workspace (> 32 MiB): rejected on
    # the host before anything is enqueued; gdn_step_frame with a workspace still takes it
    lib = gdn.load()
    B, H, D, S = 1, 512, 128, 3520
    p = gdn.Problem(B, H, D, S, 1, gdn.GDN_BF16, 1, 0.0, H * S * D, S * D, D, H * S * D, S * D, D)
    assert gdn.workspace_size(p, 1) > (32 << 20)
    x = torch.zeros((B, H, S, D), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(x)
    g = torch.ones((B, H), dtype=torch.float32, device=DEV)
    m = torch.zeros((B, H, D, D), dtype=torch.float32, device=DEV)
    code = lib.gdn_step_frame_noalloc(ctypes.byref(p), gdn._ptr(x), gdn._ptr(x), gdn._ptr(x),
                                      gdn._ptr(g), gdn._ptr(g), gdn._ptr(m), gdn._ptr(o), None, None)
    assert code == 7 and b"static scratch" in lib.gdn_last_error_message()
