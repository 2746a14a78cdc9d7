"""Calls captured into a HIP graph (through torch.cuda.CUDAGraph) and replayed.

Every call only launches kernels on the caller's stream (no memset or copy nodes), so it can be
captured. The graph below holds the fused and staged forwards, both step paths, the saving
forward with the backward from its buffer, the recomputing backward, both schedules of the
backward's reverse chain, the temporal convolution and the attention; it is replayed several
times with eager work (clearing the outputs) and synchronisations between the replays, and every
replay must reproduce the eager results bitwise (the kernels are deterministic).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
from gpu_util import random_qkv, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_graph_capture_and_replay():
    rng = np.random.default_rng(77)
    B, H, D, S, F = 1, 2, 128, 96, 6
    q, k, v = [to_dev(x, "bf16", DEV) for x in random_qkv(rng, (B, H, F * S, D), "bf16")]
    g = torch.from_numpy(rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)).to(DEV)
    b = torch.from_numpy(rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)).to(DEV)
    s0 = torch.from_numpy((0.2 * rng.standard_normal((B, H, D, D))).astype(np.float32)).to(DEV)
    d_o = to_dev(rng.standard_normal((B, H, F * S, D)).astype(np.float32), "bf16", DEV)
    qs, ks, vs = (x[:, :, :S].contiguous() for x in (q, k, v))
    g0, b0 = g[:, :, 0].contiguous(), b[:, :, 0].contiguous()
    q32, k32, v32 = (x[:, :, :S].float().contiguous() for x in (q, k, v))
    xt = torch.randn((1, 4, 8, 64), device=DEV).to(torch.bfloat16)
    wt = torch.randn((64, 3), device=DEV) * 0.3
    bt = torch.randn((64,), device=DEV) * 0.1

    # outputs and workspaces allocated before the capture
    def problem(x, F_, o_strides=None, schedule=0):
        st = x.stride()[:3]
        return gdn.Problem(B, H, D, S, F_, gdn.GDN_BF16 if x.dtype == torch.bfloat16 else gdn.GDN_F32,
                           1, 0.0, *st, *(o_strides or st), schedule)

    def ws(p, mode):
        return torch.empty(gdn.workspace_size(p, mode), dtype=torch.uint8, device=DEV)

    pf = problem(q, F)
    o_f, st_f, ws_f = torch.empty_like(q), torch.empty_like(s0), ws(pf, 0)
    o_s, st_s, ws_s = torch.empty_like(q), torch.empty_like(s0), ws(pf, 0)
    o_t, st_t, ws_t = torch.empty_like(qs), torch.empty_like(s0), ws(problem(qs, 1), 1)
    o_t32, st_t32, ws_t32 = torch.empty_like(q32), torch.empty_like(s0), ws(problem(q32, 1), 1)
    o_v = torch.empty_like(q)
    saved = torch.empty(gdn.saved_size(pf), dtype=torch.uint8, device=DEV)
    ws_v = ws(pf, 0)
    grads_s = [torch.empty_like(q) for _ in range(3)]
    ws_b3 = ws(pf, 3)
    grads_r = [torch.empty_like(q) for _ in range(3)]
    ws_b2 = ws(pf, 2)
    pc = problem(q, F, schedule=2)
    grads_c = [torch.empty_like(q) for _ in range(3)]
    ws_c2 = ws(pc, 2)
    grads_cs = [torch.empty_like(q) for _ in range(3)]
    ws_c3 = ws(pc, 3)
    yt, ct = torch.empty_like(xt), torch.empty((1, 8, 64), device=DEV, dtype=torch.bfloat16)
    oa = torch.empty_like(q)

    def calls():
        out = {}
        out["fused"] = gdn.forward_framewise(q, k, v, g, b, s0, out=o_f, state_out=st_f, workspace=ws_f,
                                             schedule="fused")
        out["staged"] = gdn.forward_framewise(q, k, v, g, b, s0, out=o_s, state_out=st_s, workspace=ws_s,
                                              schedule="staged")
        out["step"] = gdn.step_frame(qs, ks, vs, g0, b0, s0, out=o_t, state_out=st_t, workspace=ws_t)
        out["step32"] = gdn.step_frame(q32, k32, v32, g0, b0, s0, out=o_t32, state_out=st_t32,
                                       workspace=ws_t32)
        out["save"] = gdn.forward_framewise_save(q, k, v, g, b, s0, out=o_v, return_state=False,
                                                 saved=saved, workspace=ws_v)[0]
        out["bwd_saved"] = gdn.backward_framewise(q, k, v, g, b, d_o, None, None, dq=grads_s[0],
                                                  dk=grads_s[1], dv=grads_s[2], saved=saved,
                                                  workspace=ws_b3)
        out["bwd"] = gdn.backward_framewise(q, k, v, g, b, d_o, s0, None, dq=grads_r[0], dk=grads_r[1],
                                            dv=grads_r[2], workspace=ws_b2)
        out["bwd_chain"] = gdn.backward_framewise(q, k, v, g, b, d_o, s0, None, dq=grads_c[0], dk=grads_c[1],
                                                  dv=grads_c[2], workspace=ws_c2, schedule="fused")
        out["bwd_chain_saved"] = gdn.backward_framewise(q, k, v, g, b, d_o, None, None, dq=grads_cs[0],
                                                        dk=grads_cs[1], dv=grads_cs[2], saved=saved,
                                                        workspace=ws_c3, schedule="fused")
        out["tconv"] = gdn.temporal_conv(xt, wt, bt, block_frames=2, out=yt, cache_out=ct)
        out["attn"] = gdn.attention_framecausal(q, k, v, tokens_per_frame=S, out=oa)
        return out

    def flatten(out):
        flat = []
        for key in sorted(out):
            val = out[key]
            for t in (val if isinstance(val, (tuple, list)) else (val,)):
                if isinstance(t, torch.Tensor):
                    flat.append((key, t))
        return flat

    ref = [(key, t.clone()) for key, t in flatten(calls())]
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()   # warm-up on the capture stream, as torch asks before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        live = flatten(calls())
    for rep in range(3):
        for _, t in live:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (key, t), (key2, r) in zip(live, ref):
            assert key == key2
            assert torch.equal(t, r), "replay %d differs: %s" % (rep, key)
        say("replay %d: %d outputs identical" % (rep, len(live)))
