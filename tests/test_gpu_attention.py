"""Frame-causal softmax attention on the GPU (gdn_attention_framecausal through the C ABI)
against the oracle (oracle/attention.py).

Tolerance: max|d| / max|ref| <= 1e-2 (bf16 inputs and output; fp32 softmax, the weights enter
the value product in bf16).
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import gdn_synth  # noqa: E402
from gpu_util import rel_err, to_np  # noqa: E402
from oracle import attention  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_host(rng, shape):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)


def to_dev(t, layout):
    if layout == "token":   # storage [B, T, H, D]
        return t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    return t.to(DEV)


CASES = [
    # B, H, D, S, q_frames, kv_frames, q_frame0, layout
    (1, 2, 128, 40, 3, 3, 0, "head"),
    (2, 1, 64, 17, 4, 4, 0, "head"),
    (1, 2, 128, 1, 70, 70, 0, "head"),       # one token per frame: causal attention
    (1, 1, 128, 200, 1, 5, 4, "head"),       # streaming step: the last frame against the cache
    (1, 2, 64, 100, 2, 6, 2, "head"),        # later keys present, masked
    (1, 3, 128, 130, 3, 3, 0, "token"),
    (1, 2, 128, 3520, 1, 3, 2, "head"),      # a 720p frame against a 3-frame cache
    # several 256-query workgroups per head, ragged last one
    (2, 128, 128, 97, 3, 3, 0, "head"),
    (2, 128, 64, 65, 5, 6, 1, "token"),      # later keys present, masked
    # grids of at least 512 workgroups of 384 queries take the 12-wave kernel (Q in LDS)
    (2, 256, 128, 97, 3, 3, 0, "head"),
    (2, 128, 64, 65, 8, 9, 1, "token"),      # two query blocks per head, ragged, later keys masked
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_attention_matches_oracle(case):
    B, H, D, S, fq, fk, f0, layout = case
    say("attention", case)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q = bf16_host(rng, (B, H, fq * S, D))
    k = bf16_host(rng, (B, H, fk * S, D))
    v = bf16_host(rng, (B, H, fk * S, D))
    o = gdn.attention_framecausal(to_dev(q, layout), to_dev(k, layout), to_dev(v, layout),
                                  tokens_per_frame=S, q_frame0=f0)
    torch.cuda.synchronize()
    ref = attention.frame_causal_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                           S, q_frame0=f0)
    e = rel_err(to_np(o), ref)
    say("  o err %.2e" % e)
    assert e <= TOL


RESCALE_CASES = [
    # B, H, D, S, q_frames, kv_frames, q_frame0, layout, scale x sqrt(D), key ramp
    (1, 2, 128, 100, 3, 3, 0, "head", 8.0, True),
    (1, 2, 64, 77, 3, 4, 1, "head", 16.0, True),     # ragged last key tile, later keys masked
    (2, 3, 64, 40, 5, 5, 0, "token", 16.0, False),
    (1, 1, 128, 130, 2, 6, 3, "head", 12.0, True),   # streaming rows, ragged tiles
    (2, 256, 128, 40, 3, 3, 0, "head", 8.0, True),   # the 12-wave kernel
]


@pytest.mark.parametrize("case", RESCALE_CASES, ids=["-".join(map(str, c)) for c in RESCALE_CASES])
def test_attention_running_maximum_moves(case):
    """The online softmax's deferred rescale: with a large explicit scale (and keys whose norm
    grows with their index) a row's running maximum rises by more than the rescale threshold
    after its first key tile, so the accumulated weights and values are rescaled while nonzero
    (including on the masked, ragged last tile). The oracle takes the same scale."""
    B, H, D, S, fq, fk, f0, layout, mult, ramp = case
    say("attention rescale", case)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q = bf16_host(rng, (B, H, fq * S, D))
    kf = rng.standard_normal((B, H, fk * S, D)).astype(np.float32)
    if ramp:
        kf *= (1.0 + 2.0 * np.arange(fk * S, dtype=np.float32) / (fk * S))[None, None, :, None]
    k = torch.from_numpy(kf).to(torch.bfloat16)
    v = bf16_host(rng, (B, H, fk * S, D))
    scale = mult / np.sqrt(D)
    o = gdn.attention_framecausal(to_dev(q, layout), to_dev(k, layout), to_dev(v, layout),
                                  tokens_per_frame=S, q_frame0=f0, scale=scale)
    torch.cuda.synchronize()
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = attention.frame_causal_attention(qd, kd, vd, S, q_frame0=f0, scale=scale)
    # the running maximum does move after the first 64-key tile for many rows (log2 units)
    first = (qd @ kd[:, :, :64].transpose(0, 1, 3, 2)).max(axis=3) * scale / np.log(2)
    vis = [min(fk * S, (f0 + t // S + 1) * S) for t in range(fq * S)]
    full = np.array([[[(qd[b, h, t] @ kd[b, h, :vis[t]].T).max() * scale / np.log(2)
                       for t in range(fq * S)] for h in range(H)] for b in range(B)])
    moved = float(np.mean(full - first > 8.0))
    say("  rows whose maximum moves by > 8 after the first tile: %.0f%%" % (100 * moved))
    assert moved > 0.2
    e = rel_err(to_np(o), ref)
    say("  o err %.2e" % e)
    assert e <= TOL


def test_attention_deterministic_and_streaming_consistent():
    """Each frame's rows of the whole-sequence call equal a streaming call of that frame alone
    against the full key set (future keys present), bit for bit, and reruns are identical."""
    B, H, D, S, F = 1, 2, 128, 96, 4
    rng = np.random.default_rng(3)
    q, k, v = (bf16_host(rng, (B, H, F * S, D)).to(DEV) for _ in range(3))
    o1 = gdn.attention_framecausal(q, k, v, tokens_per_frame=S)
    o2 = gdn.attention_framecausal(q, k, v, tokens_per_frame=S)
    parts = [gdn.attention_framecausal(q[:, :, f * S:(f + 1) * S], k, v, tokens_per_frame=S, q_frame0=f)
             for f in range(F)]
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(torch.cat(parts, dim=2), o1)


def test_attention_880x81_full_launch():
    """The 880-token x 81-frame workload's Q, K, V (two batches, 16 heads), whole sequence;
    oracle on sampled rows of two heads."""
    w = gdn_synth.WORKLOADS["gdn_880x81_bf16"]
    S = w.S
    q, k, v = gdn_synth.qkv_torch(w, DEV)
    o = gdn.attention_framecausal(q, k, v, tokens_per_frame=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    rows = [0, 1, 879, 880, 20 * S + 5, 40 * S + 300, 80 * S, w.F * S - 1]
    for h in (0, 11):
        (qc, kc, vc), _ = gdn_synth.qkv_cpu(w, heads=[h])
        ref = attention.frame_causal_attention(qc, kc, vc, S, rows=rows)
        e = rel_err(to_np(o[:, h:h + 1, rows]), ref)
        say("  head %d sampled rows err %.2e" % (h, e))
        assert e <= TOL


def test_attention_720p_streaming_step():
    """One 720p frame (S = 3520, 16 heads) at frame 240 against the cache of frames 0..240,
    without and with a workspace (key splits); oracle on sampled rows of one head."""
    w = gdn_synth.WORKLOADS["gdn_720p_60s_bf16"]
    S, f0 = w.S, 240
    q, k, v = gdn_synth.qkv_torch(w, DEV, frames=(0, f0 + 1))
    qf = q[:, :, f0 * S:]
    o = gdn.attention_framecausal(qf, k, v, tokens_per_frame=S, q_frame0=f0)
    assert gdn.attention_workspace_size(gdn.attention_problem(qf, k, o, S, f0)) > 0
    os_ = gdn.attention_framecausal(qf, k, v, tokens_per_frame=S, q_frame0=f0, workspace="auto")
    torch.cuda.synchronize()
    rows = [0, 17, 1000, 3519]
    h = 9
    kc, vc = k[:, h:h + 1].double().cpu().numpy(), v[:, h:h + 1].double().cpu().numpy()
    qc = qf[:, h:h + 1].double().cpu().numpy()
    ref = attention.frame_causal_attention(qc, kc, vc, S, q_frame0=f0, rows=rows)
    for name, out in (("unsplit", o), ("key splits", os_)):
        e = rel_err(to_np(out[:, h:h + 1, rows]), ref)
        say("  %s: sampled rows err %.2e" % (name, e))
        assert e <= TOL
    d = rel_err(to_np(os_), to_np(o))
    say("  key splits against unsplit, all rows: %.2e" % d)
    assert d <= TOL


SPLIT_CASES = [
    # B, H, D, S, kv_frames, q_frame0, layout: one query frame against a long cache, too few
    # query blocks to fill the device, so a workspace splits the keys
    (1, 2, 128, 200, 41, 40, "head"),        # 8200 keys: ragged last key tile; ragged query block
    (1, 1, 64, 300, 30, 20, "token"),        # cache frames after the query frame present, unseen
    (2, 3, 128, 520, 12, 11, "head"),        # two query blocks per head
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=["-".join(map(str, c)) for c in SPLIT_CASES])
def test_attention_key_splits(case):
    """gdn_attention_framecausal_ws: the keys of each query block split over several
    workgroups, then merged; against the oracle, with a workspace whose entry contents are
    NaN (they must not matter), twice in a row."""
    B, H, D, S, fk, f0, layout = case
    say("attention key splits", case)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q = bf16_host(rng, (B, H, S, D))
    k = bf16_host(rng, (B, H, fk * S, D))
    v = bf16_host(rng, (B, H, fk * S, D))
    qd, kd, vd = to_dev(q, layout), to_dev(k, layout), to_dev(v, layout)
    o = torch.empty(qd.shape, dtype=torch.bfloat16, device=DEV)
    n = gdn.attention_workspace_size(gdn.attention_problem(qd, kd, o, S, f0))
    say("  workspace %d bytes" % n)
    assert n > 0
    ws = torch.full((n,), 255, dtype=torch.uint8, device=DEV)     # NaN bytes
    ref = attention.frame_causal_attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                           S, q_frame0=f0)
    for rep in range(2):
        gdn.attention_framecausal(qd, kd, vd, tokens_per_frame=S, q_frame0=f0, out=o, workspace=ws)
        torch.cuda.synchronize()
        e = rel_err(to_np(o), ref)
        say("  call %d: o err %.2e" % (rep, e))
        assert e <= TOL


def test_attention_key_splits_12_waves():
    """A single-frame call whose plan takes 12-wave workgroups with 5 key splits (48 heads of
    one 384-query block each: 240 workgroups of 50 key tiles, against 8-wave blocks of 256
    queries that would need more rounds); the oracle on sampled heads and rows."""
    B, H, D, S, fk, f0 = 1, 48, 128, 384, 41, 40
    rng = np.random.default_rng(12)
    q = bf16_host(rng, (B, H, S, D))
    k = bf16_host(rng, (B, H, fk * S, D))
    v = bf16_host(rng, (B, H, fk * S, D))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty_like(qd)
    n = gdn.attention_workspace_size(gdn.attention_problem(qd, kd, o, S, f0))
    rows_total = B * H * S
    # the plan's split count from the workspace size: part (fp32 O) + (m, l) pairs per split
    ns = n // (rows_total * (D * 4 + 8))
    say("  workspace %d bytes: %d splits" % (n, ns))
    assert ns == 5 and n == ns * rows_total * (D * 4 + 8)
    gdn.attention_framecausal(qd, kd, vd, tokens_per_frame=S, q_frame0=f0, out=o, workspace="auto")
    torch.cuda.synchronize()
    rows = [0, 100, 383]
    for h in (0, 29, 47):
        ref = attention.frame_causal_attention(q[:, h:h + 1].double().numpy(), k[:, h:h + 1].double().numpy(),
                                               v[:, h:h + 1].double().numpy(), S, q_frame0=f0, rows=rows)
        e = rel_err(to_np(o[:, h:h + 1, rows]), ref)
        say("  head %d sampled rows err %.2e" % (h, e))
        assert e <= TOL
