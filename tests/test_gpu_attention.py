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
    """One 720p frame (S = 3520, 16 heads) at frame 240 against the cache of frames 0..240;
    oracle on sampled rows of one head."""
    w = gdn_synth.WORKLOADS["gdn_720p_60s_bf16"]
    S, f0 = w.S, 240
    q, k, v = gdn_synth.qkv_torch(w, DEV, frames=(0, f0 + 1))
    o = gdn.attention_framecausal(q[:, :, f0 * S:], k, v, tokens_per_frame=S, q_frame0=f0)
    torch.cuda.synchronize()
    rows = [0, 17, 1000, 3519]
    h = 9
    kc, vc = k[:, h:h + 1].double().cpu().numpy(), v[:, h:h + 1].double().cpu().numpy()
    qc = q[:, h:h + 1, f0 * S:].double().cpu().numpy()
    ref = attention.frame_causal_attention(qc, kc, vc, S, q_frame0=f0, rows=rows)
    e = rel_err(to_np(o[:, h:h + 1, rows]), ref)
    say("  sampled rows err %.2e" % e)
    assert e <= TOL
