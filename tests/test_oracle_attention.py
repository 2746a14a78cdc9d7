"""Pins of the frame-causal softmax-attention oracle (oracle/attention.py), on the CPU.

Pinned by things it does not share:
  * one frame: torch's scaled_dot_product_attention (no mask), fp64 on the CPU;
  * one token per frame: torch's causal scaled_dot_product_attention;
  * any shape: torch's attention with the boolean frame mask (key frame <= query frame);
  * identical keys: every visible key gets the same weight, so a row is the mean of the
    visible values (closed form);
  * a streaming call (one frame's queries against the cache of frames 0..f, extra future keys
    present) equals that frame's rows of the whole-sequence call;
  * adding one vector to every key leaves each row unchanged (softmax shift invariance);
  * planted mistakes in a copy of the source, each caught by one of the above.
"""
import os

import numpy as np
import pytest
import torch

from oracle import attention

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")


def qkv(rng, B, H, T, D):
    return [rng.standard_normal((B, H, T, D)) for _ in range(3)]


def sdpa(q, k, v, **kw):
    t = [torch.from_numpy(x) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t, **kw).numpy()


def checks(mod):
    """Returns a list of failed pins."""
    bad = []
    rng = np.random.default_rng(1)
    q, k, v = qkv(rng, 1, 2, 6, 4)
    if not np.allclose(mod.frame_causal_attention(q, k, v, S=6), sdpa(q, k, v), atol=1e-12):
        bad.append("one frame")
    if not np.allclose(mod.frame_causal_attention(q, k, v, S=1), sdpa(q, k, v, is_causal=True), atol=1e-12):
        bad.append("one token per frame")
    S, F = 3, 4
    q, k, v = qkv(rng, 2, 1, S * F, 8)
    fr = np.arange(S * F) // S
    mask = torch.from_numpy(fr[None, :] <= fr[:, None])
    if not np.allclose(mod.frame_causal_attention(q, k, v, S=S), sdpa(q, k, v, attn_mask=mask), atol=1e-12):
        bad.append("frame mask")
    kk = np.repeat(k[:, :, :1], S * F, axis=2)      # identical keys
    o = mod.frame_causal_attention(q, kk, v, S=S)
    want = np.stack([v[:, :, :(t // S + 1) * S].mean(axis=2) for t in range(S * F)], axis=2)
    if not np.allclose(o, want, atol=1e-12):
        bad.append("identical keys")
    full = mod.frame_causal_attention(q, k, v, S=S)
    for f in range(F):
        part = mod.frame_causal_attention(q[:, :, f * S:(f + 1) * S], k, v, S=S, q_frame0=f)
        if not np.allclose(part, full[:, :, f * S:(f + 1) * S], atol=1e-12):
            bad.append("streaming frame %d" % f)
    u = rng.standard_normal(8)
    if not np.allclose(mod.frame_causal_attention(q, k + u, v, S=S), full, atol=1e-10):
        bad.append("shift invariance")
    rows = [0, 5, 11]
    if not np.allclose(mod.frame_causal_attention(q, k, v, S=S, rows=rows), full[:, :, rows], atol=1e-14):
        bad.append("row selection")
    return bad


def test_pins():
    assert checks(attention) == []


MUTANTS = {
    "own frame excluded": ("n = min(Tk, (f + 1) * S)", "n = min(Tk, max(1, f * S))"),
    "next frame visible": ("n = min(Tk, (f + 1) * S)", "n = min(Tk, (f + 2) * S)"),
    "no scale": ("    c = 1.0 / np.sqrt(D) if scale is None else float(scale)", "    c = 1.0"),
    "keys as values": ('out[:, :, i] = np.einsum("bhk,bhkd->bhd", p, v[:, :, :n])',
                       'out[:, :, i] = np.einsum("bhk,bhkd->bhd", p, k[:, :, :n])'),
    "frame offset ignored": ("f = q_frame0 + t // S", "f = t // S"),
    "not normalised": ("p = p / p.sum(axis=2, keepdims=True)", "p = p / p.sum(axis=2, keepdims=True).mean()"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attention_mutants_are_caught(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor must be unique: " + old
    ns = {"__name__": "attention_variant"}
    exec(compile(src.replace(old, new), "attention_variant", "exec"), ns)

    class M:
        frame_causal_attention = staticmethod(ns["frame_causal_attention"])
    try:
        caught = checks(M) != []
    except Exception:
        caught = True
    assert caught, "planted mistake not caught: " + name
