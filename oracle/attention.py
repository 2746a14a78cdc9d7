"""Oracle of frame-causal softmax attention (fp64, numpy).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may use this module; the GPU library shares no code with it.

The op is the softmax-attention counterpart of the frame-wise GDN in the pages' hybrid models:
SANA-WM interleaves softmax-attention blocks with frame-wise GDN blocks (gen-hub.ru article,
architecture section: 5 of 20 blocks; ai-papers.net, hybrid attention section), and an
all-softmax model runs out of memory on the 60 s video because its key/value cache grows with
every frame, while the GDN keeps a D x D state. SANA-Streaming's hybrid is 3.7x faster than
the all-softmax variant (jefxiong.cn digest, SANA-Streaming item).

Readings: the same frame causality as the GDN (a query of frame f sees every key of frames
0..f, all tokens of its own frame in both directions), scale 1/sqrt(D) by default, per (b, h).
q: [B, H, Tq, D] for frames q_frame0 .. q_frame0 + Tq/S - 1; k, v: [B, H, Tk, D] for frames
0 .. Tk/S - 1 (the cache, the query frames' own keys included).
"""
from __future__ import annotations

import numpy as np


def frame_causal_attention(q, k, v, S, q_frame0=0, scale=None, rows=None):
    """Returns o [B, H, Tq, D] (or only the query rows in `rows`, as [B, H, len(rows), D]).

    For each query row: scores against every visible key, softmax with the row maximum
    subtracted, weights times values."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, Tq, D = q.shape
    Tk = k.shape[2]
    c = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = range(Tq) if rows is None else list(rows)
    out = np.empty((B, H, len(rows), D))
    for i, t in enumerate(rows):
        f = q_frame0 + t // S            # the query's frame
        n = min(Tk, (f + 1) * S)          # keys of frames 0 .. f
        s = np.einsum("bhd,bhkd->bhk", q[:, :, t], k[:, :, :n]) * c
        s = s - s.max(axis=2, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=2, keepdims=True)
        out[:, :, i] = np.einsum("bhk,bhkd->bhd", p, v[:, :, :n])
    return out
