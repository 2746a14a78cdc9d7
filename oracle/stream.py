"""Frame-streaming fp64 variant of the oracle, for full-length workloads.

TEST INFRASTRUCTURE (same rules as the rest of this package). It runs the same iteration as
``gdn_oracle.c``, in the same order (scaled keys, prediction from the old state, residual,
decay-and-write, output from the new state; gen-hub.ru SANA-WM article, architecture section),
but takes one frame at a time from a callback and uses numpy fp64 matrix products for the three
products of each frame, so that one head of a 961-frame workload runs in seconds without holding
the whole sequence in memory. It is pinned by the same pin suite as the C oracle.
"""
from __future__ import annotations

import numpy as np


def forward_frames(frame_inputs, F, D, S, *, use_delta=True, key_scale=None, state_in=None,
                   keep=None):
    """One (b, h) over F frames.

    frame_inputs(f) -> (q_f, k_f, v_f, gamma_f, beta_f), q/k/v as [S, D] arrays.
    keep: frames whose outputs are returned (None = all).
    Returns (dict f -> O_f [S, D] fp64, final state [D, D] fp64).
    """
    c = 1.0 / np.sqrt(float(D) * float(S)) if key_scale is None else float(key_scale)
    M = np.zeros((D, D)) if state_in is None else np.array(state_in, dtype=np.float64)
    outs = {}
    for f in range(F):
        q, k, v, g, bt = frame_inputs(f)
        q = np.asarray(q, np.float64)
        Kt = c * np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        P = Kt @ M                                  # prediction from the old state
        R = v - float(g) * P if use_delta else v    # residual
        U = Kt.T @ R
        M = float(g) * M + float(bt) * U            # decay, then write
        if keep is None or f in keep:
            outs[f] = q @ M                         # output from the new state
    return outs, M


def forward(q, k, v, gamma, beta, state_in=None, *, use_delta=True, key_scale=None):
    """Same contract as oracle.forward (arrays [B, H, F*S, D], gates [B, H, F])."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    gamma = np.asarray(gamma, np.float64)
    beta = np.asarray(beta, np.float64)
    B, H, T, D = q.shape
    F = gamma.shape[2]
    S = T // F
    o = np.empty_like(q)
    so = np.empty((B, H, D, D))
    for b in range(B):
        for h in range(H):
            def src(f, b=b, h=h):
                sl = slice(f * S, (f + 1) * S)
                return q[b, h, sl], k[b, h, sl], v[b, h, sl], gamma[b, h, f], beta[b, h, f]
            st = None if state_in is None else state_in[b, h]
            outs, M = forward_frames(src, F, D, S, use_delta=use_delta, key_scale=key_scale,
                                     state_in=st)
            for f in range(F):
                o[b, h, f * S:(f + 1) * S] = outs[f]
            so[b, h] = M
    return o, so
