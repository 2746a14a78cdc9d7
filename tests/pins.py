"""Pins that tie the CPU oracle to facts fixed outside its own code.

Each ``pin_*`` function raises AssertionError when the oracle (or a planted-mistake variant of
it, passed as ``lib``) disagrees with:

* hand-derived worked examples (tests/golden/hand_examples.txt);
* closed forms: SANA-Video's block-causal cumulative linear attention as a masked quadratic
  sum (talk "SANA-Video ... Block Linear Diffusion Transformer", block KV cache passage), and
  the gated no-delta state as an explicit weighted sum;
* the delta-rule identity (gen-hub.ru SANA-WM article, architecture section: the write
  stores the residual between target and prediction, so a unit key recalls its value);
* the textbook token-level gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta
  Networks", ICLR 2025) at S = 1, and its frame-level Gram form for general S;
* a token-by-token brute force in pure Python;
* bounded state norms under the 1/sqrt(D*S) key scale;
* special cases (beta = 0, a single frame), step == forward, linearity and value-column
  permutation equivariance.
"""
from __future__ import annotations

import os

import numpy as np

import gdn_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_examples.txt")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def _close(a, b, tol, what):
    assert np.all(np.isfinite(a)), what + ": non-finite values"
    r = _rel(a, b)
    assert r <= tol, "%s: max|d|/max|ref| = %.3e > %.1e" % (what, r, tol)


def _inputs(rng, B, H, D, S, F, gamma=(0.8, 1.0), beta=(0.1, 0.9)):
    q = rng.standard_normal((B, H, F * S, D))
    k = rng.standard_normal((B, H, F * S, D))
    v = rng.standard_normal((B, H, F * S, D))
    g = rng.uniform(*gamma, size=(B, H, F))
    bt = rng.uniform(*beta, size=(B, H, F))
    return q, k, v, g, bt


# --------------------------------------------------------------------------- golden
def parse_golden(path=GOLDEN):
    cases, cur = [], None
    with open(path) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest.strip()}
                cases.append(cur)
            elif key == "shape":
                for item in rest.split():
                    n, val = item.split("=")
                    cur[n] = int(val)
            elif key in ("use_delta",):
                cur[key] = int(rest)
            elif key == "key_scale":
                cur[key] = None if rest.strip() == "default" else float(rest)
            elif key == "state_in" and rest.strip() == "none":
                cur[key] = None
            else:
                cur[key] = np.array([float(x) for x in rest.split()])
    return cases


def pin_golden(lib=None):
    for c in parse_golden():
        D, S, F = c["D"], c["S"], c["F"]
        st = None if c["state_in"] is None else c["state_in"].reshape(1, 1, D, D)
        o, so = oracle.forward(c["q"].reshape(1, 1, F * S, D), c["k"].reshape(1, 1, F * S, D),
                               c["v"].reshape(1, 1, F * S, D), c["gamma"].reshape(1, 1, F),
                               c["beta"].reshape(1, 1, F), st, use_delta=bool(c["use_delta"]),
                               key_scale=c["key_scale"], lib=lib)
        assert np.allclose(o.ravel(), c["o"], rtol=0, atol=1e-12), c["name"] + ": output"
        assert np.allclose(so.ravel(), c["state_out"], rtol=0, atol=1e-12), c["name"] + ": state"


# --------------------------------------------------------------------------- closed forms
def block_causal_closed_form(q, k, v, S, c):
    """O_t = sum over tokens t' in frames up to frame(t) of (q_t . c k_t') v_t'."""
    T = q.shape[0]
    fr = np.arange(T) // S
    mask = fr[None, :] <= fr[:, None]
    return ((q @ (c * k).T) * mask) @ v


def pin_block_causal(lib=None):
    rng = np.random.default_rng(11)
    for (D, S, F) in [(3, 2, 4), (4, 5, 3), (8, 1, 6), (16, 16, 3)]:
        q, k, v, _, _ = _inputs(rng, 1, 2, D, S, F)
        one = np.ones((1, 2, F))
        o, _ = oracle.forward(q, k, v, one, one, use_delta=False, lib=lib)
        c = 1.0 / np.sqrt(D * S)
        for h in range(2):
            _close(o[0, h], block_causal_closed_form(q[0, h], k[0, h], v[0, h], S, c), 1e-12,
                   "block-causal D=%d S=%d F=%d" % (D, S, F))
    # a 1-head, 2-frame slice of the block-causal bf16 workload (S = 1560, D = 64, ReLU Q/K)
    w = gdn_synth.WORKLOADS["block_causal_bf16"]
    (qv, kv, vv), _ = gdn_synth.qkv_cpu(w, heads=[3], frames=[0, 1])
    one = np.ones((1, 1, 2))
    o, _ = oracle.forward(qv, kv, vv, one, one, use_delta=False, lib=lib)
    ref = block_causal_closed_form(qv[0, 0].astype(np.float64), kv[0, 0].astype(np.float64),
                                   vv[0, 0].astype(np.float64), w.S, 1.0 / np.sqrt(w.D * w.S))
    _close(o[0, 0], ref, 1e-12, "block-causal workload slice")


def gated_nodelta_closed_form(q, k, v, g, bt, S, c, M0):
    """M_f = (prod_{f'<=f} g_f') M0 + sum_{f'<=f} (prod_{f'<g<=f} g_g) bt_f' (cK_f')^T V_f'."""
    F = len(g)
    D = q.shape[1]
    o = np.zeros_like(q)
    for f in range(F):
        M = np.prod(g[:f + 1]) * M0
        for fp in range(f + 1):
            Kf = c * k[fp * S:(fp + 1) * S]
            M = M + np.prod(g[fp + 1:f + 1]) * bt[fp] * (Kf.T @ v[fp * S:(fp + 1) * S])
        o[f * S:(f + 1) * S] = q[f * S:(f + 1) * S] @ M
    return o, M


def pin_gated_nodelta(lib=None):
    rng = np.random.default_rng(12)
    for (D, S, F) in [(4, 3, 5), (8, 8, 4), (2, 1, 7)]:
        q, k, v, g, bt = _inputs(rng, 1, 1, D, S, F)
        M0 = rng.standard_normal((1, 1, D, D))
        o, so = oracle.forward(q, k, v, g, bt, M0, use_delta=False, lib=lib)
        ro, rM = gated_nodelta_closed_form(q[0, 0], k[0, 0], v[0, 0], g[0, 0], bt[0, 0], S,
                                           1.0 / np.sqrt(D * S), M0[0, 0])
        _close(o[0, 0], ro, 1e-12, "gated no-delta output")
        _close(so[0, 0], rM, 1e-12, "gated no-delta state")


# --------------------------------------------------------------------------- delta rule
def pin_delta_identity(lib=None):
    rng = np.random.default_rng(13)
    # S = 1: a unit scaled key with beta = gamma = 1 recalls its value exactly.
    D, F = 8, 6
    c = 1.0 / np.sqrt(D)
    kt = rng.standard_normal((F, D))
    kt /= np.linalg.norm(kt, axis=1, keepdims=True)
    v = rng.standard_normal((F, D))
    M0 = rng.standard_normal((1, 1, D, D))
    one = np.ones((1, 1, F))
    o, _ = oracle.forward(kt[None, None], (kt / c)[None, None], v[None, None], one, one, M0,
                          lib=lib)
    _close(o[0, 0], v, 1e-12, "unit-key recall (S=1)")
    # frame form: orthonormal rows of cK (S <= D) recall the whole frame.
    D, S, F = 16, 5, 4
    c = 1.0 / np.sqrt(D * S)
    K, Qr, V = [], [], []
    for _ in range(F):
        basis, _ = np.linalg.qr(rng.standard_normal((D, S)))
        Qr.append(basis.T)
        K.append(basis.T / c)
        V.append(rng.standard_normal((S, D)))
    q, k, v = (np.concatenate(x)[None, None] for x in (Qr, K, V))
    one = np.ones((1, 1, F))
    o, _ = oracle.forward(q, k, v, one, one, rng.standard_normal((1, 1, D, D)), lib=lib)
    _close(o[0, 0], v[0, 0], 1e-12, "orthonormal-frame recall")


def textbook_gated_delta(q, k, v, g, bt, c, M0):
    """Token-level gated delta rule, row-vector form: M_t = g_t (I - b_t kk^T) M + b_t k v^T."""
    T, D = q.shape
    M = M0.copy()
    o = np.zeros_like(q)
    eye = np.eye(D)
    for t in range(T):
        kk = c * k[t]
        M = g[t] * (eye - bt[t] * np.outer(kk, kk)) @ M + bt[t] * np.outer(kk, v[t])
        o[t] = q[t] @ M
    return o, M


def gram_form(q, k, v, g, bt, S, c, M0):
    """Frame level: M_f = g_f (I - b_f Kt^T Kt) M + b_f Kt^T V_f, O_f = Q_f M_f."""
    T, D = q.shape
    F = T // S
    M = M0.copy()
    o = np.zeros_like(q)
    for f in range(F):
        Kt = c * k[f * S:(f + 1) * S]
        M = g[f] * (np.eye(D) - bt[f] * Kt.T @ Kt) @ M + bt[f] * Kt.T @ v[f * S:(f + 1) * S]
        o[f * S:(f + 1) * S] = q[f * S:(f + 1) * S] @ M
    return o, M


def pin_textbook(lib=None):
    rng = np.random.default_rng(14)
    D, F = 6, 9
    q, k, v, g, bt = _inputs(rng, 1, 1, D, 1, F)
    M0 = rng.standard_normal((1, 1, D, D))
    o, so = oracle.forward(q, k, v, g, bt, M0, lib=lib)
    ro, rM = textbook_gated_delta(q[0, 0], k[0, 0], v[0, 0], g[0, 0], bt[0, 0],
                                  1.0 / np.sqrt(D), M0[0, 0])
    _close(o[0, 0], ro, 1e-12, "S=1 vs textbook gated delta rule")
    _close(so[0, 0], rM, 1e-12, "S=1 state vs textbook")
    for (D, S, F) in [(8, 4, 5), (16, 32, 3)]:
        q, k, v, g, bt = _inputs(rng, 1, 1, D, S, F)
        M0 = rng.standard_normal((1, 1, D, D))
        o, so = oracle.forward(q, k, v, g, bt, M0, lib=lib)
        ro, rM = gram_form(q[0, 0], k[0, 0], v[0, 0], g[0, 0], bt[0, 0], S,
                           1.0 / np.sqrt(D * S), M0[0, 0])
        _close(o[0, 0], ro, 1e-12, "Gram form output D=%d S=%d" % (D, S))
        _close(so[0, 0], rM, 1e-12, "Gram form state D=%d S=%d" % (D, S))


# --------------------------------------------------------------------------- brute force
def brute_force_tokens(q, k, v, g, bt, S, c, use_delta, M0):
    """Pure-Python loops, token by token; every token of a frame sees the frozen old state."""
    T, D = len(q), len(q[0])
    M = [list(row) for row in M0]
    o = [[0.0] * D for _ in range(T)]
    for f in range(T // S):
        old = [list(row) for row in M]
        add = [[0.0] * D for _ in range(D)]
        for s in range(f * S, (f + 1) * S):
            kk = [c * x for x in k[s]]
            for j in range(D):
                pred = sum(kk[i] * old[i][j] for i in range(D))
                res = v[s][j] - (g[f] * pred if use_delta else 0.0)
                for i in range(D):
                    add[i][j] += kk[i] * res
        for i in range(D):
            for j in range(D):
                M[i][j] = g[f] * old[i][j] + bt[f] * add[i][j]
        for s in range(f * S, (f + 1) * S):
            for j in range(D):
                o[s][j] = sum(q[s][i] * M[i][j] for i in range(D))
    return np.array(o), np.array(M)


def pin_brute_force(lib=None):
    rng = np.random.default_rng(15)
    for use_delta in (True, False):
        D, S, F = 3, 2, 4
        q, k, v, g, bt = _inputs(rng, 1, 1, D, S, F)
        M0 = rng.standard_normal((1, 1, D, D))
        o, so = oracle.forward(q, k, v, g, bt, M0, use_delta=use_delta, lib=lib)
        ro, rM = brute_force_tokens(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                    g[0, 0].tolist(), bt[0, 0].tolist(), S,
                                    1.0 / np.sqrt(D * S), use_delta, M0[0, 0].tolist())
        _close(o[0, 0], ro, 1e-12, "brute force output")
        _close(so[0, 0], rM, 1e-12, "brute force state")
        if use_delta:
            # frame-wise is not the token-sequential rule when S > 1
            to, _ = textbook_gated_delta(q[0, 0], k[0, 0], v[0, 0],
                                         np.repeat(g[0, 0], S), np.repeat(bt[0, 0], S),
                                         1.0 / np.sqrt(D * S), M0[0, 0])
            assert _rel(o[0, 0], to) > 1e-6, "frame-wise result equals token-wise result"


# --------------------------------------------------------------------------- norms
def pin_norm_bound(lib=None):
    rng = np.random.default_rng(16)
    D, S, F = 8, 16, 20
    c = 1.0 / np.sqrt(D * S)
    q, k, v, g, bt = _inputs(rng, 1, 1, D, S, F, beta=(0.5, 1.0))
    M = 50.0 * rng.standard_normal((1, 1, D, D))
    for f in range(F):
        sl = slice(f * S, (f + 1) * S)
        Kt = c * k[0, 0, sl]
        assert bt[0, 0, f] * np.sum(Kt * Kt) <= 2.0, "scaled keys too large for the bound"
        _, Mn = oracle.step(q[:, :, sl], k[:, :, sl], v[:, :, sl], g[:, :, f], bt[:, :, f], M,
                            lib=lib)
        bound = g[0, 0, f] * np.linalg.norm(M) + bt[0, 0, f] * np.linalg.norm(Kt.T @ v[0, 0, sl])
        assert np.all(np.isfinite(Mn)), "non-finite state"
        assert np.linalg.norm(Mn) <= bound * (1 + 1e-12), "state norm above bound at frame %d" % f
        M = Mn


# --------------------------------------------------------------------------- special cases
def pin_special_cases(lib=None):
    rng = np.random.default_rng(17)
    D, S, F = 5, 3, 4
    c = 1.0 / np.sqrt(D * S)
    for use_delta in (True, False):
        q, k, v, g, _ = _inputs(rng, 1, 1, D, S, F)
        M0 = rng.standard_normal((1, 1, D, D))
        o, so = oracle.forward(q, k, v, g, np.zeros_like(g), M0, use_delta=use_delta, lib=lib)
        for f in range(F):
            Mf = np.prod(g[0, 0, :f + 1]) * M0[0, 0]
            _close(o[0, 0, f * S:(f + 1) * S], q[0, 0, f * S:(f + 1) * S] @ Mf, 1e-12,
                   "beta=0 pure decay")
        _close(so[0, 0], np.prod(g[0, 0]) * M0[0, 0], 1e-12, "beta=0 final state")
        q, k, v, g, bt = _inputs(rng, 1, 1, D, S, 1)
        o, _ = oracle.forward(q, k, v, g, bt, None, use_delta=use_delta, lib=lib)
        _close(o[0, 0], bt[0, 0, 0] * q[0, 0] @ (c * k[0, 0]).T @ v[0, 0], 1e-12,
               "single frame from zero state")


def pin_step_equals_forward(lib=None):
    rng = np.random.default_rng(18)
    B, H, D, S, F = 2, 3, 4, 5, 6
    q, k, v, g, bt = _inputs(rng, B, H, D, S, F)
    M0 = rng.standard_normal((B, H, D, D))
    o, so = oracle.forward(q, k, v, g, bt, M0, lib=lib)
    M = M0
    for f in range(F):
        sl = slice(f * S, (f + 1) * S)
        o_nc, none = oracle.step(q[:, :, sl], k[:, :, sl], v[:, :, sl], g[:, :, f], bt[:, :, f],
                                 M, commit=False, lib=lib)
        assert none is None
        of, M = oracle.step(q[:, :, sl], k[:, :, sl], v[:, :, sl], g[:, :, f], bt[:, :, f], M,
                            lib=lib)
        _close(of, o[:, :, sl], 1e-12, "step output vs forward")
        _close(o_nc, of, 0.0, "uncommitted step output")
    _close(M, so, 1e-12, "chained step state vs forward")


def pin_linearity(lib=None):
    rng = np.random.default_rng(19)
    B, H, D, S, F = 1, 2, 6, 4, 5
    for use_delta in (True, False):
        q, k, v1, g, bt = _inputs(rng, B, H, D, S, F)
        v2 = rng.standard_normal(v1.shape)
        q2 = rng.standard_normal(q.shape)
        M1 = rng.standard_normal((B, H, D, D))
        M2 = rng.standard_normal((B, H, D, D))
        run = lambda qq, vv, MM: oracle.forward(qq, k, vv, g, bt, MM, use_delta=use_delta,
                                                lib=lib)
        oa, sa = run(q, v1, M1)
        ob, sb = run(q, v2, M2)
        oc, sc = run(q, v1 + 2 * v2, M1 + 2 * M2)
        _close(oc, oa + 2 * ob, 1e-12, "linearity in (V, M0): output")
        _close(sc, sa + 2 * sb, 1e-12, "linearity in (V, M0): state")
        od, _ = run(q2, v1, M1)
        oe, _ = run(q + 3 * q2, v1, M1)
        _close(oe, oa + 3 * od, 1e-12, "linearity in Q")
        perm = rng.permutation(D)
        op, sp = run(q, v1[..., perm], M1[..., perm])
        _close(op, oa[..., perm], 1e-12, "value-column permutation: output")
        _close(sp, sa[..., perm], 1e-12, "value-column permutation: state")


ALL_PINS = [pin_golden, pin_block_causal, pin_gated_nodelta, pin_delta_identity, pin_textbook,
            pin_brute_force, pin_norm_bound, pin_special_cases, pin_step_equals_forward,
            pin_linearity]
