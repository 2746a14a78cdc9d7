"""Pins of the backward (gradient) oracle, on the CPU.

The pages define the forward recurrence only; its gradients are plain calculus. The backward
oracle (oracle/gdn_oracle.c, gdn_oracle_backward) is pinned here by things it does not share:
  * central finite differences of the forward oracle (itself pinned by tests/pins.py) for every
    input: Q, K, V, gamma, beta and the initial state, with and without the delta term,
    default and explicit key scale, with and without an upstream state gradient;
  * a closed form for one frame without the delta term, written with numpy matrix products;
  * linearity in the upstream gradients (dO, dstate_out);
  * a mutation test: plausible mistakes planted in a copy of the backward code each fail one of
    the checks above.
"""
import numpy as np
import pytest

import oracle

LOSS_TOL = 2e-7    # finite differences (h = 1e-6, fp64): observed ~1e-9


def _inputs(rng, B, H, D, S, F, with_state=True):
    q, k, v = (rng.standard_normal((B, H, F * S, D)) for _ in range(3))
    g = rng.uniform(0.8, 1.0, (B, H, F))
    b = rng.uniform(0.2, 0.9, (B, H, F))
    s0 = 0.3 * rng.standard_normal((B, H, D, D)) if with_state else None
    d_o = rng.standard_normal((B, H, F * S, D))
    d_m = rng.standard_normal((B, H, D, D))
    return q, k, v, g, b, s0, d_o, d_m


def _fd_grads(args, d_o, d_m, use_delta, key_scale, h=1e-6):
    """Central differences of L = <dO, O> + <dM, state_out> for every element of every input."""
    def loss(a):
        o, m = oracle.forward(*a, use_delta=use_delta, key_scale=key_scale)
        return float((o * d_o).sum() + (0.0 if d_m is None else (m * d_m).sum()))

    out = []
    for ai, a in enumerate(args):
        if a is None:
            out.append(None)
            continue
        num = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            ap = [None if x is None else x.copy() for x in args]
            am = [None if x is None else x.copy() for x in args]
            ap[ai][idx] += h
            am[ai][idx] -= h
            num[idx] = (loss(ap) - loss(am)) / (2 * h)
        out.append(num)
    return out


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def check_against_fd(lib, seed, use_delta, with_state, with_dm, key_scale, shape=(1, 2, 3, 2, 3)):
    rng = np.random.default_rng(seed)
    B, H, D, S, F = shape
    q, k, v, g, b, s0, d_o, d_m = _inputs(rng, B, H, D, S, F, with_state)
    if not with_dm:
        d_m = None
    got = oracle.backward(q, k, v, g, b, s0, d_o, d_m, use_delta=use_delta, key_scale=key_scale,
                          lib=lib)
    num = _fd_grads([q, k, v, g, b, s0 if with_state else np.zeros((B, H, D, D))], d_o, d_m,
                    use_delta, key_scale)
    names = ["dq", "dk", "dv", "dgamma", "dbeta", "dstate_in"]
    return {n: _rel(got[i], num[i]) for i, n in enumerate(names)}


CASES = [
    # seed, use_delta, with_state, with_dm, key_scale
    (1, True, True, True, None),
    (2, True, False, False, None),
    (3, False, True, True, None),
    (4, False, False, True, 0.37),
    (5, True, True, False, 0.61),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_backward_matches_finite_differences(case):
    errs = check_against_fd(None, *case)
    assert max(errs.values()) <= LOSS_TOL, errs


def test_backward_finite_differences_longer_chain():
    # more frames than key dims and tokens, so errors in the gradient chain compound
    errs = check_against_fd(None, 9, True, True, True, None, shape=(1, 1, 2, 3, 6))
    assert max(errs.values()) <= LOSS_TOL, errs


def test_backward_closed_form_one_frame_no_delta():
    # One frame, no delta term: M_1 = gamma M_0 + beta c K^T V and O = Q M_1, so with
    # G = Q^T dO + dM: dQ = dO M_1^T, dV = beta c K G, dK = beta c V G^T, dgamma = <G, M_0>,
    # dbeta = <G, c K^T V>, dM_0 = gamma G.
    rng = np.random.default_rng(21)
    D, S = 5, 7
    q, k, v, g, b, s0, d_o, d_m = _inputs(rng, 1, 1, D, S, 1)
    c = 1.0 / np.sqrt(D * S)
    Q, K, V, dO, M0, dM = q[0, 0], k[0, 0], v[0, 0], d_o[0, 0], s0[0, 0], d_m[0, 0]
    gg, bb = g[0, 0, 0], b[0, 0, 0]
    M1 = gg * M0 + bb * c * K.T @ V
    G = Q.T @ dO + dM
    want = [dO @ M1.T, bb * c * V @ G.T, bb * c * K @ G, np.sum(G * M0), np.sum(G * (c * K.T @ V)),
            gg * G]
    got = oracle.backward(q, k, v, g, b, s0, d_o, d_m, use_delta=False)
    got = [got[0][0, 0], got[1][0, 0], got[2][0, 0], got[3][0, 0, 0], got[4][0, 0, 0], got[5][0, 0]]
    for w, x in zip(want, got):
        np.testing.assert_allclose(x, w, rtol=1e-12, atol=1e-12)


def test_backward_linear_in_upstream_gradients():
    rng = np.random.default_rng(22)
    q, k, v, g, b, s0, d_o, d_m = _inputs(rng, 2, 2, 4, 3, 4)
    d_o2 = rng.standard_normal(d_o.shape)
    d_m2 = rng.standard_normal(d_m.shape)
    a = oracle.backward(q, k, v, g, b, s0, d_o, d_m)
    c_ = oracle.backward(q, k, v, g, b, s0, d_o2, d_m2)
    s = oracle.backward(q, k, v, g, b, s0, 2.0 * d_o + d_o2, 2.0 * d_m + d_m2)
    for x, y, z in zip(a, c_, s):
        np.testing.assert_allclose(z, 2.0 * x + y, rtol=1e-10, atol=1e-10)


MUTANTS = {
    # name: (original text, planted mistake)
    "dgamma without the residual term": ("dg -= dR[e] * P[e];", "(void)0;"),
    "no decay in the gradient chain": ("Gp[e] = g * G[e];", "Gp[e] = G[e];"),
    "dU transposed in dKt": ("acc += R[(size_t)s * D + j] * dU[(size_t)i * D + j];",
                             "acc += R[(size_t)s * D + j] * dU[(size_t)j * D + i];"),
    "sign of the prediction adjoint": ("acc += -g * dR[(size_t)s * D + j] * M[(size_t)i * D + j];",
                                       "acc += g * dR[(size_t)s * D + j] * M[(size_t)i * D + j];"),
    "key scale missing in dK": ("dk[(size_t)f * S * D + e] = c * dKt[e];",
                                "dk[(size_t)f * S * D + e] = dKt[e];"),
    "beta missing in dU": ("dU[e] = bt * G[e];", "dU[e] = G[e];"),
    "dQ from the state before the frame": (
        "acc += dOf[(size_t)s * D + j] * Mf[(size_t)i * D + j];",
        "acc += dOf[(size_t)s * D + j] * M[(size_t)i * D + j];"),
    "later frames' gradient dropped": ("G[(size_t)i * D + j] += acc;", "G[(size_t)i * D + j] = acc;"),
    "prediction path left out of the state gradient": (
        "for (int s = 0; s < S; ++s) acc += Kt[(size_t)s * D + i] * (-g * dR[(size_t)s * D + j]);",
        "for (int s = 0; s < S; ++s) acc += 0.0 * Kt[(size_t)s * D + i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutants_are_caught(name, tmp_path):
    src = oracle.source_text()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor must be unique: " + old
    lib = oracle.load_variant(src.replace(old, new), str(tmp_path))
    caught = False
    for case in CASES[:3]:
        errs = check_against_fd(lib, *case)
        if max(errs.values()) > 1e-4:
            caught = True
            break
    assert caught, "planted mistake not caught: " + name
