"""CPU oracle against its pins, and planted mistakes against the pins."""
import tempfile

import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin_streaming_variant(pin):
    # the frame-streaming numpy variant used for full-length workloads
    pin(lib="numpy")


def test_streaming_variant_keeps_selected_frames():
    from oracle import stream
    rng = np.random.default_rng(4)
    D, S, F = 8, 6, 7
    q, k, v = (rng.standard_normal((1, 1, F * S, D)) for _ in range(3))
    g = rng.uniform(0.9, 1, (1, 1, F))
    b = rng.uniform(0, 1, (1, 1, F))
    ref, ref_s = oracle.forward(q, k, v, g, b)

    def src(f):
        sl = slice(f * S, (f + 1) * S)
        return q[0, 0, sl], k[0, 0, sl], v[0, 0, sl], g[0, 0, f], b[0, 0, f]
    outs, M = stream.forward_frames(src, F, D, S, keep={0, 6})
    assert sorted(outs) == [0, 6]
    assert np.allclose(outs[6], ref[0, 0, 6 * S:], rtol=0, atol=1e-12)
    assert np.allclose(M, ref_s[0, 0], rtol=0, atol=1e-12)


def test_oracle_rejects_bad_sizes():
    z = np.zeros((1, 1, 4, 2))
    g = np.ones((1, 1, 2))
    with pytest.raises(AssertionError):
        oracle.forward(z[:, :, :3], z[:, :, :3], z[:, :, :3], g, g)


def test_oracle_threads_do_not_change_result():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((2, 3, 12, 4)) for _ in range(3))
    g = rng.uniform(0.9, 1, (2, 3, 3))
    b = rng.uniform(0, 1, (2, 3, 3))
    o1, s1 = oracle.forward(q, k, v, g, b, nthreads=1)
    o4, s4 = oracle.forward(q, k, v, g, b, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)


# Planted mistakes: (description, text in gdn_oracle.c, replacement). Every one of them must
# be caught by at least one pin.
MUTANTS = [
    ("gamma dropped from the prediction", "- g * P[(size_t)s * D + j]", "- P[(size_t)s * D + j]"),
    ("sign of the delta term flipped", "- g * P[(size_t)s * D + j]", "+ g * P[(size_t)s * D + j]"),
    ("delta term dropped", "use_delta ? Vf[(size_t)s * D + j] - g", "0 ? Vf[(size_t)s * D + j] - g"),
    ("decay dropped", "g * M[(size_t)i * D + j] + bt", "M[(size_t)i * D + j] + bt"),
    ("beta dropped", "+ bt * U[(size_t)i * D + j]", "+ U[(size_t)i * D + j]"),
    ("beta applied to the old state", "g * M[(size_t)i * D + j] + bt * U",
     "bt * g * M[(size_t)i * D + j] + U"),
    ("state transposed in the output", "Qf[(size_t)s * D + i] * M[(size_t)i * D + j]",
     "Qf[(size_t)s * D + i] * M[(size_t)j * D + i]"),
    ("state transposed in the prediction", "Kt[(size_t)s * D + i] * M[(size_t)i * D + j]",
     "Kt[(size_t)s * D + i] * M[(size_t)j * D + i]"),
    ("key scale dropped", "c * Kf[(size_t)s * D + i]", "Kf[(size_t)s * D + i]"),
    ("unscaled keys in the write", "acc += Kt[(size_t)s * D + i] * R", "acc += Kf[(size_t)s * D + i] * R"),
    ("default key scale 1/sqrt(D)", "1.0 / sqrt((double)D * (double)S)", "1.0 / sqrt((double)D)"),
    ("default key scale 1/S", "1.0 / sqrt((double)D * (double)S)", "1.0 / (double)S"),
    ("initial state ignored", "if (state_in) memcpy", "if (0) memcpy"),
    ("query read from the key", "acc += Qf[(size_t)s * D + i]", "acc += Kf[(size_t)s * D + i]"),
    ("value columns reversed in the residual", "Vf[(size_t)s * D + j] - g",
     "Vf[(size_t)s * D + (D - 1 - j)] - g"),
    ("gates of the next frame", "const double g = gamma[f];", "const double g = gamma[f + 1 < F ? f + 1 : f];"),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant):
    _, old, new = mutant
    src = oracle.source_text()
    # plant the mistake in the forward code only (the backward section repeats some lines)
    cut = src.index("/*\n * Backward (gradients) of the forward")
    fwd, rest = src[:cut], src[cut:]
    assert fwd.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.load_variant(fwd.replace(old, new) + rest, tmp)
        caught = []
        for pin in pins.ALL_PINS:
            try:
                pin(lib=lib)
            except (AssertionError, RuntimeError, IndexError, ValueError):
                caught.append(pin.__name__)
        assert caught, "no pin catches: " + mutant[0]
