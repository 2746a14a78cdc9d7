"""Pins of the 8-bit-input (E4M3) oracle, on the CPU.

The pages name low-precision inputs for the GDN kernel (mixed-precision quantisation fused with
the kernel: jefxiong.cn daily digest, SANA-Streaming item, contribution (3)) without a format;
the format here is OCP FP8 E4M3 with one scale per (b, h, f) and tensor. The oracle
(oracle/gdn_oracle.c, gdn_oracle_e4m3 and gdn_oracle_forward_fp8) is pinned by things it does
not share:
  * values of the E4M3 encoding fixed by the OCP 8-bit floating point specification (zero,
    smallest subnormal, largest subnormal, smallest normal, one, largest normal, NaN, signs);
  * every one of the 256 codes against torch's own float8_e4m3fn decoding;
  * the fp8 forward against the (separately pinned) fp64 forward run on values decoded by
    torch and scaled in numpy;
  * metamorphic relations of the scales: the output is linear in q_scale; a k_scale factor a
    and a key_scale factor 1/a cancel; v_scale scales everything when there is no initial
    state and no delta term; a scale acts only on its own (b, h, f);
  * planted mistakes in the fp8 part of the C source, each caught by one of the above.
"""
import math

import numpy as np
import pytest
import torch

import oracle

# code -> value, from the E4M3 row of the OCP 8-bit floating point specification
SPEC = {
    0x00: 0.0, 0x80: -0.0,
    0x01: 2.0 ** -9,            # smallest subnormal
    0x07: 7 * 2.0 ** -9,        # largest subnormal (0.875 * 2^-6)
    0x08: 2.0 ** -6,            # smallest normal
    0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0xB8: -1.0,
    0x77: 240.0, 0x78: 256.0,
    0x7E: 448.0, 0xFE: -448.0,  # largest normal
    0x7F: math.nan, 0xFF: math.nan,
}


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_spec(lib=None):
    bad = []
    for code, want in SPEC.items():
        got = oracle.e4m3_value(code, lib=lib)
        if math.isnan(want):
            ok = math.isnan(got)
        else:
            ok = got == want and math.copysign(1.0, got) == math.copysign(1.0, want)
        if not ok:
            bad.append((hex(code), got, want))
    return bad


def check_all_codes(lib=None):
    ours = np.array([oracle.e4m3_value(c, lib=lib) for c in range(256)])
    ref = torch_decode(np.arange(256))
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    return [hex(c) for c in np.nonzero(~same)[0]]


def test_spec_values():
    assert check_spec() == []


def test_every_code_matches_torch():
    assert check_all_codes() == []


def test_positive_codes_increase():
    v = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(v, v[1:]))


def make_inputs(rng, B, H, D, S, F, with_state=True):
    codes = [rng.integers(0, 256, (B, H, F * S, D), dtype=np.uint8) for _ in range(3)]
    for c in codes:   # no NaN codes
        c[(c & 0x7F) == 0x7F] = 0x38
    scales = [rng.uniform(0.01, 0.2, (B, H, F)) for _ in range(3)]
    g = rng.uniform(0.8, 1.0, (B, H, F))
    b = rng.uniform(0.1, 0.9, (B, H, F))
    s0 = 0.3 * rng.standard_normal((B, H, D, D)) if with_state else None
    return codes, scales, g, b, s0


def values(codes, scale, S):
    """codes [B, H, F*S, D] decoded by torch, times the scale of each token's frame."""
    return torch_decode(codes) * np.repeat(scale, S, axis=2)[..., None]


def check_forward(lib, seed, use_delta, with_state, shape=(1, 2, 8, 5, 4)):
    rng = np.random.default_rng(seed)
    B, H, D, S, F = shape
    codes, scales, g, b, s0 = make_inputs(rng, B, H, D, S, F, with_state)
    got = oracle.forward_fp8(*codes, *scales, g, b, s0, use_delta=use_delta, lib=lib)
    want = oracle.forward(*(values(c, s, S) for c, s in zip(codes, scales)), g, b, s0,
                          use_delta=use_delta)
    return max(float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-30))
               for x, y in zip(got, want))


FWD_CASES = [(1, True, True), (2, False, True), (3, True, False)]


@pytest.mark.parametrize("case", FWD_CASES, ids=[str(c) for c in FWD_CASES])
def test_forward_fp8_equals_forward_on_decoded_values(case):
    assert check_forward(None, *case) <= 1e-12


def _run(codes, scales, g, b, s0, **kw):
    return oracle.forward_fp8(*codes, *scales, g, b, s0, **kw)


def test_linear_in_q_scale():
    rng = np.random.default_rng(11)
    codes, scales, g, b, s0 = make_inputs(rng, 1, 2, 8, 5, 4)
    o1, m1 = _run(codes, scales, g, b, s0)
    o2, m2 = _run(codes, [2.5 * scales[0], scales[1], scales[2]], g, b, s0)
    np.testing.assert_allclose(o2, 2.5 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(m2, m1)


def test_key_scale_and_k_scale_cancel():
    rng = np.random.default_rng(12)
    D, S = 8, 5
    codes, scales, g, b, s0 = make_inputs(rng, 1, 2, D, S, 4)
    c = 1.0 / math.sqrt(D * S)
    o1, m1 = _run(codes, scales, g, b, s0, key_scale=c)
    o2, m2 = _run(codes, [scales[0], 3.0 * scales[1], scales[2]], g, b, s0, key_scale=c / 3.0)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(m2, m1, rtol=1e-10, atol=1e-12)


def test_v_scale_scales_everything_without_delta_and_initial_state():
    rng = np.random.default_rng(13)
    codes, scales, g, b, _ = make_inputs(rng, 1, 2, 8, 5, 4, with_state=False)
    o1, m1 = _run(codes, scales, g, b, None, use_delta=False)
    o2, m2 = _run(codes, [scales[0], scales[1], 0.5 * scales[2]], g, b, None, use_delta=False)
    np.testing.assert_allclose(o2, 0.5 * o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(m2, 0.5 * m1, rtol=1e-12, atol=1e-12)


def check_scale_locality(lib=None):
    """A k_scale change at (b=0, h=1, f=2) leaves head 0 and frames 0-1 of head 1 unchanged
    and changes frame 2 of head 1. Returns the list of violations."""
    rng = np.random.default_rng(14)
    S = 5
    codes, scales, g, b, s0 = make_inputs(rng, 1, 2, 8, S, 4)
    o1, _ = oracle.forward_fp8(*codes, *scales, g, b, s0, lib=lib)
    ks = scales[1].copy()
    ks[0, 1, 2] *= 1.7
    o2, _ = oracle.forward_fp8(codes[0], codes[1], codes[2], scales[0], ks, scales[2], g, b, s0,
                               lib=lib)
    bad = []
    if not np.array_equal(o1[0, 0], o2[0, 0]):
        bad.append("head 0 changed")
    if not np.array_equal(o1[0, 1, :2 * S], o2[0, 1, :2 * S]):
        bad.append("earlier frames changed")
    if np.array_equal(o1[0, 1, 2 * S:3 * S], o2[0, 1, 2 * S:3 * S]):
        bad.append("frame 2 unchanged")
    return bad


def test_scale_acts_on_its_own_frame():
    assert check_scale_locality() == []


MUTANTS = {
    # name: (original text, planted mistake)
    "exponent bias 8": ("mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    "subnormals read as normals": ("mag = ldexp((double)m, -9);", "mag = ldexp(1.0 + m / 8.0, -6);"),
    "NaN code read as a number": ("if (e == 15 && m == 7)\n        return NAN;",
                                  "if (e == 15 && m == 7 && 0)\n        return NAN;"),
    "sign dropped": ("return sgn ? -mag : mag;", "return mag;"),
    "one scale per head": ("const size_t frame = e / ((size_t)S * D);",
                           "const size_t frame = e / ((size_t)F * S * D);"),
    "k scale on v": ("v[e] = v_scale[frame] * gdn_oracle_e4m3(v8[e]);",
                     "v[e] = k_scale[frame] * gdn_oracle_e4m3(v8[e]);"),
    "q scale missing": ("q[e] = q_scale[frame] * gdn_oracle_e4m3(q8[e]);",
                        "q[e] = gdn_oracle_e4m3(q8[e]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutants_are_caught(name, tmp_path):
    src = oracle.source_text()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor must be unique: " + old
    lib = oracle.load_variant(src.replace(old, new), str(tmp_path))
    caught = bool(check_spec(lib)) or bool(check_all_codes(lib)) or bool(check_scale_locality(lib))
    if not caught:
        caught = any(check_forward(lib, *c) > 1e-6 for c in FWD_CASES)
    assert caught, "planted mistake not caught: " + name
