"""Pins of the block-causal temporal-conv oracle (oracle/tconv.py), on the CPU.

The pages describe the op in words (SANA-Video talk, passage on the causal FFN with temporal
conv); the oracle's training form follows that recipe literally. It is pinned by things it does
not share:
  * the streaming form (cache of the previous block's last frame) gives the same result;
  * closed forms for unit taps: identity plus bias, shift by one frame with the carried frame at
    block starts, shift the other way with zeros at block ends;
  * a single block without cache is numpy's np.convolve in 'same' mode on every (s, c) series;
  * causality: changing later blocks leaves earlier blocks' outputs alone, and the cache_out
    is the last frame;
  * planted mistakes in a copy of the oracle's source, each caught by one of the above.
"""
import os

import numpy as np
import pytest

from oracle import tconv

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "tconv.py")


def data(rng, B=2, T=6, S=3, C=4):
    x = rng.standard_normal((B, T, S, C))
    w = rng.standard_normal((C, 3))
    bias = rng.standard_normal(C)
    cache = rng.standard_normal((B, S, C))
    return x, w, bias, cache


def check_stream(mod, seed=1):
    rng = np.random.default_rng(seed)
    x, w, bias, cache = data(rng)
    worst = 0.0
    for tb in (1, 2, 3, 6):
        for ci in (None, cache):
            for bi in (None, bias):
                a, ca = mod.tconv_sequence(x, w, bi, tb, ci)
                b, cb = mod.tconv_stream(x, w, bi, tb, ci)
                worst = max(worst, float(np.abs(a - b).max()), float(np.abs(ca - cb).max()))
    return worst


def check_closed_forms(mod):
    """Returns a list of violated closed forms (both forms of the module are checked)."""
    rng = np.random.default_rng(2)
    x, _, bias, cache = data(rng, T=6)
    C = x.shape[3]
    bad = []
    for fn in (mod.tconv_sequence, mod.tconv_stream):
        for tb in (1, 2, 3):
            ident = np.tile([0.0, 1.0, 0.0], (C, 1))
            y, c_out = fn(x, ident, bias, tb, cache)
            if not np.allclose(y, x + bias, atol=1e-14):
                bad.append((fn.__name__, tb, "identity"))
            if not np.array_equal(c_out, x[:, -1]):
                bad.append((fn.__name__, tb, "cache_out"))
            left = np.tile([1.0, 0.0, 0.0], (C, 1))
            y, _ = fn(x, left, None, tb, cache)
            want = np.concatenate([cache[:, None], x[:, :-1]], axis=1)   # carried at block starts
            if not np.allclose(y, want, atol=1e-14):
                bad.append((fn.__name__, tb, "left tap"))
            y, _ = fn(x, left, None, tb, None)
            want = np.concatenate([np.zeros_like(cache)[:, None], x[:, :-1]], axis=1)
            if not np.allclose(y, want, atol=1e-14):
                bad.append((fn.__name__, tb, "left tap, no cache"))
            right = np.tile([0.0, 0.0, 1.0], (C, 1))
            y, _ = fn(x, right, None, tb, cache)
            want = np.concatenate([x[:, 1:], np.zeros_like(cache)[:, None]], axis=1)
            want[:, tb - 1::tb] = 0.0                                      # zero at block ends
            if not np.allclose(y, want, atol=1e-14):
                bad.append((fn.__name__, tb, "right tap"))
    return bad


def check_textbook(mod):
    rng = np.random.default_rng(3)
    x, w, bias, _ = data(rng, B=1, T=7, S=2, C=3)
    y, _ = mod.tconv_sequence(x, w, bias, 7, None)
    ref = np.empty_like(x)
    for s in range(2):
        for c in range(3):
            # correlation with taps (t-1, t, t+1) is convolution with the reversed taps
            ref[0, :, s, c] = np.convolve(x[0, :, s, c], w[c, ::-1], mode="same") + bias[c]
    return float(np.abs(y - ref).max())


def check_causal(mod):
    rng = np.random.default_rng(4)
    x, w, bias, cache = data(rng, T=6)
    y1, _ = mod.tconv_sequence(x, w, bias, 2, cache)
    x2 = x.copy()
    x2[:, 4:] += 1.0                     # change the last block only
    y2, _ = mod.tconv_sequence(x2, w, bias, 2, cache)
    return bool(np.array_equal(y1[:, :4], y2[:, :4])) and not np.array_equal(y1[:, 4:], y2[:, 4:])


def test_sequence_equals_stream():
    assert check_stream(tconv) <= 1e-13


def test_closed_forms():
    assert check_closed_forms(tconv) == []


def test_single_block_is_numpy_convolve():
    assert check_textbook(tconv) <= 1e-13


def test_later_blocks_do_not_reach_back():
    assert check_causal(tconv)


MUTANTS = {
    # name: (original text, planted mistake)
    "no zero token between blocks": ("            parts.append(np.zeros((B, 1, S, C)))            # the zero token between blocks\n",
                                     ""),
    "no carried token": ("            parts.append(x[:, i * block_frames - 1][:, None])  # carried last token of block i - 1\n            pos += 2",
                         "            pos += 1"),
    "taps reversed": ("    out = (weight[:, 0] * pad[:, 0:n] + weight[:, 1] * pad[:, 1:n + 1]\n           + weight[:, 2] * pad[:, 2:n + 2])",
                      "    out = (weight[:, 2] * pad[:, 0:n] + weight[:, 1] * pad[:, 1:n + 1]\n           + weight[:, 0] * pad[:, 2:n + 2])"),
    "cache is the first frame": ("    return y, x[:, T - 1].copy()", "    return y, x[:, 0].copy()"),
    "stream: cache not carried": ("        cache = blk[:, block_frames - 1].copy()", "        cache = np.zeros((B, S, C))"),
    "stream: right neighbour leaks": ("            right = blk[:, t + 1] if t + 1 < block_frames else np.zeros((B, S, C))",
                                      "            right = x[:, i * block_frames + t + 1] if i * block_frames + t + 1 < T else np.zeros((B, S, C))"),
    "bias missing": ("    if bias is not None:\n        out = out + bias", "    if bias is not None:\n        out = out + 0.0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_tconv_mutants_are_caught(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor must be unique: " + old
    ns = {"__name__": "tconv_variant"}
    exec(compile(src.replace(old, new), "tconv_variant", "exec"), ns)

    class M:
        tconv_sequence = staticmethod(ns["tconv_sequence"])
        tconv_stream = staticmethod(ns["tconv_stream"])
    caught = False
    try:
        caught = (check_stream(M) > 1e-9 or check_closed_forms(M) != [] or check_textbook(M) > 1e-9
                  or not check_causal(M))
    except Exception:      # a mistake that breaks the shapes is caught too
        caught = True
    assert caught, "planted mistake not caught: " + name
