"""Oracle of the block-causal temporal convolution with a last-token cache (fp64, numpy).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may use this module; the GPU library shares no code with it.

The op (SANA-Video talk, shadowingenglish.com, passage on the causal FFN with temporal conv):
SANA's spatial-temporal Mix-FFN convolves along time. Video is generated block by block; so
that a block cannot see the next one, training pads a zero token between consecutive blocks,
and so that a block still sees the previous one, the last token of block i is carried in as the
first token of block i + 1; the padding and carried tokens are removed after the convolution.
In streaming generation the carried token is a cache: the last frame of the previous block.

Readings (the pages give no kernel size, layout or channel count): a depthwise convolution over
latent frames with kernel size 3, centred (taps on frames t - 1, t, t + 1), zero padding, one
set of taps and a bias per channel, applied independently at every spatial token; a "token" of
the temporal axis is one latent frame. x: [B, T, S, C]; weight: [C, 3]; bias: [C] or None.
"""
from __future__ import annotations

import numpy as np


def _conv3(seq, weight, bias):
    """Plain centred depthwise conv, kernel 3, zero padding, over axis 1 of [B, n, S, C]."""
    B, n, S, C = seq.shape
    pad = np.zeros((B, n + 2, S, C))
    pad[:, 1:n + 1] = seq
    out = (weight[:, 0] * pad[:, 0:n] + weight[:, 1] * pad[:, 1:n + 1]
           + weight[:, 2] * pad[:, 2:n + 2])
    if bias is not None:
        out = out + bias
    return out


def tconv_sequence(x, weight, bias, block_frames, cache_in=None):
    """Training form: the whole sequence x [B, T, S, C] in blocks of `block_frames` frames.

    Builds the padded sequence of the pages -- block 0, then for every later block a zero
    token, the carried last token of the block before it, and the block itself -- runs one
    plain convolution over it and keeps only the outputs of the real frames. cache_in
    [B, S, C] stands for a block before the sequence (None: there is none). Returns (y [B, T,
    S, C], cache_out [B, S, C] = the last frame of the sequence)."""
    x = np.asarray(x, np.float64)
    weight = np.asarray(weight, np.float64)
    bias = None if bias is None else np.asarray(bias, np.float64)
    B, T, S, C = x.shape
    assert T % block_frames == 0, "a whole number of blocks"
    parts, keep = [], []
    pos = 0
    if cache_in is not None:           # the carried token of the block before the sequence
        parts.append(np.asarray(cache_in, np.float64)[:, None])
        pos += 1
    for i in range(T // block_frames):
        blk = x[:, i * block_frames:(i + 1) * block_frames]
        if i > 0:
            parts.append(np.zeros((B, 1, S, C)))            # the zero token between blocks
            parts.append(x[:, i * block_frames - 1][:, None])  # carried last token of block i - 1
            pos += 2
        parts.append(blk)
        keep.extend(range(pos, pos + block_frames))
        pos += block_frames
    seq = np.concatenate(parts, axis=1)
    # within the padded sequence every block but the last must end before a zero token; the
    # last one ends at the sequence end, where the conv's own zero padding plays that role
    y = _conv3(seq, weight, bias)[:, keep]
    return y, x[:, T - 1].copy()


def tconv_stream(x, weight, bias, block_frames, cache_in=None):
    """Streaming form: one block at a time, each from the cache left by the block before it
    (zeros before the first block). Returns (y, cache_out) like tconv_sequence."""
    x = np.asarray(x, np.float64)
    weight = np.asarray(weight, np.float64)
    bias = None if bias is None else np.asarray(bias, np.float64)
    B, T, S, C = x.shape
    cache = np.zeros((B, S, C)) if cache_in is None else np.asarray(cache_in, np.float64)
    y = np.empty_like(x)
    for i in range(T // block_frames):
        blk = x[:, i * block_frames:(i + 1) * block_frames]
        for t in range(block_frames):
            left = cache if t == 0 else blk[:, t - 1]
            right = blk[:, t + 1] if t + 1 < block_frames else np.zeros((B, S, C))
            out = weight[:, 0] * left + weight[:, 1] * blk[:, t] + weight[:, 2] * right
            y[:, i * block_frames + t] = out if bias is None else out + bias
        cache = blk[:, block_frames - 1].copy()
    return y, cache
