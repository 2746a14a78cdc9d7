"""Why the E4M3 forward equals the bf16 forward on the decoded values bit for bit, and when it
would not: a host emulation of how the output products group their k slots into instructions.

The fused forward forms O^T = M^T Q^T with v_mfma_f32_16x16x32_bf16: each instruction adds the
32 products of its k slots to its accumulator, and the fp32 result is rounded. The model here
rounds once per instruction (the exact sum of the exact products and the accumulator, rounded
to fp32); a second model adds the products one at a time in fp32. The bf16 path feeds Q
already scaled (s times the decoded code, exact in bf16 for a power-of-two s). The E4M3 path
feeds the decoded codes and scales the fp32 accumulator by s at the end. Scaling every product
and the accumulator by a power of two commutes with each rounding, so the two paths agree bit
for bit when both group the k slots into instructions the same way.

Loading 16 consecutive codes per lane (two k steps in one 16-byte load) regroups the slots:
step 2j then holds k = 64 j + 16 g + 0..7 for lane group g instead of 64 j + 8 g + 0..7, and
step 2j + 1 the next 8 codes of each group. Applied to one input type only, the two paths
round different partial sums and disagree in the last bits of some outputs, while both stay
within rounding of the exact product. That is the failure of the first 16-byte variant. The
kernel now uses the paired grouping for both input types (and for M^T).
"""
import math

import numpy as np
import pytest
import torch

D = 128
NATURAL = [[32 * ks + 8 * g + t for g in range(4) for t in range(8)] for ks in range(D // 32)]
PAIRED = [[64 * (ks // 2) + 16 * g + 8 * (ks % 2) + t for g in range(4) for t in range(8)]
          for ks in range(D // 32)]


def f32(x):
    return float(np.float32(x))


def bf16(x):
    """Round to bf16 (nearest even), as a Python float."""
    return float(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).float())


def e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def dot_fused(a, b, groups):
    """One output element: per instruction, the exactly rounded sum of its products and the
    accumulator, rounded to fp32."""
    acc = 0.0
    for grp in groups:
        acc = f32(math.fsum([acc] + [a[k] * b[k] for k in grp]))
    return acc


def dot_serial(a, b, groups):
    """The same, adding one product at a time in fp32 in slot order."""
    acc = 0.0
    for grp in groups:
        for k in grp:
            acc = f32(acc + f32(a[k] * b[k]))
    return acc


def cases(seed, n):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(n, D))
    codes[(codes & 0x7F) == 0x7F] = 0x38          # no NaN codes
    m = np.array([[bf16(x) for x in row] for row in rng.standard_normal((n, D)) * 0.05])
    return m, e4m3(codes)


def test_groupings_are_partitions():
    for grouping in (NATURAL, PAIRED):
        flat = sorted(k for grp in grouping for k in grp)
        assert flat == list(range(D))
        assert all(len(grp) == 32 for grp in grouping)
    assert NATURAL != PAIRED


@pytest.mark.parametrize("dot", [dot_fused, dot_serial], ids=["fused", "serial"])
@pytest.mark.parametrize("grouping", [NATURAL, PAIRED], ids=["natural", "paired"])
def test_power_of_two_scale_commutes_with_a_shared_grouping(dot, grouping):
    s = 2.0 ** -4
    m, q = cases(1, 64)
    for i in range(m.shape[0]):
        q_bf16 = [bf16(s * x) for x in q[i]]
        assert all(qb == s * x for qb, x in zip(q_bf16, q[i]))   # exact in bf16
        o_bf16 = dot(m[i], q_bf16, grouping)
        o_fp8 = f32(dot(m[i], q[i], grouping) * s)
        assert o_bf16 == o_fp8


@pytest.mark.parametrize("dot", [dot_fused, dot_serial], ids=["fused", "serial"])
def test_different_groupings_round_differently(dot):
    s = 2.0 ** -4
    m, q = cases(2, 200)
    differ = 0
    for i in range(m.shape[0]):
        o_bf16 = dot(m[i], [s * x for x in q[i]], NATURAL)
        o_fp8 = f32(dot(m[i], q[i], PAIRED) * s)
        exact = math.fsum(m[i][k] * s * q[i][k] for k in range(D))
        bound = 8 * 2.0 ** -24 * math.fsum(abs(m[i][k] * s * q[i][k]) for k in range(D))
        assert abs(o_bf16 - exact) <= bound and abs(o_fp8 - exact) <= bound
        differ += o_bf16 != o_fp8
    # both within rounding of the exact product, yet not bitwise equal
    assert differ > 10
