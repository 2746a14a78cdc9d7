"""E4M3 (8-bit Q/K/V) forward on the GPU, through the C ABI, against the CPU oracle.

Tolerance: max|d| / max|ref| <= 1e-2 (bf16 output, fp32 state), as for bf16 inputs: the codes
are decoded exactly, so the only roundings are those of the bf16 path. With power-of-two scales
the decoded values are exact bf16 values and the E4M3 path must equal the bf16 path on them
bit for bit (scaling by a power of two commutes with every rounding in the kernel).
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import frame_wise_gated_libgdn_amd as gdn  # noqa: E402
import gdn_synth  # noqa: E402
import oracle  # noqa: E402
from gpu_util import TOL, rel_err, to_np  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_case(B, H, D, S, F, with_state, seed):
    """Codes from N(0, 1) values with per-frame power-of-two scales (the generator's recipe),
    the scales then multiplied by U(0.5, 2) so that they are arbitrary fp32 values, and a few
    codes replaced by subnormals, the largest normals and zeros of both signs."""
    rng = np.random.default_rng(seed)
    codes, scales = [], []
    for _ in range(3):
        x = torch.from_numpy(rng.standard_normal((B * H * F * S, D)).astype(np.float32))
        c, s = gdn_synth.e4m3_codes(x, S, D)
        c = c.numpy().reshape(B, H, F * S, D).copy()
        special = np.array([0x01, 0x07, 0x81, 0x87, 0x7E, 0xFE, 0x00, 0x80, 0x08, 0x88], np.uint8)
        idx = rng.integers(0, c.size, 24)
        c.reshape(-1)[idx] = special[rng.integers(0, len(special), len(idx))]
        s = s.numpy().reshape(B, H, F) * rng.uniform(0.5, 2.0, (B, H, F)).astype(np.float32)
        codes.append(c)
        scales.append(s.astype(np.float32))
    g = rng.uniform(0.85, 1.0, (B, H, F)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (B, H, F)).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32) if with_state else None
    return codes, scales, g, b, s0


def to_dev_codes(c, layout):
    t = torch.from_numpy(c)
    if layout == "token":
        t = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    return t.to(DEV)


CASES = [
    # B, H, D, S, F, delta, initial state, layout
    (1, 2, 128, 200, 5, True, True, "head"),
    (1, 1, 64, 64, 7, True, False, "head"),
    (2, 2, 64, 130, 4, True, True, "token"),
    (1, 2, 128, 96, 6, False, True, "head"),
    (1, 3, 64, 33, 3, False, False, "head"),
    (1, 1, 128, 1, 9, True, True, "head"),      # one token per frame
    (1, 2, 128, 300, 1, True, False, "head"),   # one frame
    (1, 16, 128, 3520, 2, True, True, "head"),  # the 720p frame size
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_fp8_forward_matches_oracle(case):
    B, H, D, S, F, delta, with_state, layout = case
    say("fp8 forward", case)
    codes, scales, g, b, s0 = make_case(B, H, D, S, F, with_state, zlib.crc32(repr(case).encode()))
    dq, dk, dv = (to_dev_codes(c, layout) for c in codes)
    ds = [torch.from_numpy(s).to(DEV) for s in scales]
    tg, tb = torch.from_numpy(g).to(DEV), torch.from_numpy(b).to(DEV)
    ts0 = None if s0 is None else torch.from_numpy(s0).to(DEV)
    o, st = gdn.forward_framewise_fp8(dq, dk, dv, *ds, tg, tb, ts0, use_delta=delta)
    torch.cuda.synchronize()
    ro, rs = oracle.forward_fp8(*codes, *scales, g, b, s0, use_delta=delta)
    eo, es = rel_err(to_np(o), ro), rel_err(to_np(st), rs)
    say("  o %.2e state %.2e" % (eo, es))
    assert o.dtype == torch.bfloat16
    assert eo <= TOL["bf16"] and es <= 1e-4


def test_fp8_in_place_state_and_determinism():
    B, H, D, S, F = 1, 2, 128, 70, 5
    codes, scales, g, b, s0 = make_case(B, H, D, S, F, True, 41)
    dq, dk, dv = (to_dev_codes(c, "head") for c in codes)
    ds = [torch.from_numpy(s).to(DEV) for s in scales]
    tg, tb = torch.from_numpy(g).to(DEV), torch.from_numpy(b).to(DEV)
    st = torch.from_numpy(s0).to(DEV)
    o1, st1 = gdn.forward_framewise_fp8(dq, dk, dv, *ds, tg, tb, st.clone())
    o2, _ = gdn.forward_framewise_fp8(dq, dk, dv, *ds, tg, tb, st, state_out=st)  # in place
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st)


def test_fp8_generator_device_matches_host():
    w = gdn_synth.WORKLOADS["gdn_720p_60s_fp8"]
    gen = gdn_synth.TorchGen(DEV)
    codes = torch.empty((2 * w.S, w.D), dtype=torch.uint8, device=DEV)
    sc = torch.empty(2, dtype=torch.float32, device=DEV)
    gen.fill_e4m3(codes, sc, w.seed, gdn_synth.TID_V, 0, 9, 300, w.S, w.D)
    hc, hs = gdn_synth.qkv_fp8_cpu(w, heads=[9], frames=[300, 301])
    assert np.array_equal(codes.cpu().numpy(), hc[2][0, 0])
    assert np.array_equal(sc.cpu().numpy(), hs[2][0, 0])


def test_fp8_720p_full_launch():
    """The 720p 60 s shape with E4M3 inputs, as bench.py times it: bitwise equal to the bf16
    path on the decoded values (power-of-two scales), oracle on frames 0-3 of one head."""
    w = gdn_synth.WORKLOADS["gdn_720p_60s_fp8"]
    S = w.S
    say("720p fp8 workload: generating inputs on the device")
    (q8, k8, v8), (sq, sk, sv) = gdn_synth.qkv_fp8_torch(w, DEV)
    g, b = gdn_synth.gates_torch(w, DEV)
    o, st = gdn.forward_framewise_fp8(q8, k8, v8, sq, sk, sv, g, b)
    torch.cuda.synchronize()
    assert torch.isfinite(st).all()

    say("  bf16 path on the decoded values")
    ob = torch.empty_like(o)
    wide = []
    for c, s in ((q8, sq), (k8, sk), (v8, sv)):
        x = torch.empty(c.shape, dtype=torch.bfloat16, device=DEV)
        for h in range(w.H):
            x[0, h] = (c[0, h].view(torch.float8_e4m3fn).to(torch.float32).view(w.F, S, w.D)
                       * s[0, h][:, None, None]).view(w.F * S, w.D).to(torch.bfloat16)
        wide.append(x)
    del q8, k8, v8
    ob, stb = gdn.forward_framewise(*wide, g, b, out=ob)
    torch.cuda.synchronize()
    del wide
    assert torch.equal(o, ob), "E4M3 path differs from the bf16 path on the same values"
    assert torch.equal(st, stb)
    del ob

    say("  C oracle: head 3, frames 0-3")
    hc, hs = gdn_synth.qkv_fp8_cpu(w, heads=[3], frames=range(4))
    gc, bc = gdn_synth.gates_cpu(w, heads=[3], frames=range(4))
    ro, _ = oracle.forward_fp8(*hc, *hs, gc, bc)
    e = rel_err(to_np(o[:, 3:4, :4 * S]), ro)
    say("  frames 0-3 err %.3e" % e)
    assert e <= TOL["bf16"]


def test_single_token_tensor_with_short_token_stride():
    """S = F = 1: the token stride addresses nothing and may be shorter than a row; the fused
    kernel (bf16 and E4M3) must still read exactly the one row."""
    B, H, D = 1, 2, 128
    codes, scales, g, b, s0 = make_case(B, H, D, 1, 1, True, 52)
    dev = []
    for c in codes:   # storage [B, H, D] with a token stride of 8 elements
        t = torch.from_numpy(c.reshape(B, H, D)).to(DEV)
        dev.append(t.as_strided((B, H, 1, D), (H * D, D, 8, 1)))
    ds = [torch.from_numpy(s).to(DEV) for s in scales]
    tg, tb = torch.from_numpy(g).to(DEV), torch.from_numpy(b).to(DEV)
    ts0 = torch.from_numpy(s0).to(DEV)
    o, st = gdn.forward_framewise_fp8(*dev, *ds, tg, tb, ts0, schedule="fused")
    wide, wide_host = [], []
    for c, s in zip(codes, scales):
        x = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(s)[..., None]
        x = x.to(torch.bfloat16)   # arbitrary scales: the bf16 leg gets rounded values
        wide_host.append(x.to(torch.float64).numpy())
        wide.append(x.to(DEV).reshape(B, H, D).as_strided((B, H, 1, D), (H * D, D, 8, 1)))
    ob, stb = gdn.forward_framewise(*wide, tg, tb, ts0, schedule="fused")
    torch.cuda.synchronize()
    ro, rs = oracle.forward_fp8(*codes, *scales, g, b, s0)
    assert rel_err(to_np(o), ro) <= TOL["bf16"] and rel_err(to_np(st), rs) <= 1e-4
    rbo, rbs = oracle.forward(*wide_host, g, b, s0)
    assert rel_err(to_np(ob), rbo) <= TOL["bf16"] and rel_err(to_np(stb), rbs) <= 1e-4
