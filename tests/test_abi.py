"""C-ABI boundary on the CPU: the library loads, exports what the header declares, and rejects
bad arguments on the host before any device work (fake device addresses are safe here because
every call below fails validation first)."""
import ctypes
import os
import re

import pytest

import frame_wise_gated_libgdn_amd as gdn
import gdn_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgdn.h")

A = 1 << 20  # a 16-byte (and 256-byte) aligned fake address; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = gdn.load()
    names = declared_functions()
    assert {"gdn_forward_framewise", "gdn_step_frame", "gdn_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "missing export " + n


def test_abi_version_and_status_strings():
    assert gdn.abi_version() == 11
    lib = gdn.load()
    for code in range(10):
        assert lib.gdn_status_string(code)
    assert lib.gdn_status_string(99) == b"unknown status"


def prob(B=1, H=2, D=64, S=40, F=3, dtype=gdn.GDN_BF16, delta=1, layout="head"):
    T = F * S
    if layout == "head":
        st = (H * T * D, T * D, D)
    else:
        st = (T * H * D, D, H * D)
    return gdn.Problem(B, H, D, S, F, dtype, delta, 0.0, *st, *st)


def call(p, step=False, q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, si=None, o=6 * A, so=None,
         ws=8 * A, wsb=1 << 40):
    lib = gdn.load()
    fn = lib.gdn_step_frame if step else lib.gdn_forward_framewise
    pp = None if p is None else ctypes.byref(p)
    return fn(pp, q, k, v, g, b, si, o, so, ws, wsb, None)


def msg():
    return gdn.load().gdn_last_error_message().decode()


@pytest.mark.parametrize("name", gdn_synth.WORKLOAD_ORDER)
def test_workspace_size_for_workloads(name):
    w = gdn_synth.WORKLOADS[name]
    code = {"f32": gdn.GDN_F32, "bf16": gdn.GDN_BF16, "fp8": gdn.GDN_FP8_E4M3}[w.dtype]
    p = gdn.Problem(w.B, w.H, w.D, w.S, 1 if w.step_mode else w.F, code, int(w.use_delta), 0.0,
                    0, 0, w.D, 0, 0, w.D)
    n = gdn.workspace_size(p, w.step_mode)
    assert n > 0
    fused = w.dtype == "fp8" or (w.dtype == "bf16" and w.D in (64, 128) and w.B * w.H * w.F >= 1024)
    if not w.step_mode and fused:
        # two fp32 D x D states per (b, h)
        assert n >= 2 * w.B * w.H * w.D * w.D * 4
    elif not w.step_mode:
        esz = w.elem_bytes()
        # per-frame states plus at least one fp32 record per frame
        assert n >= w.B * w.H * w.F * w.D * w.D * (esz + 4 * (2 if w.use_delta else 1))


def test_step_workspace_independent_of_frames():
    # constant memory in video length (the fixed D x D state of the pages)
    sizes = {gdn.workspace_size(prob(F=f), True) for f in (1, 10, 961, 100000)}
    assert len(sizes) == 1


def test_gram_step_workspace():
    # the streaming shape (B 1, H 16, D 128, S 3520, bf16): the one-launch step's control words
    # (time-out word, 16 epochs, two flags per workgroup; 256 bytes aligned), fp32 partials of 8
    # token splits of 448 tokens (two workgroups per split, one per half of the rows: 256 in
    # all, one per CU), the new state transposed in bf16
    p = gdn.Problem(1, 16, 128, 3520, 1, gdn.GDN_BF16, 1, 0.0, 0, 0, 128, 0, 0, 128)
    ctl = (1 + 16 + 2 * 16 * 16) * 8
    ctl = (ctl + 255) // 256 * 256
    assert gdn.workspace_size(p, True) == ctl + 16 * 8 * 128 * 128 * 4 + 16 * 128 * 128 * 2
    # STAGED keeps the three launches and needs no control words
    st = gdn.Problem(1, 16, 128, 3520, 1, gdn.GDN_BF16, 1, 0.0, 0, 0, 128, 0, 0, 128, 1)
    assert gdn.workspace_size(st, True) == 16 * 8 * 128 * 128 * 4 + 16 * 128 * 128 * 2
    # heads not a multiple of 8: three launches, splits filling 256 workgroups (12 heads: 11
    # splits of 320 tokens)
    h12 = gdn.Problem(1, 12, 128, 3520, 1, gdn.GDN_BF16, 1, 0.0, 0, 0, 128, 0, 0, 128)
    assert gdn.workspace_size(h12, True) == 12 * 11 * 128 * 128 * 4 + 12 * 128 * 128 * 2
    # rows beyond 2 GiB: the whole-state step kernels
    big = gdn.Problem(1, 16, 128, 3520, 1, gdn.GDN_BF16, 1, 0.0, 0, 0, 1 << 20, 0, 0, 128)
    assert gdn.workspace_size(big, True) != gdn.workspace_size(p, True)


def test_forward_workspace_grows_with_frames():
    assert gdn.workspace_size(prob(F=20), False) > gdn.workspace_size(prob(F=10), False)


def test_null_problem():
    assert call(None) == 1
    assert "NULL" in msg()


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, 2), ("heads", 0, 2), ("tokens_per_frame", 0, 2), ("frames", 0, 2),
    ("head_dim", 48, 3), ("head_dim", 256, 3), ("dtype", 7, 3),
])
def test_bad_sizes(field, value, code):
    p = prob()
    setattr(p, field, value)
    assert call(p) == code
    assert msg()
    n = ctypes.c_size_t(123)
    assert gdn.load().gdn_workspace_size(ctypes.byref(p), 0, ctypes.byref(n)) == code
    assert n.value == 123


def test_bad_schedule():
    p = prob()
    p.schedule = 3
    assert call(p) == 2
    assert "schedule" in msg()
    p = prob(dtype=gdn.GDN_F32)
    p.schedule = 2  # fused needs bf16
    assert call(p) == 3
    p = prob(D=32)
    p.schedule = 2  # and D = 64 or 128
    assert call(p) == 3
    p = prob(D=32)
    p.schedule = 2
    assert call(p, step=True, si=7 * A, wsb=16) == 7  # step mode ignores the schedule


def test_schedule_workspace():
    staged, fused = prob(F=30), prob(F=30)
    staged.schedule, fused.schedule = 1, 2
    ns, nf = gdn.workspace_size(staged, False), gdn.workspace_size(fused, False)
    # fused: only two D x D fp32 states per (b, h) plus flags, independent of the frame count
    assert nf < ns
    fused.frames = 3000
    assert gdn.workspace_size(fused, False) == nf
    assert gdn.workspace_size(prob(F=30), False) == ns     # auto: staged for 60 items
    assert gdn.workspace_size(prob(F=3000), False) == nf   # and fused for 6000


def test_trace_arming_validation():
    lib = gdn.load()
    assert lib.gdn_set_trace(None, 0) == 0
    assert lib.gdn_set_trace(None, 3) == 1
    assert lib.gdn_set_trace(None, -1) == 2
    # a call that fails validation launches nothing
    gdn.set_trace([0x10, 0x20])
    assert call(prob(), q=None) == 1
    assert gdn.read_trace() == []
    gdn.set_trace(None)


def test_step_ignores_frames_and_requires_state():
    p = prob(F=0)
    assert call(p, step=True) == 1  # state_in missing (frames is not checked in step mode)
    assert "state_in" in msg()


def test_null_tensor_pointers():
    assert call(prob(), q=None) == 1
    assert call(prob(), o=None) == 1
    assert call(prob(), g=None) == 1


def test_misaligned_pointers_and_strides():
    assert call(prob(), k=2 * A + 8) == 5
    p = prob()
    p.qkv_stride_t = 68
    p.qkv_stride_h = 68 * 120
    assert call(p) == 5
    assert call(prob(), ws=8 * A + 16) == 5
    assert call(prob(), g=4 * A + 2) == 5


def test_bad_strides():
    p = prob()
    p.qkv_stride_t = 32  # rows of 64 elements overlap
    assert call(p) == 4
    p = prob()
    p.o_stride_h = -p.o_stride_h
    assert call(p) == 4
    p = prob(H=2)
    p.qkv_stride_h = 64  # heads interleave with tokens
    assert call(p) == 4


def test_token_major_layout_accepted_until_workspace_check():
    p = prob(layout="token")
    assert call(p, wsb=16) == 7
    assert "workspace" in msg()


def test_workspace_missing_or_small():
    p = prob()
    need = gdn.workspace_size(p, False)
    assert call(p, wsb=need - 1) == 7
    assert call(p, ws=None) == 7


def test_aliasing():
    p = prob()
    assert call(p, o=A) == 6                      # o == q
    assert call(p, o=A + 1024) == 6               # o overlaps q
    assert call(p, so=8 * A + 256) == 6           # state_out inside the workspace
    assert call(p, si=7 * A, so=7 * A + 4096) == 6  # partial overlap of the states
    assert call(p, ws=6 * A + 4096) == 6          # workspace overlaps o


def test_in_place_state_passes_alias_checks():
    # exact in-place commit is allowed: the call only fails later, at the workspace check
    p = prob()
    assert call(p, si=7 * A, so=7 * A, wsb=16) == 7


def call_bwd(p, q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, si=None, do=6 * A, dso=None, dq=9 * A,
             dk=10 * A, dv=11 * A, dg=12 * A, db=13 * A, dsi=None, ws=14 * A, wsb=1 << 40):
    lib = gdn.load()
    pp = None if p is None else ctypes.byref(p)
    return lib.gdn_backward_framewise(pp, q, k, v, g, b, si, do, dso, dq, dk, dv, dg, db, dsi, ws,
                                      wsb, None)


def test_backward_validation():
    assert call_bwd(None) == 1
    assert call_bwd(prob(), do=None) == 1
    assert call_bwd(prob(), dg=None) == 1
    assert call_bwd(prob(dtype=gdn.GDN_F32)) == 3          # bf16 only
    assert call_bwd(prob(D=32)) == 3                        # D = 64 or 128
    assert "backward" in msg()
    assert call_bwd(prob(), dq=A) == 6                      # dq == q
    assert call_bwd(prob(), dk=9 * A + 1024) == 6           # dk overlaps dq
    assert call_bwd(prob(), dsi=7 * A, dso=7 * A, wsb=16) == 7   # in-place state gradient is fine
    assert call_bwd(prob(), dsi=7 * A, dso=7 * A + 4096) == 6    # partial overlap is not
    assert call_bwd(prob(), wsb=16) == 7
    assert call_bwd(prob(), ws=14 * A + 16) == 5


def test_backward_workspace():
    p = prob(F=30)
    n = gdn.workspace_size(p, 2)
    # fp32 forward states and state gradients (F + 1 slots), the forward records and C_f records
    assert n >= 2 * (31 * 2 * 64 * 64 * 4) + 30 * 2 * 64 * 64 * 4
    assert gdn.workspace_size(prob(F=60), 2) > n
    # from saved states: only the C_f records and the state gradients (no forward records or
    # states)
    n3 = gdn.workspace_size(p, 3)
    assert n3 < n and n3 >= 31 * 2 * 64 * 64 * 4 + 30 * 2 * 64 * 64 * 4
    n4 = ctypes.c_size_t(0)
    assert gdn.load().gdn_workspace_size(ctypes.byref(p), 4, ctypes.byref(n4)) == 2


def test_backward_chain_workspace():
    """The chained schedule (explicit, or AUTO once B*H*F >= 1024) puts the ticket counter, the
    time-out flag (byte 4) and one flag per (b, h) and column group first, then two fp32
    state-gradient buffers per (b, h), and keeps no C_f records."""
    def a256(x):
        return (x + 255) // 256 * 256
    B, H, D, F = 1, 2, 64, 30
    staged, fused = prob(F=F), prob(F=F)
    staged.schedule, fused.schedule = 1, 2
    crec = B * H * F * D * D * 4
    extra = a256((2 + B * H * 4) * 4) + a256(2 * B * H * D * D * 4)
    # from saved states: the same buffers but the C records
    ns, nf = gdn.workspace_size(staged, 3), gdn.workspace_size(fused, 3)
    assert nf == ns - a256(crec) + extra, (ns, nf)
    # recomputing: the fused forward keeps only the Ghat planes (D/16 x 2 x 2 fragments of 1 KB
    # per frame) instead of the full records (planes + fp32 Bhat); one split, so no partials
    full, planes = (64 // 16) * 2 * 2 * 1024 + 4 * D * D, (64 // 16) * 2 * 2 * 1024
    ns, nf = gdn.workspace_size(staged, 2), gdn.workspace_size(fused, 2)
    assert nf == ns - a256(crec) - a256(B * H * F * full) + a256(B * H * F * planes) + extra, (ns, nf)
    assert gdn.workspace_size(prob(F=30), 2) == gdn.workspace_size(staged, 2)        # AUTO, 60 items
    big = prob(H=4, S=8, F=256)                                                       # AUTO, 1024 items
    big_f = prob(H=4, S=8, F=256)
    big_f.schedule = 2
    assert gdn.workspace_size(big, 2) == gdn.workspace_size(big_f, 2)
    assert gdn.workspace_size(big, 3) == gdn.workspace_size(big_f, 3)


def test_saved_size():
    # B=1, H=2, D=64, F=30, delta: Ghat planes (hi + lo bf16, D/16 x 2 x 2 fragments of 1 KB
    # per frame), then 256-byte aligned fp32 states for F + 1 slots
    p = prob(F=30)
    recs = 2 * 30 * (64 // 16) * 2 * 2 * 1024
    states = 2 * 31 * 64 * 64 * 4
    assert gdn.saved_size(p) == (recs + 255) // 256 * 256 + states
    assert gdn.saved_size(prob(F=30, delta=0)) == states          # no Ghat without the delta term
    n = ctypes.c_size_t(0)
    assert gdn.load().gdn_saved_size(ctypes.byref(prob(dtype=gdn.GDN_F32)), ctypes.byref(n)) == 3
    assert gdn.load().gdn_saved_size(ctypes.byref(prob(D=32)), ctypes.byref(n)) == 3


def test_saved_entry_points_validate():
    lib = gdn.load()
    p = prob(F=30)
    need = gdn.saved_size(p)
    ws = gdn.workspace_size(p, 0)
    # forward: saved required, large enough, aligned, not overlapping anything
    def fwd(saved, saved_bytes, pp=p):
        return lib.gdn_forward_framewise_save(ctypes.byref(pp), A, 2 * A, 3 * A, 4 * A, 5 * A, None,
                                              6 * A, None, saved, saved_bytes, 64 * A, ws, None)
    assert fwd(None, 0) == 1
    assert fwd(128 * A, need - 1) == 7
    assert fwd(128 * A + 16, need) == 5
    assert fwd(6 * A, need) == 6                           # overlaps o
    staged = prob(F=30)
    staged.schedule = 1
    assert fwd(128 * A, need, staged) == 3
    # backward: saved required and large enough
    ws3 = gdn.workspace_size(p, 3)
    def bwd(saved, saved_bytes):
        return lib.gdn_backward_framewise_saved(ctypes.byref(p), A, 2 * A, 3 * A, 4 * A, 5 * A, saved,
                                                saved_bytes, 6 * A, None, 7 * A, 8 * A, 9 * A, 10 * A,
                                                11 * A, None, 64 * A, ws3, None)
    assert bwd(None, 0) == 1
    assert bwd(128 * A, need - 1) == 7
    assert bwd(7 * A, need) == 6                           # dq inside the saved buffer


def call_fp8(p, q=A, k=2 * A, v=3 * A, qs=15 * A, ks=16 * A, vs=17 * A, g=4 * A, b=5 * A, si=None,
             o=6 * A, so=None, ws=8 * A, wsb=1 << 40):
    lib = gdn.load()
    pp = None if p is None else ctypes.byref(p)
    return lib.gdn_forward_framewise_fp8(pp, q, k, v, qs, ks, vs, g, b, si, o, so, ws, wsb, None)


def test_fp8_validation():
    p8 = prob(dtype=gdn.GDN_FP8_E4M3)
    assert call_fp8(None) == 1
    assert call_fp8(p8, ks=None) == 1                  # scales required
    assert call_fp8(prob()) == 3                        # bf16 data through the fp8 entry
    assert "GDN_FP8_E4M3" in msg()
    assert call(p8) == 3                                # fp8 data through the bf16 entry
    assert "gdn_forward_framewise_fp8" in msg()
    assert call(p8, step=True, si=7 * A) == 3           # no step mode
    assert call_fp8(prob(dtype=gdn.GDN_FP8_E4M3, D=32)) == 3
    p = prob(dtype=gdn.GDN_FP8_E4M3)
    p.schedule = 1
    assert call_fp8(p) == 3                             # staged: not for E4M3
    assert call_fp8(p8, qs=15 * A + 2) == 5             # scales 4-byte aligned
    assert call_fp8(p8, o=15 * A) == 6                  # o overlaps a scale array
    assert call_fp8(p8, wsb=16) == 7                    # reaches the workspace check
    n = ctypes.c_size_t(0)
    assert gdn.load().gdn_workspace_size(ctypes.byref(p8), 2, ctypes.byref(n)) == 3


def test_fp8_workspace_is_the_fused_one():
    p8, pb = prob(dtype=gdn.GDN_FP8_E4M3, F=30), prob(F=30)
    pb.schedule = 2
    assert gdn.workspace_size(p8, 0) == gdn.workspace_size(pb, 0)


def test_fused_needs_frame_rows_within_2gib():
    p = prob(F=3000)                          # auto: fused (6000 items)
    big = prob(F=3000)
    big.qkv_stride_t = 1 << 25                 # 39 rows of 2^25 bf16 elements: > 2 GiB
    big.qkv_stride_h = big.qkv_stride_t * 40 * 3000
    big.qkv_stride_b = big.qkv_stride_h * 2
    assert gdn.workspace_size(big, False) != gdn.workspace_size(p, False)   # falls back to staged
    big.schedule = 2
    assert call(big) == 3 and "2 GiB" in msg()


def test_fused_bound_counts_the_rows_past_the_frame():
    # the fused kernel addresses up to 464 rows past a frame's last one through 32-bit offsets:
    # a stride whose 40 rows fit in 2 GiB but whose 40 + 463 rows do not must not select it
    p = prob(F=3000)
    big = prob(F=3000)
    big.qkv_stride_t = 2228224                 # 39 rows: 166 MiB; 39 + 464 rows: 2.09 GiB
    big.qkv_stride_h = big.qkv_stride_t * 40 * 3000
    big.qkv_stride_b = big.qkv_stride_h * 2
    assert gdn.workspace_size(big, False) != gdn.workspace_size(p, False)   # falls back to staged
    big.schedule = 2
    assert call(big) == 3 and "2 GiB" in msg()
    ok = prob(F=3000)
    ok.qkv_stride_t = 1048576                  # 39 + 464 rows: 1006 MiB, fused
    ok.qkv_stride_h = ok.qkv_stride_t * 40 * 3000
    ok.qkv_stride_b = ok.qkv_stride_h * 2
    assert gdn.workspace_size(ok, False) == gdn.workspace_size(p, False)


def test_fused_needs_frame_output_rows_within_2gib():
    # the fused kernel also writes O through 32-bit buffer offsets: a huge o token stride
    # with small q/k/v strides must not select it
    p = prob(F=3000)
    big = prob(F=3000)
    big.o_stride_t = 1 << 25                   # 39 rows of 2^25 bf16 elements: > 2 GiB
    big.o_stride_h = big.o_stride_t * 40 * 3000
    big.o_stride_b = big.o_stride_h * 2
    assert gdn.workspace_size(big, False) != gdn.workspace_size(p, False)   # falls back to staged
    staged = prob(F=3000)
    staged.schedule = 1
    assert gdn.workspace_size(big, False) == gdn.workspace_size(staged, False)
    big.schedule = 2
    assert call(big) == 3 and "2 GiB" in msg()


def test_backward_needs_frame_rows_within_2gib():
    # the gradient kernels read K, V, Q, dO and write dK, dV, dQ through 32-bit buffer offsets
    for field in ("qkv", "o"):
        big = prob(F=3)
        setattr(big, field + "_stride_t", 1 << 25)     # 39 rows of 2^25 bf16 elements: > 2 GiB
        setattr(big, field + "_stride_h", (1 << 25) * 40 * 3)
        setattr(big, field + "_stride_b", (1 << 25) * 40 * 3 * 2)
        n = ctypes.c_size_t(0)
        assert gdn.load().gdn_workspace_size(ctypes.byref(big), 2, ctypes.byref(n)) == 3
        assert "2 GiB" in msg()
        assert call_bwd(big) == 3
    assert gdn.workspace_size(prob(F=3), 2) > 0


def tprob(B=1, T=6, S=5, C=16, tb=2, dtype=gdn.GDN_BF16):
    return gdn.TconvProblem(B, T, S, C, tb, dtype, T * S * C, S * C, C, T * S * C, S * C, C)


def call_tconv(p, x=A, w=2 * A, b=3 * A, ci=None, y=4 * A, co=None):
    lib = gdn.load()
    pp = None if p is None else ctypes.byref(p)
    return lib.gdn_tconv_forward(pp, x, w, b, ci, y, co, None)


def test_tconv_validation():
    assert call_tconv(None) == 1
    assert call_tconv(tprob(), x=None) == 1
    assert call_tconv(tprob(T=0)) == 2
    assert call_tconv(tprob(T=5, tb=2)) == 2              # whole blocks only
    assert "block_frames" in msg()
    assert call_tconv(tprob(C=12)) == 5                    # channels multiple of 8
    assert call_tconv(tprob(dtype=gdn.GDN_FP8_E4M3)) == 3
    assert call_tconv(tprob(), y=A + 64) == 6              # y overlaps x
    assert call_tconv(tprob(), ci=5 * A, co=5 * A + 32) == 6   # partial overlap of the caches
    assert call_tconv(tprob(), x=A + 8) == 5
    p = tprob()
    p.x_stride_s = 8                                       # rows of 16 channels overlap
    assert call_tconv(p) == 4


def aprob(B=1, H=2, D=128, S=40, fq=3, fk=3, f0=0):
    st = (H * fk * S * D, fk * S * D, D)
    sq = (H * fq * S * D, fq * S * D, D)
    return gdn.AttnProblem(B, H, D, S, fq, fk, f0, gdn.GDN_BF16, 0.0, *sq, *st, *sq)


def call_attn(p, q=A, k=2 * A, v=3 * A, o=4 * A):
    pp = None if p is None else ctypes.byref(p)
    return gdn.load().gdn_attention_framecausal(pp, q, k, v, o, None)


def test_attention_validation():
    assert call_attn(None) == 1
    assert call_attn(aprob(), v=None) == 1
    assert call_attn(aprob(fq=2, fk=3, f0=2)) == 2        # query frames past the key frames
    assert "within the key frames" in msg()
    assert call_attn(aprob(D=32)) == 3
    p = aprob()
    p.dtype = gdn.GDN_F32
    assert call_attn(p) == 3
    assert call_attn(aprob(), o=A + 256) == 6               # o overlaps q
    assert call_attn(aprob(), k=2 * A + 8) == 5
    big = aprob()                                             # key rows over 2 GiB: 32-bit offsets
    big.kv_stride_t = 1 << 25
    big.kv_stride_h = (1 << 25) * 3 * 40
    big.kv_stride_b = big.kv_stride_h * 2
    assert call_attn(big) == 3 and "2 GiB" in msg()


def attn_ws_size(p):
    n = ctypes.c_size_t(0)
    code = gdn.load().gdn_attention_workspace_size(None if p is None else ctypes.byref(p), ctypes.byref(n))
    return code, n.value


def call_attn_ws(p, ws, wsb, q=A, k=16 * A, v=32 * A, o=48 * A):
    return gdn.load().gdn_attention_framecausal_ws(ctypes.byref(p), q, k, v, o, ws, wsb, None)


def test_attention_workspace_validation():
    assert attn_ws_size(None)[0] == 1
    assert attn_ws_size(aprob(D=32))[0] == 3
    # a whole sequence fills the device by itself, and several query frames never split
    assert attn_ws_size(aprob(B=2, H=16, S=880, fq=81, fk=81)) == (0, 0)
    assert attn_ws_size(aprob(fq=3, fk=3)) == (0, 0)
    # one 720p frame against 961 frames: 224 workgroups of 256 queries for 256 CUs
    code, n = attn_ws_size(aprob(B=1, H=16, D=128, S=3520, fq=1, fk=961, f0=960))
    rows = 16 * 3520
    assert code == 0 and n > 0 and n % (rows * (128 * 4 + 8)) == 0
    assert 2 <= n // (rows * (128 * 4 + 8)) <= 16
    # host checks before any launch: too small, misaligned, overlapping o
    small = aprob(B=1, H=2, D=128, S=200, fq=1, fk=41, f0=40)
    code, n = attn_ws_size(small)
    assert code == 0 and n > 0
    assert call_attn_ws(small, 64 * A, n - 1) == 7 and "workspace" in msg()
    assert call_attn_ws(small, 64 * A + 16, n) == 5
    assert call_attn_ws(small, 48 * A, n) == 6 and "overlaps" in msg()


def test_trace_kinds_match_the_header():
    """The binding's trace-kind names, the header's GDN_KERNEL_* values and the library's internal
    launch kinds agree (a new kind must be added in all three)."""
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = open(os.path.join(root, "include", "libgdn.h")).read()
    kinds = {int(v): n.lower() for n, v in re.findall(r"GDN_KERNEL_(\w+)\s*=\s*(\d+)", hdr)}
    assert kinds == gdn.KERNEL_NAMES
    internal = open(os.path.join(root, "frame_wise_gated_libgdn_amd", "csrc", "gdn_internal.h")).read()
    ik = {int(v): n.lower() for n, v in re.findall(r"\bK_(\w+)\s*=\s*(\d+)", internal)}
    assert ik == kinds


def test_check_timeout_validation():
    lib = gdn.load()
    p = prob(F=3)                                 # auto: staged (6 items), no bounded waits
    assert lib.gdn_check_timeout(None, 0, A, None) == 1
    assert lib.gdn_check_timeout(ctypes.byref(p), 4, A, None) == 2
    assert "mode" in msg()
    bad = prob()
    bad.head_dim = 48
    assert lib.gdn_check_timeout(ctypes.byref(bad), 0, A, None) == 3
    # schedules without waits read nothing (the fake address is never touched)
    assert lib.gdn_check_timeout(ctypes.byref(p), 0, A, None) == 0
    assert lib.gdn_check_timeout(ctypes.byref(p), 1, A, None) == 0
    staged = prob(F=3000)
    staged.schedule = 1
    assert lib.gdn_check_timeout(ctypes.byref(staged), 0, A, None) == 0
    assert lib.gdn_check_timeout(ctypes.byref(staged), 2, A, None) == 0
    fused = prob(F=3000)
    fused.schedule = 2
    assert lib.gdn_check_timeout(ctypes.byref(fused), 0, None, None) == 1


def test_step_noalloc_validation():
    lib = gdn.load()

    def call_na(p, q=A, k=2 * A, v=3 * A, g=4 * A, b=5 * A, si=9 * A, o=6 * A, so=None):
        return lib.gdn_step_frame_noalloc(None if p is None else ctypes.byref(p), q, k, v, g, b,
                                          si, o, so, None)

    assert call_na(None) == 1
    assert call_na(prob(), q=None) == 1
    assert call_na(prob(), si=None) == 1 and "state_in" in msg()
    assert call_na(prob(), q=A + 8) == 5
    # beyond the static scratch (32 MiB): 512 heads of D = 128 at 3520 tokens need 48 MiB
    big = gdn.Problem(1, 512, 128, 3520, 1, gdn.GDN_BF16, 1, 0.0, 512 * 3520 * 128, 3520 * 128,
                      128, 512 * 3520 * 128, 3520 * 128, 128)
    assert gdn.workspace_size(big, 1) > (32 << 20)
    assert call_na(big, q=A, k=A << 12, v=A << 13, o=A << 14) == 7
    assert "static scratch" in msg()
