// C ABI of libgdn: argument validation, workspace planning and the launch sequence.
// Everything here runs on the host before any device work; the arithmetic is in
// gdn_kernels.hip.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "../../include/libgdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_msg[512] = "";

gdn_status fail(gdn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return s;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Schedule and splits chosen from the problem only, so that the workspace size is a pure
// function of it.
struct Plan {
    int mode;                   // 0 forward, 1 step, 2 backward, 3 backward from saved states
    bool fused;                 // forward: fused single pass (else staged); step: column
                                // blocks; backward: the reverse chain in the Q/dO pass
    bool fused_states;          // backward: the forward states recomputed by the fused forward
    int nsplit, split_tokens;   // partial-product kernel
    int nchunk, chunk_tokens;   // output kernel
    bool step_one;              // step: the Gram-form work may run in one launch (shape allows)
    size_t step_ctl_bytes;      // ... its time-out word, epochs and meeting flags
    size_t canon_bytes, part_bytes, mt_bytes;   // staged forward and step
    size_t ctl_bytes, chain_bytes;              // fused forward; chained backward
    size_t crec_bytes, gt_bytes;                // backward
    size_t total() const {
        if (mode >= 2)
            return align256(ctl_bytes) + align256(chain_bytes) + align256(canon_bytes) +
                   align256(part_bytes) + align256(mt_bytes) + align256(crec_bytes) + gt_bytes;
        if (mode == 1 && fused) return align256(step_ctl_bytes) + align256(part_bytes) + mt_bytes;
        return fused ? align256(ctl_bytes) + chain_bytes
                     : align256(canon_bytes) + align256(part_bytes) + mt_bytes;
    }
};

// The fused forward pays off once there are enough (b, h, f) items to fill the chip.
constexpr int64_t kFusedMinItems = 1024;

// The fused kernel reads a frame's Q, K and V rows and writes its O rows through 32-bit buffer
// offsets: for either tensor the bytes from a frame's first row to the end of its last must
// stay below 2 GiB (O is bf16 for every input type the fused kernel takes).
bool fused_rows_fit(const gdn_problem& p) {
    const int64_t esz = p.dtype == GDN_FP8_E4M3 ? 1 : 2;
    const int64_t S = p.tokens_per_frame, D = p.head_dim;
    // the fused forward also addresses kFusedRowsPast rows past the frame (they read zero and
    // drop their stores); a single-token tensor is given one row's length as its stride
    const bool one = S * (int64_t)p.frames == 1;
    const int64_t st = one ? std::max<int64_t>(p.qkv_stride_t, D) : p.qkv_stride_t;
    const int64_t ot = one ? std::max<int64_t>(p.o_stride_t, D) : p.o_stride_t;
    const int64_t rows = S - 1 + gdn::kFusedRowsPast;
    const int64_t in_span = (rows * st + D) * esz;
    const int64_t out_span = (rows * ot + D) * 2;
    return p.qkv_stride_t >= 0 && p.o_stride_t >= 0 && in_span < ((int64_t)1 << 31) &&
           out_span < ((int64_t)1 << 31);
}

bool choose_fused(const gdn_problem& p, int step_mode) {
    if (!step_mode && p.dtype == GDN_FP8_E4M3) return true;  // E4M3 runs only fused
    if (step_mode || !gdn::fused_supported(p.dtype == GDN_BF16, p.head_dim)) return false;
    if (!fused_rows_fit(p)) return false;
    if (p.schedule == GDN_SCHEDULE_FUSED) return true;
    if (p.schedule == GDN_SCHEDULE_STAGED) return false;
    return (int64_t)p.batch * p.heads * p.frames >= kFusedMinItems;
}

// The bf16 step (D = 64 / 128) reads a frame's Q rows and writes its O rows through 32-bit buffer
// offsets (rows up to S, the first past the frame, are addressed): S rows of either stride
// must stay below 2 GiB. A single-token frame is addressed with a stride of one row.
bool step_rows_fit(const gdn_problem& p) {
    const int64_t S = p.tokens_per_frame, D = p.head_dim;
    for (int64_t st : {p.qkv_stride_t, p.o_stride_t}) {
        const int64_t s = S == 1 ? std::max<int64_t>(st, D) : st;
        if (s < 0 || (S * s + D) * 2 >= ((int64_t)1 << 31)) return false;
    }
    return true;
}

bool choose_step_cols(const gdn_problem& p) {
    return gdn::step_cols_supported(p.dtype == GDN_BF16, p.head_dim) && step_rows_fit(p);
}

// The backward's reverse chain runs inside its pass over Q and dO (one workgroup per whole
// frame, ticket-ordered) once there are enough frames to fill the chip, like the fused forward;
// otherwise that pass may split frames over tokens and a separate scan runs the chain.
bool choose_bwd_chain(const gdn_problem& p) {
    if (!gdn::backward_supported(p.dtype == GDN_BF16, p.head_dim)) return false;
    if (p.schedule == GDN_SCHEDULE_FUSED) return true;
    if (p.schedule == GDN_SCHEDULE_STAGED) return false;
    return (int64_t)p.batch * p.heads * p.frames >= kFusedMinItems;
}

constexpr int kTargetGroups = 2048;  // workgroups wanted per parallel launch (256 CUs x 8)
constexpr int kStepPartials = 256;   // Gram step: partial workgroups (one per CU)
constexpr int kStepOutputs = 256;    // Gram step: output workgroups
constexpr int kStepXcdCUs = 32;      // one-launch step: workgroups per XCD (its CUs)

// mode: 0 forward, 1 step, 2 backward, 3 backward from saved states (no forward recompute)
Plan make_plan(const gdn_problem& p, int mode) {
    const int step_mode = mode == 1;
    Plan pl{};
    pl.mode = mode;
    pl.fused = mode == 0 ? choose_fused(p, 0) : mode == 1 ? choose_step_cols(p) : choose_bwd_chain(p);
    const int64_t D = p.head_dim, S = p.tokens_per_frame;
    const int64_t BH = (int64_t)p.batch * p.heads;
    const int64_t F = step_mode ? 1 : p.frames;
    const int64_t esz = p.dtype == GDN_F32 ? 4 : 2;
    const int64_t tiles64 = (S + 63) / 64;
    int64_t want;
    if (step_mode) {
        // one split per 256 tokens: enough workgroups for a single frame of a few heads
        want = (S + 255) / 256;
    } else {
        want = (kTargetGroups + BH * F - 1) / (BH * F);
    }
    want = std::max<int64_t>(1, std::min<int64_t>(want, tiles64));
    pl.split_tokens = (int)(((tiles64 + want - 1) / want) * 64);
    pl.nsplit = (int)((S + pl.split_tokens - 1) / pl.split_tokens);

    const int64_t tiles16 = (S + 15) / 16;
    // output chunks: each output workgroup first stages the D x D state, so one frame (step
    // mode) is cut into fewer, longer chunks
    const int64_t target_out = step_mode ? kTargetGroups / 4 : kTargetGroups;
    int64_t wc = (target_out + BH * F - 1) / (BH * F);
    wc = std::max<int64_t>(1, std::min<int64_t>(wc, (tiles16 + 3) / 4));
    pl.chunk_tokens = (int)(((tiles16 + wc - 1) / wc) * 16);
    pl.nchunk = (int)((S + pl.chunk_tokens - 1) / pl.chunk_tokens);

    // forward: per-frame record for the scan ([Ghat hi | Ghat lo | Bhat^T] or [Bhat^T]), fp32
    // partials only when a frame is split, per-frame states; step: per-split partials, state
    const int64_t nout = (!step_mode && p.use_delta) ? 2 : 1;
    // per-frame record: Ghat hi/lo planes in MFMA-fragment order (D/16 x 2 x ceil(D/32) KB)
    // plus Bhat (4 D^2 bytes)
    const int64_t rec = (p.use_delta ? (D / 16) * 2 * ((D + 31) / 32) * 1024 : 0) + 4 * D * D;
    pl.canon_bytes = step_mode ? 0 : (size_t)(BH * F * rec);
    pl.part_bytes = (step_mode || pl.nsplit > 1) ? (size_t)(BH * F * pl.nsplit * nout * D * D * 4) : 0;
    pl.mt_bytes = (size_t)(BH * F * D * D * esz);
    // fused: ticket counter, time-out flag and one frame flag per (b, h) and column group; two
    // fp32 state buffers per (b, h)
    pl.ctl_bytes = (size_t)(2 + BH * gdn::kChainGroups) * 4;
    pl.chain_bytes = (size_t)(2 * BH * D * D * 4);
    if (step_mode && pl.fused) {
        // Gram partials: step_halves(D) workgroups per (b, h, token split), about one per CU in
        // all, splits of at least 128 tokens (each adds a D^3 product and a D x D partial), a
        // multiple of 16; fp32 partials [BH][splits][D][D]; outputs: at most 256 tokens each;
        // the new state transposed in bf16
        const int64_t hv = gdn::step_halves((int)D);
        int64_t ns = (kStepPartials + BH * hv - 1) / (BH * hv);
        // one launch: the heads spread evenly over the 8 XCDs (B H a multiple of 8), each head's
        // workgroups on one XCD of 32 CUs, one workgroup per CU (STAGED keeps three launches)
        const int64_t hpx = BH / 8;
        pl.step_one = p.schedule != GDN_SCHEDULE_STAGED && BH % 8 == 0 && hpx * hv <= kStepXcdCUs;
        if (pl.step_one) ns = kStepXcdCUs / (hpx * hv);
        ns = std::max<int64_t>(1, std::min<int64_t>(ns, (S + 127) / 128));
        pl.split_tokens = (int)(((tiles16 + ns - 1) / ns) * 16);
        pl.nsplit = (int)((S + pl.split_tokens - 1) / pl.split_tokens);
        int64_t oc = (kStepOutputs + BH - 1) / BH;
        oc = std::max<int64_t>((tiles16 + 15) / 16, std::min<int64_t>(oc, tiles16));
        pl.chunk_tokens = (int)(((tiles16 + oc - 1) / oc) * 16);
        pl.nchunk = (int)((S + pl.chunk_tokens - 1) / pl.chunk_tokens);
        pl.part_bytes = (size_t)(BH * pl.nsplit * D * D * 4);
        pl.mt_bytes = (size_t)(BH * D * D * 2);
        pl.step_ctl_bytes = pl.step_one ? gdn::step_one_ctl_bytes(BH, pl.nsplit * hv) : 0;
        pl.canon_bytes = 0;
        pl.chain_bytes = 0;
    }
    if (mode == 2) {
        // fp32 forward states and state gradients get F + 1 slots (slot 0: initial state / its
        // gradient); the C_f records hold one fp32 D x D matrix each
        pl.mt_bytes = (size_t)(BH * (F + 1) * D * D * 4);
        pl.crec_bytes = (size_t)(BH * F * D * D * 4);
        pl.gt_bytes = pl.mt_bytes;
    }
    if (mode == 3) {
        pl.gt_bytes = (size_t)(BH * (F + 1) * D * D * 4);
        pl.crec_bytes = (size_t)(BH * F * D * D * 4);
        pl.canon_bytes = 0;   // the forward's records and states come from the saved buffer
        pl.mt_bytes = 0;
    }
    if (mode >= 2) {
        // chained: ticket counter, time-out flag and frame flags first (the time-out flag at byte
        // 4, as in the fused forward), two fp32 state-gradient buffers per (b, h), no C records
        if (pl.fused) pl.crec_bytes = 0;
        else pl.ctl_bytes = pl.chain_bytes = 0;
    }
    if (mode == 2 && pl.fused && fused_rows_fit(p)) {
        // chained, recomputing: the fused forward (no outputs) recomputes the states into the
        // layout of a saving forward's buffer: the frames' Ghat planes, then F + 1 fp32 states
        pl.fused_states = true;
        pl.canon_bytes = p.use_delta ? (size_t)(BH * F * (D / 16) * 2 * ((D + 31) / 32) * 1024) : 0;
        pl.part_bytes = 0;
        pl.mt_bytes = (size_t)(BH * (F + 1) * D * D * 4);
    }
    return pl;
}

// Buffer kept by gdn_forward_framewise_save for gdn_backward_framewise_saved: the frames' Ghat
// planes (delta rule only), then the initial state and every M_f in fp32, transposed.
struct SavedPlan {
    size_t rec_bytes;     // per frame record
    size_t recs, states;
    size_t total() const { return align256(recs) + states; }
};
SavedPlan saved_plan(const gdn_problem& p) {
    const int64_t D = p.head_dim, BH = (int64_t)p.batch * p.heads, F = p.frames;
    SavedPlan sp{};
    sp.rec_bytes = p.use_delta ? (size_t)((D / 16) * 2 * ((D + 31) / 32) * 1024) : 0;
    sp.recs = (size_t)(BH * F) * sp.rec_bytes;
    sp.states = (size_t)(BH * (F + 1) * D * D * 4);
    return sp;
}

gdn_status check_sizes(const gdn_problem* p, int mode) {
    const int step_mode = mode == 1;
    if (!p) return fail(GDN_ERR_NULL, "problem descriptor is NULL");
    if (p->batch < 1 || p->heads < 1 || p->tokens_per_frame < 1 || (!step_mode && p->frames < 1))
        return fail(GDN_ERR_SHAPE, "sizes must be >= 1 (B=%d H=%d S=%d F=%d)", p->batch, p->heads,
                    p->tokens_per_frame, p->frames);
    const int D = p->head_dim;
    if (D != 16 && D != 32 && D != 64 && D != 128)
        return fail(GDN_ERR_UNSUPPORTED, "head_dim %d not supported (16, 32, 64, 128)", D);
    if (p->dtype != GDN_F32 && p->dtype != GDN_BF16 && p->dtype != GDN_FP8_E4M3)
        return fail(GDN_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
    if (p->dtype == GDN_FP8_E4M3) {
        if (mode != 0)
            return fail(GDN_ERR_UNSUPPORTED, "E4M3 inputs: the forward over all frames only");
        if (D != 64 && D != 128)
            return fail(GDN_ERR_UNSUPPORTED, "E4M3 inputs need D = 64 or 128");
        if (p->schedule == GDN_SCHEDULE_STAGED)
            return fail(GDN_ERR_UNSUPPORTED, "E4M3 inputs run on the fused schedule only");
    }
    if (p->schedule < GDN_SCHEDULE_AUTO || p->schedule > GDN_SCHEDULE_FUSED)
        return fail(GDN_ERR_SHAPE, "schedule must be 0, 1 or 2, got %d", p->schedule);
    if (mode == 0 && p->schedule == GDN_SCHEDULE_FUSED &&
        !gdn::fused_supported(p->dtype != GDN_F32, D))
        return fail(GDN_ERR_UNSUPPORTED, "the fused schedule needs bf16 data and D = 64 or 128");
    if (mode == 0 && (p->schedule == GDN_SCHEDULE_FUSED || p->dtype == GDN_FP8_E4M3) &&
        !fused_rows_fit(*p))
        return fail(GDN_ERR_UNSUPPORTED, "the fused schedule needs a frame's q/k/v rows and its o rows within 2 GiB");
    if (mode == 2 && !gdn::backward_supported(p->dtype == GDN_BF16, D))
        return fail(GDN_ERR_UNSUPPORTED, "the backward needs bf16 data and D = 64 or 128");
    // the gradient kernels address a frame's rows through 32-bit buffer offsets
    if (mode == 2 && !fused_rows_fit(*p))
        return fail(GDN_ERR_UNSUPPORTED, "the backward needs a frame's q/k/v rows and its d_o rows within 2 GiB");
    const int64_t F = step_mode ? 1 : p->frames;
    const int64_t BH = (int64_t)p->batch * p->heads;
    // grid sizes: BH * F * splits must fit a 1-D grid; token indices f*S+s must fit int32 math
    if (BH * F * ((p->tokens_per_frame + 63) / 64) > (int64_t)1 << 30 ||
        F * (int64_t)p->tokens_per_frame > ((int64_t)1 << 31) - 1)
        return fail(GDN_ERR_SHAPE, "problem too large for one call");
    return GDN_OK;
}

// Byte extent [lo, hi) touched by a strided [B,H,T,D] tensor.
struct Span {
    const char* lo;
    const char* hi;
};
Span span_of(const void* base, int64_t B, int64_t H, int64_t T, int64_t D, int64_t sb, int64_t sh,
             int64_t st, int64_t esz) {
    const int64_t last = (B - 1) * sb + (H - 1) * sh + (T - 1) * st + (D - 1);
    return {(const char*)base, (const char*)base + (last + 1) * esz};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Strides must be non-negative and rows of distinct (b, h, t) must not overlap.
bool layout_ok(int64_t B, int64_t H, int64_t T, int64_t D, int64_t sb, int64_t sh, int64_t st) {
    if (sb < 0 || sh < 0 || st < 0) return false;
    struct Dim { int64_t n, s; } d[4] = {{B, sb}, {H, sh}, {T, st}, {D, 1}};
    Dim v[4];
    int k = 0;
    for (auto& x : d)
        if (x.n > 1) v[k++] = x;
    std::sort(v, v + k, [](const Dim& a, const Dim& b) { return a.s < b.s; });
    int64_t extent = 1;
    for (int i = 0; i < k; ++i) {
        if (v[i].s < extent) return false;
        extent = v[i].s * (v[i].n - 1) + extent;
    }
    return true;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Polls of a frame flag before a fused-schedule workgroup gives up: GDN_FUSED_SPIN_LIMIT from
// the environment (a diagnostic; 0 makes every frame after the first time out at once, so the
// time-out path can be exercised), else the default.
int fused_spin_limit() {
    const char* e = getenv("GDN_FUSED_SPIN_LIMIT");
    if (!e || !*e) return gdn::kSpinLimitDefault;
    char* end = nullptr;
    const long v = strtol(e, &end, 10);
    if (*end || v < 0 || v > (1L << 30)) return gdn::kSpinLimitDefault;
    return (int)v;
}

// scales: the three E4M3 scale arrays (gdn_forward_framewise_fp8), or NULL
// scratch: take the workspace from the library's own device scratch (ws and ws_bytes are
// ignored); every argument is validated before its address is looked up
gdn_status run(int step_mode, const gdn_problem* p, const void* q, const void* k, const void* v,
               const float* const* scales, const float* gamma, const float* beta,
               const float* state_in, void* o, float* state_out, void* ws, size_t ws_bytes,
               void* stream, void* saved = nullptr, size_t saved_bytes = 0, bool scratch = false) {
    g_msg[0] = '\0';
    gdn_status s = check_sizes(p, step_mode);
    if (s != GDN_OK) return s;
    const bool fp8 = p->dtype == GDN_FP8_E4M3;
    if (fp8 && !scales)
        return fail(GDN_ERR_UNSUPPORTED, "E4M3 inputs go through gdn_forward_framewise_fp8");
    if (!fp8 && scales)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_forward_framewise_fp8 needs dtype GDN_FP8_E4M3");
    const int64_t B = p->batch, H = p->heads, D = p->head_dim, S = p->tokens_per_frame;
    const int64_t F = step_mode ? 1 : p->frames;
    const int64_t T = F * S;
    const int64_t esz = fp8 ? 1 : p->dtype == GDN_BF16 ? 2 : 4;   // Q, K, V
    const int64_t oesz = fp8 ? 2 : esz;                             // O
    if (!q || !k || !v || !o || !gamma || !beta)
        return fail(GDN_ERR_NULL, "q, k, v, o, gamma and beta are required");
    if (fp8 && (!scales[0] || !scales[1] || !scales[2]))
        return fail(GDN_ERR_NULL, "q_scale, k_scale and v_scale are required");
    if (step_mode && !state_in) return fail(GDN_ERR_NULL, "state_in is required in step mode");
    if (!layout_ok(B, H, T, D, p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t))
        return fail(GDN_ERR_STRIDE, "q/k/v strides (%lld, %lld, %lld) overlap rows or are negative",
                    (long long)p->qkv_stride_b, (long long)p->qkv_stride_h, (long long)p->qkv_stride_t);
    if (!layout_ok(B, H, T, D, p->o_stride_b, p->o_stride_h, p->o_stride_t))
        return fail(GDN_ERR_STRIDE, "o strides (%lld, %lld, %lld) overlap rows or are negative",
                    (long long)p->o_stride_b, (long long)p->o_stride_h, (long long)p->o_stride_t);
    for (const void* ptr : {q, k, v, (const void*)o})
        if (!aligned(ptr, 16)) return fail(GDN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
    const int64_t strides[6] = {p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t,
                                p->o_stride_b,   p->o_stride_h,   p->o_stride_t};
    for (int64_t st : strides)
        if (st % 8) return fail(GDN_ERR_ALIGN, "strides must be multiples of 8 elements");
    for (const void* ptr : {(const void*)gamma, (const void*)beta, (const void*)state_in,
                            (const void*)state_out})
        if (ptr && !aligned(ptr, 4)) return fail(GDN_ERR_ALIGN, "gates and states must be 4-byte aligned");
    if (fp8)
        for (int i = 0; i < 3; ++i)
            if (!aligned(scales[i], 4)) return fail(GDN_ERR_ALIGN, "scales must be 4-byte aligned");

    const Plan pl = make_plan(*p, step_mode);
    const size_t need = pl.total();
    const SavedPlan sp = saved_plan(*p);
    if (saved && !pl.fused) return fail(GDN_ERR_UNSUPPORTED, "saving for the backward needs the fused schedule");
    if (scratch) {
        if (need > gdn::kScratchBytes)
            return fail(GDN_ERR_WORKSPACE, "this problem needs %zu bytes of workspace, more than the "
                        "library's static scratch of %zu bytes; pass a workspace to gdn_step_frame",
                        need, gdn::kScratchBytes);
        ws = nullptr;   // a library-owned array cannot overlap the caller's buffers
        ws_bytes = gdn::kScratchBytes;
    }

    const Span sq = span_of(q, B, H, T, D, p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t, esz);
    const Span sk = span_of(k, B, H, T, D, p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t, esz);
    const Span sv = span_of(v, B, H, T, D, p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t, esz);
    const Span so = span_of(o, B, H, T, D, p->o_stride_b, p->o_stride_h, p->o_stride_t, oesz);
    const Span sg = {(const char*)gamma, (const char*)(gamma + B * H * F)};
    const Span sbt = {(const char*)beta, (const char*)(beta + B * H * F)};
    const Span none = {nullptr, nullptr};
    const Span sw = ws ? Span{(const char*)ws, (const char*)ws + need} : none;
    const Span si = state_in ? Span{(const char*)state_in, (const char*)(state_in + B * H * D * D)} : none;
    const Span sso = state_out ? Span{(const char*)state_out, (const char*)(state_out + B * H * D * D)} : none;
    for (Span in : {sq, sk, sv, sg, sbt, si, sw})
        if (overlap(so, in)) return fail(GDN_ERR_ALIAS, "o overlaps an input or the workspace");
    if (fp8)
        for (int i = 0; i < 3; ++i) {
            const Span sc = {(const char*)scales[i], (const char*)(scales[i] + B * H * F)};
            if (overlap(so, sc) || overlap(sw, sc) || (state_out && overlap(sso, sc)))
                return fail(GDN_ERR_ALIAS, "an output or the workspace overlaps a scale array");
        }
    for (Span in : {sq, sk, sv, sg, sbt, so, si})
        if (overlap(sw, in)) return fail(GDN_ERR_ALIAS, "workspace overlaps an input or output");
    if (saved) {
        const Span ssv = {(const char*)saved, (const char*)saved + sp.total()};
        for (Span in : {sq, sk, sv, sg, sbt, so, si, sw, sso})
            if (overlap(ssv, in)) return fail(GDN_ERR_ALIAS, "the saved buffer overlaps another buffer");
        if (saved_bytes < sp.total())
            return fail(GDN_ERR_WORKSPACE, "saved buffer of %zu bytes needed, %zu given", sp.total(), saved_bytes);
        if (!aligned(saved, 256)) return fail(GDN_ERR_ALIGN, "the saved buffer must be 256-byte aligned");
    }
    if (state_out) {
        for (Span in : {sq, sk, sv, sg, sbt, so, sw})
            if (overlap(sso, in)) return fail(GDN_ERR_ALIAS, "state_out overlaps another buffer");
        if (state_in && state_in != state_out && overlap(sso, si))
            return fail(GDN_ERR_ALIAS, "state_out partially overlaps state_in");
    }
    if (scratch) {
        const hipError_t e = gdn::scratch_address(&ws);
        if (e != hipSuccess)
            return fail(GDN_ERR_HIP, "address of the library's scratch: %s", hipGetErrorString(e));
    }
    if (!ws || ws_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 256)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");

    gdn::Launch L{};
    L.B = (int)B; L.H = (int)H; L.D = (int)D; L.S = (int)S; L.F = (int)F;
    L.bf16 = p->dtype == GDN_BF16;
    L.fp8 = fp8;
    if (fp8) {
        L.q_scale = scales[0]; L.k_scale = scales[1]; L.v_scale = scales[2];
    }
    L.use_delta = p->use_delta != 0;
    L.c = p->key_scale > 0.f ? p->key_scale : (float)(1.0 / std::sqrt((double)D * (double)S));
    L.q = q; L.k = k; L.v = v; L.o = o;
    L.sb = p->qkv_stride_b; L.sh = p->qkv_stride_h; L.st = p->qkv_stride_t;
    L.ob = p->o_stride_b; L.oh = p->o_stride_h; L.ot = p->o_stride_t;
    L.xsb = L.sb; L.xsh = L.sh; L.xst = L.st;
    L.gamma = gamma; L.beta = beta; L.state_in = state_in; L.state_out = state_out;
    if (step_mode && pl.fused) {
        L.step_cols = 1;
        // one launch where the device holds its grid (8 XCDs with a CU for each of a head's
        // workgroups), else the three launches over the same buffers
        const int64_t W = (int64_t)pl.nsplit * gdn::step_halves((int)D);
        L.step_one = pl.step_one && gdn::step_one_device_ok((int)(B * H / 8 * W));
        L.ctl = (int*)ws;
        L.spin_limit = fused_spin_limit();
        L.part = (float*)((char*)ws + align256(pl.step_ctl_bytes));
        L.mt = (char*)ws + align256(pl.step_ctl_bytes) + align256(pl.part_bytes);
        if (S == 1) {
            L.st = std::max<int64_t>(L.st, D);
            L.ot = std::max<int64_t>(L.ot, D);
        }
    } else if (pl.fused) {
        if (saved) {
            L.save_recs = saved;
            L.save_states = (float*)((char*)saved + align256(sp.recs));
        }
        L.spin_limit = fused_spin_limit();
        L.ctl = (int*)ws;
        L.chain = (float*)((char*)ws + align256(pl.ctl_bytes));
        // the fused kernel finds the end of a frame's rows from the token stride (rows past
        // the frame read as zero); a single-token tensor may carry any token stride, which
        // addresses nothing else, so give it one row's length
        if (T == 1) {
            L.st = std::max<int64_t>(L.st, D);
            L.ot = std::max<int64_t>(L.ot, D);
        }
    } else {
        L.canon = ws;
        L.part = (float*)((char*)ws + align256(pl.canon_bytes));
        L.mt = (char*)ws + align256(pl.canon_bytes) + align256(pl.part_bytes);
    }
    L.nsplit = pl.nsplit; L.split_tokens = pl.split_tokens;
    L.nchunk = pl.nchunk; L.chunk_tokens = pl.chunk_tokens;
    const hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (step_mode) {
        e = gdn::run_step(L, st);
    } else {
        e = gdn::run_forward(L, pl.fused, st);
    }
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status run_bwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                   const float* gamma, const float* beta, const float* state_in, const void* d_o,
                   const float* d_state_out, void* dq, void* dk, void* dv, float* dgamma,
                   float* dbeta, float* d_state_in, void* ws, size_t ws_bytes, void* stream,
                   const void* saved = nullptr, size_t saved_bytes = 0) {
    g_msg[0] = '\0';
    gdn_status s = check_sizes(p, 2);
    if (s != GDN_OK) return s;
    const int64_t B = p->batch, H = p->heads, D = p->head_dim, S = p->tokens_per_frame;
    const int64_t F = p->frames, T = F * S;
    const int64_t esz = p->dtype == GDN_BF16 ? 2 : 4;
    if (!q || !k || !v || !gamma || !beta || !d_o || !dq || !dk || !dv || !dgamma || !dbeta)
        return fail(GDN_ERR_NULL, "q, k, v, gamma, beta, d_o and every gradient but d_state_in are required");
    if (!layout_ok(B, H, T, D, p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t))
        return fail(GDN_ERR_STRIDE, "q/k/v strides (%lld, %lld, %lld) overlap rows or are negative",
                    (long long)p->qkv_stride_b, (long long)p->qkv_stride_h, (long long)p->qkv_stride_t);
    if (!layout_ok(B, H, T, D, p->o_stride_b, p->o_stride_h, p->o_stride_t))
        return fail(GDN_ERR_STRIDE, "o strides (%lld, %lld, %lld) overlap rows or are negative",
                    (long long)p->o_stride_b, (long long)p->o_stride_h, (long long)p->o_stride_t);
    for (const void* ptr : {q, k, v, d_o, (const void*)dq, (const void*)dk, (const void*)dv})
        if (!aligned(ptr, 16)) return fail(GDN_ERR_ALIGN, "q, k, v, d_o and dq, dk, dv must be 16-byte aligned");
    const int64_t strides[6] = {p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t,
                                p->o_stride_b,   p->o_stride_h,   p->o_stride_t};
    for (int64_t st : strides)
        if (st % 8) return fail(GDN_ERR_ALIGN, "strides must be multiples of 8 elements");
    for (const void* ptr : {(const void*)gamma, (const void*)beta, (const void*)state_in,
                            (const void*)d_state_out, (const void*)dgamma, (const void*)dbeta,
                            (const void*)d_state_in})
        if (ptr && !aligned(ptr, 4)) return fail(GDN_ERR_ALIGN, "gates, states and their gradients must be 4-byte aligned");

    const Plan pl = make_plan(*p, saved ? 3 : 2);
    const size_t need = pl.total();
    const SavedPlan sp = saved_plan(*p);
    if (saved) {
        if (saved_bytes < sp.total())
            return fail(GDN_ERR_WORKSPACE, "saved buffer of %zu bytes needed, %zu given", sp.total(), saved_bytes);
        if (!aligned(saved, 256)) return fail(GDN_ERR_ALIGN, "the saved buffer must be 256-byte aligned");
    }
    auto qkv_span = [&](const void* x) {
        return span_of(x, B, H, T, D, p->qkv_stride_b, p->qkv_stride_h, p->qkv_stride_t, esz);
    };
    const Span none = {nullptr, nullptr};
    const Span in[] = {qkv_span(q), qkv_span(k), qkv_span(v),
                       {(const char*)gamma, (const char*)(gamma + B * H * F)},
                       {(const char*)beta, (const char*)(beta + B * H * F)},
                       state_in ? Span{(const char*)state_in, (const char*)(state_in + B * H * D * D)} : none,
                       span_of(d_o, B, H, T, D, p->o_stride_b, p->o_stride_h, p->o_stride_t, esz),
                       d_state_out ? Span{(const char*)d_state_out, (const char*)(d_state_out + B * H * D * D)} : none,
                       ws ? Span{(const char*)ws, (const char*)ws + need} : none,
                       saved ? Span{(const char*)saved, (const char*)saved + sp.total()} : none};
    const Span dsi = d_state_in ? Span{(const char*)d_state_in, (const char*)(d_state_in + B * H * D * D)} : none;
    const Span out[] = {qkv_span(dq), qkv_span(dk), qkv_span(dv),
                        {(const char*)dgamma, (const char*)(dgamma + B * H * F)},
                        {(const char*)dbeta, (const char*)(dbeta + B * H * F)}, dsi};
    const int nin = sizeof(in) / sizeof(in[0]), nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j) {
            // the state gradient may be computed in place (d_state_in == d_state_out)
            if (i == nout - 1 && j == 7 && d_state_in && (const void*)d_state_in == (const void*)d_state_out)
                continue;
            if (overlap(out[i], in[j]))
                return fail(GDN_ERR_ALIAS, "a gradient output overlaps an input, the saved buffer or the workspace");
        }
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out[j])) return fail(GDN_ERR_ALIAS, "two gradient outputs overlap");
    }
    if (saved && overlap(Span{(const char*)saved, (const char*)saved + sp.total()},
                         ws ? Span{(const char*)ws, (const char*)ws + need} : none))
        return fail(GDN_ERR_ALIAS, "the saved buffer overlaps the workspace");
    if (!ws || ws_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : (size_t)0);
    if (!aligned(ws, 256)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");

    gdn::Launch L{};
    L.B = (int)B; L.H = (int)H; L.D = (int)D; L.S = (int)S; L.F = (int)F;
    L.bf16 = p->dtype == GDN_BF16;
    L.use_delta = p->use_delta != 0;
    L.c = p->key_scale > 0.f ? p->key_scale : (float)(1.0 / std::sqrt((double)D * (double)S));
    L.q = q; L.k = k; L.v = v;
    L.sb = p->qkv_stride_b; L.sh = p->qkv_stride_h; L.st = p->qkv_stride_t;
    L.ob = p->o_stride_b; L.oh = p->o_stride_h; L.ot = p->o_stride_t;
    L.xsb = L.sb; L.xsh = L.sh; L.xst = L.st;
    L.gamma = gamma; L.beta = beta; L.state_in = state_in;
    L.d_o = d_o; L.d_state_out = d_state_out; L.d_state_in = d_state_in;
    L.dq = dq; L.dk = dk; L.dv = dv; L.dgamma = dgamma; L.dbeta = dbeta;
    char* w = (char*)ws;
    if (pl.fused) {
        L.bwd_chain = 1;
        L.spin_limit = fused_spin_limit();
        L.ctl = (int*)w;               w += align256(pl.ctl_bytes);
        L.chain = (float*)w;           w += align256(pl.chain_bytes);
    }
    L.canon = w;                       w += align256(pl.canon_bytes);
    L.part = (float*)w;                w += align256(pl.part_bytes);
    L.mt = w;                          w += align256(pl.mt_bytes);
    L.crec = w;                        w += align256(pl.crec_bytes);
    L.gt = w;
    // bytes per frame record of Ghat (and Bhat): the products' full record, or the saved planes
    L.rec_stride = (p->use_delta ? (D / 16) * 2 * ((D + 31) / 32) * 1024 : 0) + 4 * D * D;
    if (pl.fused_states) {
        L.fused_states = 1;
        L.save_recs = L.canon;
        L.save_states = (float*)L.mt;
        L.rec_stride = p->use_delta ? (D / 16) * 2 * ((D + 31) / 32) * 1024 : 0;
    }
    if (saved) {
        L.saved = 1;
        L.canon = const_cast<void*>(saved);
        L.rec_stride = (int64_t)sp.rec_bytes;
        L.mt = (char*)const_cast<void*>(saved) + align256(sp.recs);
    }
    L.nsplit = pl.nsplit; L.split_tokens = pl.split_tokens;
    L.nchunk = pl.nchunk; L.chunk_tokens = pl.chunk_tokens;
    const hipError_t e = gdn::run_backward(L, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

gdn_status run_tconv(const gdn_tconv_problem* p, const void* x, const float* weight,
                     const float* bias, const void* cache_in, void* y, void* cache_out,
                     void* stream) {
    g_msg[0] = '\0';
    if (!p) return fail(GDN_ERR_NULL, "problem descriptor is NULL");
    if (p->batch < 1 || p->frames < 1 || p->tokens < 1 || p->channels < 1 || p->block_frames < 1)
        return fail(GDN_ERR_SHAPE, "sizes must be >= 1 (B=%d T=%d S=%d C=%d block_frames=%d)",
                    p->batch, p->frames, p->tokens, p->channels, p->block_frames);
    if (p->frames % p->block_frames)
        return fail(GDN_ERR_SHAPE, "frames (%d) must be a multiple of block_frames (%d)", p->frames,
                    p->block_frames);
    if (p->dtype != GDN_F32 && p->dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "dtype %d not supported (GDN_F32, GDN_BF16)", p->dtype);
    if (p->channels % 8) return fail(GDN_ERR_ALIGN, "channels must be a multiple of 8");
    if (!x || !weight || !y) return fail(GDN_ERR_NULL, "x, weight and y are required");
    if (!aligned(weight, 16) || (bias && !aligned(bias, 16)))
        return fail(GDN_ERR_ALIGN, "weight and bias must be 16-byte aligned");
    const int64_t B = p->batch, T = p->frames, S = p->tokens, C = p->channels;
    const int64_t esz = p->dtype == GDN_BF16 ? 2 : 4;
    // one thread per 16 bytes of channels and (up to) 16 frames; the kernel indexes threads
    // in 32 bits
    if (B * S * (C / (16 / esz)) * ((T + 15) / 16) > ((int64_t)1 << 31) - 256)
        return fail(GDN_ERR_SHAPE, "problem too large for one call");
    if (!layout_ok(B, T, S, C, p->x_stride_b, p->x_stride_t, p->x_stride_s))
        return fail(GDN_ERR_STRIDE, "x strides overlap rows or are negative");
    if (!layout_ok(B, T, S, C, p->y_stride_b, p->y_stride_t, p->y_stride_s))
        return fail(GDN_ERR_STRIDE, "y strides overlap rows or are negative");
    for (const void* ptr : {x, (const void*)y, cache_in, (const void*)cache_out})
        if (ptr && !aligned(ptr, 16)) return fail(GDN_ERR_ALIGN, "x, y and the caches must be 16-byte aligned");
    for (int64_t st : {p->x_stride_b, p->x_stride_t, p->x_stride_s, p->y_stride_b, p->y_stride_t, p->y_stride_s})
        if (st % 8) return fail(GDN_ERR_ALIGN, "strides must be multiples of 8 elements");
    for (const void* ptr : {(const void*)weight, (const void*)bias})
        if (ptr && !aligned(ptr, 4)) return fail(GDN_ERR_ALIGN, "weight and bias must be 4-byte aligned");
    const Span none = {nullptr, nullptr};
    const Span sx = span_of(x, B, T, S, C, p->x_stride_b, p->x_stride_t, p->x_stride_s, esz);
    const Span sy = span_of(y, B, T, S, C, p->y_stride_b, p->y_stride_t, p->y_stride_s, esz);
    const Span sw = {(const char*)weight, (const char*)(weight + 3 * C)};
    const Span sbias = bias ? Span{(const char*)bias, (const char*)(bias + C)} : none;
    const Span sci = cache_in ? Span{(const char*)cache_in, (const char*)cache_in + B * S * C * esz} : none;
    const Span sco = cache_out ? Span{(const char*)cache_out, (const char*)cache_out + B * S * C * esz} : none;
    for (Span in : {sx, sw, sbias, sci, sco})
        if (overlap(sy, in)) return fail(GDN_ERR_ALIAS, "y overlaps an input or cache_out");
    for (Span in : {sx, sw, sbias})
        if (overlap(sco, in)) return fail(GDN_ERR_ALIAS, "cache_out overlaps an input");
    if (cache_in && cache_out && cache_in != cache_out && overlap(sco, sci))
        return fail(GDN_ERR_ALIAS, "cache_out partially overlaps cache_in");
    gdn::TconvLaunch L{};
    L.B = (int)B; L.T = (int)T; L.S = (int)S; L.C = (int)C; L.Tb = p->block_frames;
    L.bf16 = p->dtype == GDN_BF16;
    L.xsb = p->x_stride_b; L.xst = p->x_stride_t; L.xss = p->x_stride_s;
    L.ysb = p->y_stride_b; L.yst = p->y_stride_t; L.yss = p->y_stride_s;
    L.x = x; L.weight = weight; L.bias = bias; L.cache_in = cache_in; L.y = y; L.cache_out = cache_out;
    const hipError_t e = gdn::run_tconv(L, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

// Sizes, layout and limits of an attention problem (no pointers); fills the launch's shape.
gdn_status attn_shape(const gdn_attn_problem* p, gdn::AttnLaunch& L) {
    if (!p) return fail(GDN_ERR_NULL, "problem descriptor is NULL");
    if (p->batch < 1 || p->heads < 1 || p->tokens_per_frame < 1 || p->q_frames < 1 ||
        p->kv_frames < 1 || p->q_frame0 < 0)
        return fail(GDN_ERR_SHAPE, "sizes must be >= 1 and q_frame0 >= 0");
    if (p->q_frame0 + (int64_t)p->q_frames > p->kv_frames)
        return fail(GDN_ERR_SHAPE, "the query frames (%d .. %d) must lie within the key frames (0 .. %d)",
                    p->q_frame0, p->q_frame0 + p->q_frames - 1, p->kv_frames - 1);
    if (!gdn::attn_supported(p->head_dim))
        return fail(GDN_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", p->head_dim);
    if (p->dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "attention takes bf16 data");
    const int64_t B = p->batch, H = p->heads, D = p->head_dim, S = p->tokens_per_frame;
    const int64_t Tq = (int64_t)p->q_frames * S, Tk = (int64_t)p->kv_frames * S;
    if (Tk > ((int64_t)1 << 31) - 1 || B * H * ((Tq + 127) / 128) > ((int64_t)1 << 31) - 1 ||
        B * H * Tq * D * 16 > ((int64_t)1 << 62))
        return fail(GDN_ERR_SHAPE, "problem too large for one call");
    if (!layout_ok(B, H, Tq, D, p->q_stride_b, p->q_stride_h, p->q_stride_t) ||
        !layout_ok(B, H, Tk, D, p->kv_stride_b, p->kv_stride_h, p->kv_stride_t) ||
        !layout_ok(B, H, Tq, D, p->o_stride_b, p->o_stride_h, p->o_stride_t))
        return fail(GDN_ERR_STRIDE, "strides overlap rows or are negative");
    // the kernel addresses a head's key and value rows through 32-bit offsets from each tile
    if (((Tk - 1) * p->kv_stride_t + D) * 2 >= ((int64_t)1 << 31))
        return fail(GDN_ERR_UNSUPPORTED, "a head's key/value rows must lie within 2 GiB");
    for (int64_t st : {p->q_stride_b, p->q_stride_h, p->q_stride_t, p->kv_stride_b, p->kv_stride_h,
                       p->kv_stride_t, p->o_stride_b, p->o_stride_h, p->o_stride_t})
        if (st % 8) return fail(GDN_ERR_ALIGN, "strides must be multiples of 8 elements");
    L = gdn::AttnLaunch{};
    L.B = (int)B; L.H = (int)H; L.D = (int)D; L.S = (int)S; L.Tq = (int)Tq; L.Tk = (int)Tk;
    L.q_frame0 = p->q_frame0;
    L.scale = p->scale > 0.f ? p->scale : (float)(1.0 / std::sqrt((double)D));
    L.qsb = p->q_stride_b; L.qsh = p->q_stride_h; L.qst = p->q_stride_t;
    L.ksb = p->kv_stride_b; L.ksh = p->kv_stride_h; L.kst = p->kv_stride_t;
    L.osb = p->o_stride_b; L.osh = p->o_stride_h; L.ost = p->o_stride_t;
    return GDN_OK;
}

// ws == NULL: no key splits (the plain entry point)
gdn_status run_attn(const gdn_attn_problem* p, const void* q, const void* k, const void* v,
                    void* o, void* ws, size_t ws_bytes, void* stream) {
    g_msg[0] = '\0';
    gdn::AttnLaunch L;
    gdn_status st = attn_shape(p, L);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !o) return fail(GDN_ERR_NULL, "q, k, v and o are required");
    const int64_t B = L.B, H = L.H, D = L.D, Tq = L.Tq, Tk = L.Tk;
    for (const void* ptr : {q, k, v, (const void*)o})
        if (!aligned(ptr, 16)) return fail(GDN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
    const Span so = span_of(o, B, H, Tq, D, p->o_stride_b, p->o_stride_h, p->o_stride_t, 2);
    const Span ins[3] = {span_of(q, B, H, Tq, D, p->q_stride_b, p->q_stride_h, p->q_stride_t, 2),
                         span_of(k, B, H, Tk, D, p->kv_stride_b, p->kv_stride_h, p->kv_stride_t, 2),
                         span_of(v, B, H, Tk, D, p->kv_stride_b, p->kv_stride_h, p->kv_stride_t, 2)};
    for (Span in : ins)
        if (overlap(so, in)) return fail(GDN_ERR_ALIAS, "o overlaps q, k or v");
    size_t need = 0;
    gdn::attn_plan(L, ws != nullptr, &need);
    if (need) {
        if (ws_bytes < need)
            return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
        if (!aligned(ws, 256)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");
        const Span sw{(const char*)ws, (const char*)ws + need};
        if (overlap(sw, so) || overlap(sw, ins[0]) || overlap(sw, ins[1]) || overlap(sw, ins[2]))
            return fail(GDN_ERR_ALIAS, "the workspace overlaps q, k, v or o");
        const size_t part_bytes = ((size_t)L.nsplit * B * H * Tq * D * 4 + 255) / 256 * 256;
        L.part = (float*)ws;
        L.ml = (float*)((char*)ws + part_bytes);
    }
    L.q = q; L.k = k; L.v = v; L.o = o;
    const hipError_t e = gdn::run_attn(L, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_workspace_size(const gdn_problem* p, int mode, size_t* bytes_out) {
    g_msg[0] = '\0';
    if (!bytes_out) return fail(GDN_ERR_NULL, "bytes_out is NULL");
    if (mode < 0 || mode > 3) return fail(GDN_ERR_SHAPE, "mode must be 0, 1, 2 or 3, got %d", mode);
    gdn_status s = check_sizes(p, mode == 3 ? 2 : mode);
    if (s != GDN_OK) return s;
    const Plan pl = make_plan(*p, mode);
    *bytes_out = pl.total();
    return GDN_OK;
}

gdn_status gdn_forward_framewise(const gdn_problem* p, const void* q, const void* k, const void* v,
                                 const float* gamma, const float* beta, const float* state_in,
                                 void* o, float* state_out, void* workspace, size_t workspace_bytes,
                                 void* hip_stream) {
    return run(0, p, q, k, v, nullptr, gamma, beta, state_in, o, state_out, workspace,
               workspace_bytes, hip_stream);
}

gdn_status gdn_forward_framewise_fp8(const gdn_problem* p, const void* q, const void* k,
                                     const void* v, const float* q_scale, const float* k_scale,
                                     const float* v_scale, const float* gamma, const float* beta,
                                     const float* state_in, void* o, float* state_out,
                                     void* workspace, size_t workspace_bytes, void* hip_stream) {
    const float* scales[3] = {q_scale, k_scale, v_scale};
    return run(0, p, q, k, v, scales, gamma, beta, state_in, o, state_out, workspace,
               workspace_bytes, hip_stream);
}

gdn_status gdn_step_frame(const gdn_problem* p, const void* q, const void* k, const void* v,
                          const float* gamma, const float* beta, const float* state_in, void* o,
                          float* state_out, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
    return run(1, p, q, k, v, nullptr, gamma, beta, state_in, o, state_out, workspace,
               workspace_bytes, hip_stream);
}

gdn_status gdn_step_frame_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v,
                                  const float* gamma, const float* beta, const float* state_in,
                                  void* o, float* state_out, void* hip_stream) {
    return run(1, p, q, k, v, nullptr, gamma, beta, state_in, o, state_out, nullptr, 0, hip_stream,
               nullptr, 0, true);
}

gdn_status gdn_check_timeout(const gdn_problem* p, int mode, const void* workspace,
                             void* hip_stream) {
    g_msg[0] = '\0';
    if (mode < 0 || mode > 3) return fail(GDN_ERR_SHAPE, "mode must be 0, 1, 2 or 3, got %d", mode);
    gdn_status s = check_sizes(p, mode == 3 ? 2 : mode);
    if (s != GDN_OK) return s;
    const Plan pl = make_plan(*p, mode);
    // bounded waits: the fused forward, the backward's chained schedule (its reverse chain and,
    // recomputing, the fused forward that rebuilds the states) and the one-launch step
    const bool waits = mode == 1 ? pl.fused && pl.step_one : pl.fused || pl.fused_states;
    if (!waits) return GDN_OK;
    if (!workspace) return fail(GDN_ERR_NULL, "workspace is NULL");
    hipError_t e = hipStreamSynchronize((hipStream_t)hip_stream);
    if (mode == 1) {
        // the step's time-out word stays set until read here
        uint64_t word = 0;
        if (e == hipSuccess) e = hipMemcpy(&word, workspace, sizeof word, hipMemcpyDeviceToHost);
        const bool timed_out = e == hipSuccess && word == gdn::kStepTimeoutWord;
        if (timed_out) {
            const uint64_t zero = 0;
            e = hipMemcpy(const_cast<void*>(workspace), &zero, sizeof zero, hipMemcpyHostToDevice);
        }
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "reading the time-out word failed: %s", hipGetErrorString(e));
        if (timed_out)
            return fail(GDN_ERR_TIMEOUT, "a bounded wait of the one-launch step timed out; its "
                                         "state and outputs are NaN");
        return GDN_OK;
    }
    int32_t flag = 0;
    if (e == hipSuccess) e = hipMemcpy(&flag, (const char*)workspace + 4, sizeof flag, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "reading the time-out flag failed: %s", hipGetErrorString(e));
    if (flag)
        return fail(GDN_ERR_TIMEOUT, "a bounded wait of the fused schedule timed out; the outputs "
                                     "that depend on it are NaN");
    return GDN_OK;
}

gdn_status gdn_saved_size(const gdn_problem* p, size_t* bytes_out) {
    g_msg[0] = '\0';
    if (!bytes_out) return fail(GDN_ERR_NULL, "bytes_out is NULL");
    gdn_status s = check_sizes(p, 2);
    if (s != GDN_OK) return s;
    if (!fused_rows_fit(*p)) return fail(GDN_ERR_UNSUPPORTED, "the fused schedule needs a frame's q/k/v rows and its o rows within 2 GiB");
    *bytes_out = saved_plan(*p).total();
    return GDN_OK;
}
gdn_status gdn_forward_framewise_save(const gdn_problem* p, const void* q, const void* k,
                                      const void* v, const float* gamma, const float* beta,
                                      const float* state_in, void* o, float* state_out,
                                      void* saved, size_t saved_bytes, void* workspace,
                                      size_t workspace_bytes, void* hip_stream) {
    g_msg[0] = '\0';
    if (!p) return fail(GDN_ERR_NULL, "problem descriptor is NULL");
    if (!saved) return fail(GDN_ERR_NULL, "saved is required");
    gdn_status s = check_sizes(p, 2);   // what the backward supports
    if (s != GDN_OK) return s;
    if (p->schedule == GDN_SCHEDULE_STAGED)
        return fail(GDN_ERR_UNSUPPORTED, "saving for the backward runs on the fused schedule");
    gdn_problem pf = *p;
    pf.schedule = GDN_SCHEDULE_FUSED;
    return run(0, &pf, q, k, v, nullptr, gamma, beta, state_in, o, state_out, workspace,
               workspace_bytes, hip_stream, saved, saved_bytes);
}
gdn_status gdn_backward_framewise_saved(const gdn_problem* p, const void* q, const void* k,
                                        const void* v, const float* gamma, const float* beta,
                                        const void* saved, size_t saved_bytes, const void* d_o,
                                        const float* d_state_out, void* dq, void* dk, void* dv,
                                        float* dgamma, float* dbeta, float* d_state_in,
                                        void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!saved) {
        g_msg[0] = '\0';
        return fail(GDN_ERR_NULL, "saved is required");
    }
    return run_bwd(p, q, k, v, gamma, beta, nullptr, d_o, d_state_out, dq, dk, dv, dgamma, dbeta,
                   d_state_in, workspace, workspace_bytes, hip_stream, saved, saved_bytes);
}
gdn_status gdn_backward_framewise(const gdn_problem* p, const void* q, const void* k,
                                  const void* v, const float* gamma, const float* beta,
                                  const float* state_in, const void* d_o,
                                  const float* d_state_out, void* dq, void* dk, void* dv,
                                  float* dgamma, float* dbeta, float* d_state_in,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
    return run_bwd(p, q, k, v, gamma, beta, state_in, d_o, d_state_out, dq, dk, dv, dgamma, dbeta,
                   d_state_in, workspace, workspace_bytes, hip_stream);
}

gdn_status gdn_tconv_forward(const gdn_tconv_problem* p, const void* x, const float* weight,
                             const float* bias, const void* cache_in, void* y, void* cache_out,
                             void* hip_stream) {
    return run_tconv(p, x, weight, bias, cache_in, y, cache_out, hip_stream);
}

gdn_status gdn_attention_framecausal(const gdn_attn_problem* p, const void* q, const void* k,
                                     const void* v, void* o, void* hip_stream) {
    return run_attn(p, q, k, v, o, nullptr, 0, hip_stream);
}

gdn_status gdn_attention_workspace_size(const gdn_attn_problem* p, size_t* bytes_out) {
    g_msg[0] = '\0';
    if (!bytes_out) return fail(GDN_ERR_NULL, "bytes_out is NULL");
    gdn::AttnLaunch L;
    gdn_status st = attn_shape(p, L);
    if (st != GDN_OK) return st;
    gdn::attn_plan(L, true, bytes_out);
    return GDN_OK;
}

gdn_status gdn_attention_framecausal_ws(const gdn_attn_problem* p, const void* q, const void* k,
                                        const void* v, void* o, void* workspace,
                                        size_t workspace_bytes, void* hip_stream) {
    return run_attn(p, q, k, v, o, workspace, workspace_bytes, hip_stream);
}

gdn_status gdn_set_trace(void* const* events, int pairs) {
    g_msg[0] = '\0';
    if (pairs < 0 || pairs > (1 << 16)) return fail(GDN_ERR_SHAPE, "pairs must be 0..65536, got %d", pairs);
    if (pairs > 0 && !events) return fail(GDN_ERR_NULL, "events is NULL");
    gdn::set_trace(events, events ? pairs : 0);
    return GDN_OK;
}

int gdn_trace_read(gdn_trace_entry* entries, int capacity) {
    return gdn::read_trace(entries, capacity < 0 ? 0 : capacity);
}

const char* gdn_status_string(gdn_status s) {
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "null pointer";
    case GDN_ERR_SHAPE: return "bad shape";
    case GDN_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or mode";
    case GDN_ERR_STRIDE: return "bad strides";
    case GDN_ERR_ALIGN: return "misaligned pointer or stride";
    case GDN_ERR_ALIAS: return "overlapping buffers";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP runtime error";
    case GDN_ERR_TIMEOUT: return "a bounded wait timed out";
    }
    return "unknown status";
}

const char* gdn_last_error_message(void) { return g_msg; }

int gdn_abi_version(void) { return LIBGDN_ABI_VERSION; }

}  // extern "C"
