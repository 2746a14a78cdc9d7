// Launch runtime of libgdn: the order of the kernels of a forward or a step on the caller's
// stream, and the launch trace.
//
// Forward, staged:  products (gram items of every frame) -> [combine] -> scan -> products
//                   (output items of every frame).
// Forward, fused:   reset of the ticket counter and frame flags -> fused kernel.
// Step:             bf16 with D = 64 or 128: the Gram-form kernels, in one launch
//                   (step_fused) where the heads fill the XCDs, else step_partial ->
//                   step_reduce -> step_output; otherwise step_partial -> step_reduce ->
//                   products (output items of the one frame).
// Temporal conv:    one launch (the whole block or sequence).
// Attention:        one launch.
// Backward:         products + [combine] + scan (forward states) unless a saving forward kept
//                   them; then either (chained) reset + one ticket-ordered pass over Q and dO
//                   forming dQ, C_f = Q_f^T dO_f and the reverse chain of state gradients, or
//                   the same pass without the chain + [combine] + reverse scan; then the
//                   per-frame gradients of K, V, gamma and beta. States and state gradients are
//                   kept in fp32.
#include <vector>

#include "../../include/libgdn.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// Launch trace of the calling thread.
thread_local std::vector<hipEvent_t> t_trace_events;
thread_local std::vector<gdn_trace_entry> t_trace_log;

struct Launcher {
    const Launch& L;
    hipStream_t caller;
    hipError_t go(Kernel k, const Launch& A, hipStream_t s, int64_t units) {
        const size_t i = t_trace_log.size();
        const bool armed = !t_trace_events.empty();
        const bool timed = armed && 2 * i + 1 < t_trace_events.size();
        hipError_t e = hipSuccess;
        if (timed && (e = hipEventRecord(t_trace_events[2 * i], s)) != hipSuccess) return e;
        if ((e = A.step_cols ? step_launch(k, A, s) : launch_kernel(k, A, s)) != hipSuccess) return e;
        if (timed && (e = hipEventRecord(t_trace_events[2 * i + 1], s)) != hipSuccess) return e;
        if (armed) t_trace_log.push_back({(int32_t)k, s == caller ? 0 : 1, units});
        return hipSuccess;
    }
};

#define GDN_TRY(x)                          \
    do {                                    \
        const hipError_t e_ = (x);          \
        if (e_ != hipSuccess) return e_;    \
    } while (0)

}  // namespace

hipError_t run_forward(const Launch& L0, bool fused, hipStream_t s) {
    t_trace_log.clear();
    Launcher run{L0, s};
    const int64_t BH = (int64_t)L0.B * L0.H;
    const int F = L0.F;
    if (fused) {
        GDN_TRY(run.go(K_FUSED_RESET, L0, s, BH));
        return run.go(K_FUSED, L0, s, BH * F);
    }
    Launch A = L0;
    A.g0 = 0; A.gn = F; A.o0 = 0; A.on = 0;
    GDN_TRY(run.go(K_PRODUCTS, A, s, BH * F));
    if (L0.nsplit > 1) GDN_TRY(run.go(K_COMBINE, A, s, BH * F));
    A.s0 = 0; A.s1 = F;
    A.scan_in = L0.state_in;
    A.scan_out = L0.state_out;
    GDN_TRY(run.go(K_SCAN, A, s, BH * F));
    A.gn = 0; A.on = F;
    return run.go(K_PRODUCTS, A, s, BH * F);
}

hipError_t run_step(const Launch& L0, hipStream_t s) {
    t_trace_log.clear();
    Launcher run{L0, s};
    const int64_t BH = (int64_t)L0.B * L0.H;
    if (L0.step_one) return run.go(K_STEP_FUSED, L0, s, BH);
    if (L0.step_cols) {
        GDN_TRY(run.go(K_STEP_PARTIAL, L0, s, BH));
        GDN_TRY(run.go(K_STEP_REDUCE, L0, s, BH));
        return run.go(K_STEP_OUTPUT, L0, s, BH);
    }
    GDN_TRY(run.go(K_STEP_PARTIAL, L0, s, BH));
    GDN_TRY(run.go(K_STEP_REDUCE, L0, s, BH));
    Launch A = L0;
    A.F = 1;
    A.gn = 0;
    A.o0 = 0;
    A.on = 1;
    return run.go(K_PRODUCTS, A, s, BH);
}

hipError_t run_backward(const Launch& L0, hipStream_t s) {
    t_trace_log.clear();
    Launcher run{L0, s};
    const int64_t BH = (int64_t)L0.B * L0.H;
    const int F = L0.F;
    // 1. forward states: products of every frame, then the scan, M_f to slot f + 1 (slot 0:
    //    the initial state); taken from a forward's saved buffer instead when given
    if (L0.fused_states) {
        // 1'. the fused forward (ticket-ordered, no outputs) keeps each frame's Ghat planes and
        //     M_f, laid out as a saving forward's buffer; the rest runs as from saved states
        Launch A = L0;
        A.state_out = nullptr;
        A.no_output = 1;
        GDN_TRY(run.go(K_FUSED_RESET, A, s, BH));
        GDN_TRY(run.go(K_FUSED, A, s, BH * F));
    } else if (!L0.saved) {
        Launch A = L0;
        A.g0 = 0; A.gn = F; A.o0 = 0; A.on = 0;
        GDN_TRY(run.go(K_PRODUCTS, A, s, BH * F));
        if (L0.nsplit > 1) GDN_TRY(run.go(K_COMBINE, A, s, BH * F));
        A.s0 = 0; A.s1 = F;
        A.scan_in = L0.state_in;
        A.scan_out = nullptr;
        A.mt_lead = 1;
        GDN_TRY(run.go(K_SCAN_STATES, A, s, BH * F));
    }
    if (L0.bwd_chain) {
        // 2'. one ticket-ordered pass over Q and dO in descending frame order: dQ_f, C_f and the
        //     reverse chain G_f (slot f + 1), dstate_in from the workgroup of frame 0
        Launch R = L0;
        R.keep_timeout = L0.fused_states;   // a time-out of the recompute stays visible
        GDN_TRY(run.go(K_FUSED_RESET, R, s, BH));
        GDN_TRY(run.go(K_BWD_QDO, L0, s, BH * F));
        return run.go(K_BWD, L0, s, BH * F);
    }
    // 2. one pass over Q and dO: C_f = Q_f^T dO_f of every frame (its per-frame record, in the
    //    no-delta layout of the gram products; S-split partials summed by the combine kernel)
    //    and dQ_f = dO_f M_f^T from the forward states
    Launch C = L0;
    C.use_delta = 0;
    C.canon = L0.crec;
    C.g0 = 0; C.gn = F; C.o0 = 0; C.on = 0;
    GDN_TRY(run.go(K_BWD_QDO, C, s, BH * F));
    if (L0.nsplit > 1) GDN_TRY(run.go(K_COMBINE, C, s, BH * F));
    // 3. reverse scan: G_f for every frame (slot f + 1) and the gradient of the initial state
    Launch R = L0;
    R.s0 = 0; R.s1 = F + 1;
    R.scan_in = L0.d_state_out;
    R.scan_out = L0.d_state_in;
    R.mt = L0.gt;
    R.mt_lead = 1;
    GDN_TRY(run.go(K_SCAN_BWD, R, s, BH * (F + 1)));
    // 4. per-frame gradients of K, V, gamma and beta
    return run.go(K_BWD, L0, s, BH * F);
}

hipError_t run_tconv(const TconvLaunch& L, hipStream_t s) {
    t_trace_log.clear();
    const bool armed = !t_trace_events.empty();
    const bool timed = armed && t_trace_events.size() >= 2;
    hipError_t e = hipSuccess;
    if (timed && (e = hipEventRecord(t_trace_events[0], s)) != hipSuccess) return e;
    if ((e = tconv_launch(L, s)) != hipSuccess) return e;
    if (timed && (e = hipEventRecord(t_trace_events[1], s)) != hipSuccess) return e;
    if (armed) t_trace_log.push_back({(int32_t)K_TCONV, 0, (int64_t)L.B * L.T * L.S});
    return hipSuccess;
}

hipError_t run_attn(const AttnLaunch& L, hipStream_t s) {
    t_trace_log.clear();
    const bool armed = !t_trace_events.empty();
    hipError_t e = hipSuccess;
    // launch i is bracketed by trace events 2i, 2i + 1 when that many are armed
    auto launch = [&](int i, Kernel kind, hipError_t (*fn)(const AttnLaunch&, hipStream_t)) {
        const bool timed = armed && t_trace_events.size() >= (size_t)(2 * i + 2);
        hipError_t r;
        if (timed && (r = hipEventRecord(t_trace_events[2 * i], s)) != hipSuccess) return r;
        if ((r = fn(L, s)) != hipSuccess) return r;
        if (timed && (r = hipEventRecord(t_trace_events[2 * i + 1], s)) != hipSuccess) return r;
        if (armed) t_trace_log.push_back({(int32_t)kind, 0, (int64_t)L.B * L.H * L.Tq});
        return hipSuccess;
    };
    if ((e = launch(0, K_ATTN, attn_launch)) != hipSuccess) return e;
    if (L.nsplit > 1 && (e = launch(1, K_ATTN_COMBINE, attn_combine_launch)) != hipSuccess) return e;
    return hipSuccess;
}

void set_trace(void* const* events, int pairs) {
    t_trace_events.clear();
    t_trace_log.clear();
    for (int i = 0; i < 2 * pairs; ++i) t_trace_events.push_back((hipEvent_t)events[i]);
}

int read_trace(gdn_trace_entry* out, int capacity) {
    const int n = (int)t_trace_log.size();
    for (int i = 0; out && i < n && i < capacity; ++i) out[i] = t_trace_log[i];
    return n;
}

}  // namespace gdn
