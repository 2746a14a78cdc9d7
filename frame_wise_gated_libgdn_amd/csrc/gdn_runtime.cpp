// Launch runtime of libgdn: the order of the kernels of a forward or a step on the caller's
// stream, and the launch trace.
//
// Forward, staged:  products (gram items of every frame) -> [combine] -> scan -> products
//                   (output items of every frame).
// Forward, fused:   reset of the ticket counter and frame flags -> fused kernel.
// Step:             step_partial -> step_reduce -> products (output items of the one frame).
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
        if ((e = launch_kernel(k, A, s)) != hipSuccess) return e;
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
    GDN_TRY(run.go(K_STEP_PARTIAL, L0, s, BH));
    GDN_TRY(run.go(K_STEP_REDUCE, L0, s, BH));
    Launch A = L0;
    A.F = 1;
    A.gn = 0;
    A.o0 = 0;
    A.on = 1;
    return run.go(K_PRODUCTS, A, s, BH);
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
