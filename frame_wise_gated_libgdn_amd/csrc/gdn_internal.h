// Internal interface between the C-ABI layer (gdn_api.cpp), the launch runtime
// (gdn_runtime.cpp) and the kernels (gdn_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/libgdn.h"

namespace gdn {

// Argument bundle of the kernels. Strides are in elements; frame indices are absolute.
struct Launch {
    int B, H, D, S, F;
    int bf16;            // 1: Q/K/V/O are bf16; 0: fp32
    int fp8;             // 1: Q/K/V are OCP FP8 E4M3 codes with per-frame scales, O is bf16
    const float *q_scale, *k_scale, *v_scale;  // fp8: [B][H][F] scales of Q, K, V
    int use_delta;
    float c;             // key scale
    const void *q, *k, *v;
    void* o;
    int64_t sb, sh, st;  // Q/K/V strides
    int64_t ob, oh, ot;  // O strides
    int64_t xsb, xsh, xst;  // strides of the gram products' second operand (V; dO in the backward)
    int unit_scale;      // gram products without the beta c / gamma beta c^2 factors (backward)
    const float *gamma, *beta, *state_in;
    float* state_out;
    void* canon;         // workspace: per-frame record handed from the products kernel to the scan
    float* part;         // workspace: per-split fp32 partial products (when nsplit > 1)
    void* mt;            // workspace: materialised per-frame states, transposed, in the I/O type
    int spin_limit;      // fused: polls of a frame flag before a workgroup gives up (0: never
                         //   wait, every frame after the first times out)
    int* ctl;            // workspace (fused): [0] ticket counter, [1] wait time-out flag,
                         //   [2 + bh * kChainGroups + g] last frame of (b, h) whose column
                         //   group g of the state is published
    float* chain;        // workspace (fused): published states, [2][B*H][D][D] fp32, [c][n] order
    int step_cols;       // step: the Gram-form kernels of gdn_step.hip (bf16, D = 64 / 128)
    int step_one;        // step: those kernels' work in one launch (step_fused_kernel); ctl
                         //   then holds its time-out word, per-head epochs and meeting flags
    float* save_states;  // fused forward, training: fp32 states, [B*H][F + 1][D][D] transposed
                         //   (slot 0 the initial state, slot f + 1 = M_f), or NULL
    void* save_recs;     // ... and the frames' Ghat planes ([B*H][F] records of rec_stride bytes)
    int64_t rec_stride;  // bytes per frame record read by the scan (0: the full record)
    int saved;           // backward: states and Ghat records come from a forward's saved buffer
    int no_output;       // fused forward with save_states: keep the states only, form no outputs
    int keep_timeout;    // reset of the ticket counter and flags: leave the time-out flag as is
    int fused_states;    // backward: recompute the forward states with the fused forward
                         //   (no outputs) into save_recs / save_states, then run as from saved
    int bwd_chain;       // backward: the reverse chain inside the Q/dO kernel, ticket-ordered
                         //   (ctl, chain and spin_limit as in the fused forward; one flag per
                         //   (b, h) at ctl[2 + bh * kChainGroups]: the last published step)
    int nsplit;          // S splits of the gram products
    int split_tokens;    // tokens per split (multiple of 64)
    int nchunk;          // S chunks of the output products
    int chunk_tokens;    // tokens per output chunk (multiple of 16)
    // frame ranges of one launch
    int g0, gn;          // gram products (and combine) over frames [g0, g0 + gn)
    int o0, on;          // output products over frames [o0, o0 + on)
    int s0, s1;          // scan over frames [s0, s1) (backward scan: steps)
    int mt_lead;         // per-step scan outputs have F + mt_lead slots per (b, h); forward: the
                         //   initial state goes to slot 0 and M_f to slot f + 1 when set
    void* crec;          // workspace (backward): per-frame records of C_f = Q_f^T dO_f
    void* gt;            // workspace (backward): G_f = dL/dM_f (transposed, fp32), slot f + 1
    const void* d_o;     // backward: dL/dO (O strides)
    const float* d_state_out;  // backward: dL/dstate_out (NULL: zero)
    float* d_state_in;   // backward: dL/dstate_in (NULL: not returned)
    void *dq, *dk, *dv;  // backward: gradients of Q, K, V (Q/K/V strides)
    float *dgamma, *dbeta;  // backward: [B][H][F]
    const float* scan_in;  // state before frame s0 (NULL: zero)
    float* scan_out;       // state after frame s1 - 1 (NULL: not stored)
};

// Kernels the runtime can launch (also the trace kinds of the C ABI).
enum Kernel {
    K_PRODUCTS = 0, K_COMBINE = 1, K_SCAN = 2, K_STEP_PARTIAL = 3, K_STEP_REDUCE = 4,
    K_FUSED_RESET = 5, K_FUSED = 6, K_SCAN_BWD = 7, K_BWD = 8,
    K_SCAN_STATES = 9,   // the forward scan with fp32 per-frame states (backward's recompute)
    K_TCONV = 10,        // block-causal temporal convolution
    K_ATTN = 11,         // frame-causal softmax attention
    K_STEP_OUTPUT = 12,  // step (Gram-form kernels): outputs of the frame
    K_BWD_QDO = 13,      // backward: C_f = Q_f^T dO_f and dQ_f in one pass over Q and dO
    K_STEP_FUSED = 14,   // step (Gram form): partials, new state and outputs in one launch
    K_ATTN_COMBINE = 15  // softmax attention with key splits: merge of the splits' partials
};

// Arguments of the frame-causal softmax attention (gdn_attn.hip). q: [B][H][Tq][D], k, v:
// [B][H][Tk][D] (shared strides), o like q (own strides); elements, D contiguous; bf16.
// Query row t belongs to frame q_frame0 + t / S and sees keys 0 .. (frame + 1) * S - 1.
struct AttnLaunch {
    int B, H, D, S, Tq, Tk, q_frame0;
    float scale;
    int64_t qsb, qsh, qst, ksb, ksh, kst, osb, osh, ost;
    const void *q, *k, *v;
    void* o;
    // Key splits (gdn_attention_framecausal_ws, single-frame calls): nsplit workgroups share a
    // query block's key tiles, each writing its unnormalised O (part, fp32 [split][b h][t][D])
    // and its (maximum, weight sum) (ml, fp32 pairs [split][b h][t]); a second launch merges
    // them into o. nsplit = 1: one workgroup per block writes o directly. nw: waves per
    // workgroup (8 or 12), set by attn_plan.
    int nsplit, nw;
    float* part;
    float* ml;
};
bool attn_supported(int D);
// Waves per workgroup and key splits for the call (splits only when allow_split and the
// queries form one frame); bytes of workspace that the splits need (0 for nsplit = 1).
void attn_plan(AttnLaunch& L, bool allow_split, size_t* ws_bytes);
hipError_t attn_launch(const AttnLaunch& L, hipStream_t s);
hipError_t attn_combine_launch(const AttnLaunch& L, hipStream_t s);
hipError_t run_attn(const AttnLaunch& L, hipStream_t s);

// Arguments of the temporal convolution (gdn_tconv.hip). x, y: [B][T][S][C] with the strides
// below (elements, channel stride 1); caches [B][S][C] contiguous; weight [C][3], bias [C].
struct TconvLaunch {
    int B, T, S, C, Tb;
    int bf16;            // 1: x, y and the caches are bf16; 0: fp32
    int64_t xsb, xst, xss, ysb, yst, yss;
    const void* x;
    const float *weight, *bias;
    const void* cache_in;
    void* y;
    void* cache_out;
};
hipError_t tconv_launch(const TconvLaunch& L, hipStream_t s);
hipError_t run_tconv(const TconvLaunch& L, hipStream_t s);

// Fused forward: value-column groups pipelined through the frame chain (one flag each per (b, h)).
constexpr int kChainGroups = 8;
constexpr int kSpinLimitDefault = 1 << 20;  // polls of about a microsecond each
// Rows past a frame's last one that the fused forward addresses (the ragged last K/V stage, Q
// tiles prefetched ahead, O tiles of the last pass), through 32-bit offsets that read zero and
// drop stores at or past the frame's end. The host keeps (S - 1 + kFusedRowsPast) rows of
// either stride within 2 GiB, so that no such offset leaves int range or wraps into the frame.
constexpr int kFusedRowsPast = 464;

// Whether the fused single-pass forward has a kernel for this type / head size.
bool fused_supported(int bf16, int D);
// Step mode's Gram-form kernels (gdn_step.hip): whether they cover this type / head size,
// and the launch of K_STEP_PARTIAL, K_STEP_REDUCE or K_STEP_OUTPUT.
bool step_cols_supported(int bf16, int D);
// Workgroups per token split in the Gram step (each forms D / halves rows of the split's update).
constexpr int step_halves(int D) { return D == 128 ? 2 : 1; }
hipError_t step_launch(Kernel k, const Launch& L, hipStream_t s);
// One-launch step: the ctl words it needs for B*H heads of W workgroups each (time-out word,
// per-head epochs, two meeting flags per workgroup), and whether the current device can hold its
// grid (8 XCDs, each with at least `per_xcd` CUs for one workgroup each).
constexpr size_t step_one_ctl_bytes(int64_t BH, int64_t W) { return (size_t)(1 + BH + 2 * BH * W) * 8; }
bool step_one_device_ok(int per_xcd);
// Value of the one-launch step's time-out word (64-bit, at byte 0 of its workspace) once a wait
// gave up; nothing else writes it.
constexpr uint64_t kStepTimeoutWord = 0x5354455054494D45ull;
// Whether the backward has kernels for this type / head size.
bool backward_supported(int bf16, int D);

// gdn_scratch.hip: the library's own device scratch (kScratchBytes on every GPU, 256-byte
// aligned) for gdn_step_frame_noalloc; `out` receives the current device's copy.
constexpr size_t kScratchBytes = GDN_STEP_SCRATCH_BYTES;
hipError_t scratch_address(void** out);

// Enqueue one kernel on `s`. Returns the HIP error of the launch.
hipError_t launch_kernel(Kernel k, const Launch& L, hipStream_t s);

// gdn_runtime.cpp: the launch order of a forward (staged: products, scan, outputs; or fused)
// and of a step, all on stream `s`.
hipError_t run_forward(const Launch& L, bool fused, hipStream_t s);
hipError_t run_step(const Launch& L, hipStream_t s);
hipError_t run_backward(const Launch& L, hipStream_t s);
void set_trace(void* const* events, int pairs);
int read_trace(gdn_trace_entry* out, int capacity);

}  // namespace gdn
