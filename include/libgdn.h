/*
 * libgdn.h -- C ABI of libgdn, the frame-wise Gated DeltaNet (GDN) recurrence on AMD MI355X
 * (gfx950).
 *
 * The operation
 * -------------
 * Gen-hub.ru, "NVIDIA SANA-WM: минутное 720p видео с одной видеокарты", section
 * "Архитектура: четыре нетривиальных решения": SANA-WM's GDN blocks process video frame by
 * frame with a recurrent state of fixed size D x D per head; a decay gate gamma lowers the
 * weight of older frames, a delta-rule correction writes only the difference between the target
 * value and the state's current prediction, and keys are scaled by 1/sqrt(D*S) (D = head dim,
 * S = spatial tokens per frame). The pages describe this in words; libgdn computes, per (batch
 * b, head h), with M the D x D fp32 state (row = key dim, column = value dim):
 *
 *     for f = 0 .. F-1:
 *         Kt  = c K_f                         c = key_scale, default 1/sqrt(D*S)
 *         R   = V_f - gamma_f Kt M            (R = V_f when use_delta == 0)
 *         M   = gamma_f M + beta_f Kt^T R
 *         O_f = Q_f M
 *
 * Frames are causal; the S tokens of one frame all read the same state, so attention is
 * bidirectional inside a frame. With gamma = beta = 1 and use_delta = 0 this is SANA-Video's
 * block-causal cumulative linear attention (talk "SANA-Video: Efficient Video Generation with
 * Block Linear Diffusion Transformer", ICLR 2026 oral, passage on the block KV cache).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory. Every pointer is a device pointer on the current HIP device, owned by the caller.
 *   libgdn allocates no device memory and keeps no data between calls; it may be called from
 *   several host threads at once (distinct workspaces). The one exception is the static
 *   scratch array of gdn_step_frame_noalloc (below), shared by all its calls on a GPU.
 * Asynchrony. Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream) and the
 *   call returns; buffers must stay valid until the stream has passed the call. Each call only
 *   launches kernels on `hip_stream` (no memset or copy nodes, so it can be captured into a
 *   HIP graph). Two calls that share a workspace must not run concurrently.
 * Layouts. Q, K, V, O of one (b, h) are token-major rows of D contiguous elements; token
 *   t = f*S + s. Element (b, h, t, d) of Q/K/V is at
 *       base + b*qkv_stride_b + h*qkv_stride_h + t*qkv_stride_t + d      (elements)
 *   and of O at the same with the o_stride_* values. Head-major [B,H,T,D] and token-major
 *   [B,T,H,D] storage are both expressible. Gates gamma, beta are fp32 [B][H][F] contiguous
 *   (step: [B][H]). States are fp32 [B][H][D][D] contiguous, row = key dim.
 * Types. Q, K, V, O are all GDN_F32 or all GDN_BF16; states and gates are always fp32;
 *   arithmetic accumulates in fp32; bf16 outputs are rounded to nearest even. With
 *   GDN_FP8_E4M3 (gdn_forward_framewise_fp8 only) Q, K, V are 8-bit codes with per-frame
 *   scales and O is bf16.
 * Supported shapes. D in {16, 32, 64, 128}; B, H, S, F >= 1; B*H*F*S*max-stride must fit the
 *   int64 element index. Pointers to Q, K, V, O must be 16-byte aligned, the strides multiples
 *   of 8 elements, gates and states 4-byte aligned (GDN_ERR_ALIGN otherwise).
 * Gate values are not checked (that would cost a device pass); the documented domain is
 *   gamma in (0, 1], beta in [0, 1]. NaN and Inf inputs propagate.
 * Errors. Argument errors are found on the host before anything is enqueued: the call then
 *   returns a non-zero gdn_status, writes nothing and records a message for
 *   gdn_last_error_message() (per host thread). A failed launch returns GDN_ERR_HIP with the
 *   HIP error text in that message. Nothing throws or aborts across this ABI. Device faults
 *   surface at the caller's next synchronisation, as for any HIP call.
 * Determinism. Results are bitwise identical from run to run for the same inputs, shapes and
 *   workspace (fixed-order reductions, no floating-point atomics).
 */
#ifndef LIBGDN_H
#define LIBGDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LIBGDN_ABI_VERSION 11

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,         /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,        /* a size is < 1 or too large */
    GDN_ERR_UNSUPPORTED = 3,  /* head_dim or dtype not supported */
    GDN_ERR_STRIDE = 4,       /* a stride is negative or rows of one tensor overlap */
    GDN_ERR_ALIGN = 5,        /* pointer or stride alignment violated */
    GDN_ERR_ALIAS = 6,        /* an output overlaps an input (other than the allowed in-place state) */
    GDN_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than gdn_workspace_size() */
    GDN_ERR_HIP = 8,          /* a HIP runtime call failed */
    GDN_ERR_TIMEOUT = 9       /* gdn_check_timeout: a bounded wait of the fused schedule gave up */
} gdn_status;

/*
 * GDN_FP8_E4M3: Q, K, V are OCP FP8 E4M3 codes (OCP 8-bit Floating Point Specification: sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, subnormals, S.1111.111 = NaN, no infinities),
 * one byte per element (strides in elements = bytes), each with an fp32 scale per (b, h, f);
 * O is bf16. Accepted only by gdn_forward_framewise_fp8.
 */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_FP8_E4M3 = 2 } gdn_dtype;

/*
 * How a forward is run. Both schedules compute the same recurrence; results agree to rounding
 * (the state step of both splits Ghat and M into bf16 hi + lo parts; the order of fp32
 * additions differs).
 *   STAGED  products of every frame (Ghat_f, Bhat_f) into the workspace, then the frame-serial
 *           scan over those D x D records, then the outputs of every frame. Any dtype and D.
 *   FUSED   one pass: each (b, h, f) is a workgroup that computes its frame's products, waits
 *           for the state of frame f-1 of the same (b, h), applies the step, publishes M_f and
 *           writes O_f; only Q/K/V/O and the D x D states cross HBM. bf16 (or E4M3) with
 *           D = 64 or 128, and a frame's q/k/v rows and o rows each within 2 GiB
 *           (GDN_ERR_UNSUPPORTED otherwise), counting the 464 rows past the frame that the
 *           kernel addresses (and reads as zero): (S + 463) * qkv_stride_t + D elements, and
 *           (S + 463) * o_stride_t + D (a single-token tensor counts a stride of max(stride,
 *           D)). The same bound applies wherever "a frame's rows within 2 GiB" is asked below.
 *   AUTO    FUSED where supported and B*H*F >= 1024, else STAGED.
 * FUSED waits for the previous frame's state are bounded: after GDN_FUSED_SPIN_LIMIT polls
 * (environment, default 2^20, about a microsecond each) a workgroup gives up, continues with a
 * NaN state (every later output of that (b, h) is NaN) and sets the int32 time-out flag at byte
 * 4 of the workspace; the kernel always ends. gdn_check_timeout reads that flag.
 * GDN_FUSED_SPIN_LIMIT=0 times out every frame after the first at once (for exercising that
 * path).
 */
typedef enum { GDN_SCHEDULE_AUTO = 0, GDN_SCHEDULE_STAGED = 1, GDN_SCHEDULE_FUSED = 2 } gdn_schedule;

typedef struct {
    int32_t batch;             /* B */
    int32_t heads;             /* H */
    int32_t head_dim;          /* D in {16, 32, 64, 128} */
    int32_t tokens_per_frame;  /* S */
    int32_t frames;            /* F (gdn_step_frame ignores it: one frame) */
    int32_t dtype;             /* gdn_dtype of Q, K, V, O */
    int32_t use_delta;         /* 1: gated delta rule; 0: M = gamma M + beta Kt^T V */
    float   key_scale;         /* c; <= 0 selects 1/sqrt(D*S) */
    int64_t qkv_stride_b, qkv_stride_h, qkv_stride_t;   /* elements */
    int64_t o_stride_b, o_stride_h, o_stride_t;         /* elements */
    int32_t schedule;          /* a gdn_schedule; step mode: see gdn_step_frame */
} gdn_problem;

/*
 * Block-causal temporal convolution (SANA-Video talk, shadowingenglish.com, passage on the
 * causal FFN with temporal conv): the spatial-temporal Mix-FFN convolves along time; in training
 * a zero token separates consecutive blocks so that a block cannot see the next one, and the
 * last token of each block is carried in as the first token of the next; in streaming that
 * carried token is a cache. libgdn's reading: a depthwise convolution over latent frames,
 * kernel 3 centred, per spatial token and channel:
 *   y[t] = bias + w[c][0] * L(t) + w[c][1] * x[t] + w[c][2] * R(t)
 *   L(t) = x[t-1] (t > 0), cache_in (t = 0; zero when cache_in is NULL)
 *   R(t) = x[t+1], or zero when frame t ends a block ((t + 1) % block_frames == 0) or the call
 *   cache_out = x[T-1]
 * One call covers a whole sequence of T / block_frames blocks (training form) or one block from
 * the cache of the previous one (streaming form: T = block_frames).
 */
typedef struct {
    int32_t batch;             /* B */
    int32_t frames;            /* T, a multiple of block_frames */
    int32_t tokens;            /* S spatial tokens per frame */
    int32_t channels;          /* C, a multiple of 8 */
    int32_t block_frames;      /* frames per block */
    int32_t dtype;             /* GDN_F32 or GDN_BF16: x, y and the caches */
    int64_t x_stride_b, x_stride_t, x_stride_s;   /* elements; channel stride 1 */
    int64_t y_stride_b, y_stride_t, y_stride_s;   /* elements; channel stride 1 */
} gdn_tconv_problem;

/*
 *   x          input [B][T][S][C] with the x strides
 *   weight     fp32 [C][3]: taps on frames t-1, t, t+1
 *   bias       fp32 [C], or NULL (zero)
 *   cache_in   [B][S][C] contiguous, the last frame of the previous block, or NULL (zero: the
 *              first block)
 *   y          output [B][T][S][C] with the y strides; fp32 accumulation, bf16 rounded to
 *              nearest even
 *   cache_out  [B][S][C] contiguous, receives x[T-1], or NULL; may equal cache_in exactly
 * Pointers to x, y, the caches, weight and bias must be 16-byte aligned and strides multiples of 8 elements
 * (GDN_ERR_ALIGN); y and cache_out must not overlap any input (GDN_ERR_ALIAS). No workspace.
 * Asynchronous on hip_stream; errors and tracing as gdn_forward_framewise (trace kind
 * GDN_KERNEL_TCONV, units B*T*S).
 */
gdn_status gdn_tconv_forward(const gdn_tconv_problem* p, const void* x, const float* weight,
                             const float* bias, const void* cache_in, void* y, void* cache_out,
                             void* hip_stream);

/*
 * Frame-causal softmax attention: the softmax blocks that the pages' hybrid video models
 * interleave with frame-wise GDN blocks (SANA-WM: 5 of 20 blocks, gen-hub.ru article,
 * architecture section; an all-softmax model runs out of memory on the 60 s video because its
 * key/value cache grows with every frame; SANA-Streaming's hybrid is 3.7x faster than
 * all-softmax, jefxiong.cn digest). Per (b, h), a query row t of frame q_frame0 + t / S attends
 * to every key of frames 0 .. that frame (its own frame in both directions):
 *   o[t] = sum_j softmax_j(scale q[t] . k[j]) v[j],  j < min(Tk, (frame + 1) * S)
 * With q_frames = kv_frames and q_frame0 = 0 this is the whole video; with q_frames = 1 it is a
 * streaming step of frame q_frame0 against the key/value cache of frames 0 .. kv_frames - 1.
 */
typedef struct {
    int32_t batch, heads, head_dim;       /* B, H, D in {64, 128} */
    int32_t tokens_per_frame;             /* S */
    int32_t q_frames;                     /* frames of q and o: Tq = q_frames * S */
    int32_t kv_frames;                    /* frames of k and v: Tk = kv_frames * S */
    int32_t q_frame0;                     /* frame index of q's first frame */
    int32_t dtype;                        /* GDN_BF16 */
    float   scale;                        /* <= 0 selects 1/sqrt(D) */
    int64_t q_stride_b, q_stride_h, q_stride_t;    /* elements; D contiguous */
    int64_t kv_stride_b, kv_stride_h, kv_stride_t; /* shared by k and v */
    int64_t o_stride_b, o_stride_h, o_stride_t;
} gdn_attn_problem;

/*
 *   q        [B][H][Tq][D] bf16
 *   k, v     [B][H][Tk][D] bf16, the same strides; q_frame0 + q_frames <= kv_frames (every
 *            query's own frame must be present)
 *   o        [B][H][Tq][D] bf16, must not overlap q, k or v
 * fp32 softmax and accumulation; the weights enter the value product rounded to bf16. Pointers
 * 16-byte aligned, strides multiples of 8 elements; a head's Tk key (and value) rows must lie
 * within 2 GiB (GDN_ERR_UNSUPPORTED otherwise). No workspace. Asynchronous on hip_stream;
 * errors and tracing as gdn_forward_framewise (trace kind GDN_KERNEL_ATTN, units B*H*Tq).
 */
gdn_status gdn_attention_framecausal(const gdn_attn_problem* p, const void* q, const void* k,
                                     const void* v, void* o, void* hip_stream);

/*
 * The same attention with a caller-owned workspace that lets one call split each query
 * block's keys over several workgroups. A single-frame call (q_frames = 1, a streaming step)
 * has few query blocks, too few to occupy every compute unit; with splits, each workgroup takes
 * a share of the block's keys and stores its unnormalised output, running maximum and weight
 * sum in the workspace, and a second launch merges them (the usual rescaling of a softmax by
 * its maxima; trace kinds GDN_KERNEL_ATTN, then GDN_KERNEL_ATTN_COMBINE). The result equals the
 * unsplit one up to the order of fp32 rounding.
 *   gdn_attention_workspace_size   bytes the call may use (0 when it would not split: more
 *                                  than one query frame, or a grid that already fills the
 *                                  device); a pure function of the problem's sizes
 *   workspace   at least that many bytes, 256-byte aligned, not overlapping q, k, v or o
 *               (GDN_ERR_WORKSPACE / GDN_ERR_ALIGN / GDN_ERR_ALIAS otherwise); NULL runs the
 *               call unsplit, exactly as gdn_attention_framecausal. Its contents on entry do
 *               not matter; calls that share one workspace must not overlap in time.
 * Other arguments, errors and limits as gdn_attention_framecausal.
 */
gdn_status gdn_attention_workspace_size(const gdn_attn_problem* p, size_t* bytes_out);
gdn_status gdn_attention_framecausal_ws(const gdn_attn_problem* p, const void* q, const void* k,
                                        const void* v, void* o, void* workspace,
                                        size_t workspace_bytes, void* hip_stream);

/*
 * Workspace bytes needed by gdn_forward_framewise (mode = 0; also gdn_forward_framewise_save),
 * gdn_step_frame (mode = 1), gdn_backward_framewise (mode = 2) or gdn_backward_framewise_saved
 * (mode = 3) for this problem. The step-mode size does not depend on `frames`. Validates the
 * sizes in `p` (not the pointers or strides); other modes are GDN_ERR_SHAPE.
 */
gdn_status gdn_workspace_size(const gdn_problem* p, int mode, size_t* bytes_out);

/*
 * All F frames of every (b, h) in one call (the recurrence above).
 *   q, k, v      inputs, layout as above
 *   gamma, beta  fp32 [B][H][F]
 *   state_in     fp32 [B][H][D][D], or NULL for a zero initial state
 *   o            output, layout as above; must not overlap any input
 *   state_out    fp32 [B][H][D][D] state after frame F-1, or NULL; may equal state_in exactly
 *   workspace    device scratch of at least gdn_workspace_size(p, 0) bytes, 256-byte aligned;
 *                its contents on entry do not matter and are undefined afterwards
 */
gdn_status gdn_forward_framewise(const gdn_problem* p, const void* q, const void* k, const void* v,
                                 const float* gamma, const float* beta, const float* state_in,
                                 void* o, float* state_out,
                                 void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * All F frames from 8-bit inputs (the low-precision Q/K/V that SANA-Streaming fuses with its
 * GDN kernel through mixed-precision quantisation: jefxiong.cn daily digest, SANA-Streaming
 * item, contribution (3); SANA-WM's NVFP4 deployment: chatpaper.ai English abstract).
 * p->dtype must be GDN_FP8_E4M3; D = 64 or 128; the schedule is always FUSED (AUTO or FUSED
 * accepted, STAGED is GDN_ERR_UNSUPPORTED).
 *   q, k, v      E4M3 codes, [B,H,T,D] with the qkv strides (bytes); the value of an element
 *                of frame f is scale[b][h][f] * E4M3(code), with the scale of its tensor
 *   q_scale, k_scale, v_scale   fp32 [B][H][F] contiguous
 *   o            bf16 output, o strides in elements
 *   other arguments, errors and workspace (gdn_workspace_size(p, 0)) as gdn_forward_framewise.
 * The recurrence runs on the scaled values; codes are decoded exactly, products of codes
 * accumulate in fp32 and the scales are applied to those sums (K's twice in the key-key
 * product), so the result equals the bf16 path on the decoded values up to rounding order.
 */
gdn_status gdn_forward_framewise_fp8(const gdn_problem* p, const void* q, const void* k,
                                     const void* v, const float* q_scale, const float* k_scale,
                                     const float* v_scale, const float* gamma, const float* beta,
                                     const float* state_in, void* o, float* state_out,
                                     void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * One frame for streaming / autoregressive rollout: compute the frame's contribution, add it
 * to the cached state, produce the frame's output, and cache the new state only when asked
 * (the block KV cache passage of the SANA-Video talk; the chunk-causal and distilled
 * autoregressive modes of the gen-hub.ru article, section "Три режима на любой вкус"; frame
 * by frame streaming in SANA-Streaming, jefxiong.cn digest item 1).
 *   q, k, v, o   one frame: t = s in [0, S); strides as above
 *   gamma, beta  fp32 [B][H]
 *   state_in     fp32 [B][H][D][D], required
 *   state_out    NULL: the new state is not committed (a denoising pass that will be redone);
 *                otherwise it receives the new state and may equal state_in exactly
 *   workspace    at least gdn_workspace_size(p, 1) bytes, 256-byte aligned
 * bf16 data with D = 64 or 128 (and S rows of either token stride within 2 GiB) forms, per
 * token split, K^T K and K^T V and from them the split's share of the update, then the new
 * state, then the outputs. Where B*H is a multiple of 8 with B*H/8 * (2 if D = 128 else 1) <= 32,
 * p->schedule is not GDN_SCHEDULE_STAGED and the device has 8 XCDs of at least 32 CUs, the
 * three phases run in one launch (trace kind STEP_FUSED): each head's workgroups share one
 * XCD and meet twice inside the launch through its L2, waits bounded as in the FUSED forward
 * (GDN_FUSED_SPIN_LIMIT; 0 makes every meeting give up at once): a wait that gives up leaves
 * a NaN state and NaN outputs and sets the 64-bit time-out word at byte 0 of the workspace,
 * which stays set until gdn_check_timeout reads it (the meetings need the head's workgroups on
 * the GPU together, one per CU).
 * Otherwise three launches (STEP_PARTIAL, STEP_REDUCE, STEP_OUTPUT); both give the same
 * results bit for bit. Other types and head sizes use whole-state partials and the forward's
 * output kernel (STEP_PARTIAL, STEP_REDUCE, PRODUCTS). Results are bitwise reproducible.
 */
gdn_status gdn_step_frame(const gdn_problem* p, const void* q, const void* k, const void* v,
                          const float* gamma, const float* beta, const float* state_in,
                          void* o, float* state_out,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * gdn_step_frame without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, hosts that forbid hipMalloc). The
 * workspace comes from a static device array inside the library, GDN_STEP_SCRATCH_BYTES on
 * every GPU the library runs on, held until the process ends. The call allocates nothing.
 *   arguments, results and errors as gdn_step_frame; a problem whose step workspace
 *   (gdn_workspace_size(p, 1)) exceeds GDN_STEP_SCRATCH_BYTES returns GDN_ERR_WORKSPACE (before
 *   anything is enqueued; pass a workspace to gdn_step_frame instead). The first call on a
 *   device looks up that device's copy of the array (GDN_ERR_HIP if that fails).
 * Every call on one GPU shares that GPU's array, whatever the stream or host thread: calls that
 * may run at the same time on one GPU race and must be ordered by the caller (one stream, or
 * events). Nothing in the array needs to start at zero: each launch writes what the next reads
 * (the one-launch step's per-head epochs make each launch's meeting flags new whatever the
 * array held). A time-out of the one-launch step sets the word at byte 0 of the array; it is
 * not readable through gdn_check_timeout, whose workspace argument it is not.
 */
#define GDN_STEP_SCRATCH_BYTES ((size_t)32 << 20)
gdn_status gdn_step_frame_noalloc(const gdn_problem* p, const void* q, const void* k,
                                  const void* v, const float* gamma, const float* beta,
                                  const float* state_in, void* o, float* state_out,
                                  void* hip_stream);

/*
 * Gradients of gdn_forward_framewise for training: given dL/dO and dL/dstate_out of a scalar
 * loss L, returns dL/dQ, dL/dK, dL/dV, dL/dgamma, dL/dbeta and dL/dstate_in (key_scale is a
 * constant). The pages define the forward only; this is its reverse-mode derivative. With
 * G_f = dL/dM_f, Kt = c K_f, M the state before frame f and P = Kt M, R = V_f - gamma_f P:
 *     G_f      = Q_f^T dO_f + (gamma_{f+1} I - gamma_{f+1} beta_{f+1} Kt_{f+1}^T Kt_{f+1}) G_{f+1}
 *                (G_{F-1} also receives dstate_out)
 *     dQ_f     = dO_f M_f^T
 *     dV_f     = beta_f Kt G_f
 *     dK_f     = c (beta_f R G_f^T - gamma_f beta_f (Kt G_f) M^T)
 *     dgamma_f = <G_f, M> - beta_f <Kt G_f, P>,    dbeta_f = <Kt G_f, R>
 *     dstate_in = (gamma_0 I - gamma_0 beta_0 Kt_0^T Kt_0) G_0
 * (without the delta term: R = V_f, dK_f = c beta_f V_f G_f^T, dgamma_f = <G_f, M>, and the
 * chain uses gamma I). The forward states are recomputed inside the call. p->schedule picks
 * how that and the reverse chain G_f run:
 *   FUSED    the states: the fused forward without its outputs (trace kinds FUSED_RESET, FUSED)
 *            when a frame's q/k/v rows lie within 2 GiB, else as STAGED. The chain: inside the
 *            pass over Q and dO that forms Q_f^T dO_f and dQ, workgroups take frames in
 *            descending order by ticket and hand G_f on through the workspace as the fused
 *            forward hands on M_f (FUSED_RESET, BWD_QDO); then BWD for the gradients of K, V,
 *            gamma and beta. Waits are bounded as in the forward (GDN_FUSED_SPIN_LIMIT): on
 *            time-out a workgroup continues with NaN and sets the int32 time-out flag at byte 4
 *            of the workspace, and the kernel always ends. A time-out of the chain makes the
 *            gradients of the frames before it and dstate_in NaN; a time-out of the recompute
 *            makes the later states NaN, hence dQ of those frames and everything the chain
 *            forms from them.
 *   STAGED   the states: PRODUCTS, then SCAN_STATES (COMBINE between them when frames are
 *            split over tokens). The chain: the pass over Q and dO without it (BWD_QDO;
 *            COMBINE when frames are split), then a separate scan (SCAN_BWD); then BWD.
 *   AUTO     FUSED once B*H*F >= 1024, else STAGED.
 *   q, k, v, gamma, beta, state_in   the forward's inputs (state_in NULL: zero)
 *   d_o          dL/dO, layout of o (o_stride_*)
 *   d_state_out  dL/dstate_out fp32 [B][H][D][D], or NULL for zero
 *   dq, dk, dv   outputs, layout of q/k/v (qkv_stride_*), type of q
 *   dgamma, dbeta  outputs, fp32 [B][H][F]
 *   d_state_in   output fp32 [B][H][D][D], or NULL; may equal d_state_out exactly
 *   workspace    at least gdn_workspace_size(p, 2) bytes, 256-byte aligned
 * Supported: bf16 data with D = 64 or 128, a frame's q/k/v rows within 2 GiB and its d_o rows
 * within 2 GiB (GDN_ERR_UNSUPPORTED otherwise). No output may overlap an input, the workspace or
 * another output.
 */
gdn_status gdn_backward_framewise(const gdn_problem* p, const void* q, const void* k,
                                  const void* v, const float* gamma, const float* beta,
                                  const float* state_in, const void* d_o,
                                  const float* d_state_out, void* dq, void* dk, void* dv,
                                  float* dgamma, float* dbeta, float* d_state_in,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Training without recomputing the forward states: gdn_forward_framewise_save is the forward
 * (FUSED schedule; AUTO is taken as FUSED, STAGED is GDN_ERR_UNSUPPORTED) that also fills a
 * caller-owned buffer `saved` with what gdn_backward_framewise_saved needs, so that the backward
 * skips its first two launches (the frames' key-key products and the state scan).
 *   gdn_saved_size   bytes of `saved` for the problem (a pure function of it; bf16 data with
 *                    D = 64 or 128 and a frame's q/k/v rows within 2 GiB, else
 *                    GDN_ERR_UNSUPPORTED). Layout, for reference: the frames' Ghat products
 *                    (delta rule only; bf16 hi + lo planes, the library's record order), then,
 *                    256-byte aligned, the initial state and every M_f in fp32, [B][H][F+1][D][D]
 *                    with element [b][h][f+1][c][n] = M_f[n][c] (slot 0: state_in, or zero).
 *   saved            at least gdn_saved_size bytes, 256-byte aligned, must not overlap any
 *                    other argument; arguments otherwise as gdn_forward_framewise
 * gdn_backward_framewise_saved takes the same problem and inputs as the forward that filled
 * `saved` (it does not read state_in: slot 0 holds it) and computes what
 * gdn_backward_framewise computes, from the forward's own states (so the two agree to
 * rounding: the fused forward and the backward's own scan round differently); its workspace
 * is gdn_workspace_size(p, 3) bytes. p->schedule picks the reverse chain's schedule as for
 * gdn_backward_framewise (the forward's FUSED schedule does not depend on it).
 */
gdn_status gdn_saved_size(const gdn_problem* p, size_t* bytes_out);
gdn_status gdn_forward_framewise_save(const gdn_problem* p, const void* q, const void* k,
                                      const void* v, const float* gamma, const float* beta,
                                      const float* state_in, void* o, float* state_out,
                                      void* saved, size_t saved_bytes, void* workspace,
                                      size_t workspace_bytes, void* hip_stream);
gdn_status gdn_backward_framewise_saved(const gdn_problem* p, const void* q, const void* k,
                                        const void* v, const float* gamma, const float* beta,
                                        const void* saved, size_t saved_bytes, const void* d_o,
                                        const float* d_state_out, void* dq, void* dk, void* dv,
                                        float* dgamma, float* dbeta, float* d_state_in,
                                        void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Whether the last call that used `workspace` gave up a bounded wait. The FUSED schedule of
 * gdn_forward_framewise (also _fp8 and _save) and the chained schedule of the backward hand the
 * state (or its gradient) from frame to frame between workgroups; a wait for the previous frame
 * is bounded (GDN_FUSED_SPIN_LIMIT, see gdn_schedule above) and, when it gives up, the kernel
 * still ends, with NaN in every output that depends on the missing state and the int32 time-out
 * flag at byte 4 of the workspace set. This call synchronises hip_stream, so that the call on
 * it has finished, then reads that flag.
 *   p, mode    the problem and workspace mode of that call (as gdn_workspace_size: 0 forward,
 *              1 step, 2 backward, 3 backward from saved states); they select the schedule
 *   workspace  the workspace passed to that call
 * Step mode (mode 1) with a shape that may run in one launch (see gdn_step_frame): reads the
 * 64-bit time-out word at byte 0 instead, which the step never clears itself: any step call on
 * this workspace since the last check that gave up sets it, and this call clears it.
 * Returns GDN_OK when the flag is clear or the call's schedule has no bounded wait (STAGED, the
 * other step shapes; nothing is read then), GDN_ERR_TIMEOUT when it is set, GDN_ERR_HIP when
 * the synchronisation or the read fails, and the argument errors of gdn_workspace_size.
 * It blocks the host: not for use during graph capture.
 */
gdn_status gdn_check_timeout(const gdn_problem* p, int mode, const void* workspace, void* hip_stream);

/*
 * Instrumentation (launch trace). gdn_set_trace arms `pairs` pairs of caller-created,
 * timing-enabled hipEvent_t handles on the calling host thread: in every later
 * gdn_forward_framewise / gdn_step_frame call on this thread, kernel launch i (i < pairs) is
 * bracketed by events[2i] before and events[2i+1] after it, recorded on the stream the kernel
 * runs on, so hipEventElapsedTime(events[2i], events[2i+1]) is that launch's duration. The
 * events are only recorded, never waited on. pairs 0 disarms; pairs must be 0..65536. Not for
 * use during graph capture.
 * gdn_trace_read returns the number of launches of the last call on this thread while armed
 * (launches beyond `pairs` are listed but not timed) and copies up to `capacity` entries.
 */
typedef enum {
    GDN_KERNEL_PRODUCTS = 0,      /* staged: gram products or outputs of frames */
    GDN_KERNEL_COMBINE = 1,       /* staged: sum of S-split partial products */
    GDN_KERNEL_SCAN = 2,          /* staged: frame-serial state scan */
    GDN_KERNEL_STEP_PARTIAL = 3,  /* step: per-split K^T R */
    GDN_KERNEL_STEP_REDUCE = 4,   /* step: state update */
    GDN_KERNEL_FUSED_RESET = 5,   /* fused: clears the ticket counter and frame flags */
    GDN_KERNEL_FUSED = 6,         /* fused: products, state step and outputs of every frame */
    GDN_KERNEL_SCAN_BWD = 7,      /* backward: reverse scan of the state gradients */
    GDN_KERNEL_BWD = 8,           /* backward: per-frame gradients of K, V, gamma, beta */
    GDN_KERNEL_SCAN_STATES = 9,   /* backward: forward scan keeping every state in fp32 */
    GDN_KERNEL_TCONV = 10,        /* block-causal temporal convolution */
    GDN_KERNEL_ATTN = 11,         /* frame-causal softmax attention */
    GDN_KERNEL_STEP_OUTPUT = 12,  /* step, bf16 with D = 64 or 128: outputs of the frame */
    GDN_KERNEL_BWD_QDO = 13,      /* backward: Q_f^T dO_f and dQ in one pass over Q and dO */
    GDN_KERNEL_STEP_FUSED = 14,   /* step, bf16 with D = 64 or 128: partials, state, outputs */
    GDN_KERNEL_ATTN_COMBINE = 15  /* softmax attention with key splits: merge of the splits */
} gdn_kernel_kind;

typedef struct {
    int32_t kernel;   /* gdn_kernel_kind */
    int32_t stream;   /* stream of the launch: 0 = the caller's (the only one used) */
    int64_t units;    /* (b, h, frame) items. A PRODUCTS item moves 2*S*D elements of Q/K/V/O
                         (K and V read, or Q read and O written); a FUSED item moves 4*S*D
                         (K, V, Q read, O written); a BWD item 6*S*D (K, V, dO read; dQ, dK,
                         dV written) */
} gdn_trace_entry;

gdn_status gdn_set_trace(void* const* events, int pairs);
int gdn_trace_read(gdn_trace_entry* entries, int capacity);

/* Static text for a status code (never NULL). */
const char* gdn_status_string(gdn_status s);

/* Detail of the last failure on the calling host thread ("" if none). */
const char* gdn_last_error_message(void);

/* LIBGDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDN_H */
