// HIP kernels of libgdn for gfx950 (MI355X): the frame-wise Gated DeltaNet recurrence.
//
// Recurrence (gen-hub.ru, "NVIDIA SANA-WM: минутное 720p видео с одной видеокарты", section
// "Архитектура: четыре нетривиальных решения"), per (b, h), c = key scale:
//     R = V_f - gamma_f (c K_f) M,   M <- gamma_f M + beta_f (c K_f)^T R,   O_f = Q_f M.
//
// Forward (all frames):
//   1. gram products -- fully parallel over (b, h, f[, S split]). Stages K_f, V_f through LDS,
//                       contracts over the frame's tokens on MFMA:
//                         Ghat_f = gamma_f beta_f c^2 K_f^T K_f,  Bhat_f = beta_f c K_f^T V_f
//                       (gates and key scale applied in the epilogue); combine_kernel sums
//                       S-split partials when a frame was split.
//   2. scan_kernel   -- the serial part: M_f = gamma_f M - Ghat_f M + Bhat_f. This is the update
//                       above with the residual expanded (Kt^T (V - g Kt M) = Kt^T V - g Kt^T Kt M),
//                       so the frame-to-frame chain only touches D x D matrices; one workgroup
//                       owns 16 value columns of one head (columns of M evolve independently), so
//                       no workgroup waits on another. Writes each M_f (transposed, I/O type).
//   3. output products -- fully parallel O_f = Q_f M_f on MFMA.
// Gram and output items share one kernel (products_kernel); these three launches are the
// staged schedule (any dtype and D). The fused schedule (fused_kernel: bf16 or E4M3 data, D = 64
// or 128) does all three per frame in one ticket-ordered launch, handing the state from frame
// to frame through memory.
// Step (one frame from a cached state), the update as written, for fp32 data or D = 16 / 32
// (bf16 with D = 64 / 128 runs the column-block kernels of gdn_step.hip):
//   4. step_partial_kernel -- per S split: P = K M (MFMA), R = V - (gamma c) P, U_p = K^T R (MFMA).
//   5. step_reduce_kernel  -- M' = gamma M + beta c sum_p U_p; state_out; transposed copy.
//   then the output products of the one frame.
// Backward (bf16, D = 64 or 128): scan_kernel with fp32 states (forward and reverse), qdo_kernel
// (C_f = Q_f^T dO_f and dQ in one pass over Q and dO, optionally with the reverse chain) and
// bwd_kernel (dK, dV, dgamma, dbeta).
//
// MFMA: v_mfma_f32_16x16x32_bf16 for bf16 data, v_mfma_f32_16x16x4_f32 for fp32 data; fp32
// accumulation throughout. Lane l = 16 g + r of a wave holds A row r / B column r and the
// contraction slice [KL g, KL g + KL) of each KS-long step; C row 4 g + q, column r in
// register q. The contraction order inside a step is free as long as A and B agree.
#include <type_traits>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;  // threads per workgroup (4 waves of 64)

template <typename T> struct Mma;
template <> struct Mma<bf16> {
    static constexpr int KS = 32;  // contraction length of one MFMA
    static constexpr int KL = 8;   // contraction elements held by one lane
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<float> {
    static constexpr int KS = 4;
    static constexpr int KL = 1;
    typedef float frag;
    static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *(const u32x2*)p; }

// Buffer resource over `bytes` bytes at p (raw dword access; accesses past the end read zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// Eight OCP FP8 E4M3 codes (byte i = element i) to eight bf16 values (exact: every E4M3 value,
// subnormals included, is a bf16 value); gfx950's scaled conversion with a unit scale.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 w) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true))};
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

template <typename T> __device__ __forceinline__ typename Mma<T>::frag ld_frag(const T* p);
template <> __device__ __forceinline__ bf16x8 ld_frag<bf16>(const bf16* p) {
    return __builtin_bit_cast(bf16x8, ld16(p));
}
template <> __device__ __forceinline__ float ld_frag<float>(const float* p) { return *p; }

template <typename T> __device__ __forceinline__ typename Mma<T>::frag zero_frag();
template <> __device__ __forceinline__ bf16x8 zero_frag<bf16>() {
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}
template <> __device__ __forceinline__ float zero_frag<float>() { return 0.f; }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(bf16)lo, (bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Store 4 consecutive fp32 values as T.
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    *(u32x2*)p = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *(f32x4*)p = f32x4{a, b, c, d};
}

// ----------------------------------------------------------------------------------------
// LDS tile holding 64 tokens of K and V transposed: row = feature (K features 0..D-1, V
// features D..2D-1), tokens contiguous along the row. The 16-byte column blocks of each row are
// XOR-swizzled so that the transposing writes and the MFMA fragment reads spread over banks.
template <typename T, int D, int SC_ = 64> struct XTile {
    static constexpr int SC = SC_;                     // tokens per chunk
    static constexpr int RB = SC * (int)sizeof(T);     // bytes per row
    static constexpr int NCB = RB / 16;                // column blocks per row
    static constexpr int ROWS = 2 * D;
    static constexpr int BYTES = ROWS * RB;
    // XOR swizzle of the 16-byte column blocks of a row
    static __device__ __forceinline__ int swz(int row) {
        if constexpr (NCB == 8) return ((row >> 1) ^ (row >> 3)) & 7;
        else return row & (NCB - 1);
    }
    // byte offset of (row, token)
    static __device__ __forceinline__ int addr(int row, int tok) {
        const int b = tok * (int)sizeof(T);
        return row * RB + ((((b >> 4) ^ swz(row)) & (NCB - 1)) << 4) + (b & 15);
    }
};

// Global -> registers -> transposed LDS staging of one chunk of K and V. A thread moves
// VE x VE blocks (VE tokens x VE features, VE = elements per 16 bytes): VE row loads, a register
// transpose, VE row stores into the LDS tile.
template <typename T, int D, int NTH = NT, int SC = 64> struct XStage {
    using Tile = XTile<T, D, SC>;
    static constexpr int VE = 16 / (int)sizeof(T);
    static constexpr int FB = 2 * D / VE;              // feature blocks (K then V)
    static constexpr int TB = SC / VE;                 // token blocks
    static constexpr int NBLK = FB * TB;
    static constexpr int PER = (NBLK + NTH - 1) / NTH;
    u32x4 r[PER][VE];

    // tokens [t0, t0 + 64) of the frame; rows at or beyond tend are zero
    // kb, vb: token 0 of the first and second operand; kst, vst: their token strides
    __device__ __forceinline__ void load(const T* kb, const T* vb, int64_t kst, int64_t vst, int t0,
                                         int tend, int tid) {
#pragma unroll
        for (int pi = 0; pi < PER; ++pi) {
            const int blk = tid + pi * NTH;
            if (NBLK % NTH == 0 || blk < NBLK) {
                const int fb = blk % FB, tb = blk / FB;
                const bool first = fb < D / VE;
                const T* base = first ? kb + fb * VE : vb + (fb - D / VE) * VE;
                const int64_t st = first ? kst : vst;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const int tok = t0 + tb * VE + e;
                    r[pi][e] = tok < tend ? ld16(base + (int64_t)tok * st) : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    }

    // The K blocks as loaded (rows = tokens), to a row-major tile with row length kr elements
    __device__ __forceinline__ void store_key_rows(T* rows, int kr, int tid) const {
#pragma unroll
        for (int pi = 0; pi < PER; ++pi) {
            const int blk = tid + pi * NTH;
            if (NBLK % NTH == 0 || blk < NBLK) {
                const int fb = blk % FB, tb = blk / FB;
                if (fb < D / VE) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) st16(rows + (tb * VE + e) * kr + fb * VE, r[pi][e]);
                }
            }
        }
    }

    // block blk (VE tokens x VE features, rows as loaded) to the LDS tile, transposed
    static __device__ __forceinline__ void store_block(const u32x4 (&rb)[VE], int blk, char* lds) {
        const int fb = blk % FB, tb = blk / FB;
#pragma unroll
        for (int f = 0; f < VE; ++f) {
            u32x4 w;
            if constexpr (VE == 8) {
                // feature f of tokens 2c, 2c+1 -> dword c
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t a = rb[2 * c][f >> 1], b = rb[2 * c + 1][f >> 1];
                    w[c] = (f & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) w[c] = rb[c][f];
            }
            st16(lds + Tile::addr(fb * VE + f, tb * VE), w);
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int pi = 0; pi < PER; ++pi) {
            const int blk = tid + pi * NTH;
            if (NBLK % NTH == 0 || blk < NBLK) store_block(r[pi], blk, lds);
        }
    }

    // Split-operand order: the first half of the threads (whole waves) moves K's blocks, the
    // second half V's, so each wave reads through one buffer resource. Block blk1 of an operand
    // is feature block blk1 % (D / VE), token block blk1 / (D / VE).
    static constexpr int HALF = NTH / 2;
    static_assert(HALF % 64 == 0, "each operand gets whole waves");
    static constexpr int NB1 = (D / VE) * TB;
    static constexpr int PER1 = (NB1 + HALF - 1) / HALF;
    static_assert(PER1 <= PER, "split order fits the register blocks");
    static __device__ __forceinline__ int split_block(int tid, int pi) {   // -> blk, or -1
        const int op = tid / HALF, b1 = tid % HALF + pi * HALF;
        if (NB1 % HALF != 0 && b1 >= NB1) return -1;
        return (b1 / (D / VE)) * FB + op * (D / VE) + b1 % (D / VE);
    }

    // tokens [t0, t0 + SC) from buffers over the frame's rows of K (rk) and V (rv), token
    // stride stb bytes; rows past the end of a buffer read as zero
    __device__ __forceinline__ void load_rs(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int stb,
                                            int t0, int tid) {
        // the operand is a per-wave choice; readfirstlane lets the compiler keep it scalar
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_readfirstlane(tid >> 6) < HALF / 64 ? rk : rv;
#pragma unroll
        for (int pi = 0; pi < PER1; ++pi) {
            const int blk = split_block(tid, pi);
            if (blk >= 0) {
                const int fb = blk % FB % (D / VE), tb = blk / FB;
                const int vo = (t0 + tb * VE) * stb + fb * 16;
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    r[pi][e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo + e * stb, 0, 0));
            }
        }
    }

    __device__ __forceinline__ void store_rs(char* lds, int tid) const {
#pragma unroll
        for (int pi = 0; pi < PER1; ++pi) {
            const int blk = split_block(tid, pi);
            if (blk >= 0) store_block(r[pi], blk, lds);
        }
    }
};

// XStage for 8-bit (E4M3) K and V: the same blocks of 8 tokens x 8 features, loaded as 8 bytes
// per row and kept as codes while in flight; decoded to bf16 when staged into LDS.
template <int D, int NTH = NT, int SC = 64> struct XStage8 {
    using Wide = XStage<bf16, D, NTH, SC>;
    static constexpr int VE = Wide::VE, FB = Wide::FB, NBLK = Wide::NBLK, PER = Wide::PER;
    u32x2 r[PER][VE];

    __device__ __forceinline__ void load(const uint8_t* kb, const uint8_t* vb, int64_t kst, int64_t vst,
                                         int t0, int tend, int tid) {
#pragma unroll
        for (int pi = 0; pi < PER; ++pi) {
            const int blk = tid + pi * NTH;
            if (NBLK % NTH == 0 || blk < NBLK) {
                const int fb = blk % FB, tb = blk / FB;
                const bool first = fb < D / VE;
                const uint8_t* base = first ? kb + fb * VE : vb + (fb - D / VE) * VE;
                const int64_t st = first ? kst : vst;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const int tok = t0 + tb * VE + e;
                    r[pi][e] = tok < tend ? ld8(base + (int64_t)tok * st) : u32x2{0u, 0u};
                }
            }
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int pi = 0; pi < PER; ++pi) {
            const int blk = tid + pi * NTH;
            if (NBLK % NTH == 0 || blk < NBLK) {
                u32x4 rb[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) rb[e] = e4m3x8_to_bf16x8(r[pi][e]);
                Wide::store_block(rb, blk, lds);
            }
        }
    }

    // split-operand order of XStage (load_rs / store_rs), 8 bytes per row
    static constexpr int PER1 = Wide::PER1;
    __device__ __forceinline__ void load_rs(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int stb,
                                            int t0, int tid) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_readfirstlane(tid >> 6) < Wide::HALF / 64 ? rk : rv;
#pragma unroll
        for (int pi = 0; pi < PER1; ++pi) {
            const int blk = Wide::split_block(tid, pi);
            if (blk >= 0) {
                const int fb = blk % FB % (D / VE), tb = blk / FB;
                const int vo = (t0 + tb * VE) * stb + fb * 8;
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    r[pi][e] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, vo + e * stb, 0, 0));
            }
        }
    }

    __device__ __forceinline__ void store_rs(char* lds, int tid) const {
#pragma unroll
        for (int pi = 0; pi < PER1; ++pi) {
            const int blk = Wide::split_block(tid, pi);
            if (blk >= 0) {
                u32x4 rb[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) rb[e] = e4m3x8_to_bf16x8(r[pi][e]);
                Wide::store_block(rb, blk, lds);
            }
        }
    }
};

// Per-frame record handed from the products kernel to the scan, in fragment-major order so
// that every scan load instruction reads 1 KB of contiguous memory (64 lanes x 16 B):
//   Ghat planes (delta only): for wave w (state rows 16w..16w+15), plane p (hi, lo), k step ks,
//     lane l = 16 g + r: 8 bf16 = Ghat[16 w + r][32 ks + 8 g .. + 8]  (k past D never read)
//   Bhat: for column block cb, wave w, lane l = 16 g + r: 4 fp32 = Bhat[16 w + 4 g + q][16 cb + r]
template <int D> __host__ __device__ constexpr int rec_ksn() { return (D + 31) / 32; }
template <int D, bool DELTA> __host__ __device__ constexpr int rec_g_bytes() {
    return DELTA ? (D / 16) * 2 * rec_ksn<D>() * 1024 : 0;
}
template <int D, bool DELTA> __host__ __device__ constexpr int canon_bytes() {
    return rec_g_bytes<D, DELTA>() + 4 * D * D;
}
// bf16 element offset of Ghat[m][k] in plane p
template <int D> __device__ __forceinline__ int rec_g_off(int p, int m, int k) {
    const int frag = ((m >> 4) * 2 + p) * rec_ksn<D>() + (k >> 5);
    const int lane = ((k & 31) >> 3) * 16 + (m & 15);
    return (frag * 64 + lane) * 8 + (k & 7);
}
// fp32 element offset of Bhat[i][j] within the Bhat part
template <int D> __device__ __forceinline__ int rec_b_off(int i, int j) {
    const int frag = (j >> 4) * (D / 16) + (i >> 4);
    const int lane = ((i & 15) >> 2) * 16 + (j & 15);
    return (frag * 64 + lane) * 4 + (i & 3);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): 4 values to two bf16 planes (8 B each).
__device__ __forceinline__ void store_split4(bf16* hi, bf16* lo, f32x4 x) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float a = x[2 * c], b = x[2 * c + 1];
        h[c] = pack_bf16x2(a, b);
        const float ah = __builtin_bit_cast(float, h[c] << 16);
        const float bh = __builtin_bit_cast(float, h[c] & 0xFFFF0000u);
        l[c] = pack_bf16x2(a - ah, b - bh);
    }
    *(u32x2*)hi = u32x2{h[0], h[1]};
    *(u32x2*)lo = u32x2{l[0], l[1]};
}

// ----------------------------------------------------------------------------------------
// Kernel 1: per (b, h, f, split) products over the split's tokens
//   delta:    Ghat = gamma beta c^2 K^T K and Bhat = beta c K^T V
//   no delta: Bhat = beta c K^T V
// With one split the kernel writes the scan's per-frame record directly; otherwise fp32
// partials that combine_kernel sums. Item blk covers frame g0 + (blk / nsplit) % gn.
template <typename T, int D, bool DELTA>
__device__ __forceinline__ void gram_body(const Launch& L, int blk, char* lds) {
    using MM = Mma<T>;
    using X = XTile<T, D>;
    constexpr int NOUT = DELTA ? 2 * D : D;
    constexpr int TI = D / 16, TJ = NOUT / 16;
    constexpr int WI = TI >= 2 ? 2 : 1;
    constexpr int WJ = (4 / WI) < TJ ? (4 / WI) : TJ;
    constexpr int MI = TI / WI, MJ = TJ / WJ;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int p = blk % L.nsplit;
    blk /= L.nsplit;
    const int f = L.g0 + blk % L.gn, bh = blk / L.gn;
    const int b = bh / L.H, h = bh % L.H;
    const T* kb = (const T*)L.k + (int64_t)b * L.sb + (int64_t)h * L.sh + (int64_t)f * L.S * L.st;
    const T* vb = (const T*)L.v + (int64_t)b * L.xsb + (int64_t)h * L.xsh + (int64_t)f * L.S * L.xst;
    const int t0 = p * L.split_tokens;
    const int t1 = min(L.S, t0 + L.split_tokens);
    const bool active = wave < WI * WJ;
    const int wi = wave % WI, wj = wave / WI;

    f32x4 acc[MI][MJ];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int mj = 0; mj < MJ; ++mj) acc[mi][mj] = f32x4{0.f, 0.f, 0.f, 0.f};

    XStage<T, D> stg;
    stg.load(kb, vb, L.st, L.xst, t0, t1, tid);
    for (int c0 = t0; c0 < t1; c0 += X::SC) {
        __syncthreads();  // readers of the previous chunk are done
        stg.store(lds, tid);
        __syncthreads();
        if (c0 + X::SC < t1) stg.load(kb, vb, L.st, L.xst, c0 + X::SC, t1, tid);
        if (active) {
#pragma unroll
            for (int ks = 0; ks < X::SC / MM::KS; ++ks) {
                const int tok = ks * MM::KS + g * MM::KL;
                typename MM::frag af[MI];
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    af[mi] = ld_frag<T>((const T*)(lds + X::addr((wi * MI + mi) * 16 + r16, tok)));
#pragma unroll
                for (int mj = 0; mj < MJ; ++mj) {
                    const int col = (wj * MJ + mj) * 16 + r16;
                    const typename MM::frag bfr =
                        ld_frag<T>((const T*)(lds + X::addr(DELTA ? col : D + col, tok)));
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) acc[mi][mj] = MM::run(af[mi], bfr, acc[mi][mj]);
                }
            }
        }
    }

    if (!active) return;
    const int gi = bh * L.F + f;
    const float gm = L.gamma[gi], bt = L.beta[gi];
    const float sG = gm * bt * L.c * L.c, sB = L.unit_scale ? 1.f : bt * L.c;
    // Lane (r16, g) holds out[i0 + q][col], q = 0..3. It is stored transposed, [col][i0 .. i0+3]
    // (16 contiguous bytes): for Bhat this is Bhat^T; Ghat is symmetric, so its transposed
    // store is Ghat itself.
    if (L.nsplit == 1) {
        // final per-frame record: [Ghat hi bf16 | Ghat lo bf16 | Bhat^T fp32] (no delta: [Bhat^T])
        char* rec = (char*)L.canon + (int64_t)gi * canon_bytes<D, DELTA>();
        bf16* grec = (bf16*)rec;
        float* brec = (float*)(rec + rec_g_bytes<D, DELTA>());
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int i0 = (wi * MI + mi) * 16 + 4 * g;
#pragma unroll
            for (int mj = 0; mj < MJ; ++mj) {
                const int col = (wj * MJ + mj) * 16 + r16;
                const f32x4 a = acc[mi][mj];
                if (DELTA && col < D) {
                    // Ghat[col][i0 .. i0+3] (symmetric), 4 consecutive k of one fragment
                    store_split4(grec + rec_g_off<D>(0, col, i0), grec + rec_g_off<D>(1, col, i0), a * sG);
                } else {
                    *(f32x4*)(brec + rec_b_off<D>(i0, col - (DELTA ? D : 0))) = a * sB;
                }
            }
        }
    } else {
        // fp32 partial of split p: [Ghat | Bhat^T] (no delta: [Bhat^T]), summed by combine_kernel
        float* out = L.part + ((int64_t)gi * L.nsplit + p) * (int64_t)(NOUT * D);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int i0 = (wi * MI + mi) * 16 + 4 * g;
#pragma unroll
            for (int mj = 0; mj < MJ; ++mj) {
                const int col = (wj * MJ + mj) * 16 + r16;
                const float sc = DELTA && col < D ? sG : sB;
                *(f32x4*)(out + col * D + i0) = acc[mi][mj] * sc;
            }
        }
    }
}

// Sum of the S-split partials of each (b, h, f), f in [g0, g0 + gn), into the final per-frame
// record (only when the products ran with more than one split). Fixed order over the splits.
template <int D, bool DELTA>
__global__ __launch_bounds__(NT) void combine_kernel(Launch L) {
    constexpr int NOUT = DELTA ? 2 * D : D;
    constexpr int NV = NOUT * D / 4;             // float4 per frame
    constexpr int NB = (NV + NT - 1) / NT;
    const int it = blockIdx.x / NB;
    const int gi = (it / L.gn) * L.F + L.g0 + it % L.gn;  // (b h, frame) of item it
    const int v = (blockIdx.x % NB) * NT + threadIdx.x;
    if (v >= NV) return;
    const float* src = L.part + (int64_t)gi * L.nsplit * NOUT * D + 4 * v;
    f32x4 s = *(const f32x4*)src;
    for (int p = 1; p < L.nsplit; ++p) s += *(const f32x4*)(src + (int64_t)p * NOUT * D);
    char* rec = (char*)L.canon + (int64_t)gi * canon_bytes<D, DELTA>();
    const int e = 4 * v;                          // element index in [Ghat | Bhat^T], row-major [col][i]
    if (DELTA && e < D * D) {
        const int m = e / D, k = e % D;          // Ghat[m][k .. k+3]
        bf16* grec = (bf16*)rec;
        store_split4(grec + rec_g_off<D>(0, m, k), grec + rec_g_off<D>(1, m, k), s);
    } else {
        const int eb = e - (DELTA ? D * D : 0);
        const int j = eb / D, i = eb % D;        // Bhat[i .. i+3][j]
        *(f32x4*)((float*)(rec + rec_g_bytes<D, DELTA>()) + rec_b_off<D>(i, j)) = s;
    }
}

// ----------------------------------------------------------------------------------------
// Kernel 2: the frame-serial scan M_f = gamma_f M - Ghat_f M + Bhat_f over frames [s0, s1), for
// 16 value columns of one head per workgroup (columns of M evolve independently, so no workgroup waits on
// another). One wave per 16 state rows. Ghat M runs on bf16 MFMA with both operands split
// into hi + lo bf16 (hi.hi + hi.lo + lo.hi; the dropped lo.lo term is ~2^-16 of the product);
// M stays fp32 in registers (C layout) and its hi/lo planes are kept transposed in LDS as the
// B operand. Each wave's operands of the next P frames (its Ghat rows, its Bhat entries, gamma)
// sit in a register ring, loaded P frames ahead of use.
// Workgroup w lands on XCD w % 8 (round-robin dispatch); all column blocks of one head get ids
// with the same residue so that they share one XCD's L2 for Ghat_f.
template <int D, bool DELTA> struct ScanSlot {
    static constexpr int KSN = (D + 31) / 32;
    bf16x8 a[DELTA ? 2 : 1][DELTA ? KSN : 1];  // Ghat rows of this wave: [hi/lo][k step]
    f32x4 bh;                                   // Bhat[16 w + 4 g + q][col]
};
constexpr int kGammaSeg = 4000;  // frames per gamma staging (a multiple of the scan ring size)

// OT: type of the per-step outputs (the I/O type for the forward's output products; fp32 for
// the backward, whose dgamma needs the states and their gradients unrounded).
template <typename T, int D, bool DELTA, int P, bool BWD, typename OT>
__global__ __launch_bounds__(64 * (D / 16)) void scan_kernel(Launch L) {
    constexpr int NC = 16;              // value columns per workgroup
    constexpr int NCB = D / NC;         // column blocks per head
    constexpr int KSN = (D + 31) / 32;  // bf16 k steps (padded past D with zeros)
    constexpr int MR = D + 8;           // row length (bf16) of the transposed state planes
    constexpr int REC = canon_bytes<D, DELTA>();
    constexpr int CREC = canon_bytes<D, false>();  // backward: record of C_t = Q_t^T dO_t
    __shared__ __attribute__((aligned(16))) bf16 Ms[2][2][NC * MR];  // [buffer][hi, lo][col][k]
    // gamma of the current chunk of steps. Gammas come through LDS rather than scalar loads:
    // a scalar load in the step loop would share the LDS wait counter and expose a full memory
    // round trip in every step.
    __shared__ float Gam[kGammaSeg];

    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int bh = (slot / NCB) * 8 + xcd, cb = slot % NCB;
    if (bh >= L.B * L.H) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int col = cb * NC + r16;
    const int row0 = wave * 16 + 4 * g;  // this lane's 4 state rows
    const int F = L.F, s0 = L.s0, s1 = L.s1;
    const int lead = L.mt_lead;         // per-step outputs have F + lead slots per (b, h)
    const int64_t rstride = L.rec_stride ? L.rec_stride : REC;   // bytes per frame record
    const char* rec_bh = (const char*)L.canon + (int64_t)bh * F * rstride;
    const char* crec_bh = (const char*)L.crec + (int64_t)bh * F * CREC;
    OT* mt_bh = (OT*)L.mt + (int64_t)bh * (F + lead) * D * D;

    float Mc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        Mc[q] = L.scan_in ? L.scan_in[((int64_t)bh * D + row0 + q) * D + col] : 0.f;
    store_split4(&Ms[0][0][r16 * MR + row0], &Ms[0][1][r16 * MR + row0], f32x4{Mc[0], Mc[1], Mc[2], Mc[3]});
    if (!BWD && lead) store4(mt_bh + (int64_t)col * D + row0, Mc[0], Mc[1], Mc[2], Mc[3]);

    // Forward: step f applies frame f (Ghat_f, Bhat_f, gamma_f) and its result M_f goes to
    // slot f + lead. Backward (BWD, steps 0 .. F): step u with t = F - 1 - u computes
    //     G_t = gamma_{t+1} G_{t+1} - Ghat_{t+1} G_{t+1} + C_t
    // (Ghat_F = 0 and gamma_F = 1, so G_{F-1} = dstate_out + C_{F-1}; C_{-1} = 0, so the last
    // step gives the gradient of the initial state) and writes it to slot t + 1.
    // The ring has P + 1 slots: right after a step's barrier the slot freed by the previous
    // step is refilled with step f + P, so the loads stream while this step's MFMAs run.
    // The step loop body is branch-free so that the compiler keeps the ring's loads in flight
    // across iterations: loads past the last step s1-1 re-read it, and a step past the end
    // leaves the state unchanged and rewrites the last result into its own slot.
    constexpr int R = P + 1;
    ScanSlot<D, DELTA> ring[R];
    auto issue = [&](ScanSlot<D, DELTA>& r, int f) {
        f = min(f, s1 - 1);
        const int gf = BWD ? F - f : f;                  // frame of Ghat
        const bool gzero = BWD && gf >= F;               // uniform
        const char* rec = rec_bh + (int64_t)min(gf, F - 1) * rstride;
        if constexpr (DELTA) {
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) {
                const bool in = ks * 32 + g * 8 < D && !gzero;
                const char* fr = rec + ((wave * 2) * KSN + ks) * 1024 + lane * 16;
                r.a[0][ks] = in ? ld_frag<bf16>((const bf16*)fr) : zero_frag<bf16>();
                r.a[1][ks] = in ? ld_frag<bf16>((const bf16*)(fr + KSN * 1024)) : zero_frag<bf16>();
            }
        }
        const int boff = ((cb * (D / 16) + wave) * 64 + lane) * 16;
        if constexpr (BWD) {
            const int t = F - 1 - f;                     // frame of C
            const f32x4 cv = *(const f32x4*)(crec_bh + (int64_t)max(t, 0) * CREC + boff);
            r.bh = t >= 0 ? cv : f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
            r.bh = *(const f32x4*)(rec + rec_g_bytes<D, DELTA>() + boff);
        }
    };
#pragma unroll
    for (int u = 0; u < P; ++u) issue(ring[u], s0 + u);

    static_assert(kGammaSeg % R == 0, "segments must hold whole ring cycles");
    const float* gam_bh = L.gamma + (int64_t)bh * F;
    int cur = 0;
    for (int sb = s0; sb < s1; sb += kGammaSeg) {
        __syncthreads();  // the previous segment's gammas are no longer read
        for (int t = threadIdx.x; t < kGammaSeg; t += blockDim.x) {
            const int f = min(sb + t, s1 - 1);
            if constexpr (BWD) Gam[t] = F - f < F ? gam_bh[F - f] : 1.f;
            else Gam[t] = gam_bh[f];
        }
      for (int f0 = sb; f0 < sb + kGammaSeg && f0 < s1; f0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int f = f0 + u;
            const bool valid = f < s1;  // uniform
            {
                __syncthreads();  // planes of the last state complete; readers of the other buffer done
                issue(ring[(u + P) % R], f + P);  // the slot of step f - 1
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (DELTA) {
                    f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSN; ++ks) {
                        const int k = ks * 32 + g * 8;
                        const bf16x8 mh = k < D ? ld_frag<bf16>(&Ms[cur][0][r16 * MR + k]) : zero_frag<bf16>();
                        const bf16x8 ml = k < D ? ld_frag<bf16>(&Ms[cur][1][r16 * MR + k]) : zero_frag<bf16>();
                        acc = Mma<bf16>::run(ring[u].a[0][ks], mh, acc);
                        a1 = Mma<bf16>::run(ring[u].a[0][ks], ml, a1);
                        a2 = Mma<bf16>::run(ring[u].a[1][ks], mh, a2);
                    }
                    acc += a1 + a2;
                }
                const float gm = Gam[f - sb];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float mn = gm * Mc[q] - acc[q] + ring[u].bh[q];
                    Mc[q] = valid ? mn : Mc[q];
                }
                const f32x4 mv = {Mc[0], Mc[1], Mc[2], Mc[3]};
                if constexpr (DELTA)
                    store_split4(&Ms[cur ^ 1][0][r16 * MR + row0], &Ms[cur ^ 1][1][r16 * MR + row0], mv);
                const int fs = min(f, s1 - 1);
                const int os = BWD ? F - fs : fs + lead;  // output slot
                store4(mt_bh + ((int64_t)os * D + col) * D + row0, Mc[0], Mc[1], Mc[2], Mc[3]);
                cur ^= 1;
            }
        }
      }
    }

    // Each lane rewrites exactly the entries it read from scan_in, so scan_out may equal it.
    if (L.scan_out) {
#pragma unroll
        for (int q = 0; q < 4; ++q) L.scan_out[((int64_t)bh * D + row0 + q) * D + col] = Mc[q];
    }
}

// ----------------------------------------------------------------------------------------
// Kernel 3: O_f = Q_f M_f, computed as O^T = M^T Q^T so that each lane ends up with a run of
// consecutive output columns of one token (16-byte stores). The A operand rows (output columns
// j) of 16x16 tile jt are permuted: with bf16 and D >= 32, tiles 2p and 2p+1 cover columns
// 32p .. 32p+31 such that lane (r, g) receives j = 32p + 8g + 0..7 across the pair.
// LDS copy of M_f^T for the output items: rows padded by 16 bytes against bank conflicts
template <typename T, int D> struct OutStage {
    static constexpr int MR = D + 16 / (int)sizeof(T);
    static constexpr int BYTES = D * MR * (int)sizeof(T);
};

template <typename T, int D> __device__ __forceinline__ int out_col(int jt, int m) {
    if constexpr (sizeof(T) == 2 && D >= 32)
        return 32 * (jt >> 1) + 8 * (m >> 2) + 4 * (jt & 1) + (m & 3);
    else
        return 16 * jt + m;
}

template <typename T, int D>
__device__ __forceinline__ void output_body(const Launch& L, int blk, char* lds) {
    using MM = Mma<T>;
    constexpr int TJ = D / 16, KSN = (D + MM::KS - 1) / MM::KS;  // contraction padded to KS
    constexpr int MR = OutStage<T, D>::MR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int ch = blk % L.nchunk;
    blk /= L.nchunk;
    const int f = L.o0 + blk % L.on, bh = blk / L.on;
    const int b = bh / L.H, h = bh % L.H;
    const T* mt = (const T*)L.mt + ((int64_t)bh * L.F + f) * D * D;
    const T* qf = (const T*)L.q + (int64_t)b * L.sb + (int64_t)h * L.sh + (int64_t)f * L.S * L.st;
    T* of = (T*)L.o + (int64_t)b * L.ob + (int64_t)h * L.oh + (int64_t)f * L.S * L.ot;

    const int s_beg = ch * L.chunk_tokens;
    const int s_end = min(L.S, s_beg + L.chunk_tokens);
    // B operand (Q rows) of one 16-token tile; tiles past the chunk read nothing
    auto load_q = [&](int s0, typename MM::frag (&bq)[KSN]) {
        const int s = s0 + r16;
        const bool ok = s < s_end;
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            bq[ks] = ok && ks * MM::KS + g * MM::KL < D
                         ? ld_frag<T>(qf + (int64_t)s * L.st + ks * MM::KS + g * MM::KL)
                         : zero_frag<T>();
    };
    typename MM::frag bq[KSN];
    load_q(s_beg + wave * 16, bq);  // in flight while the state is staged

    // M_f^T staged once per workgroup (padded rows), then each wave's A fragments from LDS
    T* ms = (T*)lds;
    {
        // all loads in flight before the first LDS store
        constexpr int VE = 16 / (int)sizeof(T), NE = D * D / VE, PT = (NE + NT - 1) / NT;
        u32x4 x[PT];
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int e = min(tid + k * NT, NE - 1);
            x[k] = ld16(mt + (e / (D / VE)) * D + (e % (D / VE)) * VE);
        }
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int e = tid + k * NT;
            if (NE % NT == 0 || e < NE) st16(ms + (e / (D / VE)) * MR + (e % (D / VE)) * VE, x[k]);
        }
    }
    __syncthreads();
    typename MM::frag am[TJ][KSN];
#pragma unroll
    for (int jt = 0; jt < TJ; ++jt)
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            am[jt][ks] = ks * MM::KS + g * MM::KL < D
                             ? ld_frag<T>(ms + out_col<T, D>(jt, r16) * MR + ks * MM::KS + g * MM::KL)
                             : zero_frag<T>();

    for (int s0 = s_beg + wave * 16; s0 < s_end; s0 += 4 * 16) {
        const int s = s0 + r16;
        const bool ok = s < s_end;
        typename MM::frag bn[KSN];
        load_q(s0 + 4 * 16, bn);  // next tile of this wave, in flight during this one
        f32x4 acc[TJ];
#pragma unroll
        for (int jt = 0; jt < TJ; ++jt) {
            acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) acc[jt] = MM::run(am[jt][ks], bq[ks], acc[jt]);
        }
        if (ok) {
            T* orow = of + (int64_t)s * L.ot;
            if constexpr (sizeof(T) == 2 && D >= 32) {
#pragma unroll
                for (int p = 0; p < TJ / 2; ++p) {
                    const f32x4 x = acc[2 * p], y = acc[2 * p + 1];
                    st16(orow + 32 * p + 8 * g,
                         u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                               pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])});
                }
            } else {
#pragma unroll
                for (int jt = 0; jt < TJ; ++jt)
                    store4(orow + 16 * jt + 4 * g, acc[jt][0], acc[jt][1], acc[jt][2], acc[jt][3]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks) bq[ks] = bn[ks];
    }
}

// ----------------------------------------------------------------------------------------
// Products kernel: the gram items of frames [g0, g0 + gn) followed by the output items of
// frames [o0, o0 + on). Both kinds of item only stream Q/K/V/O through MFMA, so one launch can
// carry the products of one chunk of frames and the outputs of an earlier chunk whose states
// are ready, and the frame-serial scan of the chunk in between runs beside it.
template <typename T, int D, bool DELTA>
__global__ __launch_bounds__(NT, 2) void products_kernel(Launch L) {
    constexpr int GB = XTile<T, D>::BYTES, OB = OutStage<T, D>::BYTES;
    __shared__ __attribute__((aligned(16))) char lds[GB > OB ? GB : OB];
    const int ng = L.B * L.H * L.gn * L.nsplit;
    if ((int)blockIdx.x < ng)
        gram_body<T, D, DELTA>(L, blockIdx.x, lds);
    else
        output_body<T, D>(L, blockIdx.x - ng, lds);
}

// ----------------------------------------------------------------------------------------
// Fused forward (bf16 or E4M3 data, D = 64 or 128): one workgroup per (b, h, f) computes
//   1. the frame's products Ghat_f, Bhat_f (as gram_body, all S tokens, K and V staged in LDS),
//   2. the state step M_f = gamma_f M_{f-1} + Bhat_f - Ghat_f M_{f-1} on MFMA, once M_{f-1} of
//      the same (b, h) is published, then publishes M_f,
//   3. the frame's outputs O_f = Q_f M_f.
// Nothing per frame goes through HBM except Q/K/V/O themselves and the D x D state handed from
// frame to frame, so the frame-serial chain hides under the streaming of the other frames.
//
// Ordering and progress. Each workgroup takes a ticket from a counter; ticket t is frame
// t / BH of (b h) = t % BH, so a workgroup only ever waits for a smaller ticket, whose
// workgroup is already running (it took its ticket first) and waits only for smaller tickets
// in turn: the chain always completes whatever order the hardware dispatches workgroups in.
// The wait is bounded (L.spin_limit polls); on time-out the workgroup raises ctl[1], continues
// with a NaN state so the failure is visible in every later output, and still publishes, so
// the kernel always ends.
//
// Memory ordering: the state and the frame flags move only through device-coherent accesses
// (the sc1 cache policy, which the compiler also uses for agent-scope atomics: coherent across
// the chip's L2 caches on their own, so no cache write-back or invalidation is needed, which
// would also flush the streaming outputs of every other workgroup). The publisher's waves wait
// until their state stores have completed, meet at a barrier, and one lane then stores the
// frame index; the consumer's lane polls the flag, and its waves issue their state loads only
// after the barrier that follows a successful poll. States alternate between two buffers per
// (b, h): frame f + 2 overwrites the buffer of frame f only after frame f + 1, the only reader
// of it, has published. A state buffer is laid out in the lanes' own order ([wave][nb][cb]
// [lane][4 fp32]: producer and consumer use the same mapping), so that every access
// instruction covers 1 KB of contiguous memory.
//
// Wave w owns the key rows n in [w D/4, (w+1) D/4) of Ghat (as columns: Ghat is symmetric),
// of Bhat and of the state step. With tile (kb, nb) of Ghat in C layout -- lane (r, g) holds
// Ghat[16 kb + 4 g + q][n0 + 16 nb + r] -- symmetry makes it the A operand slice for rows
// n0 + 16 nb + r and k = 16 kb + 4 g + q, so the step's A operand needs no data movement: a
// 32-long MFMA k step ks takes tiles 2 ks and 2 ks + 1 in its lane slots 0-3 and 4-7. The B
// operand (M_{f-1} split into bf16 hi + lo) is laid out in LDS with the same k order.
//
// E4M3 inputs (FP8): Q, K and V arrive as 8-bit codes with one scale per (b, h, f) and tensor.
// The codes are decoded exactly to bf16 on the way into LDS or into MFMA operands, the
// products run on the codes, and the scales enter as scalars: Ghat takes k_scale^2, Bhat
// k_scale v_scale, and the output tile q_scale before rounding to bf16.
constexpr int kCoherent = 16;        // cache-policy operand of the buffer intrinsics: sc1


// Ticket counter 0, frame flags -1; the time-out flag 0 unless keep_timeout (a second ticketed
// launch in the same call keeps the first one's time-out visible).
__global__ void fused_reset_kernel(int* ctl, int n, int keep_timeout) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n && !(i == 1 && keep_timeout)) ctl[i] = i < 2 ? 0 : -1;
}

// SAVE (training): also keep what the backward needs, so that it need not recompute the forward
// states: each frame's -Ghat planes (as +Ghat, the sign flipped exactly) in the scan record
// layout at save_recs, and the initial state and every M_f in fp32, transposed, at save_states
// (slot f + 1 per frame, slot 0 the initial state). These stores come after the frame's flag,
// so they do not lengthen the frame-to-frame chain.
// OUT = false (with SAVE; the backward's recompute of the forward states): the outputs are
// not formed, so Q and O are not touched and only K and V stream.
template <int D, bool DELTA, bool FP8, bool SAVE = false, bool OUT = true>
__global__ __launch_bounds__(NT, 2) void fused_kernel(Launch L) {
    using MM = Mma<bf16>;
    constexpr int SC = 64;          // tokens per staged chunk (128 measured slower for E4M3)
    using X = XTile<bf16, D, SC>;
    static_assert(D == 64 || D == 128, "fused path: D = 64 or 128");
    constexpr int NR = D / 4;       // key rows per wave
    constexpr int NB = NR / 16;     // 16-row blocks per wave
    constexpr int CB = D / 16;      // 16-column (value) blocks
    constexpr int KB = D / 16;      // 16-long k blocks of Ghat
    constexpr int MR = D + 8;       // LDS row length (bf16) of the state planes
    constexpr int PLANE = D * MR;
    constexpr int LDS_BYTES = X::BYTES > 4 * PLANE ? X::BYTES : 4 * PLANE;
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    __shared__ int s_ticket, s_ok;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    if (tid == 0) s_ticket = atomicAdd(&L.ctl[0], 1);
    __syncthreads();
    const int BH = L.B * L.H, F = L.F, S = L.S;
    const int f = s_ticket / BH, bh = s_ticket % BH;
    const int b = bh / L.H, h = bh % L.H;
    const int nw = wave * NR;       // first key row of this wave

    // ---- 1. products over the frame's tokens
    const int64_t fo = (int64_t)b * L.sb + (int64_t)h * L.sh + (int64_t)f * S * L.st;
    f32x4 gacc[DELTA ? KB : 1][NB], bacc[NB][CB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int kb = 0; kb < (DELTA ? KB : 1); ++kb) gacc[kb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) bacc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    {
        // K and V rows of the frame through buffer resources that end with the frame's last
        // row, so the ragged last chunk reads zeros without a branch per row (the host keeps
        // a frame's rows within 2 GiB for the fused schedule)
        constexpr int ESZ = FP8 ? 1 : 2;
        const int stb = (int)L.st * ESZ;
        const int fbytes = ((S - 1) * (int)L.st + D) * ESZ;
        const __amdgpu_buffer_rsrc_t rk = buffer_over((const char*)L.k + fo * ESZ, fbytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_over((const char*)L.v + fo * ESZ, fbytes);
        typename std::conditional<FP8, XStage8<D, NT, SC>, XStage<bf16, D, NT, SC>>::type stg;
        stg.load_rs(rk, rv, stb, 0, tid);
        for (int c0 = 0; c0 < S; c0 += X::SC) {
            __syncthreads();  // readers of the previous chunk are done
            stg.store_rs(lds, tid);
            __syncthreads();
            if (c0 + X::SC < S) stg.load_rs(rk, rv, stb, c0 + X::SC, tid);
#pragma unroll
            for (int ks = 0; ks < X::SC / MM::KS; ++ks) {
                const int tok = ks * MM::KS + g * MM::KL;
                bf16x8 kn[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    kn[nb] = ld_frag<bf16>((const bf16*)(lds + X::addr(nw + 16 * nb + r16, tok)));
                if constexpr (DELTA) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const bf16x8 ki = ld_frag<bf16>((const bf16*)(lds + X::addr(16 * kb + r16, tok)));
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) gacc[kb][nb] = MM::run(ki, kn[nb], gacc[kb][nb]);
                    }
                }
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const bf16x8 vc = ld_frag<bf16>((const bf16*)(lds + X::addr(D + 16 * cb + r16, tok)));
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) bacc[nb][cb] = MM::run(kn[nb], vc, bacc[nb][cb]);
                }
            }
        }
    }
    const int gi = bh * F + f;
    const float gm = L.gamma[gi], bt = L.beta[gi];
    float sG = gm * bt * L.c * L.c, sB = bt * L.c;
    if constexpr (FP8) {
        const float sk = L.k_scale[gi];
        sG *= sk * sk;
        sB *= sk * L.v_scale[gi];
    }
    // -Ghat as bf16 hi + lo (A operand of the step), Bhat scaled in place
    uint32_t gh[DELTA ? KB : 1][NB][2], gl[DELTA ? KB : 1][NB][2];
    if constexpr (DELTA) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const float x = -sG * gacc[kb][nb][2 * c2], y = -sG * gacc[kb][nb][2 * c2 + 1];
                    const uint32_t hh = pack_bf16x2(x, y);
                    gh[kb][nb][c2] = hh;
                    gl[kb][nb][c2] = pack_bf16x2(x - __builtin_bit_cast(float, hh << 16),
                                                 y - __builtin_bit_cast(float, hh & 0xFFFF0000u));
                }
    }
    if constexpr (SAVE && DELTA) {
        // Ghat[m][k] with m = nw + 16 nb + r (symmetry) and k = 16 kb + 4 g .. + 3: 8 bytes of
        // 4 consecutive k in each plane of the record
        bf16* grec = (bf16*)L.save_recs + (int64_t)(bh * F + f) * (rec_g_bytes<D, DELTA>() / 2);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int m = nw + 16 * nb + r16, k0 = 16 * kb + 4 * g;
                const uint32_t sign = 0x80008000u;
                *(u32x2*)(grec + rec_g_off<D>(0, m, k0)) = u32x2{gh[kb][nb][0] ^ sign, gh[kb][nb][1] ^ sign};
                *(u32x2*)(grec + rec_g_off<D>(1, m, k0)) = u32x2{gl[kb][nb][0] ^ sign, gl[kb][nb][1] ^ sign};
            }
    }
    float* save_bh = SAVE ? L.save_states + (int64_t)bh * (F + 1) * D * D : nullptr;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) bacc[nb][cb] *= sB;

    // ---- 2. the state step, pipelined over kChainGroups groups of value columns: column c of
    // M_f only depends on column c of M_{f-1}, so group g of frame f starts as soon as frame f-1
    // has published its group g, and the frame-to-frame period is one group's latency.
    // groups (one 16-column block each at D = 128 and D = 64), 16-column blocks per group
    constexpr int CG = kChainGroups < CB ? kChainGroups : CB, CPG = CB / CG;
    static_assert(CB % CG == 0, "column blocks split evenly into groups");
    int* flags = L.ctl + 2 + bh * kChainGroups;
    bf16* Ph = (bf16*)lds;
    bf16* Pl = Ph + PLANE;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_over(L.chain + ((int64_t)((f + 1) & 1) * BH + bh) * D * D, D * D * 4);  // M_{f-1}
    const __amdgpu_buffer_rsrc_t rd =
        buffer_over(L.chain + ((int64_t)(f & 1) * BH + bh) * D * D, D * D * 4);        // M_f
#pragma unroll
    for (int grp = 0; grp < CG; ++grp) {
        if (tid == 0) {
            int ok = 1;
            if (f > 0) {
                int polls = 0;
                while (L.spin_limit == 0 ||
                       __hip_atomic_load(flags + grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < f - 1) {
                    if (++polls > L.spin_limit) {
                        ok = 0;
                        __hip_atomic_store(&L.ctl[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            s_ok = ok;
        }
        // also: the LDS readers of the last gram chunk (group 0) and of the previous group's
        // planes are done
        __syncthreads();
        const bool ok = s_ok != 0;

        // M_{f-1}[n][c] at this lane's C-layout positions: n = nw + 16 nb + 4 g + q,
        // c = 16 cb + r, for the group's column blocks; all loads issued before any is used
        f32x4 mp[NB][CPG];
        if (f > 0) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < CPG; ++j)
                    mp[nb][j] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rs, (((wave * NB + nb) * CB + grp * CPG + j) * 64 + lane) * 16, 0, kCoherent));
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < CPG; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        mp[nb][j][q] = L.state_in ? L.state_in[((int64_t)bh * D + nw + 16 * nb + 4 * g + q) * D +
                                                               16 * (grp * CPG + j) + r16]
                                                  : 0.f;
            if constexpr (SAVE) {   // slot 0: the initial state, transposed
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int j = 0; j < CPG; ++j)
                        *(f32x4*)(save_bh + (16 * (grp * CPG + j) + r16) * D + nw + 16 * nb + 4 * g) = mp[nb][j];
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int kb = (nw + 16 * nb) >> 4;
            const int pos = 32 * (kb >> 1) + 8 * g + 4 * (kb & 1);
#pragma unroll
            for (int j = 0; j < CPG; ++j) {
                const int cb = grp * CPG + j;
                const int c = 16 * cb + r16;
                const float nan = __builtin_nanf("");
                const f32x4 m = ok ? mp[nb][j] : f32x4{nan, nan, nan, nan};
                bacc[nb][cb] += gm * m;
                if constexpr (DELTA) store_split4(Ph + c * MR + pos, Pl + c * MR + pos, m);
            }
        }
        if constexpr (DELTA) {
            __syncthreads();
            // three passes (hi.hi, hi.lo, lo.hi) per k step, each over all of the group's
            // accumulators, so that consecutive MFMAs never depend on each other
#pragma unroll
            for (int ks = 0; ks < KB / 2; ++ks) {
                bf16x8 ah[NB], al[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    ah[nb] = __builtin_bit_cast(bf16x8, u32x4{gh[2 * ks][nb][0], gh[2 * ks][nb][1],
                                                             gh[2 * ks + 1][nb][0], gh[2 * ks + 1][nb][1]});
                    al[nb] = __builtin_bit_cast(bf16x8, u32x4{gl[2 * ks][nb][0], gl[2 * ks][nb][1],
                                                             gl[2 * ks + 1][nb][0], gl[2 * ks + 1][nb][1]});
                }
#pragma unroll
                for (int pass = 0; pass < 3; ++pass) {
                    const bf16* plane = pass == 1 ? Pl : Ph;
#pragma unroll
                    for (int j = 0; j < CPG; ++j) {
                        const int cb = grp * CPG + j;
                        const bf16x8 m = ld_frag<bf16>(plane + (16 * cb + r16) * MR + 32 * ks + 8 * g);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            bacc[nb][cb] = MM::run(pass == 2 ? al[nb] : ah[nb], m, bacc[nb][cb]);
                    }
                }
            }
        }
        // publish group grp of M_f
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < CPG; ++j) {
                const int cb = grp * CPG + j;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, bacc[nb][cb]), rd,
                                                       (((wave * NB + nb) * CB + cb) * 64 + lane) * 16, 0,
                                                       kCoherent);
            }
        __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's state stores are done
        __syncthreads();  // ... and every wave's; also: the group's planes are no longer read
        if (tid == 0) __hip_atomic_store(flags + grp, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (SAVE) {   // slot f + 1: M_f, transposed
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < CPG; ++j) {
                    const int cb = grp * CPG + j;
                    *(f32x4*)(save_bh + ((int64_t)(f + 1) * D + 16 * cb + r16) * D + nw + 16 * nb + 4 * g) = bacc[nb][cb];
                }
        }
    }
    if (f == F - 1 && L.state_out) {
        float* so = L.state_out + (int64_t)bh * D * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) so[(nw + 16 * nb + 4 * g + q) * D + 16 * cb + r16] = bacc[nb][cb][q];
    }
    if constexpr (!OUT) return;

    // ---- 3. O_f = Q_f M_f (as output_body, with bf16(M_f)^T from LDS)
    bf16* Mt = (bf16*)lds;  // [c][n]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const f32x4 x = bacc[nb][cb];
            store4(Mt + (16 * cb + r16) * MR + nw + 16 * nb + 4 * g, x[0], x[1], x[2], x[3]);
        }
    __syncthreads();
    // k slots paired over two steps: in steps 2j and 2j + 1, lane group g holds the 16
    // consecutive features 64 j + 16 g .. + 15 (the first 8 in step 2j), so that one 16-byte load
    // brings a lane's E4M3 codes for both steps. Both input types and M^T use this grouping:
    // each instruction rounds its own partial sum, and the E4M3 path (codes, then the scale on
    // the fp32 result) equals the bf16 path on the decoded values bit for bit only when the two
    // group the features alike.
    constexpr int TJ = D / 16, KSN = D / MM::KS;
    static_assert(KSN % 2 == 0 && MM::KS == 32 && MM::KL == 8, "paired k steps of 32");
    auto kslot = [&](int ks) { return 64 * (ks >> 1) + 16 * g + 8 * (ks & 1); };
    bf16x8 am[TJ][KSN];
#pragma unroll
    for (int jt = 0; jt < TJ; ++jt)
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            am[jt][ks] = ld_frag<bf16>(Mt + out_col<bf16, D>(jt, r16) * MR + kslot(ks));
    // Q tiles read and O tiles written through buffer resources that end with the frame's
    // last row, so tiles past S read zeros and drop their stores without branches; each wave
    // keeps QD tiles of Q in flight (a ring, unrolled so that every slot is a register)
    constexpr int ESZ = FP8 ? 1 : 2;
    constexpr int QD = 4;
    // rows addressed past the frame: Q loads up to 2 QD - 1 tiles of 64 ahead of the last tile
    // begun before S (plus its 16 rows), O stores up to QD - 1 tiles on, K/V one stage on
    static_assert((2 * QD - 1) * 64 + 15 < kFusedRowsPast && X::SC <= kFusedRowsPast,
                  "the host bound covers every row the fused kernel addresses");
    const __amdgpu_buffer_rsrc_t rq =
        buffer_over((const char*)L.q + fo * ESZ, ((S - 1) * (int)L.st + D) * ESZ);
    const __amdgpu_buffer_rsrc_t ro = buffer_over(
        (char*)L.o + ((int64_t)b * L.ob + (int64_t)h * L.oh + (int64_t)f * S * L.ot) * 2,
        ((S - 1) * (int)L.ot + D) * 2);
    const int qstb = (int)L.st * ESZ, ostb = (int)L.ot * 2;
    const float oscale = FP8 ? L.q_scale[gi] : 1.f;
    // Q fragments as loaded: per step 8 bf16 values, or per step pair 16 E4M3 codes decoded
    // when used
    constexpr int QN = FP8 ? KSN / 2 : KSN;
    auto load_q = [&](int s0, u32x4 (&bq)[QN]) {
        const int vo = (s0 + r16) * qstb;
#pragma unroll
        for (int i = 0; i < QN; ++i)
            bq[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rq, vo + kslot(FP8 ? 2 * i : i) * ESZ, 0, 0));
    };
    u32x4 bq[QD][QN];
#pragma unroll
    for (int d = 0; d < QD; ++d) load_q(wave * 16 + d * 64, bq[d]);
    for (int s0 = wave * 16; s0 < S; s0 += QD * 64) {
#pragma unroll
        for (int d = 0; d < QD; ++d) {
            const int st = s0 + d * 64;   // this tile; all lanes past S when st >= S
            bf16x8 bw[KSN];
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) {
                if constexpr (FP8) {
                    const u32x4 w = bq[d][ks >> 1];
                    bw[ks] = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(
                                                           (ks & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]}));
                } else {
                    bw[ks] = __builtin_bit_cast(bf16x8, bq[d][ks]);
                }
            }
            load_q(st + QD * 64, bq[d]);  // the tile QD steps ahead, into the freed slot
            f32x4 acc[TJ];
#pragma unroll
            for (int jt = 0; jt < TJ; ++jt) {
                acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSN; ++ks) acc[jt] = MM::run(am[jt][ks], bw[ks], acc[jt]);
                if constexpr (FP8) acc[jt] *= oscale;
            }
            const int oo = (st + r16) * ostb;
#pragma unroll
            for (int p = 0; p < TJ / 2; ++p) {
                const f32x4 x = acc[2 * p], y = acc[2 * p + 1];
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
                          pack_bf16x2(y[2], y[3])},
                    ro, oo + (32 * p + 8 * g) * 2, 0, 0);
            }
        }
    }
}

// ----------------------------------------------------------------------------------------
// Backward, per (b, h, f): the gradients of the frame's K, V, gamma and beta from
// G_f = dL/dM_f, the state before the frame (M_{f-1}) and the frame's K, V (dQ = dO M_f^T needs
// neither G_f nor K, V: qdo_kernel forms it on its pass over Q and dO). With Kt = c K and
// P = Kt M_{f-1} (the reverse-mode derivative of the forward update):
//     dV = beta Kt G
//     dKt = beta R G^T - gamma beta (Kt G) M_{f-1}^T,   R = V - gamma P,   dK = c dKt
//     dgamma = <G, M_{f-1}> - beta <Kt G, P>            dbeta = <Kt G, R>
// (no delta term: R = V and only the first term of dKt and of dgamma). M_{f-1} and G_f come
// from the workspace in fp32, transposed ([c][n]), and are staged in LDS as bf16. Every
// product runs transposed on MFMA, so that each lane ends up with 4 consecutive feature rows
// of one token: P^T and (Kt G)^T from A = M_{f-1}^T / G^T rows and B = K rows; their C tiles
// are then the B operand of dKt^T = G (beta R^T) + M_{f-1} (-gamma beta (Kt G)^T), with the
// k order of a 32-long step taken from two C tiles (slots 0-3 and 4-7) and the A operand read
// transposed from the same LDS copies (ds_read_tr16_b64).
// dgamma and dbeta are summed over the frame inside the workgroup in a fixed order.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Swizzled LDS layout of the backward's bf16 matrices (D x D states, token x D chunks): rows of
// D elements without padding, the 8-byte units of row r (4 elements each) permuted by XOR with
// a mask of the bits 0, 1, 3, 4 of r. The masks make the three access patterns of the backward
// free of bank conflicts, whether the LDS serves 64 banks per clock (16 lanes of a 16-byte
// access, 32 lanes of an 8-byte one) or 32: transposed reads (read_tr4: rows k0 + 8 g' + 0..3,
// units 8 (jt >> 1) + 2 (r & 3) + (jt & 1)), 16-byte fragment reads of the rows out_col(cb, r),
// and 16-byte row stores (16 lanes per row). A 16-byte access covers the unit pair 2u, 2u + 1;
// with an odd mask the pair lies swapped in LDS, so its two 8-byte halves swap in registers.
template <int D> __device__ __forceinline__ int sw_mask(int r) {
    const int b0 = r & 1, b1 = (r >> 1) & 1, b3 = (r >> 3) & 1, b4 = (r >> 4) & 1;
    if constexpr (D == 128) return b0 | b0 << 1 | (b4 ^ b3) << 2 | b1 << 3 | b3 << 4;
    else return (b0 ^ b3) | b3 << 1 | (b4 ^ b0) << 2 | b1 << 3;
}
// 16 bytes of row r, columns [c, c + 8) (c a multiple of 8), to / from a swizzled matrix
template <int D> __device__ __forceinline__ void st16_sw(bf16* X, int r, int c, u32x4 v) {
    const int m = sw_mask<D>(r);
    st16(X + r * D + (((c >> 2) ^ (m & ~1)) << 2), (m & 1) ? u32x4{v[2], v[3], v[0], v[1]} : v);
}
template <int D> __device__ __forceinline__ bf16x8 ld16_sw(const bf16* X, int r, int c) {
    const int m = sw_mask<D>(r);
    const u32x4 v = ld16(X + r * D + (((c >> 2) ^ (m & ~1)) << 2));
    return __builtin_bit_cast(bf16x8, (m & 1) ? u32x4{v[2], v[3], v[0], v[1]} : v);
}

// A operand slice of Y = X^T from a swizzled [k][n] LDS matrix X, with the rows of the 16-row
// tile jt permuted as in out_col (tiles 2p and 2p + 1 together cover 32 p .. 32 p + 31 so that
// lane (r, g) of their C tiles holds 8 consecutive rows): lane (r, g) of a 16-lane group
// receives Y[out_col(jt, r)][k0 + 4 g + j] = X[k0 + 4 g + j][out_col(jt, r)], j = 0..3.
// (ds_read_tr16_b64: in each 16-lane group, destination lane i takes element i mod 4 of the four
// b16 values at the address of source lane 4 j + i / 4; source lane 4 j + a points at row
// k0 + 4 g + j, columns out_col(jt, 4 a) .. + 3, one 8-byte unit.)
template <int D> __device__ __forceinline__ u32x2 read_tr4(const bf16* X, int k0, int jt, int r16, int g) {
    const int r = k0 + 4 * g + (r16 >> 2);
    const int u = 8 * (jt >> 1) + 2 * (r16 & 3) + (jt & 1);
    const bf16* a = X + r * D + ((u ^ sw_mask<D>(r)) << 2);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a));
}

constexpr int kBwdThreads = 512;
constexpr int kVmcnt0 = 0x0F70;   // s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt not waited for

template <int D, bool DELTA>
__global__ __launch_bounds__(kBwdThreads) void bwd_kernel(Launch L) {
    using MM = Mma<bf16>;
    constexpr int NW = kBwdThreads / 64;
    constexpr int CT = D / 16;        // 16-row tiles of a feature dimension
    constexpr int CP = CT / 2;        // tile pairs (32 features)
    constexpr int KS = D / 32;        // 32-long k steps over a feature dimension
    constexpr int PLANE = D * D;      // swizzled (sw_mask)
    __shared__ __attribute__((aligned(16))) bf16 sm[2 * PLANE];  // M_{f-1}^T, G_f^T
    __shared__ float red[2][NW];
    static_assert(D == 64 || D == 128, "backward: D = 64 or 128");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int F = L.F, S = L.S;
    const int f = blockIdx.x % F, bh = blockIdx.x / F;
    const int b = bh / L.H, h = bh % L.H;
    const int gi = bh * F + f;
    const float gm = L.gamma[gi], bt = L.beta[gi], c = L.c;
    bf16* Mp = sm;              // M_{f-1}^T [c][n]
    bf16* Gs = sm + PLANE;      // G_f^T

    // stage the two matrices (fp32 slot f of the states, f + 1 of G) as bf16 and form the frame
    // term <G_f, M_{f-1}> of dgamma from the fp32 values on the way
    float dg = 0.f, db = 0.f;
    {
        const float* mt = (const float*)L.mt + ((int64_t)bh * (F + 1) + f) * D * D;
        const float* gt = (const float*)L.gt + ((int64_t)bh * (F + 1) + f + 1) * D * D;
        constexpr int NE = D * D / 8, PT = (NE + kBwdThreads - 1) / kBwdThreads;
        f32x4 xm[PT][2], xg[PT][2];
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int e = min(tid + k * kBwdThreads, NE - 1);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                xm[k][hh] = *(const f32x4*)(mt + e * 8 + 4 * hh);
                xg[k][hh] = *(const f32x4*)(gt + e * 8 + 4 * hh);
            }
        }
        auto pack8 = [](const f32x4 (&x)[2]) {
            return u32x4{pack_bf16x2(x[0][0], x[0][1]), pack_bf16x2(x[0][2], x[0][3]),
                         pack_bf16x2(x[1][0], x[1][1]), pack_bf16x2(x[1][2], x[1][3])};
        };
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int e = tid + k * kBwdThreads;
            if (NE % kBwdThreads == 0 || e < NE) {
                const int row = e / (D / 8), cb8 = e % (D / 8);
                st16_sw<D>(Mp, row, cb8 * 8, pack8(xm[k]));
                st16_sw<D>(Gs, row, cb8 * 8, pack8(xg[k]));
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int q = 0; q < 4; ++q) dg += xm[k][hh][q] * xg[k][hh][q];
            }
        }
    }
    __syncthreads();

    const int64_t io = (int64_t)b * L.sb + (int64_t)h * L.sh + (int64_t)f * S * L.st;
    const bf16* kf = (const bf16*)L.k + io;
    const bf16* vf = (const bf16*)L.v + io;
    bf16* dkf = (bf16*)L.dk + io;
    bf16* dvf = (bf16*)L.dv + io;

    // the wave's 16-token tiles s0 = 16 wave + 16 NW i; K and V of the next tile load while the
    // current one is used (one tile ahead in registers). K, V, dK and dV go through buffer
    // resources that end with the frame's last row: rows at or past S read zero and drop their
    // stores, with no branches around the loads (the host keeps a frame's rows below 2 GiB)
    const int fbytes = ((S - 1) * (int)L.st + D) * 2, stb = (int)L.st * 2;
    const __amdgpu_buffer_rsrc_t rk = buffer_over(kf, fbytes), rv = buffer_over(vf, fbytes);
    const __amdgpu_buffer_rsrc_t rdk = buffer_over(dkf, fbytes), rdv = buffer_over(dvf, fbytes);
    auto row_off = [&](int s0) { return s0 + r16 < S ? (s0 + r16) * stb + 16 * g : fbytes; };
    bf16x8 bk[KS];
    u32x4 vv[CP];
    auto load_kv = [&](int s0, bf16x8 (&kr)[KS], u32x4 (&vr)[CP]) __attribute__((always_inline)) {
        const int off = row_off(s0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off + 64 * ks, 0, 0));
#pragma unroll
        for (int p = 0; p < CP; ++p)
            vr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off + 64 * p, 0, 0));
    };
    load_kv(wave * 16, bk, vv);
    // the first tile is complete before the loop: otherwise the compiler's wait at the loop
    // head, placed for these loads, also waits for the previous tile's stores on every pass
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    for (int s0 = wave * 16; s0 < S; s0 += NW * 16) {
        const int so = row_off(s0);
        bf16x8 nk[KS];
        u32x4 nv[CP];
        load_kv(s0 + NW * 16, nk, nv);

        // P^T and (Kt G)^T: C tiles whose rows are the features out_col(cb, 4 g + q), i.e. for
        // tile pair p, lane (r, g) holds features 32 p + 8 g + (0..7) of token r
        f32x4 pt[CT], kg[CT];
#pragma unroll
        for (int cb = 0; cb < CT; ++cb) {
            pt[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            kg[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int row = out_col<bf16, D>(cb, r16);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (DELTA) pt[cb] = MM::run(ld16_sw<D>(Mp, row, ks * 32 + 8 * g), bk[ks], pt[cb]);
                kg[cb] = MM::run(ld16_sw<D>(Gs, row, ks * 32 + 8 * g), bk[ks], kg[cb]);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep each tile's LDS reads next to its MFMAs
        }
        // residual, dV, dgamma / dbeta terms; B operands of dKt^T as bf16 pairs (natural k
        // order: slots 0-7 of step ks are features 32 ks + 8 g + 0..7)
        uint32_t b1[CT][2], b2[CT][2];
#pragma unroll
        for (int p = 0; p < CP; ++p) {
            uint32_t dvw[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int cb = 2 * p + hh;
                float rr[4], kk[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w2 = vv[p][2 * hh + (q >> 1)];
                    const float v = __builtin_bit_cast(float, (q & 1) ? (w2 & 0xFFFF0000u) : (w2 << 16));
                    const float pp = c * pt[cb][q];
                    kk[q] = c * kg[cb][q];
                    rr[q] = DELTA ? v - gm * pp : v;
                    db += kk[q] * rr[q];
                    if (DELTA) dg -= bt * kk[q] * pp;
                }
                dvw[2 * hh] = pack_bf16x2(bt * kk[0], bt * kk[1]);
                dvw[2 * hh + 1] = pack_bf16x2(bt * kk[2], bt * kk[3]);
                b1[cb][0] = pack_bf16x2(bt * rr[0], bt * rr[1]);
                b1[cb][1] = pack_bf16x2(bt * rr[2], bt * rr[3]);
                const float sc = -gm * bt;
                b2[cb][0] = pack_bf16x2(sc * kk[0], sc * kk[1]);
                b2[cb][1] = pack_bf16x2(sc * kk[2], sc * kk[3]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{dvw[0], dvw[1], dvw[2], dvw[3]}, rdv, so + 64 * p, 0, 0);
        }
        // dKt^T, a pair of 16-row tiles (32 features) at a time (not unrolled: it indexes no
        // register array, and unrolling lets the compiler hoist every LDS read)
#pragma unroll
        for (int p = 0; p < CP; ++p) {
            f32x4 ak[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 B1 = __builtin_bit_cast(bf16x8, u32x4{b1[2 * ks][0], b1[2 * ks][1],
                                                                  b1[2 * ks + 1][0], b1[2 * ks + 1][1]});
                bf16x8 B2;
                if constexpr (DELTA)
                    B2 = __builtin_bit_cast(bf16x8, u32x4{b2[2 * ks][0], b2[2 * ks][1],
                                                         b2[2 * ks + 1][0], b2[2 * ks + 1][1]});
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int jt = 2 * p + hh;
                    // slots 0-3: features 32 ks + 8 g + j; slots 4-7: 32 ks + 8 g + 4 + j
                    const u32x2 g0 = read_tr4<D>(Gs, 32 * ks, jt, r16, 2 * g);
                    const u32x2 g1 = read_tr4<D>(Gs, 32 * ks + 4, jt, r16, 2 * g);
                    ak[hh] = MM::run(__builtin_bit_cast(bf16x8, u32x4{g0[0], g0[1], g1[0], g1[1]}), B1, ak[hh]);
                    if constexpr (DELTA) {
                        const u32x2 m0 = read_tr4<D>(Mp, 32 * ks, jt, r16, 2 * g);
                        const u32x2 m1 = read_tr4<D>(Mp, 32 * ks + 4, jt, r16, 2 * g);
                        ak[hh] = MM::run(__builtin_bit_cast(bf16x8, u32x4{m0[0], m0[1], m1[0], m1[1]}), B2, ak[hh]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{pack_bf16x2(c * ak[0][0], c * ak[0][1]), pack_bf16x2(c * ak[0][2], c * ak[0][3]),
                      pack_bf16x2(c * ak[1][0], c * ak[1][1]), pack_bf16x2(c * ak[1][2], c * ak[1][3])},
                rdk, so + 64 * p, 0, 0);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bk[ks] = nk[ks];
#pragma unroll
        for (int p = 0; p < CP; ++p) vv[p] = nv[p];
    }

    // dgamma, dbeta: wave sums, then a fixed-order sum over waves
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        dg += __shfl_xor(dg, o);
        db += __shfl_xor(db, o);
    }
    if (lane == 0) {
        red[0][wave] = dg;
        red[1][wave] = db;
    }
    __syncthreads();
    if (tid == 0) {
        float sg = 0.f, sbt = 0.f;
        for (int w = 0; w < NW; ++w) {
            sg += red[0][w];
            sbt += red[1][w];
        }
        L.dgamma[gi] = sg;
        L.dbeta[gi] = sbt;
    }
}

// ----------------------------------------------------------------------------------------
// Backward, per (b, h, f): the two products that need Q and dO,
//     C_f = Q_f^T dO_f  (the per-frame term of the reverse chain)   and   dQ_f = dO_f M_f^T,
// in one pass over Q and dO (dQ needs only the forward state M_f, not G_f). Chunks of 64 tokens
// of Q and dO go through registers into LDS as rows (token-major, as in memory); the next
// chunk's loads are in flight while the current chunk is used. C contracts over tokens on MFMA
// with both operands read transposed from the row tiles (ds_read_tr16_b64): A = Q^T, B = dO.
// Wave w owns the C row tiles ja = RW w .. RW w + RW - 1 against every column tile jb; lane
// (r, g) of tile (ja, jb) holds C[i0 + q][out_col(jb, r)], i0 = out_col(ja, 4 g), q = 0..3
// ("C layout" below). dQ^T = M_f dO^T runs with A = M_f read transposed from an LDS copy of
// M_f^T and B = dO rows: wave w takes the 16 chunk rows out_col(w, r), r = 0..15. Every LDS
// matrix uses the swizzled layout of sw_mask. Q and dO are read through L.q and L.d_o with
// their own strides.
//
// Without CHAIN, one workgroup per (b, h, f, token split): C goes to the per-frame record the
// reverse scan reads (L.canon, the no-delta record layout of the gram products), or with
// several splits to fp32 partials (L.part) that combine_kernel sums.
//
// With CHAIN (whole frames), the reverse chain runs inside the kernel, ticket-ordered like the
// fused forward: ticket k takes frame t = F - 1 - k / BH of (b h) = k mod BH, and after its
// pass over Q and dO the workgroup forms
//     G_t = gamma_{t+1} G_{t+1} - Ghat_{t+1} G_{t+1} + C_t      (step u = F - 1 - t)
// from G_{t+1}, which the workgroup of ticket k - BH published (G_F = dstate_out, or zero, with
// gamma_F = 1 and Ghat_F = 0), and publishes G_t in turn. Ghat_{t+1} comes from the forward's
// per-frame records (L.canon, L.rec_stride bytes apart, +Ghat as bf16 hi/lo planes); the
// product Ghat G runs on MFMA with both operands split into hi + lo (hi.hi + hi.lo + lo.hi),
// G_{t+1} as the B operand from LDS planes [column][row]. G_t goes to the state-gradient slot
// t + 1 (fp32, transposed) for the gradient kernel; the workgroup of frame 0 also forms
// dstate_in = gamma_0 G_0 - Ghat_0 G_0. A workgroup only waits for a smaller ticket, whose
// workgroup is already running, so the chain always completes. Hand-off as in the fused
// forward: G moves through two fp32 buffers per (b, h) (step u writes buffer u mod 2) with
// device-coherent (sc1) accesses in the lanes' own order, in kBwdChainGroups groups of columns
// with one flag each (the last step that published the group), so that the next frame starts
// on a group as soon as it is published. Step u + 2 writes a group of buffer u mod 2 only after
// step u + 1, the only reader of it, has published that group (after its loads of it were
// used). The wait is bounded by L.spin_limit polls, after which the workgroup raises the
// time-out flag L.ctl[1], continues with a NaN G_{t+1} (so the state gradients of frame t and
// every earlier frame are NaN) and still publishes.
constexpr int kQdoThreads = 256;
constexpr int kBwdChainGroups = 4;   // column groups of the backward's chain hand-off

// Barrier for LDS hand-offs only: waits for this wave's LDS accesses, not for its global loads
// and stores (__syncthreads would also drain the prefetch of the next chunk and the dQ stores).
__device__ __forceinline__ void lds_sync() { __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, bool CHAIN, bool DELTA>
__global__ __launch_bounds__(kQdoThreads, 2) void qdo_kernel(Launch L) {
    using MM = Mma<bf16>;
    constexpr int NW = kQdoThreads / 64;
    constexpr int SC = 16 * NW;              // tokens per chunk: one 16-token dQ tile per wave
    constexpr int CT = D / 16, CP = CT / 2, KS = D / 32;
    constexpr int RW = CT / NW;              // C row tiles per wave
    constexpr int FB = D / 8;                // 16-byte blocks per token row
    constexpr int NLD = SC * FB / kQdoThreads;
    static_assert(D == 64 || D == 128, "backward: D = 64 or 128");
    static_assert(NW == 4 && (SC * FB) % kQdoThreads == 0 && (D * FB) % kQdoThreads == 0,
                  "four waves, whole rows per chunk");
    static_assert(!CHAIN || 2 * D * D <= (D + 2 * SC) * D, "the G planes fit in the chunk LDS");
    __shared__ __attribute__((aligned(16))) bf16 sm[(D + 2 * SC) * D];   // swizzled (sw_mask)
    __shared__ int s_ticket, s_ok;
    bf16* Mn = sm;               // M_f^T [c][n]
    bf16* Qt = sm + D * D;       // Q chunk [token][feature]
    bf16* Ot = Qt + SC * D;      // dO chunk [token][feature]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int F = L.F, S = L.S, BH = L.B * L.H;
    int f, bh, p;
    if constexpr (CHAIN) {
        if (tid == 0) s_ticket = atomicAdd(&L.ctl[0], 1);
        __syncthreads();
        f = F - 1 - s_ticket / BH;
        bh = s_ticket % BH;
        p = 0;
    } else {
        int blk = blockIdx.x;
        p = blk % L.nsplit;
        blk /= L.nsplit;
        f = blk % F;
        bh = blk / F;
    }
    const int b = bh / L.H, h = bh % L.H;
    const int gi = bh * F + f;
    const int t0 = CHAIN ? 0 : p * L.split_tokens, t1 = CHAIN ? S : min(S, t0 + L.split_tokens);
    const int64_t io = (int64_t)b * L.sb + (int64_t)h * L.sh + (int64_t)f * S * L.st;
    const bf16* qf = (const bf16*)L.q + io;
    bf16* dqf = (bf16*)L.dq + io;
    const bf16* of = (const bf16*)L.d_o + (int64_t)b * L.ob + (int64_t)h * L.oh + (int64_t)f * S * L.ot;

    // M_f^T (fp32 state slot f + 1) to LDS as bf16
    {
        const float* mt = (const float*)L.mt + ((int64_t)bh * (F + 1) + f + 1) * D * D;
        constexpr int PT = D * FB / kQdoThreads;
        f32x4 x[PT][2];
#pragma unroll
        for (int k = 0; k < PT; ++k)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) x[k][hh] = *(const f32x4*)(mt + (tid + k * kQdoThreads) * 8 + 4 * hh);
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int e = tid + k * kQdoThreads;
            st16_sw<D>(Mn, e / FB, (e % FB) * 8,
                       u32x4{pack_bf16x2(x[k][0][0], x[k][0][1]), pack_bf16x2(x[k][0][2], x[k][0][3]),
                             pack_bf16x2(x[k][1][0], x[k][1][1]), pack_bf16x2(x[k][1][2], x[k][1][3])});
        }
    }

    // tokens [c0, c0 + SC) of Q and dO into registers; rows at or beyond t1 are zero. Q, dO and
    // dQ go through buffer resources that end with the frame's last row, and rows past t1 are
    // addressed at that end: they read zero and drop their stores, with no branches (the host
    // keeps a frame's rows below 2 GiB), so the compiler can count the accesses in flight
    const int qbytes = ((S - 1) * (int)L.st + D) * 2, obytes = ((S - 1) * (int)L.ot + D) * 2;
    const int qstb = (int)L.st * 2, ostb = (int)L.ot * 2;
    const __amdgpu_buffer_rsrc_t rbq = buffer_over(qf, qbytes), rbo = buffer_over(of, obytes);
    const __amdgpu_buffer_rsrc_t rbdq = buffer_over(dqf, qbytes);
    u32x4 rq[NLD], ro[NLD];
    auto load = [&](int c0) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int e = tid + i * kQdoThreads, tok = c0 + e / FB, fb = e % FB;
            const bool in = tok < t1;
            rq[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rbq, in ? tok * qstb + fb * 16 : qbytes, 0, 0));
            ro[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rbo, in ? tok * ostb + fb * 16 : obytes, 0, 0));
        }
    };

    f32x4 acc[RW][CT];
#pragma unroll
    for (int a = 0; a < RW; ++a)
#pragma unroll
        for (int jb = 0; jb < CT; ++jb) acc[a][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ja0 = RW * wave;

    load(t0);
    // the first chunk is complete before the loop: otherwise the compiler's wait at the loop
    // head, placed for these loads, also waits for the previous chunk's dQ stores on every pass
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    for (int c0 = t0; c0 < t1; c0 += SC) {
        lds_sync();   // the previous chunk's readers are done (first pass: M_f^T is written)
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int e = tid + i * kQdoThreads, row = e / FB, fb = e % FB;
            st16_sw<D>(Qt, row, fb * 8, rq[i]);
            st16_sw<D>(Ot, row, fb * 8, ro[i]);
        }
        lds_sync();
        load(c0 + SC);   // past the end: zeros, no memory access
        __builtin_amdgcn_sched_barrier(0);   // issued here, a whole chunk ahead of their use

        // C += Q^T dO over the chunk's tokens, 32 at a time (k slots 0-7 of lane group g:
        // tokens k0 + 8 g + 0..7, the same in both operands)
#pragma unroll
        for (int k0 = 0; k0 < SC; k0 += 32) {
            bf16x8 af[RW];
#pragma unroll
            for (int a = 0; a < RW; ++a) {
                const u32x2 x0 = read_tr4<D>(Qt, k0, ja0 + a, r16, 2 * g);
                const u32x2 x1 = read_tr4<D>(Qt, k0 + 4, ja0 + a, r16, 2 * g);
                af[a] = __builtin_bit_cast(bf16x8, u32x4{x0[0], x0[1], x1[0], x1[1]});
            }
#pragma unroll
            for (int jb = 0; jb < CT; ++jb) {
                const u32x2 x0 = read_tr4<D>(Ot, k0, jb, r16, 2 * g);
                const u32x2 x1 = read_tr4<D>(Ot, k0 + 4, jb, r16, 2 * g);
                const bf16x8 bfr = __builtin_bit_cast(bf16x8, u32x4{x0[0], x0[1], x1[0], x1[1]});
#pragma unroll
                for (int a = 0; a < RW; ++a) acc[a][jb] = MM::run(af[a], bfr, acc[a][jb]);
            }
        }

        // dQ^T = M_f dO^T for the wave's 16 tokens (chunk rows out_col(wave, r): the fragment
        // reads of the swizzled tile are then free of bank conflicts), 32 features at a time
        const int trow = out_col<bf16, 64>(wave, r16);
        const int s = c0 + trow;
        const int so = s < t1 ? s * qstb + 16 * g : qbytes;
        bf16x8 bo[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bo[ks] = ld16_sw<D>(Ot, trow, ks * 32 + 8 * g);
#pragma unroll
        for (int pp = 0; pp < CP; ++pp) {
            f32x4 aq[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const u32x2 n0 = read_tr4<D>(Mn, 32 * ks, 2 * pp + hh, r16, 2 * g);
                    const u32x2 n1 = read_tr4<D>(Mn, 32 * ks + 4, 2 * pp + hh, r16, 2 * g);
                    aq[hh] = MM::run(__builtin_bit_cast(bf16x8, u32x4{n0[0], n0[1], n1[0], n1[1]}), bo[ks], aq[hh]);
                }
            }
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{pack_bf16x2(aq[0][0], aq[0][1]), pack_bf16x2(aq[0][2], aq[0][3]),
                      pack_bf16x2(aq[1][0], aq[1][1]), pack_bf16x2(aq[1][2], aq[1][3])},
                rbdq, so + 64 * pp, 0, 0);
        }
    }

    // row of C-layout register q of tile (a, .) is ri(a) + q; column of tile jb is out_col(jb, r)
    auto ri = [&](int a) { const int ja = ja0 + a; return 32 * (ja >> 1) + 8 * g + 4 * (ja & 1); };

    if constexpr (!CHAIN) {
#pragma unroll
        for (int a = 0; a < RW; ++a) {
            const int i0 = ri(a);
#pragma unroll
            for (int jb = 0; jb < CT; ++jb) {
                const int j = out_col<bf16, D>(jb, r16);
                if (L.nsplit == 1)
                    *(f32x4*)((float*)((char*)L.canon + (int64_t)gi * canon_bytes<D, false>()) + rec_b_off<D>(i0, j)) =
                        acc[a][jb];
                else
                    *(f32x4*)(L.part + ((int64_t)gi * L.nsplit + p) * (D * D) + j * D + i0) = acc[a][jb];
            }
        }
    } else {
        const int u = F - 1 - f;   // chain step
        // dst -= Ghat_fr src, with src (fp32, C layout) split into bf16 hi/lo planes
        // [column][row] in LDS as the B operand and Ghat_fr (A rows out_col(ja, r), i.e. the
        // C-layout rows ri(a) + q of the product) from frame fr's record
        auto ghat_step = [&](const f32x4 (&src)[RW][CT], f32x4 (&dst)[RW][CT], int fr) {
            bf16* Ph = sm;
            bf16* Pl = sm + D * D;
            __syncthreads();   // earlier readers of the LDS are done
#pragma unroll
            for (int a = 0; a < RW; ++a)
#pragma unroll
                for (int jb = 0; jb < CT; ++jb) {
                    const int j = out_col<bf16, D>(jb, r16);
                    const int off = j * D + (((ri(a) >> 2) ^ sw_mask<D>(j)) << 2);
                    store_split4(Ph + off, Pl + off, src[a][jb]);
                }
            __syncthreads();
            constexpr int KSN = rec_ksn<D>();
            const char* rec = (const char*)L.canon + ((int64_t)bh * F + fr) * L.rec_stride;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 ah[RW], al[RW];
#pragma unroll
                for (int a = 0; a < RW; ++a) {
                    const int m = out_col<bf16, D>(ja0 + a, r16);
                    const char* fa = rec + (((m >> 4) * 2) * KSN + ks) * 1024 + (16 * g + (m & 15)) * 16;
                    ah[a] = ld_frag<bf16>((const bf16*)fa);
                    al[a] = ld_frag<bf16>((const bf16*)(fa + KSN * 1024));
                }
#pragma unroll
                for (int jb = 0; jb < CT; ++jb) {
                    const int j = out_col<bf16, D>(jb, r16);
                    const bf16x8 bh_ = ld16_sw<D>(Ph, j, 32 * ks + 8 * g);
                    const bf16x8 bl_ = ld16_sw<D>(Pl, j, 32 * ks + 8 * g);
#pragma unroll
                    for (int a = 0; a < RW; ++a) {
                        f32x4 x = MM::run(ah[a], bh_, f32x4{0.f, 0.f, 0.f, 0.f});
                        x = MM::run(ah[a], bl_, x);
                        x = MM::run(al[a], bh_, x);
                        dst[a][jb] -= x;
                    }
                }
            }
        };

        // The step runs over kBwdChainGroups groups of column tiles (columns of G evolve
        // independently): group c of G_t needs only group c of G_{t+1}, so the next frame's
        // workgroup starts on group c as soon as this one has published it, and the
        // frame-to-frame period is one group's latency.
        constexpr int CG = kBwdChainGroups, TPG = CT / CG;   // groups, column tiles per group
        static_assert(CT % CG == 0 && CG <= kChainGroups, "column tiles split evenly into groups");
        int* flags = L.ctl + 2 + bh * kChainGroups;
        const __amdgpu_buffer_rsrc_t rs =
            buffer_over(L.chain + ((int64_t)((u + 1) & 1) * BH + bh) * D * D, D * D * 4);   // G_{t+1}
        const __amdgpu_buffer_rsrc_t rd =
            buffer_over(L.chain + ((int64_t)(u & 1) * BH + bh) * D * D, D * D * 4);         // G_t
        auto cidx = [&](int a, int jb) { return (((wave * RW + a) * CT + jb) * 64 + lane) * 16; };
        const float gnext = u > 0 ? L.gamma[gi + 1] : 1.f;

        // Ghat_{t+1} rows of this wave (A operand, hi and lo, every k step), loaded before the
        // first wait
        constexpr int KSN = rec_ksn<D>();
        bf16x8 ga[DELTA ? RW : 1][DELTA ? KS : 1][2];
        if constexpr (DELTA) {
            if (u > 0) {
                const char* rec = (const char*)L.canon + ((int64_t)bh * F + f + 1) * L.rec_stride;
#pragma unroll
                for (int a = 0; a < RW; ++a) {
                    const int m = out_col<bf16, D>(ja0 + a, r16);
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const char* fa = rec + (((m >> 4) * 2) * KSN + ks) * 1024 + (16 * g + (m & 15)) * 16;
                        ga[a][ks][0] = ld_frag<bf16>((const bf16*)fa);
                        ga[a][ks][1] = ld_frag<bf16>((const bf16*)(fa + KSN * 1024));
                    }
                }
            }
        }
        bf16* Ph = sm;            // G_{t+1} planes [column][row], the group's columns only
        bf16* Pl = sm + D * D;
#pragma unroll
        for (int grp = 0; grp < CG; ++grp) {
            if (tid == 0) {
                int ok = 1;
                if (u > 0) {
                    int polls = 0;
                    while (L.spin_limit == 0 ||
                           __hip_atomic_load(flags + grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < u - 1) {
                        if (++polls > L.spin_limit) {
                            ok = 0;
                            __hip_atomic_store(&L.ctl[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                s_ok = ok;
            }
            // also: the LDS readers of the last chunk (group 0) are done
            __syncthreads();
            const bool ok = s_ok != 0;
            // group grp of G_{t+1} in C layout (dstate_out for t = F - 1)
            f32x4 gn[RW][TPG];
#pragma unroll
            for (int a = 0; a < RW; ++a)
#pragma unroll
                for (int jj = 0; jj < TPG; ++jj) {
                    const int jb = grp * TPG + jj;
                    if (u > 0) {
                        gn[a][jj] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, cidx(a, jb), 0, kCoherent));
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            gn[a][jj][q] = L.d_state_out ? L.d_state_out[((int64_t)bh * D + ri(a) + q) * D +
                                                                         out_col<bf16, D>(jb, r16)]
                                                         : 0.f;
                    }
                }
            const float nan = __builtin_nanf("");
            // G_t = C_t + gamma_{t+1} G_{t+1} - Ghat_{t+1} G_{t+1}, for the group's columns
#pragma unroll
            for (int a = 0; a < RW; ++a)
#pragma unroll
                for (int jj = 0; jj < TPG; ++jj) {
                    if (!ok) gn[a][jj] = f32x4{nan, nan, nan, nan};
                    acc[a][grp * TPG + jj] += gnext * gn[a][jj];
                }
            if constexpr (DELTA) {
                if (u > 0) {
#pragma unroll
                    for (int a = 0; a < RW; ++a)
#pragma unroll
                        for (int jj = 0; jj < TPG; ++jj) {
                            const int j = out_col<bf16, D>(grp * TPG + jj, r16);
                            const int off = j * D + (((ri(a) >> 2) ^ sw_mask<D>(j)) << 2);
                            store_split4(Ph + off, Pl + off, gn[a][jj]);
                        }
                    __syncthreads();
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int jj = 0; jj < TPG; ++jj) {
                            const int j = out_col<bf16, D>(grp * TPG + jj, r16);
                            const bf16x8 bh_ = ld16_sw<D>(Ph, j, 32 * ks + 8 * g);
                            const bf16x8 bl_ = ld16_sw<D>(Pl, j, 32 * ks + 8 * g);
#pragma unroll
                            for (int a = 0; a < RW; ++a) {
                                f32x4 x = MM::run(ga[a][ks][0], bh_, f32x4{0.f, 0.f, 0.f, 0.f});
                                x = MM::run(ga[a][ks][0], bl_, x);
                                x = MM::run(ga[a][ks][1], bh_, x);
                                acc[a][grp * TPG + jj] -= x;
                            }
                        }
                }
            }
            // publish group grp of G_t
#pragma unroll
            for (int a = 0; a < RW; ++a)
#pragma unroll
                for (int jj = 0; jj < TPG; ++jj)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[a][grp * TPG + jj]), rd,
                                                           cidx(a, grp * TPG + jj), 0, kCoherent);
            __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are done
            __syncthreads();                                          // ... and every wave's
            if (tid == 0) __hip_atomic_store(flags + grp, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // state-gradient slot t + 1 for the gradient kernel: G_t transposed, [column][row]
        float* gt = (float*)L.gt + ((int64_t)bh * (F + 1) + f + 1) * D * D;
#pragma unroll
        for (int a = 0; a < RW; ++a)
#pragma unroll
            for (int jb = 0; jb < CT; ++jb) *(f32x4*)(gt + out_col<bf16, D>(jb, r16) * D + ri(a)) = acc[a][jb];

        // frame 0: dstate_in = gamma_0 G_0 - Ghat_0 G_0
        if (f == 0 && L.d_state_in) {
            const float g0 = L.gamma[gi];
            f32x4 ds[RW][CT];
#pragma unroll
            for (int a = 0; a < RW; ++a)
#pragma unroll
                for (int jb = 0; jb < CT; ++jb) ds[a][jb] = g0 * acc[a][jb];
            if constexpr (DELTA) ghat_step(acc, ds, 0);
#pragma unroll
            for (int a = 0; a < RW; ++a)
#pragma unroll
                for (int jb = 0; jb < CT; ++jb)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        L.d_state_in[((int64_t)bh * D + ri(a) + q) * D + out_col<bf16, D>(jb, r16)] = ds[a][jb][q];
        }
    }
}

// ----------------------------------------------------------------------------------------
// Kernel 4: one frame, partial sums over the split's tokens of U = K^T R, with
// R = V - (gamma c) K M (delta) or R = V (no delta). The prediction P = K M runs on MFMA with M
// (state_in) rounded to the I/O type. For bf16 data U is accumulated as K^T V + K^T (-gamma c P):
// V is an exact bf16 input and only the small prediction term is rounded to bf16. For fp32
// data R is formed in fp32. Each 64-token chunk of K and V is staged in LDS twice: transposed
// (rows = features; the U product contracts over tokens) and, for K, row-major (the prediction
// contracts over features). M is staged once per workgroup, transposed, in the I/O type.
// Token grouping inside a step of the U product: for bf16, a 32-token group is two 16-token
// tiles; lane group g holds tokens {4g..4g+3} of the first tile and {16+4g..16+4g+3} of the
// second (exactly the rows of the prediction's C fragments). For fp32, step q of a 16-token
// tile gives lane group g the token 4g + q.
// The partial is stored transposed, part[p][j][i] = U_p[i][j], 16 contiguous bytes per lane.
template <int D> constexpr int step_threads() { return 64 * (D / 16 > 4 ? D / 16 : 4); }

template <typename T, int D, bool DELTA>
__global__ __launch_bounds__(step_threads<D>()) void step_partial_kernel(Launch L) {
    using MM = Mma<T>;
    using X = XTile<T, D>;
    constexpr int SNT = step_threads<D>();   // one wave per 16-column tile (at least 4 waves)
    constexpr int TJ = D / 16;
    constexpr int NWJ = TJ;                   // waves with work
    constexpr int JW = 1;                     // 16-column tiles per wave
    constexpr int KSN = (D + MM::KS - 1) / MM::KS;  // contraction over D, padded to KS
    constexpr int DP = KSN * MM::KS;          // padded feature count
    constexpr int RT = sizeof(T) == 2 ? 2 : 1; // 16-token tiles per U step group
    constexpr int TG = 16 * RT;               // tokens per group
    constexpr int KR = DP + 16 / (int)sizeof(T);   // row length (elements) of the row-major K copy
    constexpr int MR = DP + 16 / (int)sizeof(T);   // row length of the transposed M copy
    __shared__ __attribute__((aligned(16))) char lds[X::BYTES];
    __shared__ __attribute__((aligned(16))) T krow[DELTA ? X::SC * KR : 1];
    constexpr bool MT = DELTA && sizeof(T) == 2;   // bf16: M staged transposed; fp32: read directly
    __shared__ __attribute__((aligned(16))) T mt[MT ? D * MR : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int p = blockIdx.x % L.nsplit, bh = blockIdx.x / L.nsplit;
    const int b = bh / L.H, h = bh % L.H;
    const int64_t io = (int64_t)b * L.sb + (int64_t)h * L.sh;
    const T* kb = (const T*)L.k + io;
    const T* vb = (const T*)L.v + io;
    const int t0 = p * L.split_tokens, t1 = min(L.S, t0 + L.split_tokens);
    const bool active = wave < NWJ;
    const float gc = L.gamma[bh] * L.c;

    // two chunks of K and V in flight: chunk c is loaded while chunk c - 2 is computed
    XStage<T, D, SNT> sa, sb;
    sa.load(kb, vb, L.st, L.st, t0, t1, tid);
    sb.load(kb, vb, L.st, L.st, t0 + X::SC, t1, tid);

    // B operand of the prediction: M[i][j] for this wave's columns, all key rows. bf16: from a
    // transposed copy mt[j][i] (i past D is zero); fp32: one element per lane, read directly
    // (lanes of a group read consecutive columns).
    typename MM::frag bm[JW][KSN];
    if constexpr (DELTA && !MT) {
        if (active) {
            const float* M = L.state_in + (int64_t)bh * D * D;
#pragma unroll
            for (int jl = 0; jl < JW; ++jl)
#pragma unroll
                for (int ks = 0; ks < KSN; ++ks)
                    bm[jl][ks] = M[(ks * 4 + g) * D + (wave * JW + jl) * 16 + r16];
        }
    }
    if constexpr (DELTA && DP > D) {
        for (int e = tid; e < X::SC * (DP - D); e += SNT) krow[(e / (DP - D)) * KR + D + e % (DP - D)] = (T)0.f;
    }
    if constexpr (MT) {
        const float* M = L.state_in + (int64_t)bh * D * D;
        // one 8 x 8 block of M per thread (D/8 x D/8 blocks <= SNT): 16 loads in flight, bf16
        // conversion and a register transpose, then 8 row stores of 16 bytes into mt
        constexpr int NBK = D / 8;
        static_assert(NBK * NBK <= SNT, "one 8x8 block of M per thread");
        if (tid < NBK * NBK) {
            const int bi = tid / NBK, bj = tid % NBK;
            f32x4 x[8][2];
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) x[e][hh] = *(const f32x4*)(M + (8 * bi + e) * D + 8 * bj + 4 * hh);
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const int hh = cc >> 2, q = cc & 3;
                st16(mt + (8 * bj + cc) * MR + 8 * bi,
                     u32x4{pack_bf16x2(x[0][hh][q], x[1][hh][q]), pack_bf16x2(x[2][hh][q], x[3][hh][q]),
                           pack_bf16x2(x[4][hh][q], x[5][hh][q]), pack_bf16x2(x[6][hh][q], x[7][hh][q])});
            }
        }
        if constexpr (DP > D) {
            for (int e = tid; e < D * (DP - D); e += SNT) mt[(e / (DP - D)) * MR + D + e % (DP - D)] = (T)0.f;
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int jl = 0; jl < JW; ++jl) {
                const int j = (wave * JW + jl) * 16 + r16;
#pragma unroll
                for (int ks = 0; ks < KSN; ++ks)
                    bm[jl][ks] = ld_frag<T>(mt + j * MR + ks * MM::KS + g * MM::KL);
            }
        }
    }

    f32x4 acc[TJ][JW];
#pragma unroll
    for (int it = 0; it < TJ; ++it)
#pragma unroll
        for (int jl = 0; jl < JW; ++jl) acc[it][jl] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto chunk = [&](XStage<T, D, SNT>& stg, int c0) {
        __syncthreads();
        stg.store(lds, tid);
        if constexpr (DELTA) stg.store_key_rows(krow, KR, tid);  // row-major K copy of the chunk
        __syncthreads();
        if (c0 + 2 * X::SC < t1) stg.load(kb, vb, L.st, L.st, c0 + 2 * X::SC, t1, tid);
        if (!active) return;
#pragma unroll
        for (int tg = 0; tg < X::SC; tg += TG) {
            // prediction P = K M (fp32, C layout): rows 4g+q of each 16-token tile, column
            // (wave tile jl, r16)
            f32x4 pr[RT][JW];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                for (int jl = 0; jl < JW; ++jl) pr[rt][jl] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (DELTA) {
#pragma unroll
                    for (int ks = 0; ks < KSN; ++ks) {
                        const typename MM::frag ak =
                            ld_frag<T>(krow + (tg + rt * 16 + r16) * KR + ks * MM::KS + g * MM::KL);
#pragma unroll
                        for (int jl = 0; jl < JW; ++jl) pr[rt][jl] = MM::run(ak, bm[jl][ks], pr[rt][jl]);
                    }
                }
            }
            if constexpr (sizeof(T) == 2) {
                // U += K^T V + K^T (-gamma c P): V enters exactly (bf16 input); only the
                // prediction term is rounded to bf16 for the MFMA.
#pragma unroll
                for (int jl = 0; jl < JW; ++jl) {
                    const int vrow = D + (wave * JW + jl) * 16 + r16;
                    const u32x2 vlo = *(const u32x2*)(lds + X::addr(vrow, tg + 4 * g));
                    const u32x2 vhi = *(const u32x2*)(lds + X::addr(vrow, tg + 16 + 4 * g));
                    const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{vlo[0], vlo[1], vhi[0], vhi[1]});
                    bf16x8 bp;
                    if (DELTA)
                        bp = __builtin_bit_cast(
                            bf16x8, u32x4{pack_bf16x2(-gc * pr[0][jl][0], -gc * pr[0][jl][1]),
                                          pack_bf16x2(-gc * pr[0][jl][2], -gc * pr[0][jl][3]),
                                          pack_bf16x2(-gc * pr[1][jl][0], -gc * pr[1][jl][1]),
                                          pack_bf16x2(-gc * pr[1][jl][2], -gc * pr[1][jl][3])});
#pragma unroll
                    for (int it = 0; it < TJ; ++it) {
                        const int krw = it * 16 + r16;
                        const u32x2 lo = *(const u32x2*)(lds + X::addr(krw, tg + 4 * g));
                        const u32x2 hi = *(const u32x2*)(lds + X::addr(krw, tg + 16 + 4 * g));
                        const bf16x8 ak = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                        acc[it][jl] = MM::run(ak, bv, acc[it][jl]);
                        if (DELTA) acc[it][jl] = MM::run(ak, bp, acc[it][jl]);
                    }
                }
            } else {
                // fp32 data: the residual R = V - gamma c P is formed and contracted in fp32
#pragma unroll
                for (int jl = 0; jl < JW; ++jl) {
                    const int vrow = D + (wave * JW + jl) * 16 + r16;
                    const f32x4 vv = *(const f32x4*)(lds + X::addr(vrow, tg + 4 * g));
                    float R[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) R[q] = DELTA ? vv[q] - gc * pr[0][jl][q] : vv[q];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int it = 0; it < TJ; ++it) {
                            const float ak = *(const float*)(lds + X::addr(it * 16 + r16, tg + 4 * g + q));
                            acc[it][jl] = Mma<float>::run(ak, R[q], acc[it][jl]);
                        }
                }
            }
        }
    };
    for (int c0 = t0; c0 < t1; c0 += 2 * X::SC) {
        chunk(sa, c0);
        if (c0 + X::SC < t1) chunk(sb, c0 + X::SC);
    }
    if (!active) return;
    float* out = L.part + ((int64_t)bh * L.nsplit + p) * D * D;
#pragma unroll
    for (int it = 0; it < TJ; ++it)
#pragma unroll
        for (int jl = 0; jl < JW; ++jl) {
            const int j = (wave * JW + jl) * 16 + r16;
            *(f32x4*)(out + j * D + it * 16 + 4 * g) = acc[it][jl];
        }
}

// Kernel 5: M' = gamma M + beta c sum_p U_p (fixed order over p); state_out on commit;
// transposed copy of M' in the I/O type for the output products. Thread: 4 key rows x 1 column.
// The partials of a thread are loaded in batches of 16 (indices clamped, extra terms masked) so
// that their loads are in flight together.
template <typename T, int D>
__global__ __launch_bounds__(NT) void step_reduce_kernel(Launch L) {
    constexpr int NQ = D * D / 4;
    constexpr int NB = (NQ + NT - 1) / NT;
    constexpr int BATCH = 16;
    const int bh = blockIdx.x / NB;
    const int t = (blockIdx.x % NB) * NT + threadIdx.x;
    if (t >= NQ) return;
    const int i0 = (t % (D / 4)) * 4, j = t / (D / 4);
    const float gm = L.gamma[bh], bc = L.beta[bh] * L.c;
    const float* part = L.part + (int64_t)bh * L.nsplit * D * D + j * D + i0;  // [p][j][i]
    const float* min_ = L.state_in + (int64_t)bh * D * D;
    float m0[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) m0[q] = min_[(i0 + q) * D + j];  // issued with the first batch
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
    const int np = L.nsplit;
    for (int p0 = 0; p0 < np; p0 += BATCH) {
        f32x4 x[BATCH];
#pragma unroll
        for (int e = 0; e < BATCH; ++e) x[e] = *(const f32x4*)(part + (int64_t)min(p0 + e, np - 1) * D * D);
#pragma unroll
        for (int e = 0; e < BATCH; ++e) u += p0 + e < np ? x[e] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = gm * m0[q] + bc * u[q];
    if (L.state_out) {
#pragma unroll
        for (int q = 0; q < 4; ++q) L.state_out[(int64_t)bh * D * D + (i0 + q) * D + j] = m[q];
    }
    store4((T*)L.mt + ((int64_t)bh * D + j) * D + i0, m[0], m[1], m[2], m[3]);
}

// ----------------------------------------------------------------------------------------
constexpr int kScanAhead = 4;  // frames of scan operands kept in flight

template <typename T, int D, bool DELTA> static hipError_t launch(Kernel k, const Launch& L,
                                                                 hipStream_t s) {
    const int BH = L.B * L.H;
    switch (k) {
    case K_PRODUCTS: {
        const int64_t n = (int64_t)BH * ((int64_t)L.gn * L.nsplit + (int64_t)L.on * L.nchunk);
        if (n == 0) return hipSuccess;
        hipLaunchKernelGGL((products_kernel<T, D, DELTA>), dim3((unsigned)n), dim3(NT), 0, s, L);
        break;
    }
    case K_COMBINE: {
        constexpr int NB = ((DELTA ? 2 * D : D) * D / 4 + NT - 1) / NT;
        if (L.gn == 0) return hipSuccess;
        hipLaunchKernelGGL((combine_kernel<D, DELTA>), dim3(BH * L.gn * NB), dim3(NT), 0, s, L);
        break;
    }
    case K_SCAN: {
        if (L.s1 <= L.s0) return hipSuccess;
        const int units = (BH + 7) / 8 * 8 * (D / 16);
        hipLaunchKernelGGL((scan_kernel<T, D, DELTA, kScanAhead, false, T>), dim3(units), dim3(64 * (D / 16)),
                           0, s, L);
        break;
    }
    case K_SCAN_STATES: {
        if (L.s1 <= L.s0) return hipSuccess;
        const int units = (BH + 7) / 8 * 8 * (D / 16);
        hipLaunchKernelGGL((scan_kernel<T, D, DELTA, kScanAhead, false, float>), dim3(units),
                           dim3(64 * (D / 16)), 0, s, L);
        break;
    }
    case K_FUSED_RESET: {
        const int n = 2 + BH * kChainGroups;
        hipLaunchKernelGGL(fused_reset_kernel, dim3((n + NT - 1) / NT), dim3(NT), 0, s, L.ctl, n, L.keep_timeout);
        break;
    }
    case K_FUSED: {
        if constexpr (std::is_same<T, bf16>::value && (D == 64 || D == 128)) {
            if (L.fp8)
                hipLaunchKernelGGL((fused_kernel<D, DELTA, true>), dim3(BH * L.F), dim3(NT), 0, s, L);
            else if (L.save_states && L.no_output)
                hipLaunchKernelGGL((fused_kernel<D, DELTA, false, true, false>), dim3(BH * L.F), dim3(NT), 0, s, L);
            else if (L.save_states)
                hipLaunchKernelGGL((fused_kernel<D, DELTA, false, true>), dim3(BH * L.F), dim3(NT), 0, s, L);
            else
                hipLaunchKernelGGL((fused_kernel<D, DELTA, false>), dim3(BH * L.F), dim3(NT), 0, s, L);
        } else {
            return hipErrorInvalidValue;
        }
        break;
    }
    case K_SCAN_BWD: {
        if (L.s1 <= L.s0) return hipSuccess;
        const int units = (BH + 7) / 8 * 8 * (D / 16);
        hipLaunchKernelGGL((scan_kernel<T, D, DELTA, kScanAhead, true, float>), dim3(units),
                           dim3(64 * (D / 16)), 0, s, L);
        break;
    }
    case K_BWD: {
        if constexpr (std::is_same<T, bf16>::value && (D == 64 || D == 128)) {
            hipLaunchKernelGGL((bwd_kernel<D, DELTA>), dim3(BH * L.F), dim3(kBwdThreads), 0, s, L);
        } else {
            return hipErrorInvalidValue;
        }
        break;
    }
    case K_BWD_QDO: {
        if constexpr (std::is_same<T, bf16>::value && (D == 64 || D == 128)) {
            if (L.bwd_chain)
                hipLaunchKernelGGL((qdo_kernel<D, true, DELTA>), dim3(BH * L.F), dim3(kQdoThreads), 0, s, L);
            else
                hipLaunchKernelGGL((qdo_kernel<D, false, false>), dim3(BH * L.F * L.nsplit), dim3(kQdoThreads), 0, s, L);
        } else {
            return hipErrorInvalidValue;
        }
        break;
    }
    case K_STEP_PARTIAL:
        hipLaunchKernelGGL((step_partial_kernel<T, D, DELTA>), dim3(BH * L.nsplit), dim3(step_threads<D>()),
                           0, s, L);
        break;
    case K_STEP_REDUCE: {
        constexpr int NB = (D * D / 4 + NT - 1) / NT;
        hipLaunchKernelGGL((step_reduce_kernel<T, D>), dim3(BH * NB), dim3(NT), 0, s, L);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// bf16_data: bf16 or E4M3 inputs (E4M3 runs only on the fused kernel)
bool fused_supported(int bf16_data, int D) { return bf16_data && (D == 64 || D == 128); }
bool backward_supported(int bf16_data, int D) { return bf16_data && (D == 64 || D == 128); }

hipError_t launch_kernel(Kernel k, const Launch& L, hipStream_t s) {
    const bool dl = L.use_delta != 0;
#define GDN_CASE(T, D) \
    case D: return dl ? launch<T, D, true>(k, L, s) : launch<T, D, false>(k, L, s);
    if (L.bf16 || L.fp8) {
        switch (L.D) { GDN_CASE(bf16, 16) GDN_CASE(bf16, 32) GDN_CASE(bf16, 64) GDN_CASE(bf16, 128) }
    } else {
        switch (L.D) { GDN_CASE(float, 16) GDN_CASE(float, 32) GDN_CASE(float, 64) GDN_CASE(float, 128) }
    }
#undef GDN_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
