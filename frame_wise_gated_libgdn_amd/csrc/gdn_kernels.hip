// HIP kernels of libgdn for gfx950 (MI355X): the frame-wise Gated DeltaNet recurrence.
//
// Recurrence (gen-hub.ru, "NVIDIA SANA-WM: минутное 720p видео с одной видеокарты", section
// "Архитектура: четыре нетривиальных решения"), per (b, h), c = key scale:
//     R = V_f - gamma_f (c K_f) M,   M <- gamma_f M + beta_f (c K_f)^T R,   O_f = Q_f M.
//
// Forward (all frames), three kernels:
//   1. gram_kernel   -- fully parallel over (b, h, f[, S split]). Stages K_f, V_f through LDS,
//                       contracts over the frame's tokens on MFMA:
//                         Ghat_f = gamma_f beta_f c^2 K_f^T K_f,  Bhat_f = beta_f c K_f^T V_f
//                       (gates and key scale applied in the epilogue).
//   2. scan_kernel   -- the serial part: M_f = gamma_f M - Ghat_f M + Bhat_f. This is the update
//                       above with the residual expanded (Kt^T (V - g Kt M) = Kt^T V - g Kt^T Kt M),
//                       so the frame-to-frame chain only touches D x D matrices; one workgroup
//                       owns 16 value columns of one head (columns of M evolve independently), so
//                       no workgroup waits on another. Writes each M_f (transposed, I/O type).
//   3. output_kernel -- fully parallel O_f = Q_f M_f on MFMA.
// Step (one frame from a cached state), the update as written:
//   4. step_partial_kernel -- per S split: P = K M (MFMA), R = V - (gamma c) P, U_p = K^T R (MFMA).
//   5. step_reduce_kernel  -- M' = gamma M + beta c sum_p U_p; state_out; transposed copy.
//   then output_kernel with one frame.
//
// MFMA: v_mfma_f32_16x16x32_bf16 for bf16 data, v_mfma_f32_16x16x4_f32 for fp32 data; fp32
// accumulation throughout. Lane l = 16 g + r of a wave holds A row r / B column r and the
// contraction slice [KL g, KL g + KL) of each KS-long step; C row 4 g + q, column r in
// register q. The contraction order inside a step is free as long as A and B agree.
#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
template <typename T, int D> struct XTile {
    static constexpr int SC = 64;                      // tokens per chunk
    static constexpr int RB = SC * (int)sizeof(T);     // bytes per row
    static constexpr int NCB = RB / 16;                // column blocks per row
    static constexpr int ROWS = 2 * D;
    static constexpr int BYTES = ROWS * RB;
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
template <typename T, int D> struct XStage {
    static constexpr int VE = 16 / (int)sizeof(T);
    static constexpr int FB = 2 * D / VE;              // feature blocks (K then V)
    static constexpr int TB = XTile<T, D>::SC / VE;    // token blocks
    static constexpr int NBLK = FB * TB;
    static constexpr int PER = (NBLK + NT - 1) / NT;
    u32x4 r[PER][VE];

    // tokens [t0, t0 + 64) of the frame; rows at or beyond tend are zero
    __device__ __forceinline__ void load(const T* kb, const T* vb, int64_t st, int t0, int tend,
                                         int tid) {
#pragma unroll
        for (int pi = 0; pi < PER; ++pi) {
            const int blk = tid + pi * NT;
            if (NBLK % NT == 0 || blk < NBLK) {
                const int fb = blk % FB, tb = blk / FB;
                const T* base = fb < D / VE ? kb + fb * VE : vb + (fb - D / VE) * VE;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const int tok = t0 + tb * VE + e;
                    r[pi][e] = tok < tend ? ld16(base + (int64_t)tok * st) : u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int pi = 0; pi < PER; ++pi) {
            const int blk = tid + pi * NT;
            if (NBLK % NT == 0 || blk < NBLK) {
                const int fb = blk % FB, tb = blk / FB;
#pragma unroll
                for (int f = 0; f < VE; ++f) {
                    u32x4 w;
                    if constexpr (VE == 8) {
                        // feature f of tokens 2c, 2c+1 -> dword c
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint32_t a = r[pi][2 * c][f >> 1], b = r[pi][2 * c + 1][f >> 1];
                            w[c] = (f & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
                        }
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c) w[c] = r[pi][c][f];
                    }
                    st16(lds + XTile<T, D>::addr(fb * VE + f, tb * VE), w);
                }
            }
        }
    }
};

// ----------------------------------------------------------------------------------------
// Kernel 1: per (b, h, f, split) partial products over the split's tokens
//   delta:    part = [ gamma beta c^2 K^T K | beta c K^T V ]   (two D x D fp32 blocks)
//   no delta: part = [ beta c K^T V ]
template <typename T, int D, bool DELTA>
__global__ __launch_bounds__(NT, 2) void gram_kernel(Launch L) {
    using MM = Mma<T>;
    using X = XTile<T, D>;
    constexpr int NOUT = DELTA ? 2 * D : D;
    constexpr int TI = D / 16, TJ = NOUT / 16;
    constexpr int WI = TI >= 2 ? 2 : 1;
    constexpr int WJ = (4 / WI) < TJ ? (4 / WI) : TJ;
    constexpr int MI = TI / WI, MJ = TJ / WJ;
    __shared__ __attribute__((aligned(16))) char lds[X::BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    int blk = blockIdx.x;
    const int p = blk % L.nsplit;
    blk /= L.nsplit;
    const int f = blk % L.F, bh = blk / L.F;
    const int b = bh / L.H, h = bh % L.H;
    const int64_t fo = (int64_t)b * L.sb + (int64_t)h * L.sh + (int64_t)f * L.S * L.st;
    const T* kb = (const T*)L.k + fo;
    const T* vb = (const T*)L.v + fo;
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
    stg.load(kb, vb, L.st, t0, t1, tid);
    for (int c0 = t0; c0 < t1; c0 += X::SC) {
        __syncthreads();  // readers of the previous chunk are done
        stg.store(lds, tid);
        __syncthreads();
        if (c0 + X::SC < t1) stg.load(kb, vb, L.st, c0 + X::SC, t1, tid);
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
    const float sG = gm * bt * L.c * L.c, sB = bt * L.c;
    float* out = L.part + ((int64_t)gi * L.nsplit + p) * (int64_t)(NOUT * D);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int i0 = (wi * MI + mi) * 16 + 4 * g;
#pragma unroll
        for (int mj = 0; mj < MJ; ++mj) {
            const int col = (wj * MJ + mj) * 16 + r16;
            const bool isG = DELTA && col < D;
            const float s = isG ? sG : sB;
            float* dst = out + (isG ? 0 : (DELTA ? D * D : 0)) + (isG ? col : col - (DELTA ? D : 0));
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[(i0 + q) * D] = acc[mi][mj][q] * s;
        }
    }
}

// ----------------------------------------------------------------------------------------
// Kernel 2: the frame-serial scan. One workgroup per (b, h, 16 value columns).
// Workgroup w lands on XCD w % 8 (round-robin dispatch); all column blocks of one head are
// given ids with the same residue so that they share one XCD's L2 for Ghat_f.
template <typename T, int D, bool DELTA>
__global__ __launch_bounds__(NT) void scan_kernel(Launch L) {
    constexpr int NC = 16;              // value columns per workgroup
    constexpr int NCB = D / NC;         // column blocks per head
    constexpr int TI = D / 16;
    constexpr int NW = TI < 4 ? TI : 4; // waves that hold state rows
    constexpr int IT = TI / NW;         // 16-row tiles per wave
    constexpr int GP = D + 4;           // padded Ghat row (floats)
    constexpr int GV = (D * D / 4 + NT - 1) / NT;  // float4 of Ghat per thread
    constexpr int NOUT = DELTA ? 2 * D : D;
    __shared__ __attribute__((aligned(16))) float Gs[DELTA ? D * GP : 4];
    __shared__ __attribute__((aligned(16))) float Ms[2][D * NC];

    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int bh = (slot / NCB) * 8 + xcd, cb = slot % NCB;
    if (bh >= L.B * L.H) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const bool active = wave < NW;
    const int col = cb * NC + r16;
    const int64_t pstride = (int64_t)NOUT * D;  // floats per partial
    const float* part_bh = L.part + (int64_t)bh * L.F * L.nsplit * pstride;
    T* mt_bh = (T*)L.mt + (int64_t)bh * L.F * D * D;

    float Mc[IT][4];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = ((active ? wave : 0) * IT + it) * 16 + 4 * g + q;
            Mc[it][q] = L.state_in ? L.state_in[((int64_t)bh * D + row) * D + col] : 0.f;
            if (active) Ms[0][row * NC + r16] = Mc[it][q];
        }

    // Next frame's Ghat (whole D x D, float4 per thread) and Bhat (this wave's C-layout
    // entries), summed over the S splits. The split loop is outermost so that all loads of one
    // split are independent and in flight together.
    f32x4 gpre[GV];
    float bpre[IT][4];
    auto load_next = [&](int f) {
        const float* src = part_bh + (int64_t)f * L.nsplit * pstride;
        for (int p = 0; p < L.nsplit; ++p) {
            const float* sp = src + p * pstride;
            if (DELTA) {
#pragma unroll
                for (int v = 0; v < GV; ++v) {
                    const int i4 = tid + v * NT;
                    const f32x4 x = i4 * 4 < D * D ? *(const f32x4*)(sp + 4 * i4) : f32x4{0.f, 0.f, 0.f, 0.f};
                    gpre[v] = p == 0 ? x : gpre[v] + x;
                }
            }
            if (active) {
                const float* bp = sp + (DELTA ? D * D : 0);
#pragma unroll
                for (int it = 0; it < IT; ++it)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float x = bp[((wave * IT + it) * 16 + 4 * g + q) * D + col];
                        bpre[it][q] = p == 0 ? x : bpre[it][q] + x;
                    }
            }
        }
    };
    load_next(0);

    int cur = 0;
    for (int f = 0; f < L.F; ++f) {
        if (DELTA) {
#pragma unroll
            for (int v = 0; v < GV; ++v) {
                const int i4 = tid + v * NT;
                if (i4 * 4 < D * D) {
                    const int row = (4 * i4) / D, c4 = (4 * i4) % D;
                    *(f32x4*)&Gs[row * GP + c4] = gpre[v];
                }
            }
        }
        float Bc[IT][4];
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int q = 0; q < 4; ++q) Bc[it][q] = bpre[it][q];
        __syncthreads();
        if (f + 1 < L.F) load_next(f + 1);
        if (active) {
            f32x4 acc[IT];
#pragma unroll
            for (int it = 0; it < IT; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (DELTA) {
#pragma unroll 8
                for (int ks = 0; ks < D / 4; ++ks) {
                    const float bm = Ms[cur][(4 * ks + g) * NC + r16];
#pragma unroll
                    for (int it = 0; it < IT; ++it) {
                        const float ag = Gs[((wave * IT + it) * 16 + r16) * GP + 4 * ks + g];
                        acc[it] = Mma<float>::run(ag, bm, acc[it]);
                    }
                }
            }
            const float gm = L.gamma[bh * L.F + f];
            T* mt = mt_bh + ((int64_t)f * D + col) * D;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int row0 = (wave * IT + it) * 16 + 4 * g;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    Mc[it][q] = gm * Mc[it][q] - acc[it][q] + Bc[it][q];
                    Ms[cur ^ 1][(row0 + q) * NC + r16] = Mc[it][q];
                }
                store4(mt + row0, Mc[it][0], Mc[it][1], Mc[it][2], Mc[it][3]);
            }
        }
        cur ^= 1;
        __syncthreads();
    }

    if (active && L.state_out) {
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = (wave * IT + it) * 16 + 4 * g + q;
                L.state_out[((int64_t)bh * D + row) * D + col] = Mc[it][q];
            }
    }
}

// ----------------------------------------------------------------------------------------
// Kernel 3: O_f = Q_f M_f, computed as O^T = M^T Q^T so that each lane ends up with a run of
// consecutive output columns of one token (16-byte stores). The A operand rows (output columns
// j) of 16x16 tile jt are permuted: with bf16 and D >= 32, tiles 2p and 2p+1 cover columns
// 32p .. 32p+31 such that lane (r, g) receives j = 32p + 8g + 0..7 across the pair.
template <typename T, int D> __device__ __forceinline__ int out_col(int jt, int m) {
    if constexpr (sizeof(T) == 2 && D >= 32)
        return 32 * (jt >> 1) + 8 * (m >> 2) + 4 * (jt & 1) + (m & 3);
    else
        return 16 * jt + m;
}

template <typename T, int D>
__global__ __launch_bounds__(NT, 2) void output_kernel(Launch L) {
    using MM = Mma<T>;
    constexpr int TJ = D / 16, KSN = (D + MM::KS - 1) / MM::KS;  // contraction padded to KS
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    int blk = blockIdx.x;
    const int ch = blk % L.nchunk;
    blk /= L.nchunk;
    const int f = blk % L.F, bh = blk / L.F;
    const int b = bh / L.H, h = bh % L.H;
    const T* mt = (const T*)L.mt + ((int64_t)bh * L.F + f) * D * D;
    const T* qf = (const T*)L.q + (int64_t)b * L.sb + (int64_t)h * L.sh + (int64_t)f * L.S * L.st;
    T* of = (T*)L.o + (int64_t)b * L.ob + (int64_t)h * L.oh + (int64_t)f * L.S * L.ot;

    typename MM::frag am[TJ][KSN];
#pragma unroll
    for (int jt = 0; jt < TJ; ++jt)
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            am[jt][ks] = ks * MM::KS + g * MM::KL < D
                             ? ld_frag<T>(mt + out_col<T, D>(jt, r16) * D + ks * MM::KS + g * MM::KL)
                             : zero_frag<T>();

    const int s_beg = ch * L.chunk_tokens;
    const int s_end = min(L.S, s_beg + L.chunk_tokens);
    for (int s0 = s_beg + wave * 16; s0 < s_end; s0 += 4 * 16) {
        const int s = s0 + r16;
        const bool ok = s < s_end;
        typename MM::frag bq[KSN];
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            bq[ks] = ok && ks * MM::KS + g * MM::KL < D
                         ? ld_frag<T>(qf + (int64_t)s * L.st + ks * MM::KS + g * MM::KL)
                         : zero_frag<T>();
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
    }
}

// ----------------------------------------------------------------------------------------
// Kernel 4: one frame, partial sums over the split's tokens of U = K^T R, with
// R = V - (gamma c) K M (delta) or R = V (no delta). The prediction P = K M runs on MFMA with M
// (state_in) rounded to the I/O type. For bf16 data U is accumulated as K^T V + K^T (-gamma c P):
// V is an exact bf16 input and only the small prediction term is rounded to bf16. For fp32
// data R is formed in fp32. K and V of each 64-token chunk are staged transposed in LDS; the
// prediction's K rows are read directly.
// Token grouping inside a step of the U product: for bf16, a 32-token group is two 16-token
// tiles; lane group g holds tokens {4g..4g+3} of the first tile and {16+4g..16+4g+3} of the
// second (exactly the rows of the prediction's C fragments). For fp32, step q of a 16-token
// tile gives lane group g the token 4g + q.
template <typename T, int D, bool DELTA>
__global__ __launch_bounds__(NT) void step_partial_kernel(Launch L) {
    using MM = Mma<T>;
    using X = XTile<T, D>;
    constexpr int TJ = D / 16;
    constexpr int NWJ = TJ < 4 ? TJ : 4;      // waves with work
    constexpr int JW = TJ / NWJ;              // 16-column tiles per wave
    constexpr int KSN = (D + MM::KS - 1) / MM::KS;  // contraction over D, padded to KS
    constexpr int RT = sizeof(T) == 2 ? 2 : 1; // 16-token tiles per U step group
    constexpr int TG = 16 * RT;               // tokens per group
    __shared__ __attribute__((aligned(16))) char lds[X::BYTES];

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

    // B operand of the prediction: M[i][j] for this wave's columns, all key rows
    typename MM::frag bm[JW][KSN];
    if (DELTA && active) {
        const float* M = L.state_in + (int64_t)bh * D * D;
#pragma unroll
        for (int jl = 0; jl < JW; ++jl) {
            const int j = (wave * JW + jl) * 16 + r16;
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) {
                if constexpr (sizeof(T) == 2) {
                    float m[8];
                    const bool in = ks * 32 + g * 8 < D;
#pragma unroll
                    for (int e = 0; e < 8; ++e) m[e] = in ? M[(ks * 32 + g * 8 + e) * D + j] : 0.f;
                    bm[jl][ks] = __builtin_bit_cast(
                        bf16x8, u32x4{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]),
                                      pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7])});
                } else {
                    bm[jl][ks] = M[(ks * 4 + g) * D + j];
                }
            }
        }
    }

    f32x4 acc[TJ][JW];
#pragma unroll
    for (int it = 0; it < TJ; ++it)
#pragma unroll
        for (int jl = 0; jl < JW; ++jl) acc[it][jl] = f32x4{0.f, 0.f, 0.f, 0.f};

    XStage<T, D> stg;
    stg.load(kb, vb, L.st, t0, t1, tid);
    for (int c0 = t0; c0 < t1; c0 += X::SC) {
        __syncthreads();
        stg.store(lds, tid);
        __syncthreads();
        if (c0 + X::SC < t1) stg.load(kb, vb, L.st, c0 + X::SC, t1, tid);
        if (!active) continue;
#pragma unroll 1
        for (int tg = 0; tg < X::SC; tg += TG) {
            // prediction P = K M (fp32, C layout): rows 4g+q of each 16-token tile, column
            // (wave tile jl, r16)
            f32x4 pr[RT][JW];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                for (int jl = 0; jl < JW; ++jl) pr[rt][jl] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (DELTA) {
                    const int s = c0 + tg + rt * 16 + r16;
                    const bool ok = s < t1;
#pragma unroll
                    for (int ks = 0; ks < KSN; ++ks) {
                        const typename MM::frag ak =
                            ok && ks * MM::KS + g * MM::KL < D
                                ? ld_frag<T>(kb + (int64_t)s * L.st + ks * MM::KS + g * MM::KL)
                                : zero_frag<T>();
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
                        const int krow = it * 16 + r16;
                        const u32x2 lo = *(const u32x2*)(lds + X::addr(krow, tg + 4 * g));
                        const u32x2 hi = *(const u32x2*)(lds + X::addr(krow, tg + 16 + 4 * g));
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
    }
    if (!active) return;
    float* out = L.part + ((int64_t)bh * L.nsplit + p) * D * D;
#pragma unroll
    for (int it = 0; it < TJ; ++it)
#pragma unroll
        for (int jl = 0; jl < JW; ++jl) {
            const int j = (wave * JW + jl) * 16 + r16;
#pragma unroll
            for (int q = 0; q < 4; ++q) out[(it * 16 + 4 * g + q) * D + j] = acc[it][jl][q];
        }
}

// Kernel 5: M' = gamma M + beta c sum_p U_p (fixed order over p); state_out on commit;
// transposed copy of M' in the I/O type for the output kernel. Thread: 4 key rows x 1 column.
template <typename T, int D>
__global__ __launch_bounds__(NT) void step_reduce_kernel(Launch L) {
    constexpr int NQ = D * D / 4;
    constexpr int NB = (NQ + NT - 1) / NT;
    const int bh = blockIdx.x / NB;
    const int t = (blockIdx.x % NB) * NT + threadIdx.x;
    if (t >= NQ) return;
    const int j = t % D, i0 = (t / D) * 4;
    const float gm = L.gamma[bh], bc = L.beta[bh] * L.c;
    const float* part = L.part + (int64_t)bh * L.nsplit * D * D;
    float m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int idx = (i0 + q) * D + j;
        float u = 0.f;
        for (int p = 0; p < L.nsplit; ++p) u += part[(int64_t)p * D * D + idx];
        m[q] = gm * L.state_in[(int64_t)bh * D * D + idx] + bc * u;
    }
    if (L.state_out) {
#pragma unroll
        for (int q = 0; q < 4; ++q) L.state_out[(int64_t)bh * D * D + (i0 + q) * D + j] = m[q];
    }
    store4((T*)L.mt + ((int64_t)bh * D + j) * D + i0, m[0], m[1], m[2], m[3]);
}

// ----------------------------------------------------------------------------------------
// Optional stage events (tracing): event i is recorded after kernel i (event 0 before the first).
static inline void mark(const Launch& L, int i) {
    if (i < L.nev && L.ev[i]) (void)hipEventRecord(L.ev[i], L.stream);
}

template <typename T, int D, bool DELTA> static hipError_t fwd(const Launch& L) {
    const int BH = L.B * L.H;
    mark(L, 0);
    hipLaunchKernelGGL((gram_kernel<T, D, DELTA>), dim3(BH * L.F * L.nsplit), dim3(NT), 0,
                       L.stream, L);
    mark(L, 1);
    const int units = (BH + 7) / 8 * 8 * (D / 16);
    hipLaunchKernelGGL((scan_kernel<T, D, DELTA>), dim3(units), dim3(NT), 0, L.stream, L);
    mark(L, 2);
    hipLaunchKernelGGL((output_kernel<T, D>), dim3(BH * L.F * L.nchunk), dim3(NT), 0, L.stream, L);
    mark(L, 3);
    return hipGetLastError();
}

template <typename T, int D, bool DELTA> static hipError_t stp(const Launch& L) {
    const int BH = L.B * L.H;
    mark(L, 0);
    hipLaunchKernelGGL((step_partial_kernel<T, D, DELTA>), dim3(BH * L.nsplit), dim3(NT), 0,
                       L.stream, L);
    mark(L, 1);
    constexpr int NB = (D * D / 4 + NT - 1) / NT;
    hipLaunchKernelGGL((step_reduce_kernel<T, D>), dim3(BH * NB), dim3(NT), 0, L.stream, L);
    mark(L, 2);
    Launch L1 = L;
    L1.F = 1;
    hipLaunchKernelGGL((output_kernel<T, D>), dim3(BH * L.nchunk), dim3(NT), 0, L.stream, L1);
    mark(L, 3);
    return hipGetLastError();
}


#define GDN_DISPATCH(FN, L)                                                                  \
    do {                                                                                     \
        const bool dl = (L).use_delta != 0;                                                  \
        if ((L).bf16) {                                                                      \
            switch ((L).D) {                                                                 \
            case 16: return dl ? FN<bf16, 16, true>(L) : FN<bf16, 16, false>(L);             \
            case 32: return dl ? FN<bf16, 32, true>(L) : FN<bf16, 32, false>(L);             \
            case 64: return dl ? FN<bf16, 64, true>(L) : FN<bf16, 64, false>(L);             \
            case 128: return dl ? FN<bf16, 128, true>(L) : FN<bf16, 128, false>(L);          \
            }                                                                                \
        } else {                                                                             \
            switch ((L).D) {                                                                 \
            case 16: return dl ? FN<float, 16, true>(L) : FN<float, 16, false>(L);           \
            case 32: return dl ? FN<float, 32, true>(L) : FN<float, 32, false>(L);           \
            case 64: return dl ? FN<float, 64, true>(L) : FN<float, 64, false>(L);           \
            case 128: return dl ? FN<float, 128, true>(L) : FN<float, 128, false>(L);        \
            }                                                                                \
        }                                                                                    \
        return hipErrorInvalidValue;                                                         \
    } while (0)

hipError_t launch_forward(const Launch& L) { GDN_DISPATCH(fwd, L); }
hipError_t launch_step(const Launch& L) { GDN_DISPATCH(stp, L); }

}  // namespace gdn
