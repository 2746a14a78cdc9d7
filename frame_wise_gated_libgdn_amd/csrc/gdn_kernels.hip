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
//                       (gates and key scale applied in the epilogue); combine_kernel sums
//                       S-split partials when a frame was split.
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
// partials that combine_kernel sums.
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

// Sum of the S-split partials of each (b, h, f) into the final per-frame record (only when the
// products kernel ran with more than one split). Fixed order over the splits.
template <int D, bool DELTA>
__global__ __launch_bounds__(NT) void combine_kernel(Launch L) {
    constexpr int NOUT = DELTA ? 2 * D : D;
    constexpr int NV = NOUT * D / 4;             // float4 per frame
    constexpr int NB = (NV + NT - 1) / NT;
    const int gi = blockIdx.x / NB;
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
// Kernel 2: the frame-serial scan M_f = gamma_f M - Ghat_f M + Bhat_f, for 16 value columns of
// one head per workgroup (columns of M evolve independently, so no workgroup waits on
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

template <typename T, int D, bool DELTA, int P>
__global__ __launch_bounds__(64 * (D / 16)) void scan_kernel(Launch L) {
    constexpr int NC = 16;              // value columns per workgroup
    constexpr int NCB = D / NC;         // column blocks per head
    constexpr int KSN = (D + 31) / 32;  // bf16 k steps (padded past D with zeros)
    constexpr int MR = D + 8;           // row length (bf16) of the transposed state planes
    constexpr int REC = canon_bytes<D, DELTA>();
    __shared__ __attribute__((aligned(16))) bf16 Ms[2][2][NC * MR];  // [buffer][hi, lo][col][k]
    // gamma_f of the current chunk of frames. Gammas come through LDS rather than scalar loads:
    // a scalar load in the frame loop would share the LDS wait counter and expose a full memory
    // round trip in every frame.
    __shared__ float Gam[kGammaSeg];

    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int bh = (slot / NCB) * 8 + xcd, cb = slot % NCB;
    if (bh >= L.B * L.H) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int col = cb * NC + r16;
    const int row0 = wave * 16 + 4 * g;  // this lane's 4 state rows
    const int F = L.F;
    const char* rec_bh = (const char*)L.canon + (int64_t)bh * F * REC;
    T* mt_bh = (T*)L.mt + (int64_t)bh * F * D * D;

    float Mc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        Mc[q] = L.state_in ? L.state_in[((int64_t)bh * D + row0 + q) * D + col] : 0.f;
    store_split4(&Ms[0][0][r16 * MR + row0], &Ms[0][1][r16 * MR + row0], f32x4{Mc[0], Mc[1], Mc[2], Mc[3]});

    // The ring has P + 1 slots: right after a frame's barrier the slot freed by the previous
    // frame is refilled with frame f + P, so the loads stream while this frame's MFMAs run.
    // The frame loop body is branch-free so that the compiler keeps the ring's loads in flight
    // across iterations: loads past the last frame re-read frame F-1, and a frame past the end
    // leaves M unchanged and rewrites M_{F-1} into its own slot.
    constexpr int R = P + 1;
    ScanSlot<D, DELTA> ring[R];
    auto issue = [&](ScanSlot<D, DELTA>& r, int f) {
        f = min(f, F - 1);
        const char* rec = rec_bh + (int64_t)f * REC;
        if constexpr (DELTA) {
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) {
                const bool in = ks * 32 + g * 8 < D;
                const char* fr = rec + ((wave * 2) * KSN + ks) * 1024 + lane * 16;
                r.a[0][ks] = in ? ld_frag<bf16>((const bf16*)fr) : zero_frag<bf16>();
                r.a[1][ks] = in ? ld_frag<bf16>((const bf16*)(fr + KSN * 1024)) : zero_frag<bf16>();
            }
        }
        r.bh = *(const f32x4*)(rec + rec_g_bytes<D, DELTA>() + ((cb * (D / 16) + wave) * 64 + lane) * 16);
    };
#pragma unroll
    for (int u = 0; u < P; ++u) issue(ring[u], u);

    static_assert(kGammaSeg % R == 0, "segments must hold whole ring cycles");
    const float* gam_bh = L.gamma + (int64_t)bh * F;
    int cur = 0;
    for (int sb = 0; sb < F; sb += kGammaSeg) {
        __syncthreads();  // the previous segment's gammas are no longer read
        for (int t = threadIdx.x; t < kGammaSeg; t += blockDim.x) Gam[t] = gam_bh[min(sb + t, F - 1)];
      for (int f0 = sb; f0 < sb + kGammaSeg && f0 < F; f0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int f = f0 + u;
            const bool valid = f < F;  // uniform
            {
                __syncthreads();  // planes of M_{f-1} complete; readers of the other buffer done
                issue(ring[(u + P) % R], f + P);  // the slot of frame f - 1
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
                const int fs = min(f, F - 1);
                store4(mt_bh + ((int64_t)fs * D + col) * D + row0, Mc[0], Mc[1], Mc[2], Mc[3]);
                cur ^= 1;
            }
        }
      }
    }

    if (L.state_out) {
#pragma unroll
        for (int q = 0; q < 4; ++q) L.state_out[((int64_t)bh * D + row0 + q) * D + col] = Mc[q];
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
constexpr int kScanAhead = 4;  // frames of scan operands kept in flight

// Optional stage events (tracing): event i is recorded after kernel i (event 0 before the first).
static inline void mark(const Launch& L, int i) {
    if (i < L.nev && L.ev[i]) (void)hipEventRecord(L.ev[i], L.stream);
}

template <typename T, int D, bool DELTA> static hipError_t fwd(const Launch& L) {
    const int BH = L.B * L.H;
    mark(L, 0);
    hipLaunchKernelGGL((gram_kernel<T, D, DELTA>), dim3(BH * L.F * L.nsplit), dim3(NT), 0,
                       L.stream, L);
    if (L.nsplit > 1) {
        constexpr int NB = ((DELTA ? 2 * D : D) * D / 4 + NT - 1) / NT;
        hipLaunchKernelGGL((combine_kernel<D, DELTA>), dim3(BH * L.F * NB), dim3(NT), 0, L.stream, L);
    }
    mark(L, 1);
    const int units = (BH + 7) / 8 * 8 * (D / 16);
    hipLaunchKernelGGL((scan_kernel<T, D, DELTA, kScanAhead>), dim3(units), dim3(64 * (D / 16)), 0,
                       L.stream, L);
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
