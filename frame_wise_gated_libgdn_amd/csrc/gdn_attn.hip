// Frame-causal softmax attention: the softmax blocks that the hybrid video models interleave
// with frame-wise GDN blocks (SANA-WM: gen-hub.ru article, architecture section; SANA-Streaming:
// jefxiong.cn digest). A query of frame f attends to every key of frames 0..f (its own frame in
// both directions), o = softmax(scale q k^T) v, per (b, h). Queries may be a later slice of the
// frames than the keys (a streaming step against the cache of all frames so far).
//
// One workgroup of 4 waves takes 128 queries of one (b, h); a wave owns 32 of them (two 16-query
// MFMA tiles) and walks the visible keys in tiles of 64:
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = the wave's Q rows,
//     held in registers for the whole call), so lane (r, g) holds the scores of query r for
//     keys 4 g .. 4 g + 3 of each 16-key block;
//   * online softmax per query in that layout (exp2 of one fma with scale * log2 e folded in;
//     row maxima across the four lanes of a query by lane exchange; the running maximum moves
//     only by more than 8 in log2 units, so most tiles skip rescaling the accumulators);
//   * O^T += V^T P^T: the score tiles are the B operand as they stand, taking the k order of a
//     32-key step as keys {4 g + j} then {16 + 4 g + j} from two 16-key tiles; the A operand V^T
//     is read in that same order with transposed LDS reads (ds_read_tr16_b64).
// K/V tiles go from global memory straight into LDS (gfx950's 16-byte global_load_lds), double
// buffered, so the next tile is in flight while this one is used and no registers hold it: the
// tile lands unpadded, one 1 KB stretch per instruction, and bank conflicts are avoided by the
// choice of source chunk per lane (an XOR swizzle of each row's 16-byte chunks). Key tiles that
// every query of the workgroup sees completely skip the mask; the others mask per element.
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kAttnThreads = 256;
constexpr int kKT = 64;        // keys per tile

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(bf16)lo, (bf16)hi});
}

// XOR swizzle of the 16-byte chunks of a key row in an unpadded [key][dim] LDS tile with CH
// chunks per row: chunk c of row r is stored at chunk c ^ swz(r). The masks (functions of the
// bits b_i of r) keep both reads of the tile free of bank conflicts whether the LDS serves 64
// banks per clock (16 lanes of a 16-byte access, 32 lanes of an 8-byte one) or 32 (8 and 16
// lanes): K fragment reads (rows 16 kt + 0..15, one chunk) and V^T reads (rows k0 + 4 g + 0..3,
// chunks 2d and 2d + 1, 8 bytes per lane).
template <int CH> __device__ __forceinline__ int swz(int r) {
    const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
    if constexpr (CH == 16) return (b3 ^ b2) | b0 << 1 | b1 << 2 | b2 << 3;
    else return (b3 ^ b2) | b1 << 1 | (b0 ^ b2) << 2;
}

// lane (r, g) of each 16-lane group receives X[k0 + 4 g + j][c0 + r], j = 0..3, from a swizzled
// [key][dim] LDS tile (ds_read_tr16_b64: destination lane i takes element i mod 4 of the four
// b16 values at the address of source lane 4 j + i / 4, so source lane s points at row
// k0 + 4 g + s / 4, columns c0 + 4 (s mod 4) .. + 3: chunk c0 / 8 + (s mod 4) / 2, half s mod 2)
template <int D> __device__ __forceinline__ u32x2 read_tr(const bf16* X, int k0, int c0, int r, int g) {
    constexpr int CH = D / 8;
    const int row = k0 + 4 * g + (r >> 2);
    const int c = c0 / 8 + ((r & 3) >> 1);
    const bf16* a = X + row * D + ((c ^ swz<CH>(row)) * 8) + 4 * (r & 1);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a));
}

// number of keys visible to query row t (keys of frames 0 .. its frame)
__device__ __forceinline__ int visible(const AttnLaunch& L, int t) {
    const int64_t n = (int64_t)(L.q_frame0 + t / L.S + 1) * L.S;
    return n < L.Tk ? (int)n : L.Tk;
}

// QT 16-query tiles per wave: each K / V^T fragment read from LDS feeds QT MFMAs
template <int D, int QT>
__global__ __launch_bounds__(kAttnThreads, QT >= 4 ? 1 : 2) void attn_kernel(AttnLaunch L) {
    constexpr int kQW = 16 * QT;     // queries per wave
    constexpr int kQB = 4 * kQW;     // queries per workgroup
    constexpr int KSD = D / 32;           // k steps over the head dim
    constexpr int DT = D / 16;            // 16-dim tiles of O
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int NKT = kKT / 16;         // 16-key tiles per key tile
    constexpr int SLOTS = kKT * CH;       // 16-byte slots of one operand tile
    constexpr int INSTR = 2 * SLOTS / (64 * 4);   // load instructions per wave per tile (K and V)
    static_assert(SLOTS % 64 == 0 && (2 * SLOTS) % 256 == 0, "whole instructions per wave");
    __shared__ __attribute__((aligned(16))) bf16 tiles[2][2][kKT * D];   // [buffer][K, V]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    // XCD-aware order: workgroup i runs on XCD i mod 8; XCD x takes the contiguous stretch
    // [x n8, (x + 1) n8) of the (b h)-major, query-block-minor order, so that the workgroups
    // resident on one XCD are neighbouring query blocks of the same head and share its K/V tiles
    // through that XCD's L2 (the grid is padded to 8 n8 workgroups; the padding returns at once)
    const int nqb = (L.Tq + kQB - 1) / kQB;
    const int n8 = (L.B * L.H * nqb + 7) / 8;
    const int item = (int)(blockIdx.x % 8) * n8 + (int)(blockIdx.x / 8);
    if (item >= L.B * L.H * nqb) return;
    const int bh = item / nqb, qb = item % nqb;
    const int b = bh / L.H, h = bh % L.H;
    const int qw0 = qb * kQB + wave * kQW;    // first query of this wave

    // the wave's Q rows as B operands; rows past Tq repeat the last row (never stored)
    bf16x8 qf[QT][KSD];
    int nlim[QT];
    {
        const bf16* qbase = (const bf16*)L.q + (int64_t)b * L.qsb + (int64_t)h * L.qsh;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int t = min(qw0 + 16 * qt + r, L.Tq - 1);
            nlim[qt] = visible(L, t);
#pragma unroll
            for (int k = 0; k < KSD; ++k)
                qf[qt][k] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qbase + (int64_t)t * L.qst + 32 * k + 8 * g));
        }
    }
    // keys every query of the workgroup sees, and the keys any of them sees
    const int kfull = visible(L, qb * kQB);
    const int kmax = visible(L, min(qb * kQB + kQB, L.Tq) - 1);

    const bf16* kbase = (const bf16*)L.k + (int64_t)b * L.ksb + (int64_t)h * L.ksh;
    const bf16* vbase = (const bf16*)L.v + (int64_t)b * L.ksb + (int64_t)h * L.ksh;
    // tile of keys k0 .. k0 + kKT - 1 into buffer buf: instruction ins of the workgroup fills
    // slots 64 ins .. 64 ins + 63 of the K | V pair; rows past Tk are loaded clamped (finite
    // values: their scores are masked and their weights are zero)
    auto issue = [&](int k0, int buf) {
#pragma unroll
        for (int i = 0; i < INSTR; ++i) {
            const int ins = wave * INSTR + i;
            const bool isv = ins * 64 >= SLOTS;              // the same for the whole wave
            const int u = ins * 64 + lane - (isv ? SLOTS : 0);
            const int row = u / CH, c = (u % CH) ^ swz<CH>(row);
            const bf16* src = (isv ? vbase : kbase) + (int64_t)min(k0 + row, L.Tk - 1) * L.kst + c * 8;
            bf16* dst = &tiles[buf][isv ? 1 : 0][(ins * 64 - (isv ? SLOTS : 0)) * 8];
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };

    const float c2 = L.scale * 1.4426950408889634f;   // scores in log2 units
    float m[QT], l[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        m[qt] = -__builtin_inff();
        l[qt] = 0.f;
    }
    f32x4 oacc[DT][QT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    int buf = 0;
    for (int k0 = 0; k0 < kmax; k0 += kKT, buf ^= 1) {
        // this wave's loads of tile k0 are done; after the barrier every wave's are, and every
        // wave is done reading the other buffer (the previous tile), which the next tile fills
        __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (k0 + kKT < kmax) issue(k0 + kKT, buf ^ 1);
        const bf16* ks = tiles[buf][0];
        const bf16* vs = tiles[buf][1];

        // S^T = K Q^T for 64 keys x 32 queries
        f32x4 sacc[NKT][QT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) sacc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KSD; ++k)
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const int row = 16 * kt + r;
                const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(ks + row * D + (((4 * k + g) ^ swz<CH>(row)) * 8)));
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) sacc[kt][qt] = mfma(a, qf[qt][k], sacc[kt][qt]);
            }
        if (k0 + kKT > kfull) {   // a tile some query does not see completely
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (k0 + 16 * kt + 4 * g + q >= nlim[qt]) sacc[kt][qt][q] = -__builtin_inff();
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            // tile maximum on the raw scores (the scale is positive), across the query's 4 lanes
            float tmax = -__builtin_inff();
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int q = 0; q < 4; ++q) tmax = __builtin_fmaxf(tmax, sacc[kt][qt][q]);
            tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
            // the running maximum (log2 units) moves only when the tile's exceeds it by more than
            // 8, so weights stay below 2^8 and most tiles skip the rescale; exact, since the
            // final normalisation uses the same maximum. Finite after the first tile (key 0 is
            // visible to every query).
            const float cand = tmax * c2;
            const bool move = cand > m[qt] + 8.f;
            if (__any(move)) {
                const float mnew = move ? cand : m[qt];
                const float alpha = __builtin_amdgcn_exp2f(m[qt] - mnew);
                l[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
                m[qt] = mnew;
            }
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][qt][q], c2, -m[qt]));
                    sacc[kt][qt][q] = p;
                    sum += p;
                }
            l[qt] += sum;
        }
        // O^T += V^T P^T, two 32-key steps
#pragma unroll
        for (int ks2 = 0; ks2 < NKT / 2; ++ks2) {
            bf16x8 pb[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const f32x4 x = sacc[2 * ks2][qt], y = sacc[2 * ks2 + 1][qt];
                pb[qt] = __builtin_bit_cast(bf16x8, u32x4{pack2(x[0], x[1]), pack2(x[2], x[3]),
                                                          pack2(y[0], y[1]), pack2(y[2], y[3])});
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x2 v0 = read_tr<D>(vs, 32 * ks2, 16 * dt, r, g);
                const u32x2 v1 = read_tr<D>(vs, 32 * ks2 + 16, 16 * dt, r, g);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = mfma(a, pb[qt], oacc[dt][qt]);
            }
        }
    }

    // normalise and store: lane (r, g) holds O[query 16 qt + r][dims 16 dt + 4 g .. + 3]
    bf16* obase = (bf16*)L.o + (int64_t)b * L.osb + (int64_t)h * L.osh;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        float lt_ = l[qt];
        lt_ += __shfl_xor(lt_, 16);
        lt_ += __shfl_xor(lt_, 32);
        const float inv = 1.f / lt_;
        const int t = qw0 + 16 * qt + r;
        if (t < L.Tq) {
            bf16* orow = obase + (int64_t)t * L.ost;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 x = oacc[dt][qt] * inv;
                *(u32x2*)(orow + 16 * dt + 4 * g) = u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])};
            }
        }
    }
}

}  // namespace

bool attn_supported(int D) { return D == 64 || D == 128; }

template <int D, int QT> hipError_t launch_qt(const AttnLaunch& L, hipStream_t s) {
    constexpr int kQB = 4 * 16 * QT;
    const int64_t items = (int64_t)L.B * L.H * ((L.Tq + kQB - 1) / kQB);
    const int64_t blocks = (items + 7) / 8 * 8;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<D, QT>), dim3((unsigned)blocks), dim3(kAttnThreads), 0, s, L);
    return hipGetLastError();
}

constexpr int kAttnQT = 2;   // 16-query tiles per wave (4: one wave per SIMD, measured slower)

hipError_t attn_launch(const AttnLaunch& L, hipStream_t s) {
    if (L.D == 128) return launch_qt<128, kAttnQT>(L, s);
    if (L.D == 64) return launch_qt<64, kAttnQT>(L, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
