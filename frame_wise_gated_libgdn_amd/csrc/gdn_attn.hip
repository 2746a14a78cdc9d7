// Frame-causal softmax attention: the softmax blocks that the hybrid video models interleave
// with frame-wise GDN blocks (SANA-WM: gen-hub.ru article, architecture section; SANA-Streaming:
// jefxiong.cn digest). A query of frame f attends to every key of frames 0..f (its own frame in
// both directions), o = softmax(scale q k^T) v, per (b, h). Queries may be a later slice of the
// frames than the keys (a streaming step against the cache of all frames so far).
//
// One workgroup of 8 waves takes 256 queries of one (b, h); a wave owns 32 of them and walks the
// visible keys in tiles of 64. Products run on v_mfma_f32_32x32x16_bf16 (on gfx950 it sustains
// about 2.4 PFLOP/s, the 16x16x32 form about 1.45): lane l = 32 g + r holds A row r and B column
// r over the contraction slice [8 g, 8 g + 8), and C rows 8 i + 4 g + q (register 4 i + q) of
// column r.
//   * S^T = K Q^T per 32-key block: A = K rows from LDS, B = the wave's Q rows, held in
//     registers for the whole call; lane (r, g) ends up with the scores of query r for keys
//     8 i + 4 g + q of each 32-key block (16 per block);
//   * online softmax per query in that layout (exp2 of one fma with scale * log2 e folded in;
//     the two lanes of a query meet by one lane exchange; the running maximum moves only by
//     more than 8 in log2 units, so most tiles skip rescaling the accumulators);
//   * O^T += V^T P^T per 16-key step s: B = P^T is registers 8 (s mod 2) .. + 7 of score block
//     s / 2 as they stand, so k slot t of lane group g is key 16 s + 4 g + (t mod 4) + 8 (t / 4);
//     the A operand V^T is read in that same order with transposed LDS reads (ds_read_tr16_b64,
//     two per fragment).
// K/V tiles go from global memory straight into LDS (gfx950's 16-byte global_load_lds), double
// buffered (two arrays, the tile loop unrolled by two, so that the compiler keeps the next tile's
// loads in flight across this tile's LDS reads), and no registers hold the next tile: the
// tile lands unpadded, one 1 KB stretch per instruction, and bank conflicts are avoided by the
// choice of source chunk per lane (an XOR swizzle of each row's 16-byte chunks). Key tiles that
// every query of the workgroup sees completely skip the mask; the others mask per element.
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kKT = 64;        // keys per tile
constexpr int kQW = 32;        // queries per wave
// waves per workgroup (one workgroup per CU, two waves per SIMD). They share each K/V tile, so
// 8 halve the tile traffic per query against 4; measured on the 880 x 81 sequence and on 720p
// streaming frames (224 workgroups) 8 were faster throughout (43.3 against 47.0 ms, 100.5 against
// 117.1 ms at frame 960)
constexpr int kNW = 8;
constexpr int kQB = kNW * kQW; // queries per workgroup

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(bf16)lo, (bf16)hi});
}

// XOR swizzle of the 16-byte chunks of a key row in an unpadded [key][dim] LDS tile with CH
// chunks per row: chunk c of row r is stored at chunk c ^ swz(r). The masks (XOR combinations of
// the bits b_i of r) keep both reads of the tile free of bank conflicts whether the LDS serves
// 64 banks per clock (16 lanes of a 16-byte access, 32 lanes of an 8-byte one) or 32 (8 and 16
// lanes): K fragment reads (rows 32 kb + 0..31, one chunk per 32 lanes) and V^T reads (per
// 16-lane group 4 rows and 2 chunks; the four groups of a wave at rows +0 / +4, dims +0 / +16;
// 8 bytes per lane).
template <int CH> __device__ __forceinline__ int swz(int r) {
    const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
    if constexpr (CH == 16) return b0 | b1 << 1 | (b0 ^ b2) << 2 | (b1 ^ b3) << 3;
    else return b1 | (b0 ^ b2) << 1 | (b0 ^ b1 ^ b3) << 2;
}

// Slice of the A operand V^T for one 32-dim block: lane l = 32 g + r receives
// X[krow + 4 g + j][c0 + r], j = 0..3, from a swizzled [key][dim] LDS tile. ds_read_tr16_b64
// gives destination lane i of each 16-lane group element i mod 4 of the four b16 values at the
// address of source lane 4 j + i / 4; so source lane s of group q = l / 16 points at row
// krow + 4 (q / 2) + s / 4, dims c0 + 16 (q mod 2) + 4 (s mod 4) .. + 3.
template <int D> __device__ __forceinline__ u32x2 read_vt(const bf16* X, int krow, int c0, int lane) {
    constexpr int CH = D / 8;
    const int q = lane >> 4, s = lane & 15;
    const int row = krow + 4 * (q >> 1) + (s >> 2);
    const int col = c0 + 16 * (q & 1) + 4 * (s & 3);
    const bf16* a = X + row * D + (((col >> 3) ^ swz<CH>(row)) * 8) + (col & 7);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a));
}

// number of keys visible to query row t (keys of frames 0 .. its frame)
__device__ __forceinline__ int visible(const AttnLaunch& L, int t) {
    const int64_t n = (int64_t)(L.q_frame0 + t / L.S + 1) * L.S;
    return n < L.Tk ? (int)n : L.Tk;
}

template <int D>
__global__ __launch_bounds__(64 * kNW, 1) void attn_kernel(AttnLaunch L) {
    constexpr int KS = D / 16;            // 16-long k steps over the head dim (scores)
    constexpr int DB = D / 32;            // 32-dim blocks of O
    constexpr int KB = kKT / 32;          // 32-key blocks per tile
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int SLOTS = kKT * CH;       // 16-byte slots of one operand tile
    constexpr int INSTR = 2 * SLOTS / (64 * kNW);   // load instructions per wave per tile (K and V)
    static_assert(SLOTS % 64 == 0 && (2 * SLOTS) % (64 * kNW) == 0, "whole instructions per wave");
    // the two buffers are separate arrays and the tile loop is unrolled by two, so that every
    // LDS read names its buffer statically: the compiler can then tell the reads of one buffer
    // from the direct-to-LDS loads into the other, and does not wait for those before them
    __shared__ __attribute__((aligned(16))) bf16 tile0[2][kKT * D];   // [K, V] of even tiles
    __shared__ __attribute__((aligned(16))) bf16 tile1[2][kKT * D];   // [K, V] of odd tiles

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, g = lane >> 5;
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

    // the wave's Q rows as B operands (lane (r, g): query qw0 + r, dims 16 ks + 8 g .. + 7);
    // rows past Tq repeat the last row (never stored)
    bf16x8 qf[KS];
    int nlim;
    {
        const bf16* qbase = (const bf16*)L.q + (int64_t)b * L.qsb + (int64_t)h * L.qsh;
        const int t = min(qw0 + r, L.Tq - 1);
        nlim = visible(L, t);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qbase + (int64_t)t * L.qst + 16 * ks + 8 * g));
    }
    // keys every query of the workgroup sees, and the keys any of them sees
    const int kfull = visible(L, qb * kQB);
    const int kmax = visible(L, min(qb * kQB + kQB, L.Tq) - 1);

    const bf16* kbase = (const bf16*)L.k + (int64_t)b * L.ksb + (int64_t)h * L.ksh;
    const bf16* vbase = (const bf16*)L.v + (int64_t)b * L.ksb + (int64_t)h * L.ksh;
    // tile of keys k0 .. k0 + kKT - 1 into buffer buf: instruction ins of the workgroup fills
    // slots 64 ins .. 64 ins + 63 of the K | V pair; rows past Tk are loaded clamped (finite
    // values: their scores are masked and their weights are zero)
    auto issue = [&](int k0, bf16 (&tl)[2][kKT * D]) {
#pragma unroll
        for (int i = 0; i < INSTR; ++i) {
            const int ins = wave * INSTR + i;
            const bool isv = ins * 64 >= SLOTS;              // the same for the whole wave
            const int u = ins * 64 + lane - (isv ? SLOTS : 0);
            const int row = u / CH, c = (u % CH) ^ swz<CH>(row);
            const bf16* src = (isv ? vbase : kbase) + (int64_t)min(k0 + row, L.Tk - 1) * L.kst + c * 8;
            bf16* dst = &tl[isv ? 1 : 0][(ins * 64 - (isv ? SLOTS : 0)) * 8];
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };

    const float c2 = L.scale * 1.4426950408889634f;   // scores in log2 units
    float m = -__builtin_inff(), l = 0.f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;

    // one tile of keys k0 .. k0 + kKT - 1, held in cur; the next tile goes into nxt
    auto step = [&](int k0, bf16 (&cur)[2][kKT * D], bf16 (&nxt)[2][kKT * D]) __attribute__((always_inline)) {
        // this wave's loads of tile k0 are done; after the barrier every wave's are, and every
        // wave is done reading the other buffer (the previous tile), which the next tile fills
        __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (k0 + kKT < kmax) issue(k0 + kKT, nxt);
        const bf16* kt = cur[0];
        const bf16* vt = cur[1];

        // S^T = K Q^T for 64 keys x 32 queries
        f32x16 sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int row = 32 * kb + r;
                const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(kt + row * D + (((2 * ks + g) ^ swz<CH>(row)) * 8)));
                sacc[kb] = mfma32(a, qf[ks], sacc[kb]);
            }
        if (k0 + kKT > kfull) {   // a tile some query does not see completely
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (k0 + 32 * kb + 8 * (j >> 2) + 4 * g + (j & 3) >= nlim) sacc[kb][j] = -__builtin_inff();
        }
        // tile maximum on the raw scores (the scale is positive), across the query's two lanes
        float tmax = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) tmax = __builtin_fmaxf(tmax, sacc[kb][j]);
        tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
        // the running maximum (log2 units) moves only when the tile's exceeds it by more than 8,
        // so weights stay below 2^8 and most tiles skip the rescale; exact, since the final
        // normalisation uses the same maximum. Finite after the first tile (key 0 is visible to
        // every query).
        const float cand = tmax * c2;
        const bool move = cand > m + 8.f;
        if (__any(move)) {
            const float mnew = move ? cand : m;
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m = mnew;
        }
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][j], c2, -m));
                sacc[kb][j] = p;
                sum += p;
            }
        l += sum;
        // O^T += V^T P^T, four 16-key steps
#pragma unroll
        for (int s = 0; s < kKT / 16; ++s) {
            const int o = 8 * (s & 1);
            const f32x16& x = sacc[s >> 1];
            const bf16x8 pb = __builtin_bit_cast(
                bf16x8, u32x4{pack2(x[o], x[o + 1]), pack2(x[o + 2], x[o + 3]), pack2(x[o + 4], x[o + 5]),
                              pack2(x[o + 6], x[o + 7])});
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x2 v0 = read_vt<D>(vt, 16 * s, 32 * db, lane);
                const u32x2 v1 = read_vt<D>(vt, 16 * s + 8, 32 * db, lane);
                oacc[db] = mfma32(__builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]}), pb, oacc[db]);
            }
        }
    };
    issue(0, tile0);
    for (int k0 = 0; k0 < kmax; k0 += 2 * kKT) {
        step(k0, tile0, tile1);
        if (k0 + kKT < kmax) step(k0 + kKT, tile1, tile0);
    }

    // normalise and store: lane (r, g) holds O[query qw0 + r][dims 32 db + 8 i + 4 g .. + 3] in
    // registers 4 i .. 4 i + 3 of block db
    bf16* obase = (bf16*)L.o + (int64_t)b * L.osb + (int64_t)h * L.osh;
    const float inv = 1.f / (l + __shfl_xor(l, 32));
    const int t = qw0 + r;
    if (t < L.Tq) {
        bf16* orow = obase + (int64_t)t * L.ost;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * i;
                *(u32x2*)(orow + 32 * db + 8 * i + 4 * g) =
                    u32x2{pack2(oacc[db][j] * inv, oacc[db][j + 1] * inv), pack2(oacc[db][j + 2] * inv, oacc[db][j + 3] * inv)};
            }
    }
}

}  // namespace

bool attn_supported(int D) { return D == 64 || D == 128; }

template <int D> hipError_t launch_d(const AttnLaunch& L, hipStream_t s) {
    const int64_t items = (int64_t)L.B * L.H * ((L.Tq + kQB - 1) / kQB);
    const int64_t blocks = (items + 7) / 8 * 8;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<D>), dim3((unsigned)blocks), dim3(64 * kNW), 0, s, L);
    return hipGetLastError();
}

hipError_t attn_launch(const AttnLaunch& L, hipStream_t s) {
    if (L.D == 128) return launch_d<128>(L, s);
    if (L.D == 64) return launch_d<64>(L, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
