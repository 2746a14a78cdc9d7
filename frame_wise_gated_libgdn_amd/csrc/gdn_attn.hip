// Frame-causal softmax attention: the softmax blocks that the hybrid video models interleave
// with frame-wise GDN blocks (SANA-WM: gen-hub.ru article, architecture section; SANA-Streaming:
// jefxiong.cn digest). A query of frame f attends to every key of frames 0..f (its own frame in
// both directions), o = softmax(scale q k^T) v, per (b, h). Queries may be a later slice of the
// frames than the keys (a streaming step against the cache of all frames so far).
//
// One workgroup of 8 or 12 waves takes 256 or 384 queries of one (b, h); a wave owns 32 of
// them and walks the visible keys in tiles of 64. Products run on v_mfma_f32_32x32x16_bf16 (on
// gfx950 it sustains about 2.4 PFLOP/s, the 16x16x32 form about 1.45): lane l = 32 g + r holds
// A row r and B column r over the contraction slice [8 g, 8 g + 8), and C rows 8 i + 4 g + q
// (register 4 i + q) of column r.
//   * S^T = K Q^T per 32-key block: A = K rows from LDS, B = the wave's Q rows, held in
//     registers for the whole call (in LDS with 12 waves); lane (r, g) ends up with the scores
//     of query r for keys 8 i + 4 g + q of each 32-key block (16 per block);
//   * online softmax per query in that layout (exp2 of one fma with scale * log2 e folded in;
//     the two lanes of a query meet by one lane exchange; the running maximum moves only by
//     more than 8 in log2 units, so most tiles skip rescaling the accumulators; the normaliser
//     is the fp32 sum of the bf16 weights the products use);
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
// Instruction scheduling is left to the compiler: forcing one wave's softmax to interleave
// with its next tile's products measured slower (the two waves of a SIMD overlap each other's
// products and vector work; one wave's vector work does not run in its own products' shadow).
#include <stdint.h>

#include <algorithm>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kKT = 64;        // keys per tile
constexpr int kQW = 32;        // queries per wave
// Waves per workgroup (one workgroup per CU): 8 (two per SIMD, Q in registers) or 12 (three
// per SIMD, Q in LDS, so that registers fit 168 per lane). They share each K/V tile, so more
// waves stream fewer tiles per query. Measured on the 880 x 81 sequence and on 720p streaming
// frames: 8 waves beat 4 throughout (43.3 against 47.0 ms, 100.5 against 117.1 ms at frame
// 960); 12 beat 8 on the whole sequence (40.3 against 40.9-43.2 ms) but lose on one frame,
// whose 10 query blocks per head of 384 leave CUs idle (117 against 95-98 ms). The launcher
// takes 12 when the grid has at least two workgroups per CU.
constexpr int kQBMax = 12 * kQW;   // queries per workgroup at most

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
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

// byte offset of read_vt's address for rows krow = 8 h (mod 16) and dims c0 = 32 db, within a
// tile: the 16-key step s adds s 16 D 2 bytes (row bits 4 and up leave the swizzle unchanged)
template <int D> __device__ __forceinline__ uint32_t vt_off(int h, int db, int lane) {
    constexpr int CH = D / 8;
    const int q = lane >> 4, s = lane & 15;
    const int row = 8 * h + 4 * (q >> 1) + (s >> 2);
    const int col = 32 * db + 16 * (q & 1) + 4 * (s & 3);
    return (uint32_t)((row * D + (((col >> 3) ^ swz<CH>(row)) * 8) + (col & 7)) * 2);
}

// number of keys visible to query row t (keys of frames 0 .. its frame)
__device__ __forceinline__ int visible(const AttnLaunch& L, int t) {
    const int64_t n = (int64_t)(L.q_frame0 + t / L.S + 1) * L.S;
    return n < L.Tk ? (int)n : L.Tk;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_kernel(AttnLaunch L) {
    constexpr int QB = NW * kQW;          // queries per workgroup
    constexpr bool QLDS = NW > 8;         // Q fragments from LDS instead of registers
    constexpr int KS = D / 16;            // 16-long k steps over the head dim (scores)
    constexpr int DB = D / 32;            // 32-dim blocks of O
    constexpr int KB = kKT / 32;          // 32-key blocks per tile
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int SLOTS = kKT * CH;       // 16-byte slots of one operand tile
    constexpr int NI = 2 * SLOTS / 64;                 // load instructions per tile (K and V)
    constexpr int INSTR = (NI + NW - 1) / NW;          // at most, per wave (wave w: w, w + NW, ..)
    static_assert(SLOTS % 64 == 0, "whole instructions");
    // the two buffers are separate arrays and the tile loop is unrolled by two, so that every
    // LDS read names its buffer statically: the compiler can then tell the reads of one buffer
    // from the direct-to-LDS loads into the other, and does not wait for those before them.
    // Their larger alignment places them first in LDS, below 64 KB, so that every V^T read of
    // either buffer takes its buffer, half and 16-key step in the instruction's immediate offset
    // (with the Q rows first, each tile added its 96 KB base to eight lane offsets)
    __shared__ __attribute__((aligned(1024))) bf16 tile0[2][kKT * D];   // [K, V] of even tiles
    __shared__ __attribute__((aligned(1024))) bf16 tile1[2][kKT * D];   // [K, V] of odd tiles
    // with QLDS, each wave's Q rows, [query][dim] swizzled as the K tiles
    __shared__ __attribute__((aligned(16))) bf16 qs[QLDS ? NW : 1][QLDS ? kQW * D : 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, g = lane >> 5;
    // XCD-aware order: workgroup i runs on XCD i mod 8; XCD x takes the contiguous stretch
    // [x n8, (x + 1) n8) of the (b h)-major, query-block-minor order, so that the workgroups
    // resident on one XCD are neighbouring query blocks of the same head and share its K/V tiles
    // through that XCD's L2 (the grid is padded to 8 n8 workgroups; the padding returns at once).
    // Within a head the query blocks go last to first: later blocks see more keys, and starting
    // the longest first keeps the end of the launch short (a list-scheduling model of the
    // 880 x 81 sequence, 32 CUs per XCD: 0.2% over the even split of the work, against 4.2%
    // first to last)
    // With key splits the order is (b h, split)-major: the resident workgroups of an XCD are
    // then neighbouring query blocks of one split, which read the same key tiles.
    const int nqb = (L.Tq + QB - 1) / QB;
    const int NS = L.nsplit;
    const int nitems = L.B * L.H * NS * nqb;
    const int n8 = (nitems + 7) / 8;
    const int item = (int)(blockIdx.x % 8) * n8 + (int)(blockIdx.x / 8);
    if (item >= nitems) return;
    const int bhs = item / nqb, qb = nqb - 1 - item % nqb;
    const int bh = bhs / NS, sp = bhs % NS;
    const int b = bh / L.H, h = bh % L.H;
    const int qw0 = qb * QB + wave * kQW;    // first query of this wave

    // the wave's Q rows as B operands (lane (r, g): query qw0 + r, dims 16 ks + 8 g .. + 7);
    // rows past Tq repeat the last row (never stored)
    const bf16* qw = qs[QLDS ? wave : 0];
    bf16x8 qf[QLDS ? 1 : KS];
    int nlim;
    {
        const bf16* qbase = (const bf16*)L.q + (int64_t)b * L.qsb + (int64_t)h * L.qsh;
        const int t = min(qw0 + r, L.Tq - 1);
        nlim = visible(L, t);
        u32x4 x[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) x[ks] = *(const u32x4*)(qbase + (int64_t)t * L.qst + 16 * ks + 8 * g);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (QLDS) *(u32x4*)(qs[wave] + r * D + (((2 * ks + g) ^ swz<CH>(r)) * 8)) = x[ks];
            else qf[ks] = __builtin_bit_cast(bf16x8, x[ks]);
        }
    }
    // per-lane byte offsets of the V^T reads (read_vt) for the two halves of a 16-key step and
    // each 32-dim block
    uint32_t voff[2][DB];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < DB; ++db) voff[hh][db] = vt_off<D>(hh, db, lane);
    // keys every query of the workgroup sees, and the keys any of them sees; this split's
    // share of the latter, [kbeg, kend), in whole tiles (all of it without splits; with
    // splits, every query of the block sees every key: the queries form one frame)
    const int kfull = visible(L, qb * QB);
    const int kmax = visible(L, min(qb * QB + QB, L.Tq) - 1);
    const int ntile = (kmax + kKT - 1) / kKT;
    const int kbeg = (int)((int64_t)sp * ntile / NS) * kKT;
    const int kend = min((int)((int64_t)(sp + 1) * ntile / NS) * kKT, kmax);

    const bf16* kbase = (const bf16*)L.k + (int64_t)b * L.ksb + (int64_t)h * L.ksh;
    const bf16* vbase = (const bf16*)L.v + (int64_t)b * L.ksb + (int64_t)h * L.ksh;
    // tile of keys k0 .. k0 + kKT - 1 into buffer buf: instruction ins of the workgroup fills
    // slots 64 ins .. 64 ins + 63 of the K | V pair; rows past Tk are loaded clamped (finite
    // values: their scores are masked and their weights are zero). A uniform base per tile and
    // a 32-bit offset per lane (the host keeps a head's key rows below 2 GiB): each lane's row
    // and swizzled chunk offsets are the same for every tile and are computed once, so a load
    // costs one clamp and one add per tile (recomputing them cost about 30 vector instructions
    // per tile)
    const int kstb = (int)L.kst * 2;
    uint32_t roff[INSTR], coff[INSTR];
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
        const int ins = wave + NW * i;
        const bool isv = ins * 64 >= SLOTS;
        const int u = ins * 64 + lane - (isv ? SLOTS : 0);
        const int row = u / CH, c = (u % CH) ^ swz<CH>(row);
        roff[i] = (uint32_t)(row * kstb);
        coff[i] = (uint32_t)(c * 16);
    }
    auto issue = [&](int k0, bf16 (&tl)[2][kKT * D]) {
        const char* ksrc = (const char*)kbase + (int64_t)k0 * kstb;
        const char* vsrc = (const char*)vbase + (int64_t)k0 * kstb;
        // the last row's offset, or the tile's last (at most 63 rows on: below 2 GiB)
        const uint32_t limoff = (uint32_t)(min(L.Tk - 1 - k0, kKT - 1) * kstb);
#pragma unroll
        for (int i = 0; i < INSTR; ++i) {
            const int ins = wave + NW * i;
            if (NI % NW && ins >= NI) break;                 // the same for the whole wave
            const bool isv = ins * 64 >= SLOTS;              // the same for the whole wave
            const char* src = (isv ? vsrc : ksrc) + (min(roff[i], limoff) + coff[i]);
            bf16* dst = &tl[isv ? 1 : 0][(ins * 64 - (isv ? SLOTS : 0)) * 8];
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };

    const float c2 = L.scale * 1.4426950408889634f;   // scores in log2 units
    const bf16x2 ones2 = bf16x2{(bf16)1.f, (bf16)1.f};
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
        if (k0 + kKT < kend) issue(k0 + kKT, nxt);
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
                bf16x8 qb_;
                if constexpr (QLDS) qb_ = __builtin_bit_cast(bf16x8, *(const u32x4*)(qw + r * D + (((2 * ks + g) ^ swz<CH>(r)) * 8)));
                else qb_ = qf[ks];
                sacc[kb] = mfma32(a, qb_, sacc[kb]);
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
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) sacc[kb][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][j], c2, -m));
        // O^T += V^T P^T, four 16-key steps. The normaliser sums the same bf16 weights that the
        // products take, two per instruction (v_dot2c_f32_bf16 against (1, 1), fp32 sum)
#pragma unroll
        for (int s = 0; s < kKT / 16; ++s) {
            const int o = 8 * (s & 1);
            const f32x16& x = sacc[s >> 1];
            const u32x4 pw = u32x4{pack2(x[o], x[o + 1]), pack2(x[o + 2], x[o + 3]), pack2(x[o + 4], x[o + 5]),
                                   pack2(x[o + 6], x[o + 7])};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = pw[e];   // through a scalar: a bit cast of a vector lane itself reads lane 0 on this compiler
                l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones2, l, false);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x2 v0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)((const char*)vt + voff[0][db] + s * 16 * D * 2)));
                const u32x2 v1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)((const char*)vt + voff[1][db] + s * 16 * D * 2)));
                oacc[db] = mfma32(__builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]}), pb, oacc[db]);
            }
        }
    };
    if (kbeg < kend) issue(kbeg, tile0);
    for (int k0 = kbeg; k0 < kend; k0 += 2 * kKT) {
        step(k0, tile0, tile1);
        if (k0 + kKT < kend) step(k0 + kKT, tile1, tile0);
    }

    // lane (r, g) holds O[query qw0 + r][dims 32 db + 8 i + 4 g .. + 3] in registers
    // 4 i .. 4 i + 3 of block db
    const float lsum = l + __shfl_xor(l, 32);
    const int t = qw0 + r;
    if (NS > 1) {
        // this split's unnormalised O, its maximum (log2 units; the same in both lanes of a
        // query) and its weight sum, for the merge
        if (t < L.Tq) {
            const int64_t row = (int64_t)(sp * L.B * L.H + bh) * L.Tq + t;
            float* prow = L.part + row * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = 4 * i;
                    *(f32x4*)(prow + 32 * db + 8 * i + 4 * g) =
                        f32x4{oacc[db][j], oacc[db][j + 1], oacc[db][j + 2], oacc[db][j + 3]};
                }
            if (g == 0) *(f32x2*)(L.ml + 2 * row) = f32x2{m, lsum};
        }
        return;
    }
    // normalise and store
    bf16* obase = (bf16*)L.o + (int64_t)b * L.osb + (int64_t)h * L.osh;
    const float inv = 1.f / lsum;
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

// Merge of the key splits: per query row, M = max_s m_s, w_s = 2^(m_s - M),
// o = sum_s w_s O_s / sum_s w_s l_s in split order, rounded to bf16. 32 lanes per row, 4
// dimensions each (D = 128; 16 lanes at D = 64), 256 threads per workgroup.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnLaunch L) {
    constexpr int LPR = D / 4;                 // lanes per row
    constexpr int RPB = 256 / LPR;             // rows per workgroup
    const int64_t nrow = (int64_t)L.B * L.H * L.Tq;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    if (row >= nrow) return;
    const int c = 4 * (threadIdx.x % LPR);
    const int NS = L.nsplit;
    float M = -__builtin_inff();
    for (int s = 0; s < NS; ++s) M = __builtin_fmaxf(M, L.ml[2 * (s * nrow + row)]);
    float den = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < NS; ++s) {
        const int64_t rs = s * nrow + row;
        const f32x2 ml = *(const f32x2*)(L.ml + 2 * rs);
        const float w = __builtin_amdgcn_exp2f(ml[0] - M);
        den += w * ml[1];
        acc += w * *(const f32x4*)(L.part + rs * D + c);
    }
    const float inv = 1.f / den;
    const int bh = (int)(row / L.Tq), t = (int)(row % L.Tq);
    const int b = bh / L.H, h = bh % L.H;
    bf16* orow = (bf16*)L.o + (int64_t)b * L.osb + (int64_t)h * L.osh + (int64_t)t * L.ost;
    *(u32x2*)(orow + c) = u32x2{pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv)};
}

}  // namespace

bool attn_supported(int D) { return D == 64 || D == 128; }

// Waves per workgroup: 12 where the grid then has at least two workgroups per CU (256 CUs),
// else 8. Key splits (when allowed, for a single-frame call whose grid leaves CUs idle): the
// count of splits that minimises the estimated length of the launch, rounds of 256 workgroups
// times the tiles each takes, with each split at least 16 tiles long; a 12-wave workgroup's
// tile counts 0.93 of the 8-wave one's per query (the two measured on one CU's worth of work).
void attn_plan(AttnLaunch& L, bool allow_split, size_t* ws_bytes) {
    constexpr int kCUs = 256, kMinTiles = 16, kMaxSplit = 16;
    auto items = [&](int nw) { return (int64_t)L.B * L.H * ((L.Tq + nw * kQW - 1) / (nw * kQW)); };
    L.nw = items(12) >= 2 * kCUs ? 12 : 8;
    L.nsplit = 1;
    const int64_t S = L.S;
    if (allow_split && L.Tq == S) {
        const int64_t kmax = std::min<int64_t>((int64_t)(L.q_frame0 + 1) * S, L.Tk);
        const int64_t tiles = (kmax + kKT - 1) / kKT;
        // cost in query-tile units: rounds x (queries per workgroup x tiles per split)
        auto cost = [&](int nw, int ns) {
            const int64_t n = items(nw) * ns;
            return (double)((n + kCUs - 1) / kCUs) * nw * kQW * ((tiles + ns - 1) / ns) * (nw == 12 ? 0.93 : 1.0);
        };
        double best = 0.;
        int bnw = 0, bns = 1;
        for (int nw : {8, 12})
            for (int ns = 2; ns <= kMaxSplit && tiles / ns >= kMinTiles; ++ns)
                if (bnw == 0 || cost(nw, ns) < best) {
                    best = cost(nw, ns);
                    bnw = nw;
                    bns = ns;
                }
        if (bnw && best < 0.97 * cost(L.nw, 1)) {   // a split must gain more than its merge costs
            L.nw = bnw;
            L.nsplit = bns;
        }
    }
    const int64_t rows = (int64_t)L.B * L.H * L.Tq;
    *ws_bytes = L.nsplit > 1 ? (size_t)(((L.nsplit * rows * L.D * 4 + 255) / 256) * 256 + L.nsplit * rows * 8) : 0;
}

template <int D, int NW> hipError_t launch_nw(const AttnLaunch& L, hipStream_t s) {
    const int64_t items = (int64_t)L.B * L.H * L.nsplit * ((L.Tq + NW * kQW - 1) / (NW * kQW));
    const int64_t blocks = (items + 7) / 8 * 8;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<D, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, L);
    return hipGetLastError();
}

template <int D> hipError_t launch_d(const AttnLaunch& L, hipStream_t s) {
    return L.nw == 12 ? launch_nw<D, 12>(L, s) : launch_nw<D, 8>(L, s);
}

hipError_t attn_launch(const AttnLaunch& L, hipStream_t s) {
    if (L.nsplit < 1 || (L.nsplit > 1 && (!L.part || !L.ml)) || (L.nw != 8 && L.nw != 12))
        return hipErrorInvalidValue;
    if (L.D == 128) return launch_d<128>(L, s);
    if (L.D == 64) return launch_d<64>(L, s);
    return hipErrorInvalidValue;
}

hipError_t attn_combine_launch(const AttnLaunch& L, hipStream_t s) {
    const int64_t rows = (int64_t)L.B * L.H * L.Tq;
    const int rpb = 256 / (L.D / 4);
    const int64_t blocks = (rows + rpb - 1) / rpb;
    if (blocks > 0x7FFFFFFF || L.nsplit < 2) return hipErrorInvalidValue;
    if (L.D == 128)
        hipLaunchKernelGGL((attn_combine_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, s, L);
    else if (L.D == 64)
        hipLaunchKernelGGL((attn_combine_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, s, L);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
