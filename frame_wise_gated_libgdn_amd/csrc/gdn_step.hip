// Step mode for bf16 data with D = 64 or 128: one frame from a cached state (gen-hub.ru, "NVIDIA
// SANA-WM: минутное 720p видео с одной видеокарты", section "Архитектура: четыре нетривиальных
// решения"; streaming by frames: jefxiong.cn digest, item 1):
//     R = V - gamma (c K) M,   M' = gamma M + beta (c K)^T R,   O = Q M'.
// With the residual expanded, (c K)^T R = c (K^T V) - gamma c^2 (K^T K) M, so the part of the
// update that runs over the frame's tokens is the pair of products G = K^T K and B = K^T V, which
// split over tokens without the state; the state enters once per split, through a D x D x D
// product. Three launches on the stream:
//   1. step_gram_kernel, one workgroup of 8 waves per (b, h, token split p) (one per CU at the
//      streaming shape): K and V of the split go from global memory straight into LDS (16-byte
//      direct loads in stages of 112 tokens at D = 128, the next stage loading while one is
//      used; XOR-swizzled 16-byte chunks), [G_p | B_p] = K_p^T [K_p | V_p] accumulates on v_mfma_f32_32x32x16_bf16
//      (every operand a transposed LDS read), then U_p = B_p - gamma c G_p M with -gamma c G_p
//      and M in bf16, stored as a partial of 24 bits per value. K and V cross HBM once.
//   2. step_sum_kernel, one workgroup per (b, h, 32 x 32 tile): M' = gamma M + beta c sum_p U_p
//      in split order, state_out, and the bf16 transposed copy M'^T.
//   3. step_output_kernel, one workgroup per (b, h, chunk of at most 256 tokens): M'^T staged
//      through LDS into registers (the A operand of every tile), O^T = M'^T Q^T per 16-token
//      tile with 16-byte stores; the chunk's Q loads stay in flight across the staging barrier.
// Nothing waits on another workgroup inside a launch; the stream orders the three, so results
// are bitwise reproducible. (A single launch that hands partials and states between
// workgroups through device-coherent memory was slower: each such hand-off costs a memory
// round trip of microseconds under load, more than a launch boundary.)
#include <stdint.h>

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kGramThreads = 512;   // Gram kernel: 8 waves, one workgroup per CU
constexpr int kSumThreads = 256;    // sum kernel: one 32 x 32 tile of 16 fp32 per lane, 4 per thread
constexpr int kOutThreads = 256;    // output kernel: 4 waves
constexpr int kQD = 4;              // 16-token output tiles per wave (a chunk has at most 16)

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_bf16: lane l = 32 g + r holds A row r and B column r over the contraction
// slice [8 g, 8 g + 8), and C rows 8 i + 4 g + q (register 4 i + q) of column r
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(bf16)lo, (bf16)hi});
}

__device__ __forceinline__ bf16x8 join(u32x2 lo, u32x2 hi) {
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// cache-policy operand of the buffer intrinsics for device-scope accesses (sc1). Loads are
// served by the L2 of the XCD they run on, never by a CU's own L1, which may hold lines from
// before a hand-off. Stores write through to memory (and are then read back from memory, not
// from the L2: 1.3 against 0.5 us measured for a hand-off within an XCD): used for the outputs
// and the partials, so that the L2 does not write them back when the launch ends. At the
// streaming shape that ends the one-launch step 1.6 us sooner for the outputs and 0.5 us
// sooner for the partials, net of their slower read-back.
constexpr int kDeviceScope = 16;

// The partials travel in 24 bits per value: the top three bytes of each fp32 (sign, exponent and
// 15 fraction bits), rounded to nearest (ties away from zero), four values in 12 bytes. A
// partial keeps 16 significant bits, against the 8 of the bf16 operands of the products that
// form it; the sum of the partials and the state stay fp32. A NaN is truncated and made quiet,
// so that it stays a NaN whatever its payload; a finite value past the largest 24-bit one
// rounds to infinity.
__device__ __forceinline__ u32x3 pack24(f32x4 x) {
    uint32_t t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // through a scalar: a bit cast of a vector lane itself reads lane 0 on this compiler
        const float f = x[q];
        const uint32_t b = __builtin_bit_cast(uint32_t, f);
        t[q] = (b & 0x7FFFFFFFu) > 0x7F800000u ? b >> 8 | 0x4000u : (b + 0x80u) >> 8;
    }
    return u32x3{t[0] | t[1] << 24, t[1] >> 8 | t[2] << 16, t[2] >> 16 | t[3] << 8};
}
__device__ __forceinline__ f32x4 unpack24(u32x3 d) {
    const uint32_t t0 = d[0] & 0xFFFFFFu, t1 = d[0] >> 24 | (d[1] & 0xFFFFu) << 8;
    const uint32_t t2 = d[1] >> 16 | (d[2] & 0xFFu) << 16, t3 = d[2] >> 8;
    return f32x4{__builtin_bit_cast(float, t0 << 8), __builtin_bit_cast(float, t1 << 8),
                 __builtin_bit_cast(float, t2 << 8), __builtin_bit_cast(float, t3 << 8)};
}
constexpr int kPartBytes = 12;   // bytes per lane and register group of a partial

// Barrier on LDS accesses only: this wave's LDS accesses are complete, then s_barrier. Unlike
// __syncthreads() it does not wait for outstanding global loads (its workgroup release fence
// lowers to vmcnt(0)).
__device__ __forceinline__ void lds_barrier() { __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------- Gram kernel
// Stage of the split in LDS: K and V of TB tokens, [token][D] bf16 rows without padding (56 KB
// for the pair). Two stages are resident (separate arrays, so that the compiler can tell reads
// of one from the direct loads into the other).
template <int D> struct GramLds {
    static constexpr int TB = D == 128 ? 112 : 224;   // tokens per stage (a multiple of 16)
    static constexpr int TILE = TB * D;               // bf16 elements of one K or V stage
};

// XOR swizzle of the 16-byte chunks of a token row of a [token][D] stage (CH = D / 8 chunks per
// row): chunk c of row r is stored at chunk c ^ swz(r). The masks keep the transposed reads below
// (per 16-lane group 4 rows and 2 neighbouring chunks; the four groups of a wave at rows +0 / +4,
// columns +0 / +16; 8 bytes per lane) free of bank conflicts with 64 or 32 banks per clock.
template <int CH> __device__ __forceinline__ int gswz(int r) {
    const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
    if constexpr (CH == 16) return b0 | b1 << 1 | (b0 ^ b2) << 2 | (b1 ^ b3) << 3;
    else return b1 | (b0 ^ b2) << 1 | (b0 ^ b1 ^ b3) << 2;
}

// Lane l = 32 g + r receives X[krow + 4 g + j][c0 + r], j = 0..3, from a swizzled [row][W]
// bf16 LDS matrix (W elements per row, chunk c of row r stored at chunk c ^ gswz(r)):
// ds_read_tr16_b64 gives destination lane i of each 16-lane group element i mod 4 of the four
// b16 values at the address of source lane 4 j + i / 4; so source lane s of group q = l / 16
// points at row krow + 4 (q / 2) + s / 4, columns c0 + 16 (q mod 2) + 4 (s mod 4) .. + 3. krow is
// a multiple of 8 and the swizzle depends on the row's low 4 bits only, so the address of a read
// at row krow + 16 k is a per-lane offset (tr_off, for krow = 0 or 8) plus 16 k rows.
template <int W> __device__ __forceinline__ int tr_off(int krow, int c0, int lane) {
    const int q = lane >> 4, s = lane & 15;
    const int row = krow + 4 * (q >> 1) + (s >> 2);
    const int col = c0 + 16 * (q & 1) + 4 * (s & 3);
    return row * W + (((col >> 3) ^ gswz<W / 8>(row)) * 8) + (col & 7);
}
__device__ __forceinline__ u32x2 read_tr(const bf16* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}
// Element (row, col) of the same swizzled [row][W] layout (col a multiple of 4 for 8-byte and of
// 8 for 16-byte accesses)
template <int W> __device__ __forceinline__ int sw_off(int row, int col) {
    return row * W + (((col >> 3) ^ gswz<W / 8>(row)) * 8) + (col & 7);
}

// Contraction operand over the 16 rows kr .. kr + 15 (kr a multiple of 16) of a [row][W] matrix
// for one 32-column block, whose per-lane offsets for rows 0 and 8 are o0 and o8: lane (r, g)
// holds column c0 + r at rows kr + 4 g + 0..3 (slots 0-3) and kr + 8 + 4 g + 0..3 (slots 4-7).
// A and B operands use the same row order, so the product sums over the 16 rows.
template <int W> __device__ __forceinline__ bf16x8 frag(const bf16* X, int kr, int o0, int o8) {
    return join(read_tr(X + kr * W + o0), read_tr(X + kr * W + o8));
}
// The same with the slots of tokens at or past `valid` zeroed (the ragged end of a split; the
// rows there hold copies of the split's last row, so the other operand stays finite)
__device__ __forceinline__ bf16x8 mask_tail(bf16x8 x, int krow, int lane, int valid) {
    const int t0 = krow + 4 * (lane >> 5);
    const u32x4 v = __builtin_bit_cast(u32x4, x);
    const uint32_t m0 = (t0 < valid ? 0xFFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
    const uint32_t m1 = (t0 + 2 < valid ? 0xFFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
    const uint32_t m2 = (t0 + 8 < valid ? 0xFFFFu : 0u) | (t0 + 9 < valid ? 0xFFFF0000u : 0u);
    const uint32_t m3 = (t0 + 10 < valid ? 0xFFFFu : 0u) | (t0 + 11 < valid ? 0xFFFF0000u : 0u);
    return __builtin_bit_cast(bf16x8, u32x4{v[0] & m0, v[1] & m1, v[2] & m2, v[3] & m3});
}

// Role ((b h) * nsplit + p) * HV + hr: split p of (b, h), rows [hr DR, hr DR + DR) of U (DR =
// D / HV key features; HV = step_halves(D)). The workgroup forms those rows of [G | B] = K^T
// [K | V] over the split's tokens (DR rows; 2 D columns: D of G, then D of B). Wave w owns RTW x
// CTW tiles of 32 x 32: local rows 32 RTW (w mod 2), columns 32 CTW (w / 2); waves 0-3 hold G,
// waves 4-7 hold B. The epilogue writes -gamma c G (transposed) and M to LDS in bf16 and the B
// waves finish their tiles as U_p = B_p + (-gamma c G_p) M. The partial goes to
// part[role][tile][i][lane][12 bytes] (registers 4 i .. 4 i + 3 of the C layout in 24 bits
// each, pack24), tile = local 32-row block * (D / 32) + 32-column block of U.
// `last()` runs in every wave once the split's last stage has landed, before its products
// (for global loads into registers that the caller wants in flight early; no LDS access).
template <int D, bool DELTA, class Hook>
__device__ __forceinline__ void gram_phase(const Launch& L, int bh, int p, int hr, int role,
                                           bf16 (&st0)[2][GramLds<D>::TILE],
                                           bf16 (&st1)[2][GramLds<D>::TILE],
                                           bf16 (&ms)[DELTA ? D * D : 8], Hook&& last) {
    using GL = GramLds<D>;
    constexpr int HV = step_halves(D), DR = D / HV;
    constexpr int TB = GL::TB, CH = D / 8;
    constexpr int SLOTS = TB * CH;                    // 16-byte slots of one K (or V) stage
    constexpr int INSTR = 2 * SLOTS / kGramThreads;   // direct loads per thread per stage
    static_assert(SLOTS % 64 == 0 && (2 * SLOTS) % kGramThreads == 0, "whole wave instructions");
    static_assert(SLOTS % (64 * INSTR) == 0, "the K / V boundary falls between waves");
    constexpr int RTW = DR / 64, CTW = D / 64;        // 32 x 32 tiles per wave: rows, columns
    constexpr int NTL = (DR / 32) * (D / 32);         // tiles of this workgroup's rows of U
    static_assert(2 * RTW * 4 * CTW * 32 * 32 == 2 * DR * D, "eight waves cover the rows of [G | B]");
    static_assert(D * DR <= 2 * GL::TILE, "the epilogue's copy of G fits in one stage buffer");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int r = lane & 31, g = lane >> 5;
    const int b = bh / L.H, h = bh % L.H;
    const int t0 = p * L.split_tokens, t1 = min(L.S, t0 + L.split_tokens);
    const int ntok = t1 - t0, nst = (ntok + TB - 1) / TB;
    const int64_t io = (int64_t)b * L.sb + (int64_t)h * L.sh;
    const bf16* kb = (const bf16*)L.k + io;
    const bf16* vb = (const bf16*)L.v + io;

    // the state, for the epilogue: thread t < D^2 / 32 holds rows 4 (t / (D / 8)) .. + 3, columns
    // 8 (t mod (D / 8)) .. + 7 of M; loaded first, so that the stage loads queue behind it
    constexpr int MB = D * D / 32;
    static_assert(MB <= kGramThreads, "one 4 x 8 block of M per thread");
    const bool mthread = DELTA && tid < MB;
    const int mj0 = 4 * (tid / (D / 8)), mn0 = 8 * (tid % (D / 8));
    f32x4 mx[4][2];
    if (mthread) {
        const float* M = L.state_in + (int64_t)bh * D * D + mj0 * D + mn0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) mx[e][hh] = *(const f32x4*)(M + e * D + 4 * hh);
    }

    // stage n (tokens t0 + n TB ..) into buffer tl: instruction ins of the workgroup fills slots
    // 64 ins .. 64 ins + 63 of the K | V pair (lane i's 16 bytes land at slot 64 ins + i; the
    // lane picks the source chunk that the swizzle puts there); rows past the split load its
    // last row and are zeroed in the operands
    auto issue = [&](int n, bf16 (&tl)[2][GL::TILE]) {
        const int s0 = t0 + n * TB;
#pragma unroll
        for (int i = 0; i < INSTR; ++i) {
            const int ins = wave * INSTR + i;
            const bool isv = ins * 64 >= SLOTS;
            const int u = ins * 64 + lane - (isv ? SLOTS : 0);
            const int row = u / CH, c = (u % CH) ^ gswz<CH>(row);
            const bf16* src = (isv ? vb : kb) + (int64_t)min(s0 + row, t1 - 1) * L.st + c * 8;
            bf16* dst = &tl[isv ? 1 : 0][(ins * 64 - (isv ? SLOTS : 0)) * 8];
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };
    issue(0, st0);
    if (mthread) {
        // M in bf16 for the epilogue's B operand (16-byte rows of the swizzled [k][n] layout);
        // the stage-0 loads stay in flight (issued after M's)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *(u32x4*)(ms + sw_off<D>(mj0 + e, mn0)) =
                u32x4{pack2(mx[e][0][0], mx[e][0][1]), pack2(mx[e][0][2], mx[e][0][3]),
                      pack2(mx[e][1][0], mx[e][1][1]), pack2(mx[e][1][2], mx[e][1][3])};
    }

    const int rt0 = RTW * (wave & 1), ct0 = CTW * (wave >> 1);
    const bool gwave = ct0 < D / 32;            // this wave's block lies in G
    const bool busy = DELTA || !gwave;          // without the delta term G is not needed
    // per-lane offsets of the operand reads (rows 0 and 8 of a 16-token step): A = the wave's
    // key features of K, B = its columns of K (G) or of V (B)
    const int bc0 = gwave ? 32 * ct0 : 32 * ct0 - D;
    int oa[RTW][2], ob[CTW][2];
#pragma unroll
    for (int a = 0; a < RTW; ++a)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) oa[a][h8] = tr_off<D>(8 * h8, hr * DR + 32 * (rt0 + a), lane);
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) ob[c][h8] = tr_off<D>(8 * h8, bc0 + 32 * c, lane);
    f32x16 acc[RTW][CTW];
#pragma unroll
    for (int a = 0; a < RTW; ++a)
#pragma unroll
        for (int c = 0; c < CTW; ++c)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[a][c][j] = 0.f;

    // stage n from buffer cur, with stage n + 1 loading into nxt meanwhile. This wave's direct
    // loads of stage n are complete (an explicit wait: the barrier's fence waits for LDS
    // accesses only, and the compiler's own wait is not placed before every stage), so after
    // the barrier every wave's are, and every wave is past its reads of stage n - 1 from nxt
    // before the next loads go there. The loads of the other buffer are issued only after the
    // barrier, so the compiler, which tells the two arrays apart, adds no wait for them before
    // the reads of cur.
    auto stage = [&](int n, bf16 (&cur)[2][GL::TILE], bf16 (&nxt)[2][GL::TILE]) __attribute__((always_inline)) {
        __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (n + 1 < nst) issue(n + 1, nxt);
        else last();
        const int valid = min(TB, ntok - n * TB);
        if (busy) {
            const bf16* kt = cur[0];
            const bf16* bt = gwave ? cur[0] : cur[1];   // B operand: K (G) or V (B)
            // every 16-token step of the stage; the operands of step kk + 1 are read while the
            // products of step kk run (two register sets); steps past `valid` add zeros (their
            // A slots are masked)
            constexpr int NK = TB / 16;
            bf16x8 fa[2][RTW], fb[2][CTW];
            auto load = [&](int kk, int set) __attribute__((always_inline)) {
                const int kr = 16 * kk;
#pragma unroll
                for (int a = 0; a < RTW; ++a) fa[set][a] = mask_tail(frag<D>(kt, kr, oa[a][0], oa[a][1]), kr, lane, valid);
#pragma unroll
                for (int c = 0; c < CTW; ++c) fb[set][c] = frag<D>(bt, kr, ob[c][0], ob[c][1]);
            };
            load(0, 0);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                if (kk + 1 < NK) load(kk + 1, (kk + 1) & 1);
#pragma unroll
                for (int a = 0; a < RTW; ++a)
#pragma unroll
                    for (int c = 0; c < CTW; ++c) acc[a][c] = mfma32(fa[kk & 1][a], fb[kk & 1][c], acc[a][c]);
            }
        }
    };
    for (int n = 0; n < nst; n += 2) {
        stage(n, st0, st1);
        if (n + 1 < nst) stage(n + 1, st1, st0);
    }

    if constexpr (DELTA) {
        // every wave is done with the stages: -gamma c G^T into stage buffer 0 as a swizzled
        // [k][i] bf16 matrix (k the D key features, i this workgroup's DR rows; 8-byte stores of
        // the C layout's 4 consecutive rows)
        lds_barrier();
        bf16* gs = &st0[0][0];
        const float ngc = -L.gamma[bh] * L.c;
        if (gwave) {
#pragma unroll
            for (int a = 0; a < RTW; ++a)
#pragma unroll
                for (int c = 0; c < CTW; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f32x16& x = acc[a][c];
                        *(u32x2*)(gs + sw_off<DR>(32 * (ct0 + c) + r, 32 * (rt0 + a) + 8 * i + 4 * g)) =
                            u32x2{pack2(ngc * x[4 * i], ngc * x[4 * i + 1]), pack2(ngc * x[4 * i + 2], ngc * x[4 * i + 3])};
                    }
        }
        lds_barrier();
        if (!gwave) {
            // U = B + (-gamma c G) M over the D key features, 16 at a time; both operands by
            // transposed reads in the same row order: A from G^T (rows k, columns i), B from M
            // (rows k, columns n)
            int ga[RTW][2], gb[CTW][2];
#pragma unroll
            for (int a = 0; a < RTW; ++a)
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) ga[a][h8] = tr_off<DR>(8 * h8, 32 * (rt0 + a), lane);
#pragma unroll
            for (int c = 0; c < CTW; ++c)
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) gb[c][h8] = tr_off<D>(8 * h8, 32 * (ct0 + c) - D, lane);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                bf16x8 fa[RTW], fb[CTW];
#pragma unroll
                for (int a = 0; a < RTW; ++a) fa[a] = frag<DR>(gs, 16 * ks, ga[a][0], ga[a][1]);
#pragma unroll
                for (int c = 0; c < CTW; ++c) fb[c] = frag<D>(ms, 16 * ks, gb[c][0], gb[c][1]);
#pragma unroll
                for (int a = 0; a < RTW; ++a)
#pragma unroll
                    for (int c = 0; c < CTW; ++c) acc[a][c] = mfma32(fa[a], fb[c], acc[a][c]);
            }
        }
    }
    if (!gwave) {
        // register group i of every lane: one contiguous 768 bytes per store instruction,
        // written through (so that the end of the launch need not write them back)
        constexpr int RB = NTL * 4 * 64 * kPartBytes;   // bytes of one role's partial
        const __amdgpu_buffer_rsrc_t rp = buffer_over((const char*)L.part + (int64_t)role * RB, RB);
#pragma unroll
        for (int a = 0; a < RTW; ++a)
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
                const int tile = (rt0 + a) * (D / 32) + (ct0 + c - D / 32);
                const f32x16& x = acc[a][c];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b96(
                        pack24(f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]}), rp,
                        ((tile * 4 + i) * 64 + lane) * kPartBytes, 0, kDeviceScope);
            }
    }
}

template <int D, bool DELTA>
__global__ __launch_bounds__(kGramThreads, 1) void step_gram_kernel(Launch L) {
    constexpr int HV = step_halves(D);
    __shared__ __attribute__((aligned(16))) bf16 st0[2][GramLds<D>::TILE];   // K, V of even stages
    __shared__ __attribute__((aligned(16))) bf16 st1[2][GramLds<D>::TILE];   // K, V of odd stages
    __shared__ __attribute__((aligned(16))) bf16 ms[DELTA ? D * D : 8];      // M in bf16, [k][n]
    // workgroup i runs on XCD i mod 8; XCD x takes the contiguous stretch [x n8, (x + 1) n8) of
    // the roles in order, so the two halves of a split read its K and V through one L2 and the
    // splits of one (b, h) share its state there (the grid is padded to 8 n8 workgroups; the
    // padding returns at once)
    const int nrole = L.B * L.H * L.nsplit * HV;
    const int n8 = (nrole + 7) / 8;
    const int role = (int)(blockIdx.x % 8) * n8 + (int)(blockIdx.x / 8);
    if (role >= nrole) return;
    const int hr = role % HV, bh = role / HV / L.nsplit, p = role / HV % L.nsplit;
    gram_phase<D, DELTA>(L, bh, p, hr, role, st0, st1, ms, [] {});
}

// ------------------------------------------------------------------------------ sum kernel
// One 32 x 32 tile (rt, ct) of the new state of one (b, h), on 256 threads: thread thr takes
// registers 4 (thr / 64) .. + 3 of lane thr mod 64 of the partial layout, i.e. rows 32 rt +
// 8 (thr / 64) + 4 g + 0..3 of column 32 ct + r (lane = 32 g + r); a wave reads 1 KB in a row. M' = gamma M + beta c
// sum_p U_p, summed in split order; state_out (when committing) and the bf16 transposed copy M'^T.
// COH: the partials were stored by other workgroups of the same launch and are read with
// device-scope loads; poison: the partials are incomplete, M' is NaN.
template <int D, bool COH>
__device__ __forceinline__ void sum_tile(const Launch& L, int bh, int tile, int thr, bool poison) {
    constexpr int NT = (D / 32) * (D / 32), HV = step_halves(D), RTH = D / 32 / HV;
    constexpr int NTL = NT / HV;                     // tiles of one workgroup's partial
    const int lane = thr & 63, part = thr >> 6;
    const int rt = tile / (D / 32), ct = tile % (D / 32);
    const int hr = rt / RTH, lt = (rt % RTH) * (D / 32) + ct;   // half and local tile of the partial
    const int i = 32 * rt + 8 * part + 4 * (lane >> 5), j = 32 * ct + (lane & 31);
    const int NS = L.nsplit;
    // partial of split p: role ((b h) NS + p) HV + hr; consecutive splits are HV NTL tiles apart
    constexpr int RB = NTL * 4 * 64 * kPartBytes;   // bytes of one role's partial
    const char* head = (const char*)L.part + (int64_t)bh * NS * HV * RB;
    const int src = (((hr * NTL + lt) * 4 + part) * 64 + lane) * kPartBytes;   // bytes into the head
    const __amdgpu_buffer_rsrc_t rp = buffer_over(head, NS * HV * RB);
    const float* min_ = L.state_in + (int64_t)bh * D * D;
    float m0[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) m0[qq] = min_[(i + qq) * D + j];
    constexpr int BATCH = 8;   // partials in flight
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < NS; p0 += BATCH) {
        f32x4 x[BATCH];
#pragma unroll
        for (int e = 0; e < BATCH; ++e) {
            const int off = src + min(p0 + e, NS - 1) * HV * RB;
            if constexpr (COH)
                x[e] = unpack24(__builtin_amdgcn_raw_buffer_load_b96(rp, off, 0, kDeviceScope));
            else
                x[e] = unpack24(__builtin_amdgcn_raw_buffer_load_b96(rp, off, 0, 0));
        }
#pragma unroll
        for (int e = 0; e < BATCH; ++e)
            if (p0 + e < NS) u += x[e];
    }
    const float gm = L.gamma[bh], bc = L.beta[bh] * L.c;
    float m[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) m[qq] = poison ? __builtin_nanf("") : gm * m0[qq] + bc * u[qq];
    if (L.state_out) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) L.state_out[(int64_t)bh * D * D + (i + qq) * D + j] = m[qq];
    }
    *(u32x2*)((bf16*)L.mt + (int64_t)bh * D * D + j * D + i) = u32x2{pack2(m[0], m[1]), pack2(m[2], m[3])};
}

template <int D>
__global__ __launch_bounds__(kSumThreads) void step_sum_kernel(Launch L) {
    constexpr int NT = (D / 32) * (D / 32);
    sum_tile<D, false>(L, blockIdx.x / NT, blockIdx.x % NT, threadIdx.x, false);
}

// ---------------------------------------------------------------------------- output kernel
// Output column of row m of 16-row tile jt of the A operand M'^T: tiles 2p and 2p + 1 cover
// columns 32p .. 32p + 31 so that lane (r, g) of their C tiles holds 8 consecutive columns.
__device__ __forceinline__ int out_col(int jt, int m) { return 32 * (jt >> 1) + 8 * (m >> 2) + 4 * (jt & 1) + (m & 3); }

// M'^T in the output kernel's LDS: unpadded rows whose 8-byte units are permuted by XOR with
// a mask of the row's bits 0, 1, 3, 4, free of bank conflicts for 16-byte row stores and for
// the 16-byte reads of the rows out_col(jt, r) (64 or 32 banks per clock). A 16-byte access
// covers the unit pair 2u, 2u + 1; with an odd mask the pair lies swapped in LDS, so the two
// 8-byte halves swap in registers.
template <int D> __device__ __forceinline__ int out_mask(int r) {
    const int b0 = r & 1, b1 = (r >> 1) & 1, b3 = (r >> 3) & 1, b4 = (r >> 4) & 1;
    if constexpr (D == 128) return b0 | b0 << 1 | (b4 ^ b3) << 2 | b1 << 3 | b3 << 4;
    else return (b0 ^ b3) | b3 << 1 | (b4 ^ b0) << 2 | b1 << 3;
}
template <int D> __device__ __forceinline__ int out_off(int r, int c) {   // c: a multiple of 8
    return r * D + (((c >> 2) ^ (out_mask<D>(r) & ~1)) << 2);
}
__device__ __forceinline__ u32x4 half_swap(u32x4 v, bool sw) { return sw ? u32x4{v[2], v[3], v[0], v[1]} : v; }
template <int D> struct OutLds {
    static constexpr int BYTES = D * D * 2;    // M'^T, swizzled (out_mask)
};

// O = Q M' for tokens [chunk * chunk_tokens, + chunk_tokens) of one (b, h): wave w takes the
// 16-token tiles w, w + 4, .. (at most kQD), computed as O^T = M'^T Q^T so that lane (r, g)
// ends up with 8 consecutive output columns of token r.
template <int D>
__global__ __launch_bounds__(kOutThreads, 2) void step_output_kernel(Launch L) {
    constexpr int KSN = D / 32, TJ = D / 16;
    __shared__ __attribute__((aligned(16))) char lds[OutLds<D>::BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / L.nchunk, ch = blockIdx.x % L.nchunk;
    const int b = bh / L.H, h = bh % L.H;
    const int S = L.S;
    const int s_beg = ch * L.chunk_tokens, s_end = min(S, s_beg + L.chunk_tokens);

    // M'^T loads first, then the chunk's Q rows (B operand: lane (r, g) holds
    // Q[t][32 ks + 8 g .. + 7]) through a buffer resource ending with the frame's last row:
    // rows past S read zero and their stores drop
    constexpr int NE = D * D / 8, PT = NE / kOutThreads;
    static_assert(NE % kOutThreads == 0, "whole rows per thread");
    const bf16* mt = (const bf16*)L.mt + (int64_t)bh * D * D;
    u32x4 x[PT];
#pragma unroll
    for (int k = 0; k < PT; ++k) x[k] = *(const u32x4*)(mt + (tid + k * kOutThreads) * 8);
    const int qstb = (int)L.st * 2, ostb = (int)L.ot * 2;
    const __amdgpu_buffer_rsrc_t rq =
        buffer_over((const bf16*)L.q + (int64_t)b * L.sb + (int64_t)h * L.sh, ((S - 1) * (int)L.st + D) * 2);
    const __amdgpu_buffer_rsrc_t ro =
        buffer_over((bf16*)L.o + (int64_t)b * L.ob + (int64_t)h * L.oh, ((S - 1) * (int)L.ot + D) * 2);
    u32x4 bq[kQD][KSN];
#pragma unroll
    for (int d = 0; d < kQD; ++d) {
        const int row = min(s_beg + 16 * (wave + 4 * d) + r, S);
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            bq[d][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, row * qstb + (32 * ks + 8 * g) * 2, 0, 0));
    }
    bf16* ms = (bf16*)lds;   // M'^T, swizzled
#pragma unroll
    for (int k = 0; k < PT; ++k) {
        const int e = tid + k * kOutThreads, row = e / (D / 8), c = (e % (D / 8)) * 8;
        *(u32x4*)(ms + out_off<D>(row, c)) = half_swap(x[k], out_mask<D>(row) & 1);
    }
    // LDS-only barrier: the chunk's Q loads stay in flight, each tile waits for its own rows
    lds_barrier();
    bf16x8 am[TJ][KSN];
#pragma unroll
    for (int jt = 0; jt < TJ; ++jt)
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            am[jt][ks] = __builtin_bit_cast(bf16x8, half_swap(*(const u32x4*)(ms + out_off<D>(out_col(jt, r), 32 * ks + 8 * g)),
                                                              out_mask<D>(out_col(jt, r)) & 1));

#pragma unroll
    for (int d = 0; d < kQD; ++d) {
        const int st = s_beg + 16 * (wave + 4 * d);
        if (st < s_end) {
            f32x4 acc[TJ];
#pragma unroll
            for (int jt = 0; jt < TJ; ++jt) {
                acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KSN; ++ks) acc[jt] = mfma(am[jt][ks], __builtin_bit_cast(bf16x8, bq[d][ks]), acc[jt]);
            }
            const int oo = min(st + r, S) * ostb;
#pragma unroll
            for (int pp = 0; pp < TJ / 2; ++pp) {
                const f32x4 y0 = acc[2 * pp], y1 = acc[2 * pp + 1];
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{pack2(y0[0], y0[1]), pack2(y0[2], y0[3]), pack2(y1[0], y1[1]), pack2(y1[2], y1[3])}, ro,
                    oo + (32 * pp + 8 * g) * 2, 0, kDeviceScope);
            }
        }
    }
}

// ---------------------------------------------------------------------- one-launch step
// The three phases above in one launch, for shapes where every (b, h) gets its W = nsplit * HV
// workgroups on one XCD: workgroup i runs on XCD i mod 8 (the hardware hands workgroups to the
// XCDs in turn), and XCD x takes the heads x hpx .. x hpx + hpx - 1 (hpx = B H / 8), W
// workgroups each, at most one per CU. Phase A is the Gram kernel's work, then the W
// workgroups of the head meet; phase B: workgroup r forms the 32 x 32 tiles r, r + W, .. of
// M' (the sum kernel's work); they meet again; phase C: workgroup r forms the outputs of its
// chunk of ceil(S / 16 / W) 16-token tiles (the output kernel's work, by 8 waves). Every phase
// keeps the arithmetic and summation order of its kernel, so the results are those of the
// three launches, bit for bit.
//
// Hand-offs. The partials, M'^T and the meeting flags are written with plain stores, which land
// in the L2 of the writer's XCD (measured: a flag is seen about 0.4 us after it is stored, 1.1 us
// with device-scope stores, which write through), and read with device-scope loads, which that
// L2 serves and a CU's own L1 does not; workgroups of one head share that L2, so nothing waits
// for HBM. A meeting: every wave waits until its stores have completed, the workgroup meets at a
// barrier, one lane stores the tag
//     T_k = (epoch + 1) << 8 | k << 4 | xcc
// at flag[k][b h][r], and one wave polls the W flags of the head until each holds T_k. The
// epoch of a head (ctl word 1 + b h) is read at the start and advanced by workgroup 0 of the
// head after the second meeting, so each launch's tags differ from whatever the buffer held; the
// XCC id (hardware register) in the tag makes a head whose workgroups landed on different XCDs,
// whose L2 caches do not see each other's stores, fail to meet instead of reading stale data.
// Waits are bounded (spin_limit polls; 0 gives up at once): a workgroup that gives up stores
// kStepTimeout in ctl word 0 and goes on with NaN (a NaN state after the first meeting, NaN
// outputs after the second), so the kernel always ends. The meetings need the head's W
// workgroups resident together: the host launches this kernel only where the grid fits one
// workgroup per CU on every XCD.
//
// ctl (64-bit words): [0] time-out word, [1 + b h] epoch of (b, h),
// [1 + B H + (k B H + b h) W + r] flag of workgroup r at meeting k.
constexpr uint64_t kStepTimeout = kStepTimeoutWord;
constexpr int kOutBatch = 2;   // one-launch step: 16-token output tiles per wave and batch

template <int D, bool DELTA>
__global__ __launch_bounds__(kGramThreads, 1) void step_fused_kernel(Launch L) {
    constexpr int HV = step_halves(D);
    constexpr int KSN = D / 32, TJ = D / 16, NT = (D / 32) * (D / 32);
    constexpr int NW = kGramThreads / 64;
    __shared__ __attribute__((aligned(16))) bf16 st0[2][GramLds<D>::TILE];
    __shared__ __attribute__((aligned(16))) bf16 st1[2][GramLds<D>::TILE];
    __shared__ __attribute__((aligned(16))) bf16 ms[DELTA ? D * D : 8];
    __shared__ int s_bad;
    static_assert(D * D <= 2 * GramLds<D>::TILE, "M'^T fits in one stage buffer");

    const int BH = L.B * L.H, W = L.nsplit * HV, hpx = BH / 8;
    const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8);
    const int bh = xcd * hpx + slot / W, r = slot % W;
    if (slot >= hpx * W) return;
    const int p = r / HV, hr = r % HV;
    const int role = (bh * L.nsplit + p) * HV + hr;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint64_t* ctl = (uint64_t*)L.ctl;
    uint64_t* flags = ctl + 1 + BH;

    // tags of this launch (wave 0 stores and polls them)
    uint64_t tag0 = 0;
    if (wave == 0) {
        const uint64_t ep = __hip_atomic_load(ctl + 1 + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u;   // HW_REG_XCC_ID[3:0]
        tag0 = ((ep + 1) << 8) | xcc;
    }
    // meeting k of the head's W workgroups; returns true when a wait gave up. PEND: loads this
    // wave issued after its last store, left in flight (the counter retires in issue order, so
    // waiting until at most PEND remain waits for every store); the barrier waits for LDS only
    auto meet = [&](int k, auto pend) __attribute__((always_inline)) {
        constexpr int PEND = decltype(pend)::value;
        if constexpr (PEND == 0) __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
        else if constexpr (PEND == 4) __asm__ __volatile__("s_waitcnt vmcnt(4)" ::: "memory");
        else if constexpr (PEND == 8) __asm__ __volatile__("s_waitcnt vmcnt(8)" ::: "memory");
        else static_assert(PEND < 0, "no wait for this count");
        lds_barrier();
        if (wave == 0) {
            const uint64_t tag = tag0 | ((uint64_t)k << 4);
            uint64_t* fl = flags + ((int64_t)k * BH + bh) * W;
            if (lane == 0) __hip_atomic_store(fl + r, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            bool ok = false;   // spin_limit 0: every meeting gives up at once
            for (int it = 0; it < L.spin_limit; ++it) {
                const bool mine = lane >= W || __hip_atomic_load(fl + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
                ok = __all(mine);
                if (ok) break;
            }
            if (lane == 0) {
                if (!ok) __hip_atomic_store(ctl, kStepTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (k == 1 && r == 0)   // every workgroup of the head has read the epoch
                    __hip_atomic_store(ctl + 1 + bh, (tag0 >> 8), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_bad = !ok;
            }
        }
        lds_barrier();
        return s_bad != 0;
    };

    // phase C's Q rows (B operand: lane (q16, g4) holds Q[t][32 ks + 8 g4 .. + 7]); rows past S
    // read zero
    const int S = L.S;
    const int b = bh / L.H, h = bh % L.H;
    const int q16 = lane & 15, g4 = lane >> 4;
    const int ctk = ((S + 15) / 16 + W - 1) / W * 16;
    const int s_beg = r * ctk, s_end = min(S, s_beg + ctk);
    const int qstb = (int)L.st * 2, ostb = (int)L.ot * 2;
    const __amdgpu_buffer_rsrc_t rq =
        buffer_over((const bf16*)L.q + (int64_t)b * L.sb + (int64_t)h * L.sh, ((S - 1) * (int)L.st + D) * 2);
    const __amdgpu_buffer_rsrc_t ro =
        buffer_over((bf16*)L.o + (int64_t)b * L.ob + (int64_t)h * L.oh, ((S - 1) * (int)L.ot + D) * 2);
    u32x4 bq[kOutBatch][KSN];
    auto load_q = [&](int d0) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < kOutBatch; ++d) {
            const int row = min(s_beg + 16 * (wave + NW * (d0 + d)) + q16, S);
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks)
                bq[d][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, row * qstb + (32 * ks + 8 * g4) * 2, 0, 0));
        }
    };

    // phase A
    gram_phase<D, DELTA>(L, bh, p, hr, role, st0, st1, ms, [] {});
    const bool bad1 = meet(0, std::integral_constant<int, 0>());

    // phase B: tiles r, r + W, .. of M', 256 threads each
    for (int t = r + W * (tid >> 8); t < NT; t += 2 * W) sum_tile<D, true>(L, bh, t, tid & 255, bad1);
    // phase C's first Q rows load during the second meeting: issued after phase B's stores (the
    // empty asm keeps the compiler from moving them earlier), which the meeting waits for alone
    __asm__ __volatile__("" ::: "memory");
    load_q(0);
    const bool bad2 = meet(1, std::integral_constant<int, kOutBatch * KSN>());

    // phase C: M'^T through LDS into registers, then the chunk's tiles, kOutBatch per wave at a time
    constexpr int NE = D * D / 8, PT = NE / kGramThreads;
    static_assert(NE % kGramThreads == 0, "whole rows of M'^T per thread");
    const __amdgpu_buffer_rsrc_t rm = buffer_over((const bf16*)L.mt + (int64_t)bh * D * D, D * D * 2);
    bf16* mst = &st0[0][0];
    {
        u32x4 x[PT];
#pragma unroll
        for (int k = 0; k < PT; ++k)
            x[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rm, (tid + k * kGramThreads) * 16, 0, kDeviceScope));
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int e = tid + k * kGramThreads, row = e / (D / 8), c = (e % (D / 8)) * 8;
            *(u32x4*)(mst + out_off<D>(row, c)) = half_swap(bad2 ? u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u} : x[k],
                                                            out_mask<D>(row) & 1);
        }
    }
    lds_barrier();
    bf16x8 am[TJ][KSN];
#pragma unroll
    for (int jt = 0; jt < TJ; ++jt)
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            am[jt][ks] = __builtin_bit_cast(bf16x8, half_swap(*(const u32x4*)(mst + out_off<D>(out_col(jt, q16), 32 * ks + 8 * g4)),
                                                              out_mask<D>(out_col(jt, q16)) & 1));
    const int ntile = max(0, (s_end - s_beg + 15) / 16);
    for (int d0 = 0; NW * d0 < ntile; d0 += kOutBatch) {
        if (d0 > 0) load_q(d0);
#pragma unroll
        for (int d = 0; d < kOutBatch; ++d) {
            const int st = s_beg + 16 * (wave + NW * (d0 + d));
            if (st < s_end) {
                f32x4 acc[TJ];
#pragma unroll
                for (int jt = 0; jt < TJ; ++jt) {
                    acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSN; ++ks) acc[jt] = mfma(am[jt][ks], __builtin_bit_cast(bf16x8, bq[d][ks]), acc[jt]);
                }
                const int oo = min(st + q16, S) * ostb;
#pragma unroll
                for (int pp = 0; pp < TJ / 2; ++pp) {
                    const f32x4 y0 = acc[2 * pp], y1 = acc[2 * pp + 1];
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4{pack2(y0[0], y0[1]), pack2(y0[2], y0[3]), pack2(y1[0], y1[1]), pack2(y1[2], y1[3])}, ro,
                        oo + (32 * pp + 8 * g4) * 2, 0, kDeviceScope);
                }
            }
        }
    }
}

template <int D> hipError_t launch_d(Kernel k, const Launch& L, hipStream_t s) {
    const int64_t BH = (int64_t)L.B * L.H;
    switch (k) {
    case K_STEP_PARTIAL: {
        const int64_t n = (BH * L.nsplit * step_halves(D) + 7) / 8 * 8;
        if (n > 0x7FFFFFFF || L.split_tokens % 16) return hipErrorInvalidValue;
        if (L.use_delta)
            hipLaunchKernelGGL((step_gram_kernel<D, true>), dim3((unsigned)n), dim3(kGramThreads), 0, s, L);
        else
            hipLaunchKernelGGL((step_gram_kernel<D, false>), dim3((unsigned)n), dim3(kGramThreads), 0, s, L);
        break;
    }
    case K_STEP_REDUCE: {
        const int64_t n = BH * (D / 32) * (D / 32);
        if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL((step_sum_kernel<D>), dim3((unsigned)n), dim3(kSumThreads), 0, s, L);
        break;
    }
    case K_STEP_FUSED: {
        const int64_t n = BH * L.nsplit * step_halves(D);
        if (BH % 8 || n > 8 * 32 || L.split_tokens % 16 || !L.ctl) return hipErrorInvalidValue;
        if (L.use_delta)
            hipLaunchKernelGGL((step_fused_kernel<D, true>), dim3((unsigned)n), dim3(kGramThreads), 0, s, L);
        else
            hipLaunchKernelGGL((step_fused_kernel<D, false>), dim3((unsigned)n), dim3(kGramThreads), 0, s, L);
        break;
    }
    case K_STEP_OUTPUT: {
        const int64_t n = BH * L.nchunk;
        if (n > 0x7FFFFFFF || L.chunk_tokens > 4 * 16 * kQD) return hipErrorInvalidValue;
        hipLaunchKernelGGL((step_output_kernel<D>), dim3((unsigned)n), dim3(kOutThreads), 0, s, L);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool step_cols_supported(int bf16, int D) { return bf16 && (D == 64 || D == 128); }

bool step_one_device_ok(int per_xcd) {
    constexpr int kMaxDevices = 64;
    static int cached[kMaxDevices];   // 0 unknown, else 1 + CUs per XCD (0 when not 8 XCDs)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    int c = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (c == 0) {
        int xcc = 0, cu = 0;
        if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return false;
        c = 1 + (xcc == 8 ? cu / 8 : 0);
        __atomic_store_n(&cached[dev], c, __ATOMIC_RELAXED);
    }
    return per_xcd >= 1 && c - 1 >= per_xcd;
}

hipError_t step_launch(Kernel k, const Launch& L, hipStream_t s) {
    if (!L.bf16) return hipErrorInvalidValue;
    switch (L.D) {
    case 64: return launch_d<64>(k, L, s);
    case 128: return launch_d<128>(k, L, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
