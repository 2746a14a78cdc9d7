// Step mode for bf16 data with D = 64 or 128: one frame from a cached state, the update as
// written (gen-hub.ru, "NVIDIA SANA-WM: минутное 720p видео с одной видеокарты", section
// "Архитектура: четыре нетривиальных решения"; streaming by frames: jefxiong.cn digest, item 1):
//     P = (c K) M,   R = V - gamma P,   M' = gamma M + beta (c K)^T R,   O = Q M'.
//
// Columns of M' only depend on the same columns of M (R's column j needs column j of M), so the
// update splits into independent blocks of 32 value columns. Three launches on the stream:
//   1. step_partials_kernel, one workgroup per (b, h, column block J, token split p):
//      P = K M[:, J] on MFMA for each 16-token tile (A = K rows, B = M[:, J] in bf16, held in
//      registers), then U_p[:, J] = K^T (V[:, J] - gamma c P) accumulated over the split (A = K^T
//      by transposed LDS reads, B = V[:, J] exact plus the bf16-rounded prediction term),
//      stored as an fp32 partial. K and V come in 64-token chunks through registers (three in
//      flight while one is used): each wave loads its 16 K rows in the prediction's A-operand
//      layout, so the prediction runs from registers, then writes them into LDS unpadded with
//      an XOR swizzle of each row's 16-byte chunks; one barrier per chunk (LDS double
//      buffered). The column blocks of one (b, h, split) read the same K rows and are
//      placed on one XCD (workgroup i runs on XCD i mod 8), so K comes from that XCD's L2
//      after its first read.
//   2. step_merge_kernel, one workgroup per (b, h, J, 32 rows): M' = gamma M + beta c sum_p U_p
//      in split order, state_out, and the bf16 transposed copy M'^T.
//   3. step_output_kernel, one workgroup per (b, h, chunk of at most 256 tokens): M'^T staged
//      through LDS into registers (the A operand of every tile), O^T = M'^T Q^T per 16-token
//      tile with 16-byte stores, every Q tile of the chunk loaded before the first product.
// Nothing waits on another workgroup inside a launch; the stream orders the three, so results
// are bitwise reproducible. (A single launch that hands partials and states between
// workgroups through device-coherent memory was slower: each such hand-off costs a memory
// round trip of microseconds under load, more than a launch boundary.)
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

constexpr int kThreads = 256;   // 4 waves
constexpr int kCW = 32;         // value columns per partial role
constexpr int kSC = 64;         // tokens per staged chunk
constexpr int kRing = 2;        // staged chunks in LDS
constexpr int kStages = 3;      // chunks in registers (in flight while one is used)
constexpr int kQD = 4;          // 16-token output tiles per wave (a chunk has at most 16)

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// XOR swizzle of the 16-byte chunks of row r of an unpadded LDS tile with CH chunks per row:
// chunk c of row r is stored at chunk c ^ swz(r). The masks (functions of the bits b_i of r) make
// the tile's accesses free of bank conflicts whether the LDS serves 64 banks per clock (16 lanes
// of a 16-byte access, 32 lanes of an 8-byte one) or 32 (8 and 16 lanes):
//   CH = 16, 8 (K chunk, D = 128, 64): 16-byte row stores (16 rows, one chunk each) and
//            transposed reads (rows k0 + 4 g + 0..3, two neighbouring chunks);
//   CH = 4 (V chunk): transposed reads of two neighbouring chunks (the stores fill whole rows).
template <int CH> __device__ __forceinline__ int swz(int r) {
    const int b0 = r & 1, b1 = (r >> 1) & 1, b2 = (r >> 2) & 1, b3 = (r >> 3) & 1;
    if constexpr (CH == 16) return (b3 ^ b2) | b0 << 1 | b1 << 2 | b2 << 3;
    else if constexpr (CH == 8) return (b3 ^ b2) | b1 << 1 | (b0 ^ b2) << 2;
    else return (b1 ^ b2) << 1;
}
// The prediction tile [kCW][kSC] (8-byte accesses, 16 rows x 4 units): unit u of row r is
// stored at unit u ^ (r mod 16).
__device__ __forceinline__ int pct_off(int row, int col) { return row * kSC + ((((col >> 2) ^ row) & 15) << 2); }

// Lane (r, g) of each 16-lane group receives X[k0 + 4 g + j][c0 + r], j = 0..3, from a swizzled
// [row][CH chunks] bf16 LDS tile (ds_read_tr16_b64: destination lane i takes element i mod 4 of
// the four values at the address of source lane 4 j + i / 4, so source lane s points at row
// k0 + 4 g + s / 4, columns c0 + 4 (s mod 4) .. + 3).
template <int CH> __device__ __forceinline__ u32x2 read_tr(const bf16* X, int k0, int c0, int r, int g) {
    const int row = k0 + 4 * g + (r >> 2);
    const int c = c0 / 8 + ((r & 3) >> 1);
    const bf16* a = X + row * CH * 8 + ((c ^ swz<CH>(row)) * 8) + 4 * (r & 1);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a));
}

// Barrier of the staged loop: this wave's LDS accesses are complete, then s_barrier. Unlike
// __syncthreads() it does not wait for outstanding global loads (its workgroup release fence
// lowers to vmcnt(0), which would drain the chunks in flight into registers).
__device__ __forceinline__ void lds_barrier() { __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D> struct PartLds {
    static constexpr int KB = kSC * D * 2;     // K chunk [token][D]
    static constexpr int VB = kSC * kCW * 2;   // V chunk [token][kCW]
    static constexpr int BUF = KB + VB;
    static constexpr int PB = kCW * kSC * 2;   // prediction tile [kCW][kSC] (pct_off)
    static constexpr int MTOFF = kRing * (BUF + PB);   // M[:, J]^T in bf16: [kCW][D + 8]
    static constexpr int BYTES = MTOFF + kCW * (D + 8) * 2;
};
template <int D> struct OutLds {
    static constexpr int BYTES = D * D * 2;    // M'^T, swizzled (out_mask)
};

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

// Partial of role ((b h) * nsplit + p) * NJ + J.
template <int D, bool DELTA>
__device__ void partial_body(const Launch& L, int role, char* lds) {
    constexpr int NJ = D / kCW, CHK = D / 8, KSN = D / 32, RT = D / 64;
    static_assert(kSC * (kCW / 8) == kThreads, "one 16-byte slot of V per thread and chunk");
    using PL = PartLds<D>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int NS = L.nsplit;
    const int q = role / NJ, J = role % NJ;
    const int bh = q / NS, p = q % NS;
    const int b = bh / L.H, h = bh % L.H;
    const int t0 = p * L.split_tokens, t1 = min(L.S, t0 + L.split_tokens);
    const int64_t io = (int64_t)b * L.sb + (int64_t)h * L.sh;
    const bf16* kb = (const bf16*)L.k + io;
    const bf16* vb = (const bf16*)L.v + io + kCW * J;

    // M[:, J] (B operand of the prediction) goes through LDS once per workgroup, transposed
    // and in bf16: thread t < (D / 8) (kCW / 8) loads the 8 x 8 block (rows 8 (t / 4), columns
    // kCW J + 8 (t mod 4)) with 16-byte loads and stores its columns as rows of mts[j][k]
    constexpr int NBK = (D / 8) * (kCW / 8);
    static_assert(NBK <= kThreads, "one 8 x 8 block of M per thread");
    const bool mthread = DELTA && tid < NBK;
    f32x4 mx[8][2];
    if (mthread) {
        const float* M = L.state_in + (int64_t)bh * D * D + (8 * (tid / (kCW / 8))) * D + kCW * J + 8 * (tid % (kCW / 8));
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) mx[e][hh] = *(const f32x4*)(M + e * D + 4 * hh);
    }

    // A chunk of tokens c0 .. c0 + kSC - 1 in registers: wave w holds K rows 16 w .. 16 w + 15
    // as the prediction's A operand (lane (r, g): row 16 w + r, features 32 ks + 8 g .. + 7);
    // thread t holds the 16 bytes of V that go to slot t of the V tile (row t / 4, stored chunk
    // t mod 4, the row's chunk (t mod 4) ^ swz(row)). Rows past the split load its last row and
    // are replaced by zeros, so they add nothing.
    struct Stage {
        u32x4 k[KSN];
        u32x4 v;
    };
    const int vrow = tid >> 2, vchunk = (tid & 3) ^ swz<kCW / 8>(tid >> 2);
    auto load = [&](Stage& st, int c0) {
        const bf16* kr = kb + (int64_t)min(c0 + 16 * wave + r, t1 - 1) * L.st + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks) st.k[ks] = *(const u32x4*)(kr + 32 * ks);
        st.v = *(const u32x4*)(vb + (int64_t)min(c0 + vrow, t1 - 1) * L.st + vchunk * 8);
    };
    Stage sg[kStages];   // chunks n + 1 .. n + kStages are in flight while chunk n is used
#pragma unroll
    for (int i = 0; i < kStages; ++i)
        if (t0 + i * kSC < t1) load(sg[i], t0 + i * kSC);

    bf16x8 bm[DELTA ? 2 : 1][DELTA ? KSN : 1];
    if constexpr (DELTA) {
        bf16* mts = (bf16*)(lds + PL::MTOFF);   // [kCW][D + 8]
        if (mthread) {
            const int k0 = 8 * (tid / (kCW / 8)), j0 = 8 * (tid % (kCW / 8));
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int hh = c >> 2, qq = c & 3;
                *(u32x4*)(mts + (j0 + c) * (D + 8) + k0) =
                    u32x4{pack2(mx[0][hh][qq], mx[1][hh][qq]), pack2(mx[2][hh][qq], mx[3][hh][qq]),
                          pack2(mx[4][hh][qq], mx[5][hh][qq]), pack2(mx[6][hh][qq], mx[7][hh][qq])};
            }
        }
        lds_barrier();
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks)
                bm[ct][ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(mts + (16 * ct + r) * (D + 8) + 32 * ks + 8 * g));
    }
    const float gc = L.gamma[bh] * L.c;

    f32x4 acc[RT][2];
#pragma unroll
    for (int it = 0; it < RT; ++it)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[it][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk n: the prediction from the stage's registers, the stage into LDS buffer n % 2 (with
    // the prediction tile), the stage refilled with chunk n + kStages, one barrier, the U
    // product. Buffer n % 2 was last read for chunk n - 2, which every wave finished before the
    // barrier of chunk n - 1.
    auto chunk = [&](Stage& st, int c0, int n) {
        const int buf = n & 1;
        bf16* kc = (bf16*)(lds + buf * PL::BUF);
        bf16* vc = (bf16*)(lds + buf * PL::BUF + PL::KB);
        bf16* pct = (bf16*)(lds + kRing * PL::BUF + buf * PL::PB);   // -gamma c P^T: [kCW][kSC]
        const int tv = t1 - c0;   // tokens of the split left, from this chunk on
        const u32x4 z = {0u, 0u, 0u, 0u};
        const int krow = 16 * wave + r;
        u32x4 kx[KSN];
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks) kx[ks] = krow < tv ? st.k[ks] : z;
        if constexpr (DELTA) {
            // C lane (r, g) holds P[16 wave + 4 g + q][16 ct + r]
            f32x4 pa[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) pa[ct] = mfma(__builtin_bit_cast(bf16x8, kx[ks]), bm[ct][ks], pa[ct]);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                *(u32x2*)(pct + pct_off(16 * ct + r, 16 * wave + 4 * g)) =
                    u32x2{pack2(-gc * pa[ct][0], -gc * pa[ct][1]), pack2(-gc * pa[ct][2], -gc * pa[ct][3])};
        }
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks)
            *(u32x4*)(kc + krow * D + (((4 * ks + g) ^ swz<CHK>(krow)) * 8)) = kx[ks];
        *(u32x4*)(vc + tid * 8) = vrow < tv ? st.v : z;
        if (c0 + kStages * kSC < t1) load(st, c0 + kStages * kSC);
        lds_barrier();
        // U[i][j] += sum over the chunk's tokens of K[t][i] (V[t][j] - gamma c P[t][j]); the k
        // order of a 32-token step is tokens {4 g + e} then {16 + 4 g + e}, in A and B alike
#pragma unroll
        for (int tg = 0; tg < kSC; tg += 32) {
            bf16x8 bv[2], bp[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                bv[ct] = join(read_tr<kCW / 8>(vc, tg, 16 * ct, r, g), read_tr<kCW / 8>(vc, tg + 16, 16 * ct, r, g));
                if constexpr (DELTA) {
                    bp[ct] = join(*(const u32x2*)(pct + pct_off(16 * ct + r, tg + 4 * g)),
                                  *(const u32x2*)(pct + pct_off(16 * ct + r, tg + 16 + 4 * g)));
                }
            }
#pragma unroll
            for (int it = 0; it < RT; ++it) {
                const int i0 = 16 * (wave * RT + it);
                const bf16x8 ak = join(read_tr<CHK>(kc, tg, i0, r, g), read_tr<CHK>(kc, tg + 16, i0, r, g));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    acc[it][ct] = mfma(ak, bv[ct], acc[it][ct]);
                    if constexpr (DELTA) acc[it][ct] = mfma(ak, bp[ct], acc[it][ct]);
                }
            }
        }
    };
    for (int c0 = t0, n = 0; c0 < t1; c0 += kStages * kSC, n += kStages) {
#pragma unroll
        for (int i = 0; i < kStages; ++i)
            if (c0 + i * kSC < t1) chunk(sg[i], c0 + i * kSC, n + i);
    }

    // partial of split p in the lanes' own order: part[(b h) J][p][tile][lane][4 fp32], tile
    // (row tile) * 2 + (column tile)
    float* pp = L.part + ((int64_t)(bh * NJ + J) * NS + p) * D * kCW;
#pragma unroll
    for (int it = 0; it < RT; ++it)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
            *(f32x4*)(pp + (((wave * RT + it) * 2 + ct) * 64 + lane) * 4) = acc[it][ct];
}

template <int D, bool DELTA>
__global__ __launch_bounds__(kThreads, 2) void step_partials_kernel(Launch L) {
    constexpr int NJ = D / kCW;
    __shared__ __attribute__((aligned(16))) char lds[PartLds<D>::BYTES];
    const int NG = L.B * L.H * L.nsplit;   // (b, h, split) groups
    // workgroup i runs on XCD i mod 8: the NJ column blocks of a group share an XCD
    const int xcd = blockIdx.x % 8, k = blockIdx.x / 8;
    const int q = (k / NJ) * 8 + xcd, J = k % NJ;
    if (q >= NG) return;
    partial_body<D, DELTA>(L, q * NJ + J, lds);
}

// M' = gamma M + beta c sum_p U_p for rows 32 rb .. 32 rb + 31 of column block J of one (b, h);
// thread t handles tile 4 rb + t / 64 of the partial layout at lane t mod 64: rows
// 16 (2 rb + t / 128) + 4 g + q, column 32 J + 16 ((t / 64) mod 2) + r.
template <int D>
__global__ __launch_bounds__(kThreads) void step_merge_kernel(Launch L) {
    constexpr int NJ = D / kCW, NRB = D / 32;
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int rb = blockIdx.x % NRB, J = (blockIdx.x / NRB) % NJ, bh = blockIdx.x / (NRB * NJ);
    const int tile = 4 * rb + (tid >> 6);
    const int i = 16 * (tile >> 1) + 4 * g, j = kCW * J + 16 * (tile & 1) + r;
    const int NS = L.nsplit;
    const float* part = L.part + (int64_t)(bh * NJ + J) * NS * D * kCW + (tile * 64 + lane) * 4;
    const float* min_ = L.state_in + (int64_t)bh * D * D;
    float m0[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) m0[qq] = min_[(i + qq) * D + j];
    constexpr int BATCH = 8;   // partials in flight
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < NS; p0 += BATCH) {
        f32x4 x[BATCH];
#pragma unroll
        for (int e = 0; e < BATCH; ++e) x[e] = *(const f32x4*)(part + (int64_t)min(p0 + e, NS - 1) * D * kCW);
#pragma unroll
        for (int e = 0; e < BATCH; ++e)
            if (p0 + e < NS) u += x[e];
    }
    const float gm = L.gamma[bh], bc = L.beta[bh] * L.c;
    float m[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) m[qq] = gm * m0[qq] + bc * u[qq];
    if (L.state_out) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) L.state_out[(int64_t)bh * D * D + (i + qq) * D + j] = m[qq];
    }
    *(u32x2*)((bf16*)L.mt + (int64_t)bh * D * D + j * D + i) = u32x2{pack2(m[0], m[1]), pack2(m[2], m[3])};
}

// O = Q M' for tokens [chunk * chunk_tokens, + chunk_tokens) of one (b, h): wave w takes the
// 16-token tiles w, w + 4, .. (at most kQD), computed as O^T = M'^T Q^T so that lane (r, g)
// ends up with 8 consecutive output columns of token r.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void step_output_kernel(Launch L) {
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
    constexpr int NE = D * D / 8, PT = NE / kThreads;
    static_assert(NE % kThreads == 0, "whole rows per thread");
    const bf16* mt = (const bf16*)L.mt + (int64_t)bh * D * D;
    u32x4 x[PT];
#pragma unroll
    for (int k = 0; k < PT; ++k) x[k] = *(const u32x4*)(mt + (tid + k * kThreads) * 8);
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
        const int e = tid + k * kThreads, row = e / (D / 8), c = (e % (D / 8)) * 8;
        *(u32x4*)(ms + out_off<D>(row, c)) = half_swap(x[k], out_mask<D>(row) & 1);
    }
    __syncthreads();
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
                    oo + (32 * pp + 8 * g) * 2, 0, 0);
            }
        }
    }
}

template <int D> hipError_t launch_d(Kernel k, const Launch& L, hipStream_t s) {
    constexpr int NJ = D / kCW;
    const int64_t BH = (int64_t)L.B * L.H;
    switch (k) {
    case K_STEP_PARTIAL: {
        const int64_t n = (BH * L.nsplit + 7) / 8 * 8 * NJ;
        if (n > 0x7FFFFFFF || L.split_tokens % kSC) return hipErrorInvalidValue;
        if (L.use_delta)
            hipLaunchKernelGGL((step_partials_kernel<D, true>), dim3((unsigned)n), dim3(kThreads), 0, s, L);
        else
            hipLaunchKernelGGL((step_partials_kernel<D, false>), dim3((unsigned)n), dim3(kThreads), 0, s, L);
        break;
    }
    case K_STEP_REDUCE:
        hipLaunchKernelGGL((step_merge_kernel<D>), dim3((unsigned)(BH * NJ * (D / 32))), dim3(kThreads), 0, s, L);
        break;
    case K_STEP_OUTPUT: {
        const int64_t n = BH * L.nchunk;
        if (n > 0x7FFFFFFF || L.chunk_tokens > 4 * 16 * kQD) return hipErrorInvalidValue;
        hipLaunchKernelGGL((step_output_kernel<D>), dim3((unsigned)n), dim3(kThreads), 0, s, L);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool step_cols_supported(int bf16, int D) { return bf16 && (D == 64 || D == 128); }

hipError_t step_launch(Kernel k, const Launch& L, hipStream_t s) {
    if (!L.bf16) return hipErrorInvalidValue;
    switch (L.D) {
    case 64: return launch_d<64>(k, L, s);
    case 128: return launch_d<128>(k, L, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
