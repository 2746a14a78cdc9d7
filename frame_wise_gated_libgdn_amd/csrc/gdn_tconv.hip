// Block-causal temporal convolution with a last-frame cache (SANA-Video talk, passage on the
// causal FFN with temporal conv): a depthwise convolution over latent frames, kernel 3 centred,
// in which a block's last frame sees zero on its right (the zero token between blocks) and a
// block's first frame sees the previous block's last frame on its left (the carried token; the
// cache when the previous block came in an earlier call).
//
//   y[t] = bias + w0 * L(t) + w1 * x[t] + w2 * R(t)
//   L(t) = x[t-1] for t > 0; cache_in (or 0) for t = 0
//   R(t) = x[t+1] unless t + 1 ends a block or the call (then 0)
//   cache_out = x[T-1]
//
// HBM-bound streaming (tconv_kernel; one-frame calls have tconv_frame_kernel below). A thread
// owns 16 bytes of channels of one (b, s) and TF consecutive frames: it loads the TF + 2 frames
// of its window at once (addresses clamped into the tensor, out-of-range values replaced by
// selects after the loads, so no load sits behind a branch), and writes TF outputs with 16-byte
// stores. Consecutive threads walk channels, then frame
// chunks, so the one-frame halos of neighbouring chunks are read close together in time (from
// L2). The thread of the first chunk reads cache_in and writes cache_out, so the two may be the
// same buffer.
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTconvThreads = 256;
constexpr int kTconvFrames = 16;   // frames per thread (long calls)

template <typename T> struct Vec;
template <> struct Vec<float> {
    static constexpr int N = 4;
    // whole-vector casts: a cast of one ext-vector element lvalue reads element 0
    static __device__ __forceinline__ void unpack(u32x4 w, float (&v)[N]) {
        const f32x4 f = __builtin_bit_cast(f32x4, w);
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = f[i];
    }
    static __device__ __forceinline__ u32x4 pack(const float (&v)[N]) {
        return __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]});
    }
};
template <> struct Vec<__bf16> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(u32x4 w, float (&v)[N]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
        }
    }
    static __device__ __forceinline__ u32x4 pack(const float (&v)[N]) {
        // round to nearest even (gfx950 converts pairs in one instruction)
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2 * i], (__bf16)v[2 * i + 1]});
        return w;
    }
};

template <typename T, int TF>
__global__ __launch_bounds__(kTconvThreads) void tconv_kernel(TconvLaunch L) {
    using V = Vec<T>;
    constexpr int N = V::N;
    // 32-bit index arithmetic: the host keeps the thread count below 2^31
    const uint32_t ncv = (uint32_t)L.C / N;
    const uint32_t ntc = (uint32_t)(L.T + TF - 1) / TF;
    uint32_t r = blockIdx.x * (uint32_t)kTconvThreads + threadIdx.x;
    const int cv = (int)(r % ncv);
    r /= ncv;
    const int tc = (int)(r % ntc);
    r /= ntc;
    const int s = (int)(r % (uint32_t)L.S);
    r /= (uint32_t)L.S;
    if (r >= (uint32_t)L.B) return;
    const int b = (int)r;
    const int c0 = cv * N;
    const int t0 = tc * TF;
    const T* xs = (const T*)L.x + (int64_t)b * L.xsb + (int64_t)s * L.xss + c0;
    const int64_t cache_off = ((int64_t)b * L.S + s) * L.C + c0;

    // window: frames t0 - 1 .. t0 + TF; slot 0 is the left neighbour of frame t0
    u32x4 raw[TF + 2];
    {
        const T* left = t0 > 0 ? xs + (int64_t)(t0 - 1) * L.xst
                               : (L.cache_in ? (const T*)L.cache_in + cache_off : xs);
        raw[0] = *(const u32x4*)left;
    }
#pragma unroll
    for (int i = 1; i < TF + 2; ++i) {
        const int t = min(t0 - 1 + i, L.T - 1);
        raw[i] = *(const u32x4*)(xs + (int64_t)t * L.xst);
    }
    // the frame for cache_out (the last one), read by the first chunk's threads; the others
    // re-read a frame of their own window instead of branching around the load
    const bool keep_cache = tc == 0 && L.cache_out;
    const u32x4 last = *(const u32x4*)(xs + (int64_t)(keep_cache ? L.T - 1 : min(t0, L.T - 1)) * L.xst);

    // taps of the N channels: 3 N consecutive floats (16-byte aligned: c0 is a multiple of N
    // and 3 N floats are a whole number of 16-byte words), bias likewise
    float w0[N], w1[N], w2[N], bs[N];
    {
        f32x4 tw[3 * N / 4], tb[N / 4];
#pragma unroll
        for (int k = 0; k < 3 * N / 4; ++k) tw[k] = *(const f32x4*)(L.weight + 3 * c0 + 4 * k);
#pragma unroll
        for (int k = 0; k < N / 4; ++k)
            tb[k] = L.bias ? *(const f32x4*)(L.bias + c0 + 4 * k) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < N; ++j) {
            w0[j] = tw[(3 * j) / 4][(3 * j) % 4];
            w1[j] = tw[(3 * j + 1) / 4][(3 * j + 1) % 4];
            w2[j] = tw[(3 * j + 2) / 4][(3 * j + 2) % 4];
            bs[j] = tb[j / 4][j % 4];
        }
    }
    float prev[N], cur[N], next[N];
    V::unpack(raw[0], prev);
    if (t0 == 0 && !L.cache_in) {
#pragma unroll
        for (int j = 0; j < N; ++j) prev[j] = 0.f;
    }
    V::unpack(raw[1], cur);
    T* ys = (T*)L.y + (int64_t)b * L.ysb + (int64_t)s * L.yss + c0;
#pragma unroll
    for (int i = 0; i < TF; ++i) {
        const int t = t0 + i;
        V::unpack(raw[i + 2], next);
        const bool right = t + 1 < L.T && (t + 1) % L.Tb != 0;
        float out[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float nx = right ? next[j] : 0.f;
            out[j] = __builtin_fmaf(w2[j], nx, __builtin_fmaf(w1[j], cur[j], __builtin_fmaf(w0[j], prev[j], bs[j])));
        }
        if (t < L.T) *(u32x4*)(ys + (int64_t)t * L.yst) = V::pack(out);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            prev[j] = cur[j];
            cur[j] = next[j];
        }
    }
    if (keep_cache) *(u32x4*)((T*)L.cache_out + cache_off) = last;
}

// One frame (T = 1, a streaming call of a one-frame block): y = bias + w0 * cache_in + w1 * x
// (the right neighbour is past the call, so zero) and cache_out = x. A thread owns one 16-byte
// channel chunk at P (b, s) positions, q + p * NQ for p = 0..P-1, so that each of its P slices is
// coalesced across the threads; it issues all 2 P loads before the first use, the grid is small
// enough to be resident at once, and the taps are loaded once per thread. Each position's
// cache_in is read before its cache_out is written by the same thread, so the two may be the
// same buffer.
constexpr int kTconvPos = 4;

template <typename T, int P>
__global__ __launch_bounds__(kTconvThreads) void tconv_frame_kernel(TconvLaunch L) {
    using V = Vec<T>;
    constexpr int N = V::N;
    const uint32_t ncv = (uint32_t)L.C / N;
    const uint32_t npos = (uint32_t)L.B * (uint32_t)L.S;
    const uint32_t nq = (npos + P - 1) / P;
    const uint32_t r = blockIdx.x * (uint32_t)kTconvThreads + threadIdx.x;
    const int cv = (int)(r % ncv);
    const uint32_t q = r / ncv;
    if (q >= nq) return;
    const int c0 = cv * N;

    u32x4 xv[P], cv_in[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const uint32_t pos = min(q + p * nq, npos - 1);   // past the end: re-read the last (unused)
        const int b = (int)(pos / (uint32_t)L.S), s = (int)(pos % (uint32_t)L.S);
        xv[p] = *(const u32x4*)((const T*)L.x + (int64_t)b * L.xsb + (int64_t)s * L.xss + c0);
        cv_in[p] = L.cache_in ? *(const u32x4*)((const T*)L.cache_in + (int64_t)pos * L.C + c0)
                              : u32x4{0u, 0u, 0u, 0u};
    }
    float w0[N], w1[N], bs[N];
    {
        f32x4 tw[3 * N / 4], tb[N / 4];
#pragma unroll
        for (int k = 0; k < 3 * N / 4; ++k) tw[k] = *(const f32x4*)(L.weight + 3 * c0 + 4 * k);
#pragma unroll
        for (int k = 0; k < N / 4; ++k)
            tb[k] = L.bias ? *(const f32x4*)(L.bias + c0 + 4 * k) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < N; ++j) {
            w0[j] = tw[(3 * j) / 4][(3 * j) % 4];
            w1[j] = tw[(3 * j + 1) / 4][(3 * j + 1) % 4];
            bs[j] = tb[j / 4][j % 4];
        }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const uint32_t pos = q + p * nq;
        if (pos < npos) {
            const int b = (int)(pos / (uint32_t)L.S), s = (int)(pos % (uint32_t)L.S);
            float cur[N], left[N], out[N];
            V::unpack(xv[p], cur);
            V::unpack(cv_in[p], left);
#pragma unroll
            for (int j = 0; j < N; ++j) out[j] = __builtin_fmaf(w1[j], cur[j], __builtin_fmaf(w0[j], left[j], bs[j]));
            *(u32x4*)((T*)L.y + (int64_t)b * L.ysb + (int64_t)s * L.yss + c0) = V::pack(out);
            if (L.cache_out) *(u32x4*)((T*)L.cache_out + (int64_t)pos * L.C + c0) = xv[p];
        }
    }
}

template <typename T, int TF> hipError_t launch_tf(const TconvLaunch& L, hipStream_t s) {
    constexpr int N = Vec<T>::N;
    const int64_t threads = (int64_t)L.B * L.S * (L.C / N) * ((L.T + TF - 1) / TF);
    const int64_t blocks = (threads + kTconvThreads - 1) / kTconvThreads;
    if (blocks * kTconvThreads > 0x7FFFFFFF) return hipErrorInvalidValue;   // 32-bit indices
    hipLaunchKernelGGL((tconv_kernel<T, TF>), dim3((unsigned)blocks), dim3(kTconvThreads), 0, s, L);
    return hipGetLastError();
}

// one frame: tconv_frame_kernel; otherwise frames per thread to fit short calls (a streaming
// block of a few frames) or long ones
template <typename T> hipError_t launch_t(const TconvLaunch& L, hipStream_t s) {
    if (L.T <= 1) {
        constexpr int N = Vec<T>::N;
        const int64_t nq = ((int64_t)L.B * L.S + kTconvPos - 1) / kTconvPos;
        const int64_t threads = nq * (L.C / N);
        const int64_t blocks = (threads + kTconvThreads - 1) / kTconvThreads;
        if (blocks * kTconvThreads > 0x7FFFFFFF || (int64_t)L.B * L.S > 0x7FFFFFFF)
            return hipErrorInvalidValue;   // 32-bit indices
        hipLaunchKernelGGL((tconv_frame_kernel<T, kTconvPos>), dim3((unsigned)blocks), dim3(kTconvThreads), 0, s, L);
        return hipGetLastError();
    }
    if (L.T <= 4) return launch_tf<T, 4>(L, s);
    return launch_tf<T, kTconvFrames>(L, s);
}

}  // namespace

hipError_t tconv_launch(const TconvLaunch& L, hipStream_t s) {
    return L.bf16 ? launch_t<__bf16>(L, s) : launch_t<float>(L, s);
}

}  // namespace gdn
