// Internal interface between the C-ABI layer (gdn_api.cpp) and the kernels (gdn_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Argument bundle of one launch sequence. Strides are in elements.
struct Launch {
    int B, H, D, S, F;
    int bf16;            // 1: Q/K/V/O are bf16; 0: fp32
    int use_delta;
    float c;             // key scale
    const void *q, *k, *v;
    void* o;
    int64_t sb, sh, st;  // Q/K/V strides
    int64_t ob, oh, ot;  // O strides
    const float *gamma, *beta, *state_in;
    float* state_out;
    void* canon;         // workspace: per-frame record handed from the products kernel to the scan
    float* part;         // workspace: per-split fp32 partial products (when nsplit > 1)
    void* mt;            // workspace: materialised per-frame states, transposed, in the I/O type
    int nsplit;          // S splits of the partial-product kernel
    int split_tokens;    // tokens per split (multiple of 64)
    int nchunk;          // S chunks of the output kernel
    int chunk_tokens;    // tokens per output chunk (multiple of 16)
    hipStream_t stream;
    hipEvent_t ev[4];    // optional stage events (nev of them)
    int nev;
};

// Enqueue the whole forward (all frames) / one streaming step. Return the HIP error of the
// launches (hipSuccess when all were enqueued).
hipError_t launch_forward(const Launch& L);
hipError_t launch_step(const Launch& L);

}  // namespace gdn
