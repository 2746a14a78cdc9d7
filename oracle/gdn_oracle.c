/*
 * gdn_oracle.c -- plain fp64 reference for the frame-wise Gated DeltaNet (GDN) recurrence.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library. The GPU library (frame_wise_gated_libgdn_amd) never calls it,
 * includes none of it and shares no code with it.
 *
 * What is computed, and where it comes from
 * -----------------------------------------
 * Gen-hub.ru, "NVIDIA SANA-WM: минутное 720p видео с одной видеокарты", section
 * "Архитектура: четыре нетривиальных решения":
 *   - GDN keeps a recurrent state of fixed size D x D per head, whatever the video length;
 *   - it is processed frame by frame ("покадровая" GDN);
 *   - a decay gate gamma lowers the weight of older frames;
 *   - a delta-rule correction writes into the state only the difference between the target
 *     value and the value the state currently predicts;
 *   - keys are scaled by 1/sqrt(D*S), D = head dim, S = spatial tokens per frame.
 * The pages give these steps in words only. The equations taken here (one state update per
 * frame; the S tokens of a frame all read the state left by the previous frame):
 *
 *     Kt  = c * K_f                      c = key_scale (default 1/sqrt(D*S))
 *     P   = Kt * M                       prediction of the frame's values from the old state
 *     R   = V_f - gamma_f * P            delta-rule residual (R = V_f when use_delta == 0)
 *     U   = Kt^T * R
 *     M   = gamma_f * M + beta_f * U     decay, then write
 *     O_f = Q_f * M                      every token of frame f reads the state after frame f
 *
 * With gamma = beta = 1 and use_delta = 0 this is the additive block state of SANA-Video's
 * block-causal linear attention (talk "SANA-Video: Efficient Video Generation with Block Linear
 * Diffusion Transformer", ICLR 2026 oral, passage on the block KV cache: the D x D state of block
 * i is the state of block i-1 plus block i's own K^T V contribution).
 *
 * Orientation: M[i][j], row i = key dimension, column j = value dimension (row-vector
 * convention, O = Q M).
 *
 * Layout of every array (all fp64, contiguous, row-major):
 *     q, k, v, o        [B][H][F*S][D]    token t = f*S + s
 *     gamma, beta       [B][H][F]
 *     state_in/out      [B][H][D][D]
 *
 * The loops are written for a reader, not for speed. Threads (OpenMP) run independent (b, h)
 * pairs only; each pair is computed by one thread in the order above.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One (b, h) pair over F frames. M holds the running state on entry and on exit. */
static void gdn_head(int D, int S, int F, int use_delta, double c,
                     const double* q, const double* k, const double* v,
                     const double* gamma, const double* beta,
                     double* M, double* o,
                     double* Kt, double* P, double* R, double* U)
{
    for (int f = 0; f < F; ++f) {
        const double* Kf = k + (size_t)f * S * D;
        const double* Vf = v + (size_t)f * S * D;
        const double* Qf = q + (size_t)f * S * D;
        double* Of = o + (size_t)f * S * D;
        const double g = gamma[f];
        const double bt = beta[f];

        /* scaled keys */
        for (int s = 0; s < S; ++s)
            for (int i = 0; i < D; ++i)
                Kt[(size_t)s * D + i] = c * Kf[(size_t)s * D + i];

        /* prediction P = Kt M (old state) */
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int i = 0; i < D; ++i)
                    acc += Kt[(size_t)s * D + i] * M[(size_t)i * D + j];
                P[(size_t)s * D + j] = acc;
            }

        /* residual R = V - gamma P, or R = V without the delta term */
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < D; ++j)
                R[(size_t)s * D + j] = use_delta ? Vf[(size_t)s * D + j] - g * P[(size_t)s * D + j]
                                                 : Vf[(size_t)s * D + j];

        /* U = Kt^T R */
        for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int s = 0; s < S; ++s)
                    acc += Kt[(size_t)s * D + i] * R[(size_t)s * D + j];
                U[(size_t)i * D + j] = acc;
            }

        /* state update M = gamma M + beta U */
        for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j)
                M[(size_t)i * D + j] = g * M[(size_t)i * D + j] + bt * U[(size_t)i * D + j];

        /* output O = Q M (new state) */
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int i = 0; i < D; ++i)
                    acc += Qf[(size_t)s * D + i] * M[(size_t)i * D + j];
                Of[(size_t)s * D + j] = acc;
            }
    }
}

/*
 * Forward over all F frames for every (b, h).
 * key_scale <= 0 selects the default 1/sqrt(D*S).
 * state_in may be NULL (zero initial state); state_out may be NULL (not returned).
 * nthreads <= 0 lets OpenMP choose. Returns 0 on success, 1 on bad sizes, 2 on a NULL
 * required pointer, 3 when scratch memory cannot be allocated.
 */
int gdn_oracle_forward(int B, int H, int D, int S, int F, int use_delta, double key_scale,
                       const double* q, const double* k, const double* v,
                       const double* gamma, const double* beta, const double* state_in,
                       double* o, double* state_out, int nthreads)
{
    if (B < 1 || H < 1 || D < 1 || S < 1 || F < 1) return 1;
    if (!q || !k || !v || !gamma || !beta || !o) return 2;
    const double c = key_scale > 0.0 ? key_scale : 1.0 / sqrt((double)D * (double)S);
    const int nbh = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int bh = 0; bh < nbh; ++bh) {
        const size_t tok = (size_t)F * S * D;
        double* M = (double*)calloc((size_t)D * D, sizeof(double));
        double* U = (double*)malloc((size_t)D * D * sizeof(double));
        double* Kt = (double*)malloc((size_t)S * D * sizeof(double));
        double* P = (double*)malloc((size_t)S * D * sizeof(double));
        double* R = (double*)malloc((size_t)S * D * sizeof(double));
        if (!M || !U || !Kt || !P || !R) {
            failed |= 1;
        } else {
            if (state_in) memcpy(M, state_in + (size_t)bh * D * D, (size_t)D * D * sizeof(double));
            gdn_head(D, S, F, use_delta, c, q + bh * tok, k + bh * tok, v + bh * tok,
                     gamma + (size_t)bh * F, beta + (size_t)bh * F, M, o + bh * tok, Kt, P, R, U);
            if (state_out) memcpy(state_out + (size_t)bh * D * D, M, (size_t)D * D * sizeof(double));
        }
        free(M); free(U); free(Kt); free(P); free(R);
    }
    (void)nthreads;
    return failed ? 3 : 0;
}

/*
 * One streaming step: a single frame from a given state (the cached-state rollout of the
 * SANA-Video talk's block KV cache passage and the chunk-causal / distilled autoregressive
 * modes of the gen-hub.ru article, section "Три режима на любой вкус").
 * q, k, v, o: [B][H][S][D]; gamma, beta: [B][H]; state_in: [B][H][D][D] (required).
 * state_out == NULL means the new state is not committed (it is computed and dropped).
 */
int gdn_oracle_step(int B, int H, int D, int S, int use_delta, double key_scale,
                    const double* q, const double* k, const double* v,
                    const double* gamma, const double* beta, const double* state_in,
                    double* o, double* state_out, int nthreads)
{
    if (!state_in) return 2;
    return gdn_oracle_forward(B, H, D, S, 1, use_delta, key_scale, q, k, v, gamma, beta,
                              state_in, o, state_out, nthreads);
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
