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

/*
 * Low-precision inputs: Q, K and V given as 8-bit floating-point codes with one fp32 scale per
 * (b, h, frame) for each tensor (the mixed-precision quantisation that SANA-Streaming fuses with
 * its GDN kernel: jefxiong.cn daily digest, SANA-Streaming item, contribution (3); SANA-WM's
 * NVFP4 deployment: chatpaper.ai English abstract). The code format is OCP FP8 E4M3 (OCP 8-bit
 * Floating Point Specification, E4M3): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities.
 * An element's value is scale[b][h][f] * E4M3(code). The recurrence then runs unchanged on
 * those values (gdn_oracle_forward).
 */
double gdn_oracle_e4m3(unsigned code)
{
    const int sgn = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);                 /* 2^(1-7) * (m / 8) */
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -mag : mag;
}

/* q8, k8, v8: codes [B][H][F*S][D]; q_scale, k_scale, v_scale: [B][H][F]. Other arguments and
   return codes as gdn_oracle_forward. */
int gdn_oracle_forward_fp8(int B, int H, int D, int S, int F, int use_delta, double key_scale,
                           const unsigned char* q8, const unsigned char* k8, const unsigned char* v8,
                           const double* q_scale, const double* k_scale, const double* v_scale,
                           const double* gamma, const double* beta, const double* state_in,
                           double* o, double* state_out, int nthreads)
{
    if (B < 1 || H < 1 || D < 1 || S < 1 || F < 1) return 1;
    if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale) return 2;
    const size_t n = (size_t)B * H * F * S * D;
    double* q = (double*)malloc(n * sizeof(double));
    double* k = (double*)malloc(n * sizeof(double));
    double* v = (double*)malloc(n * sizeof(double));
    int rc = 3;
    if (q && k && v) {
        for (size_t e = 0; e < n; ++e) {
            const size_t frame = e / ((size_t)S * D);       /* (b h) * F + f */
            q[e] = q_scale[frame] * gdn_oracle_e4m3(q8[e]);
            k[e] = k_scale[frame] * gdn_oracle_e4m3(k8[e]);
            v[e] = v_scale[frame] * gdn_oracle_e4m3(v8[e]);
        }
        rc = gdn_oracle_forward(B, H, D, S, F, use_delta, key_scale, q, k, v, gamma, beta, state_in,
                                o, state_out, nthreads);
    }
    free(q); free(k); free(v);
    return rc;
}

/*
 * Backward (gradients) of the forward above for a scalar loss L whose gradients with respect
 * to the outputs are given: d_o = dL/dO [B][H][F*S][D] and d_state_out = dL/dstate_out
 * [B][H][D][D] (NULL: zero). Returns dq, dk, dv [B][H][F*S][D], dgamma, dbeta [B][H][F] and,
 * when d_state_in is not NULL, dL/dstate_in [B][H][D][D]. key_scale is a constant (no gradient).
 *
 * The pages define only the forward; this is its reverse-mode derivative, written as the adjoint
 * of each forward line, visited in reverse order. For frame f, with G = dL/dM_f accumulated from
 * later frames and from state_out:
 *     O_f = Q_f M_f              ->  dQ_f = dO_f M_f^T ;  G += Q_f^T dO_f
 *     M_f = gamma M + beta U     ->  dU = beta G ;  dgamma_f = <G, M> ;  dbeta_f = <G, U> ;
 *                                    G_prev = gamma G
 *     U = Kt^T R                 ->  dKt = R dU^T ;  dR = Kt dU
 *     R = V - gamma P            ->  dV_f = dR ;  dP = -gamma dR ;  dgamma_f -= <dR, P>
 *                                    (R = V without the delta term: dV_f = dR, no dP)
 *     P = Kt M                   ->  dKt += dP M^T ;  G_prev += Kt^T dP
 *     Kt = c K_f                 ->  dK_f = c dKt
 * where M is the state before frame f. The forward states are recomputed first and kept.
 */
static void gdn_head_backward(int D, int S, int F, int use_delta, double c,
                              const double* q, const double* k, const double* v,
                              const double* gamma, const double* beta, const double* d_o,
                              double* Ms, double* G, double* dq, double* dk, double* dv,
                              double* dgamma, double* dbeta,
                              double* Kt, double* P, double* R, double* U, double* dU,
                              double* dR, double* dKt, double* Gp)
{
    const size_t DD = (size_t)D * D;
    /* forward states: Ms[0] = state before frame 0, Ms[f + 1] = state after frame f */
    for (int f = 0; f < F; ++f) {
        const double* Kf = k + (size_t)f * S * D;
        const double* Vf = v + (size_t)f * S * D;
        const double* M = Ms + (size_t)f * DD;
        double* Mn = Ms + (size_t)(f + 1) * DD;
        for (size_t e = 0; e < (size_t)S * D; ++e) Kt[e] = c * Kf[e];
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int i = 0; i < D; ++i) acc += Kt[(size_t)s * D + i] * M[(size_t)i * D + j];
                R[(size_t)s * D + j] = use_delta ? Vf[(size_t)s * D + j] - gamma[f] * acc
                                                 : Vf[(size_t)s * D + j];
            }
        for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int s = 0; s < S; ++s) acc += Kt[(size_t)s * D + i] * R[(size_t)s * D + j];
                Mn[(size_t)i * D + j] = gamma[f] * M[(size_t)i * D + j] + beta[f] * acc;
            }
    }

    for (int f = F - 1; f >= 0; --f) {
        const double* Qf = q + (size_t)f * S * D;
        const double* Kf = k + (size_t)f * S * D;
        const double* Vf = v + (size_t)f * S * D;
        const double* dOf = d_o + (size_t)f * S * D;
        const double* M = Ms + (size_t)f * DD;         /* state before frame f */
        const double* Mf = Ms + (size_t)(f + 1) * DD;  /* state after frame f */
        const double g = gamma[f], bt = beta[f];

        /* O_f = Q_f M_f */
        for (int s = 0; s < S; ++s)
            for (int i = 0; i < D; ++i) {
                double acc = 0.0;
                for (int j = 0; j < D; ++j) acc += dOf[(size_t)s * D + j] * Mf[(size_t)i * D + j];
                dq[(size_t)f * S * D + (size_t)s * D + i] = acc;
            }
        for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int s = 0; s < S; ++s) acc += Qf[(size_t)s * D + i] * dOf[(size_t)s * D + j];
                G[(size_t)i * D + j] += acc;
            }

        /* recompute the frame's intermediates: Kt, P, R, U */
        for (size_t e = 0; e < (size_t)S * D; ++e) Kt[e] = c * Kf[e];
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int i = 0; i < D; ++i) acc += Kt[(size_t)s * D + i] * M[(size_t)i * D + j];
                P[(size_t)s * D + j] = acc;
                R[(size_t)s * D + j] = use_delta ? Vf[(size_t)s * D + j] - g * acc : Vf[(size_t)s * D + j];
            }
        for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int s = 0; s < S; ++s) acc += Kt[(size_t)s * D + i] * R[(size_t)s * D + j];
                U[(size_t)i * D + j] = acc;
            }

        /* M_f = gamma M + beta U */
        double dg = 0.0, db = 0.0;
        for (size_t e = 0; e < DD; ++e) {
            dU[e] = bt * G[e];
            dg += G[e] * M[e];
            db += G[e] * U[e];
            Gp[e] = g * G[e];
        }

        /* U = Kt^T R */
        for (int s = 0; s < S; ++s)
            for (int i = 0; i < D; ++i) {
                double acc = 0.0;
                for (int j = 0; j < D; ++j) acc += R[(size_t)s * D + j] * dU[(size_t)i * D + j];
                dKt[(size_t)s * D + i] = acc;
            }
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int i = 0; i < D; ++i) acc += Kt[(size_t)s * D + i] * dU[(size_t)i * D + j];
                dR[(size_t)s * D + j] = acc;
            }

        /* R = V - gamma P */
        for (size_t e = 0; e < (size_t)S * D; ++e) dv[(size_t)f * S * D + e] = dR[e];
        if (use_delta) {
            for (size_t e = 0; e < (size_t)S * D; ++e) dg -= dR[e] * P[e];
            /* P = Kt M with dP = -gamma dR */
            for (int s = 0; s < S; ++s)
                for (int i = 0; i < D; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < D; ++j) acc += -g * dR[(size_t)s * D + j] * M[(size_t)i * D + j];
                    dKt[(size_t)s * D + i] += acc;
                }
            for (int i = 0; i < D; ++i)
                for (int j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int s = 0; s < S; ++s) acc += Kt[(size_t)s * D + i] * (-g * dR[(size_t)s * D + j]);
                    Gp[(size_t)i * D + j] += acc;
                }
        }

        /* Kt = c K_f */
        for (size_t e = 0; e < (size_t)S * D; ++e) dk[(size_t)f * S * D + e] = c * dKt[e];
        dgamma[f] = dg;
        dbeta[f] = db;
        memcpy(G, Gp, DD * sizeof(double));
    }
}

int gdn_oracle_backward(int B, int H, int D, int S, int F, int use_delta, double key_scale,
                        const double* q, const double* k, const double* v,
                        const double* gamma, const double* beta, const double* state_in,
                        const double* d_o, const double* d_state_out,
                        double* dq, double* dk, double* dv, double* dgamma, double* dbeta,
                        double* d_state_in, int nthreads)
{
    if (B < 1 || H < 1 || D < 1 || S < 1 || F < 1) return 1;
    if (!q || !k || !v || !gamma || !beta || !d_o || !dq || !dk || !dv || !dgamma || !dbeta)
        return 2;
    const double c = key_scale > 0.0 ? key_scale : 1.0 / sqrt((double)D * (double)S);
    const int nbh = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int bh = 0; bh < nbh; ++bh) {
        const size_t tok = (size_t)F * S * D, DD = (size_t)D * D, SD = (size_t)S * D;
        double* Ms = (double*)calloc((size_t)(F + 1) * DD, sizeof(double));
        double* G = (double*)calloc(DD, sizeof(double));
        double* U = (double*)malloc(DD * sizeof(double));
        double* dU = (double*)malloc(DD * sizeof(double));
        double* Gp = (double*)malloc(DD * sizeof(double));
        double* Kt = (double*)malloc(SD * sizeof(double));
        double* P = (double*)malloc(SD * sizeof(double));
        double* R = (double*)malloc(SD * sizeof(double));
        double* dR = (double*)malloc(SD * sizeof(double));
        double* dKt = (double*)malloc(SD * sizeof(double));
        if (!Ms || !G || !U || !dU || !Gp || !Kt || !P || !R || !dR || !dKt) {
            failed |= 1;
        } else {
            if (state_in) memcpy(Ms, state_in + (size_t)bh * DD, DD * sizeof(double));
            if (d_state_out) memcpy(G, d_state_out + (size_t)bh * DD, DD * sizeof(double));
            gdn_head_backward(D, S, F, use_delta, c, q + bh * tok, k + bh * tok, v + bh * tok,
                              gamma + (size_t)bh * F, beta + (size_t)bh * F, d_o + bh * tok, Ms, G,
                              dq + bh * tok, dk + bh * tok, dv + bh * tok, dgamma + (size_t)bh * F,
                              dbeta + (size_t)bh * F, Kt, P, R, U, dU, dR, dKt, Gp);
            if (d_state_in) memcpy(d_state_in + (size_t)bh * DD, G, DD * sizeof(double));
        }
        free(Ms); free(G); free(U); free(dU); free(Gp); free(Kt); free(P); free(R); free(dR); free(dKt);
    }
    (void)nthreads;
    return failed ? 3 : 0;
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
