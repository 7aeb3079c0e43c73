/*
 * linattn_oracle.c -- plain fp64 CPU oracle for causal / decode / non-causal
 * linear attention with the feature map phi(x) = elu(x) + 1.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no source, header, table or helper with the HIP library: it is the
 * slow, obviously-correct definition that the GPU path is compared against.
 *
 * Sources (web pages, cited by title and section):
 *  - "Attention Kernel Mask" (allenlu2009.github.io, 2024-11-17), section
 *    "Cumsum" (the plain-words cumulative-sum derivation): the running key sum
 *    S_t = S_{t-1} + k_t, the running context Z_t = Z_{t-1} + k_t v_t^T, the
 *    normaliser D_t = q_t^T S_t + eps and the output out_t = q_t^T Z_t / D_t;
 *    causality means position t only sees positions <= t.
 *  - The same page, "How to accelerate causal linear attention", mode 2 (pure
 *    sequential / RNN mode): one token at a time with a fixed-size state, which
 *    is the decode step below.
 *  - The same page, "Non-causal Bi-Directional Attention Kernel" and its
 *    remark that non-causal attention reads the inputs once: one global
 *    Z = sum_t phi(k_t) v_t^T and S = sum_t phi(k_t) applied to every query.
 *  - "Segment-Wise Attention" (GitHub issue on an Infini-attention
 *    implementation): the compressive memory is an associative matrix whose
 *    update and retrieval follow the linear-attention rule of "Transformers
 *    are RNNs" (Katharopoulos et al. 2020), carried from segment to segment.
 *    That paper's feature map is elu(x) + 1; the printed recurrence uses raw
 *    q, k, and the reading taken here applies phi to both q and k.
 *
 * Conventions: every input tensor is contiguous [BH][N][d] float (bf16 and
 * fp32 inputs are both exact in float); all arithmetic and all outputs are
 * double.  The state Z of one head is [d][d] row-major with Z[j][c] = sum over
 * tokens of phi(k)_j * v_c (key dimension first), S is [d].
 *
 * Parity pins: brute-force quadratic masked evaluation, an independent chunked
 * evaluator, closed forms and invariants (see the oracle pin tests).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* elu(x) + 1 with elu's alpha = 1: x + 1 above zero, exp(x) at or below it.
 * Both branches give 1 at x = 0. */
static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Causal linear attention over N tokens of each of BH heads, recurrent form
 * ("Attention Kernel Mask", section "Cumsum"), with phi applied to q and k:
 *   f = phi(k_t);  Z += f v_t^T;  S += f;
 *   g = phi(q_t);  out_t = (g^T Z) / (g . S + eps)
 * The update comes before the readout, so token t attends to itself.
 * z_in / s_in (may be NULL = zeros) give the state carried in from earlier
 * segments ("Segment-Wise Attention"); z_out / s_out (may be NULL) receive the
 * state after the last token.  out may be NULL (state only).
 */
void oracle_causal(long BH, long N, long d, double eps,
                   const float *q, const float *k, const float *v,
                   const double *z_in, const double *s_in,
                   double *out, double *z_out, double *s_out)
{
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < BH; ++h) {
        double *Z = (double *)calloc((size_t)(d * d), sizeof(double));
        double *S = (double *)calloc((size_t)d, sizeof(double));
        double *f = (double *)malloc((size_t)d * sizeof(double));
        double *g = (double *)malloc((size_t)d * sizeof(double));
        long t, j, c;
        if (z_in) memcpy(Z, z_in + h * d * d, (size_t)(d * d) * sizeof(double));
        if (s_in) memcpy(S, s_in + h * d, (size_t)d * sizeof(double));
        for (t = 0; t < N; ++t) {
            const float *kt = k + (h * N + t) * d;
            const float *vt = v + (h * N + t) * d;
            const float *qt = q + (h * N + t) * d;
            for (j = 0; j < d; ++j) f[j] = phi((double)kt[j]);
            for (j = 0; j < d; ++j) {
                for (c = 0; c < d; ++c) Z[j * d + c] += f[j] * (double)vt[c];
                S[j] += f[j];
            }
            if (!out) continue;
            for (j = 0; j < d; ++j) g[j] = phi((double)qt[j]);
            {
                double den = 0.0;
                double *ot = out + (h * N + t) * d;
                for (j = 0; j < d; ++j) den += g[j] * S[j];
                den += eps;
                for (c = 0; c < d; ++c) {
                    double num = 0.0;
                    for (j = 0; j < d; ++j) num += g[j] * Z[j * d + c];
                    ot[c] = num / den;
                }
            }
        }
        if (z_out) memcpy(z_out + h * d * d, Z, (size_t)(d * d) * sizeof(double));
        if (s_out) memcpy(s_out + h * d, S, (size_t)d * sizeof(double));
        free(Z); free(S); free(f); free(g);
    }
}

/*
 * One generation step for each of BH heads ("Attention Kernel Mask", mode 2,
 * pure sequential / RNN mode: fixed memory, no KV cache).  q, k, v are [BH][d];
 * Z [BH][d][d] and S [BH][d] are updated in place, then read:
 *   Z += phi(k) v^T;  S += phi(k);  out = phi(q)^T Z / (phi(q) . S + eps)
 */
void oracle_decode_step(long BH, long d, double eps,
                        const float *q, const float *k, const float *v,
                        double *Z, double *S, double *out)
{
    long h;
#pragma omp parallel for schedule(static)
    for (h = 0; h < BH; ++h) {
        double *Zh = Z + h * d * d, *Sh = S + h * d;
        const float *qh = q + h * d, *kh = k + h * d, *vh = v + h * d;
        double den = 0.0;
        long j, c;
        for (j = 0; j < d; ++j) {
            double fj = phi((double)kh[j]);
            for (c = 0; c < d; ++c) Zh[j * d + c] += fj * (double)vh[c];
            Sh[j] += fj;
        }
        for (j = 0; j < d; ++j) den += phi((double)qh[j]) * Sh[j];
        den += eps;
        for (c = 0; c < d; ++c) {
            double num = 0.0;
            for (j = 0; j < d; ++j) num += phi((double)qh[j]) * Zh[j * d + c];
            out[h * d + c] = num / den;
        }
    }
}

/*
 * Non-causal (bidirectional) linear attention ("Attention Kernel Mask",
 * section "Non-causal Bi-Directional Attention Kernel"): every query sees all
 * N keys of its head through one global state
 *   Z = sum_t phi(k_t) v_t^T,  S = sum_t phi(k_t),
 *   out_t = phi(q_t)^T Z / (phi(q_t) . S + eps).
 * z_out / s_out (may be NULL) receive the global state; out may be NULL.
 */
void oracle_noncausal(long BH, long N, long d, double eps,
                      const float *q, const float *k, const float *v,
                      double *out, double *z_out, double *s_out)
{
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < BH; ++h) {
        double *Z = (double *)calloc((size_t)(d * d), sizeof(double));
        double *S = (double *)calloc((size_t)d, sizeof(double));
        double *g = (double *)malloc((size_t)d * sizeof(double));
        long t, j, c;
        for (t = 0; t < N; ++t) {
            const float *kt = k + (h * N + t) * d;
            const float *vt = v + (h * N + t) * d;
            for (j = 0; j < d; ++j) {
                double fj = phi((double)kt[j]);
                for (c = 0; c < d; ++c) Z[j * d + c] += fj * (double)vt[c];
                S[j] += fj;
            }
        }
        for (t = 0; out && t < N; ++t) {
            const float *qt = q + (h * N + t) * d;
            double *ot = out + (h * N + t) * d;
            double den = 0.0;
            for (j = 0; j < d; ++j) g[j] = phi((double)qt[j]);
            for (j = 0; j < d; ++j) den += g[j] * S[j];
            den += eps;
            for (c = 0; c < d; ++c) {
                double num = 0.0;
                for (j = 0; j < d; ++j) num += g[j] * Z[j * d + c];
                ot[c] = num / den;
            }
        }
        if (z_out) memcpy(z_out + h * d * d, Z, (size_t)(d * d) * sizeof(double));
        if (s_out) memcpy(s_out + h * d, S, (size_t)d * sizeof(double));
        free(Z); free(S); free(g);
    }
}

/*
 * Compressive memory of one segment ("Segment-Wise Attention": the memory is
 * an associative matrix, read and updated with the linear-attention rule of
 * "Transformers are RNNs", and the thread's read divides the retrieved memory
 * by the retrieved norm term).  Every query of the segment reads only what
 * the earlier segments left in the memory:
 *   out_t = phi(q_t)^T M / (phi(q_t) . n + eps)   with (M, n) = (z_in, s_in),
 * and then the memory takes in the whole segment:
 *   z_out = M + sum_t phi(k_t) v_t^T,  s_out = n + sum_t phi(k_t).
 * z_in / s_in may be NULL (zeros: the first segment reads 0 / eps); out,
 * z_out, s_out may be NULL (not written).
 */
void oracle_memory(long BH, long N, long d, double eps,
                   const float *q, const float *k, const float *v,
                   const double *z_in, const double *s_in,
                   double *out, double *z_out, double *s_out)
{
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < BH; ++h) {
        double *mem = (double *)calloc((size_t)(d * d), sizeof(double));
        double *norm = (double *)calloc((size_t)d, sizeof(double));
        double *fq = (double *)malloc((size_t)d * sizeof(double));
        long t, i, c;
        if (z_in) memcpy(mem, z_in + h * d * d, (size_t)(d * d) * sizeof(double));
        if (s_in) memcpy(norm, s_in + h * d, (size_t)d * sizeof(double));
        /* the read, from the memory of the earlier segments */
        for (t = 0; out && t < N; ++t) {
            const float *qrow = q + (h * N + t) * d;
            double *orow = out + (h * N + t) * d;
            double retrieved_norm = eps;
            for (i = 0; i < d; ++i) fq[i] = phi((double)qrow[i]);
            for (i = 0; i < d; ++i) retrieved_norm += fq[i] * norm[i];
            for (c = 0; c < d; ++c) {
                double retrieved = 0.0;
                for (i = 0; i < d; ++i) retrieved += fq[i] * mem[i * d + c];
                orow[c] = retrieved / retrieved_norm;
            }
        }
        /* the update, with every key and value of the segment */
        for (t = 0; t < N; ++t) {
            const float *krow = k + (h * N + t) * d;
            const float *vrow = v + (h * N + t) * d;
            for (i = 0; i < d; ++i) {
                const double fk = phi((double)krow[i]);
                for (c = 0; c < d; ++c) mem[i * d + c] += fk * (double)vrow[c];
                norm[i] += fk;
            }
        }
        if (z_out) memcpy(z_out + h * d * d, mem, (size_t)(d * d) * sizeof(double));
        if (s_out) memcpy(s_out + h * d, norm, (size_t)d * sizeof(double));
        free(mem); free(norm); free(fq);
    }
}

/*
 * Unnormalised causal linear attention: the chunk formulas of "Attention
 * Kernel Mask" (section "How to accelerate causal linear attention", the
 * chunk-sequential and materialised modes) as printed, with no denominator.
 * Per head, with phi on q and k:
 *   W = W_in + sum_{i<=t} phi(k_i) v_i^T,   out_t = phi(q_t)^T W.
 * w_in (may be NULL = zeros) is the carried-in context.  The key sums of the
 * normalised form do not enter; the carried state is the same Z.
 */
void oracle_causal_unnormalized(long BH, long N, long d,
                                const float *q, const float *k, const float *v,
                                const double *w_in, double *out)
{
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < BH; ++h) {
        double *W = (double *)calloc((size_t)(d * d), sizeof(double));
        double *phik = (double *)malloc((size_t)d * sizeof(double));
        double *phiq = (double *)malloc((size_t)d * sizeof(double));
        long t, a, b;
        if (w_in) memcpy(W, w_in + h * d * d, (size_t)(d * d) * sizeof(double));
        for (t = 0; t < N; ++t) {
            const float *krow = k + (h * N + t) * d, *vrow = v + (h * N + t) * d, *qrow = q + (h * N + t) * d;
            double *orow = out + (h * N + t) * d;
            for (a = 0; a < d; ++a) phik[a] = phi((double)krow[a]);
            for (a = 0; a < d; ++a)
                for (b = 0; b < d; ++b) W[a * d + b] += phik[a] * (double)vrow[b];
            for (a = 0; a < d; ++a) phiq[a] = phi((double)qrow[a]);
            for (b = 0; b < d; ++b) {
                double acc = 0.0;
                for (a = 0; a < d; ++a) acc += phiq[a] * W[a * d + b];
                orow[b] = acc;
            }
        }
        free(W); free(phik); free(phiq);
    }
}

/* Derivative of phi: 1 above zero, exp(x) at or below it (both sides give 1
 * at x = 0, so phi is continuously differentiable). */
static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

/*
 * Gradients of the causal form -- the backward pass of a training step,
 * which "Attention Kernel Mask" names (the "Training-Backward" row of its
 * table under "Causal Attention Training and Inferencing"; training needs
 * every output, the cumsum problem of its "Causal linear attention" notes)
 * but does not write out.  They are the exact derivatives of oracle_causal's
 * definition.  With f_t = phi(k_t), g_t = phi(q_t), Z_t, S_t the running
 * state (state_in included) and D_t = g_t . S_t + eps, out_t = Z_t^T g_t / D_t,
 * for an upstream gradient dout_t (and dz_out, ds_out reaching the final
 * state; NULL = zeros):
 *   dn_t = dout_t / D_t,  dD_t = -(dout_t . out_t) / D_t
 *   dq_t = (Z_t dn_t + S_t dD_t) * phi'(q_t)                 (forward sweep)
 *   R_t = dz_out + sum_{u>=t} g_u dn_u^T,  r_t = ds_out + sum_{u>=t} g_u dD_u
 *   dk_t = (R_t v_t + r_t) * phi'(k_t),  dv_t = R_t^T f_t     (reverse sweep)
 *   dz_in = R_0,  ds_in = r_0
 * (Segment-Wise Attention discusses detaching the carried memory from the
 * graph: that is dz_out = ds_out = NULL and ignoring dz_in, ds_in.)
 * dout, dq, dk, dv: [BH][N][d]; dz_* [BH][d][d]; ds_* [BH][d]; dz_in / ds_in
 * may be NULL.
 */
void oracle_causal_bwd(long BH, long N, long d, double eps,
                       const float *q, const float *k, const float *v, const float *dout,
                       const double *z_in, const double *s_in,
                       const double *dz_out, const double *ds_out,
                       double *dq, double *dk, double *dv, double *dz_in, double *ds_in)
{
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < BH; ++h) {
        double *Z = (double *)calloc((size_t)(d * d), sizeof(double));
        double *S = (double *)calloc((size_t)d, sizeof(double));
        double *R = (double *)calloc((size_t)(d * d), sizeof(double));
        double *r = (double *)calloc((size_t)d, sizeof(double));
        double *dn = (double *)malloc((size_t)(N * d + 1) * sizeof(double));
        double *dD = (double *)malloc((size_t)(N + 1) * sizeof(double));
        double *f = (double *)malloc((size_t)d * sizeof(double));
        double *g = (double *)malloc((size_t)d * sizeof(double));
        double *o = (double *)malloc((size_t)d * sizeof(double));
        long t, j, c;
        if (z_in) memcpy(Z, z_in + h * d * d, (size_t)(d * d) * sizeof(double));
        if (s_in) memcpy(S, s_in + h * d, (size_t)d * sizeof(double));
        /* forward sweep: the state after token t, the output, dq_t */
        for (t = 0; t < N; ++t) {
            const float *kt = k + (h * N + t) * d, *vt = v + (h * N + t) * d;
            const float *qt = q + (h * N + t) * d, *dot = dout + (h * N + t) * d;
            double den = 0.0, dodo = 0.0;
            for (j = 0; j < d; ++j) f[j] = phi((double)kt[j]);
            for (j = 0; j < d; ++j) {
                for (c = 0; c < d; ++c) Z[j * d + c] += f[j] * (double)vt[c];
                S[j] += f[j];
            }
            for (j = 0; j < d; ++j) g[j] = phi((double)qt[j]);
            for (j = 0; j < d; ++j) den += g[j] * S[j];
            den += eps;
            for (c = 0; c < d; ++c) {
                double num = 0.0;
                for (j = 0; j < d; ++j) num += g[j] * Z[j * d + c];
                o[c] = num / den;
                dodo += (double)dot[c] * o[c];
            }
            dD[t] = -dodo / den;
            for (c = 0; c < d; ++c) dn[t * d + c] = (double)dot[c] / den;
            for (j = 0; j < d; ++j) {
                double acc = S[j] * dD[t];
                for (c = 0; c < d; ++c) acc += Z[j * d + c] * dn[t * d + c];
                dq[(h * N + t) * d + j] = acc * dphi((double)qt[j]);
            }
        }
        /* reverse sweep: the adjoint state R_t, r_t (token t included), dk_t, dv_t */
        if (dz_out) memcpy(R, dz_out + h * d * d, (size_t)(d * d) * sizeof(double));
        if (ds_out) memcpy(r, ds_out + h * d, (size_t)d * sizeof(double));
        for (t = N - 1; t >= 0; --t) {
            const float *kt = k + (h * N + t) * d, *vt = v + (h * N + t) * d;
            const float *qt = q + (h * N + t) * d;
            for (j = 0; j < d; ++j) g[j] = phi((double)qt[j]);
            for (j = 0; j < d; ++j) {
                for (c = 0; c < d; ++c) R[j * d + c] += g[j] * dn[t * d + c];
                r[j] += g[j] * dD[t];
            }
            for (j = 0; j < d; ++j) f[j] = phi((double)kt[j]);
            for (j = 0; j < d; ++j) {
                double acc = r[j];
                for (c = 0; c < d; ++c) acc += R[j * d + c] * (double)vt[c];
                dk[(h * N + t) * d + j] = acc * dphi((double)kt[j]);
            }
            for (c = 0; c < d; ++c) {
                double acc = 0.0;
                for (j = 0; j < d; ++j) acc += R[j * d + c] * f[j];
                dv[(h * N + t) * d + c] = acc;
            }
        }
        if (dz_in) memcpy(dz_in + h * d * d, R, (size_t)(d * d) * sizeof(double));
        if (ds_in) memcpy(ds_in + h * d, r, (size_t)d * sizeof(double));
        free(Z); free(S); free(R); free(r); free(dn); free(dD); free(f); free(g); free(o);
    }
}
