/*
 * la_oracle.c -- slow, plain fp64 CPU reference for causal kernelized linear
 * attention in fast-weight form.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no header, helper or constant with
 * the GPU path.
 *
 * Every function is the plain definition written out, one token at a time,
 * in double precision.  Inputs are widened exactly from the stored fp32 /
 * bf16 values by the caller.
 *
 * Sources (pages, by title and section):
 *  - "Attention is also an FFN" (kwkr.cn/news/587576):
 *      sec. 2.1  kernel factorisation, state S_i = sum_{j<=i} phi(k_j) v_j^T and
 *                its outer-product recurrence; query y_i = phi(q_i)^T S_i
 *      sec. 3.2  decayed recurrence S_t = lambda S_{t-1} + phi(k_t) v_t^T
 *      sec. 4.1  elu+1 feature map; single-token step updates the state first
 *                and then queries it; the state starts at zero
 *      sec. 4.2  normaliser z_i = z_{i-1} + phi(k_i), output divided by
 *                phi(q_i)^T z_i plus a small eps; the decay may also be put on z
 *      sec. 5.1  ReLU named beside elu+1 as a feature map with a controlled
 *                output range
 *  - "From standard attention to linear attention" (tqpw.cn/news/561043):
 *      sec. 3    non-causal closed form with S = sum phi(k) v^T, Z = sum phi(k)
 *      sec. 4.1  elu(x)+1 with alpha = 1
 *      sec. 4.2  random cos/sin features of omega . x scaled by 1/sqrt(m),
 *                with a prefactor exp(|x|^2/2) h(x) and an optional h such as
 *                exp(-|x|^2/2)
 *      sec. 6    autoregressive step: S += k v^T, Z += k, then query; the
 *                forward takes a key padding mask and a key sequence of its
 *                own length (cross attention)
 *      sec. 2    cross attention: N queries against M keys and values
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes): update-then-query (inclusive state); the decay multiplies z as well
 * as S; the denominator is (phi(q)^T z + eps); the random-feature map is
 * phi(x) = exp(-|x'|^2/2)/sqrt(m) [cos(omega x'), sin(omega x')] with
 * x' = s x, cosine block first; the two other prefactors the section's
 * formula allows are 1/sqrt(m) (h = exp(-|x|^2/2) cancelling exp(|x|^2/2):
 * the Gaussian kernel) and exp(+|x'|^2/2)/sqrt(m) (h = 1: the kernel
 * exp(x'.y')).  A key padding mask removes a key's term phi(k_j) v_j^T and
 * phi(k_j) from every sum; positions keep their indices, so the decay of the
 * other keys is unchanged.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

enum {
    ORC_PHI_ELU1 = 0,
    ORC_PHI_TRIG_RF = 1,          /* prefactor exp(-|x'|^2/2) / sqrt(m) */
    ORC_PHI_RELU = 2,
    ORC_PHI_TRIG_RF_PLAIN = 3,    /* prefactor 1 / sqrt(m) */
    ORC_PHI_TRIG_RF_SOFTMAX = 4   /* prefactor exp(+|x'|^2/2) / sqrt(m) */
};

/* Feature map of one vector x[dk] -> out[F].
 * ELU1: F = dk, phi(x)_f = x_f + 1 if x_f > 0 else exp(x_f)   (elu, alpha=1, plus 1)
 * RELU: F = dk, phi(x)_f = x_f if x_f > 0 else 0
 * TRIG_RF*: F = 2m, x' = scale * x, u_r = omega_r . x',
 *          phi = c(x') * [cos u_1..cos u_m, sin u_1..sin u_m] with
 *          c = exp(-|x'|^2/2)/sqrt(m) (TRIG_RF), 1/sqrt(m) (PLAIN),
 *          exp(+|x'|^2/2)/sqrt(m) (SOFTMAX) */
void orc_phi(int kind, const double* x, int dk, int m, const double* omega,
             double scale, double* out)
{
    if (kind == ORC_PHI_ELU1) {
        for (int f = 0; f < dk; ++f)
            out[f] = x[f] > 0.0 ? x[f] + 1.0 : exp(x[f]);
        return;
    }
    if (kind == ORC_PHI_RELU) {
        for (int f = 0; f < dk; ++f)
            out[f] = x[f] > 0.0 ? x[f] : 0.0;
        return;
    }
    double* xs = (double*)malloc(sizeof(double) * (size_t)dk);
    double nrm2 = 0.0;
    for (int f = 0; f < dk; ++f) {
        xs[f] = scale * x[f];
        nrm2 += xs[f] * xs[f];
    }
    double c;
    if (kind == ORC_PHI_TRIG_RF) c = exp(-0.5 * nrm2) / sqrt((double)m);
    else if (kind == ORC_PHI_TRIG_RF_SOFTMAX) c = exp(0.5 * nrm2) / sqrt((double)m);
    else c = 1.0 / sqrt((double)m);
    for (int r = 0; r < m; ++r) {
        double u = 0.0;
        for (int f = 0; f < dk; ++f) u += omega[(size_t)r * dk + f] * xs[f];
        out[r] = c * cos(u);
        out[m + r] = c * sin(u);
    }
    free(xs);
}

static int feat_dim(int kind, int dk, int m)
{
    return (kind == ORC_PHI_ELU1 || kind == ORC_PHI_RELU) ? dk : 2 * m;
}

/* Causal forward over nbh independent (batch, head) rows.
 *   q,k [nbh][N][dk], v [nbh][N][dv], lam [nbh], S0 [nbh][F][dv] / z0 [nbh][F]
 *   (NULL = zero state), kpm [nbh][N] key padding mask (nonzero = the key
 *   adds nothing; NULL = none), y [nbh][N][dv], S_out / z_out (NULL = not written),
 *   kappa [nbh][N] (NULL = not computed): the cancellation factor
 *   |phi q|^T zbar / |phi(q)^T z + eps| with zbar the same recurrence on |phi(k)|.
 * Per token: S <- lam S + phi(k) v^T ; z <- lam z + phi(k) ;
 *            y = phi(q)^T S / (phi(q)^T z + eps). */
void orc_causal(const double* q, const double* k, const double* v,
                long nbh, long N, int dk, int dv, int kind, int m,
                const double* omega, double scale, const double* lam, double eps,
                const unsigned char* kpm,
                const double* S0, const double* z0,
                double* y, double* S_out, double* z_out, double* kappa)
{
    const int F = feat_dim(kind, dk, m);
    double* S = (double*)malloc(sizeof(double) * (size_t)F * dv);
    double* z = (double*)malloc(sizeof(double) * (size_t)F);
    double* zb = (double*)malloc(sizeof(double) * (size_t)F);
    double* pk = (double*)malloc(sizeof(double) * (size_t)F);
    double* pq = (double*)malloc(sizeof(double) * (size_t)F);
    for (long bh = 0; bh < nbh; ++bh) {
        const double L = lam[bh];
        if (S0) memcpy(S, S0 + (size_t)bh * F * dv, sizeof(double) * (size_t)F * dv);
        else memset(S, 0, sizeof(double) * (size_t)F * dv);
        if (z0) memcpy(z, z0 + (size_t)bh * F, sizeof(double) * (size_t)F);
        else memset(z, 0, sizeof(double) * (size_t)F);
        for (int f = 0; f < F; ++f) zb[f] = fabs(z[f]);
        for (long i = 0; i < N; ++i) {
            const double* ki = k + ((size_t)bh * N + i) * dk;
            const double* qi = q + ((size_t)bh * N + i) * dk;
            const double* vi = v + ((size_t)bh * N + i) * dv;
            orc_phi(kind, ki, dk, m, omega, scale, pk);
            orc_phi(kind, qi, dk, m, omega, scale, pq);
            if (kpm && kpm[(size_t)bh * N + i])  /* padded key: no term */
                for (int f = 0; f < F; ++f) pk[f] = 0.0;
            for (int f = 0; f < F; ++f) {
                double* Sf = S + (size_t)f * dv;
                for (int d = 0; d < dv; ++d) Sf[d] = L * Sf[d] + pk[f] * vi[d];
                z[f] = L * z[f] + pk[f];
                zb[f] = L * zb[f] + fabs(pk[f]);
            }
            double den = 0.0, denb = 0.0;
            for (int f = 0; f < F; ++f) {
                den += pq[f] * z[f];
                denb += fabs(pq[f]) * zb[f];
            }
            double* yi = y + ((size_t)bh * N + i) * dv;
            for (int d = 0; d < dv; ++d) {
                double num = 0.0;
                for (int f = 0; f < F; ++f) num += pq[f] * S[(size_t)f * dv + d];
                yi[d] = num / (den + eps);
            }
            if (kappa) kappa[(size_t)bh * N + i] = denb / fabs(den + eps);
        }
        if (S_out) memcpy(S_out + (size_t)bh * F * dv, S, sizeof(double) * (size_t)F * dv);
        if (z_out) memcpy(z_out + (size_t)bh * F, z, sizeof(double) * (size_t)F);
    }
    free(S); free(z); free(zb); free(pk); free(pq);
}

/* Non-causal forward: S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j) over the
 * whole sequence (no decay), then y_i = phi(q_i)^T S / (phi(q_i)^T z + eps). */
void orc_noncausal(const double* q, const double* k, const double* v,
                   long nbh, long N, int dk, int dv, int kind, int m,
                   const double* omega, double scale, double eps, double* y)
{
    const int F = feat_dim(kind, dk, m);
    double* S = (double*)malloc(sizeof(double) * (size_t)F * dv);
    double* z = (double*)malloc(sizeof(double) * (size_t)F);
    double* p = (double*)malloc(sizeof(double) * (size_t)F);
    for (long bh = 0; bh < nbh; ++bh) {
        memset(S, 0, sizeof(double) * (size_t)F * dv);
        memset(z, 0, sizeof(double) * (size_t)F);
        for (long j = 0; j < N; ++j) {
            const double* kj = k + ((size_t)bh * N + j) * dk;
            const double* vj = v + ((size_t)bh * N + j) * dv;
            orc_phi(kind, kj, dk, m, omega, scale, p);
            for (int f = 0; f < F; ++f) {
                for (int d = 0; d < dv; ++d) S[(size_t)f * dv + d] += p[f] * vj[d];
                z[f] += p[f];
            }
        }
        for (long i = 0; i < N; ++i) {
            const double* qi = q + ((size_t)bh * N + i) * dk;
            orc_phi(kind, qi, dk, m, omega, scale, p);
            double den = 0.0;
            for (int f = 0; f < F; ++f) den += p[f] * z[f];
            double* yi = y + ((size_t)bh * N + i) * dv;
            for (int d = 0; d < dv; ++d) {
                double num = 0.0;
                for (int f = 0; f < F; ++f) num += p[f] * S[(size_t)f * dv + d];
                yi[d] = num / (den + eps);
            }
        }
    }
    free(S); free(z); free(p);
}

/* Cross attention, non-causal: Nq queries against Nk keys and values of the
 * same (batch, head) row.  S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j)
 * over the keys j that kpm (per row, Nk bytes; NULL = none) does not mark,
 * then y_i = phi(q_i)^T S / (phi(q_i)^T z + eps) for every query. */
void orc_cross(const double* q, const double* k, const double* v,
               long nbh, long Nq, long Nk, int dk, int dv, int kind, int m,
               const double* omega, double scale, double eps,
               const unsigned char* kpm, double* y)
{
    const int F = feat_dim(kind, dk, m);
    double* S = (double*)malloc(sizeof(double) * (size_t)F * dv);
    double* z = (double*)malloc(sizeof(double) * (size_t)F);
    double* p = (double*)malloc(sizeof(double) * (size_t)F);
    for (long bh = 0; bh < nbh; ++bh) {
        memset(S, 0, sizeof(double) * (size_t)F * dv);
        memset(z, 0, sizeof(double) * (size_t)F);
        for (long j = 0; j < Nk; ++j) {
            if (kpm && kpm[(size_t)bh * Nk + j]) continue;
            const double* kj = k + ((size_t)bh * Nk + j) * dk;
            const double* vj = v + ((size_t)bh * Nk + j) * dv;
            orc_phi(kind, kj, dk, m, omega, scale, p);
            for (int f = 0; f < F; ++f) {
                for (int d = 0; d < dv; ++d) S[(size_t)f * dv + d] += p[f] * vj[d];
                z[f] += p[f];
            }
        }
        for (long i = 0; i < Nq; ++i) {
            const double* qi = q + ((size_t)bh * Nq + i) * dk;
            orc_phi(kind, qi, dk, m, omega, scale, p);
            double den = 0.0;
            for (int f = 0; f < F; ++f) den += p[f] * z[f];
            double* yi = y + ((size_t)bh * Nq + i) * dv;
            for (int d = 0; d < dv; ++d) {
                double num = 0.0;
                for (int f = 0; f < F; ++f) num += p[f] * S[(size_t)f * dv + d];
                yi[d] = num / (den + eps);
            }
        }
    }
    free(S); free(z); free(p);
}

/* One recurrent decode step on nbh head-states, in place:
 *   q,k [nbh][dk], v [nbh][dv], S [nbh][F][dv], z [nbh][F], y [nbh][dv].
 * S <- lam S + phi(k) v^T ; z <- lam z + phi(k) ; y = phi(q)^T S / (phi(q)^T z + eps). */
void orc_decode_step(const double* q, const double* k, const double* v,
                     long nbh, int dk, int dv, int kind, int m,
                     const double* omega, double scale, const double* lam, double eps,
                     double* S, double* z, double* y)
{
    const int F = feat_dim(kind, dk, m);
    double* pk = (double*)malloc(sizeof(double) * (size_t)F);
    double* pq = (double*)malloc(sizeof(double) * (size_t)F);
    for (long bh = 0; bh < nbh; ++bh) {
        const double L = lam[bh];
        double* Sb = S + (size_t)bh * F * dv;
        double* zb = z + (size_t)bh * F;
        orc_phi(kind, k + (size_t)bh * dk, dk, m, omega, scale, pk);
        orc_phi(kind, q + (size_t)bh * dk, dk, m, omega, scale, pq);
        const double* vb = v + (size_t)bh * dv;
        for (int f = 0; f < F; ++f) {
            for (int d = 0; d < dv; ++d)
                Sb[(size_t)f * dv + d] = L * Sb[(size_t)f * dv + d] + pk[f] * vb[d];
            zb[f] = L * zb[f] + pk[f];
        }
        double den = 0.0;
        for (int f = 0; f < F; ++f) den += pq[f] * zb[f];
        for (int d = 0; d < dv; ++d) {
            double num = 0.0;
            for (int f = 0; f < F; ++f) num += pq[f] * Sb[(size_t)f * dv + d];
            y[(size_t)bh * dv + d] = num / (den + eps);
        }
    }
    free(pk); free(pq);
}

/* Vector-Jacobian product of the feature map: dx = J_phi(x)^T dp for one
 * vector x[dk] and a gradient dp[F] with respect to phi(x).
 * ELU1: d phi_f / d x_f = 1 for x_f > 0, exp(x_f) otherwise.
 * RELU: 1 for x_f > 0, 0 otherwise.
 * TRIG_RF*: with x' = scale x, u_r = omega_r . x', phi = c [cos u, sin u] and
 *   c = exp(s |x'|^2 / 2) / sqrt(m) (s = -1, 0, +1 by kind):
 *   d phi / d x' = s x' phi^T + c [-sin u_r omega_r | cos u_r omega_r], so
 *   dx = scale (s x' (phi . dp) + c sum_r omega_r (-sin u_r dp_r + cos u_r dp_{m+r})). */
void orc_phi_vjp(int kind, const double* x, int dk, int m, const double* omega,
                 double scale, const double* dp, double* dx)
{
    if (kind == ORC_PHI_ELU1) {
        for (int f = 0; f < dk; ++f) dx[f] = dp[f] * (x[f] > 0.0 ? 1.0 : exp(x[f]));
        return;
    }
    if (kind == ORC_PHI_RELU) {
        for (int f = 0; f < dk; ++f) dx[f] = x[f] > 0.0 ? dp[f] : 0.0;
        return;
    }
    const double s = kind == ORC_PHI_TRIG_RF ? -1.0 : (kind == ORC_PHI_TRIG_RF_SOFTMAX ? 1.0 : 0.0);
    double* xs = (double*)malloc(sizeof(double) * (size_t)dk);
    double nrm2 = 0.0;
    for (int f = 0; f < dk; ++f) {
        xs[f] = scale * x[f];
        nrm2 += xs[f] * xs[f];
        dx[f] = 0.0;
    }
    const double c = exp(0.5 * s * nrm2) / sqrt((double)m);
    double phidp = 0.0;
    for (int r = 0; r < m; ++r) {
        double u = 0.0;
        for (int f = 0; f < dk; ++f) u += omega[(size_t)r * dk + f] * xs[f];
        const double cu = cos(u), su = sin(u);
        phidp += c * cu * dp[r] + c * su * dp[m + r];
        const double w = c * (-su * dp[r] + cu * dp[m + r]);
        for (int f = 0; f < dk; ++f) dx[f] += w * omega[(size_t)r * dk + f];
    }
    for (int f = 0; f < dk; ++f) dx[f] = scale * (dx[f] + s * xs[f] * phidp);
    free(xs);
}

/* Gradients of the causal forward (reverse mode of the recurrence of
 * orc_causal), for the loss L = sum_i g_i . y_i + <dS_out, S_{N-1}> +
 * <dz_out, z_{N-1}>.  Per (batch, head) row:
 *   forward, token order: S_i, z_i, den_i = phi(q_i).z_i + eps, y_i;
 *     dnum_i = g_i / den_i,  dden_i = -(g_i . y_i) / den_i,
 *     d phi(q_i) = S_i dnum_i + z_i dden_i,  dq_i = J_phi(q_i)^T d phi(q_i);
 *     and, forward mode in lambda, T_i = dS_i/dlambda = lambda T_{i-1} + S_{i-1}
 *     (t_i likewise; T = 0 before token 0, S_{-1} = S0), so that
 *     dlambda = sum_i [dnum_i . T_i^T phi(q_i) + dden_i t_i . phi(q_i)]
 *             + <dS_out, T_{N-1}> + <dz_out, t_{N-1}>;
 *   reverse, adjoint of the state: U_{N-1} = dS_out + phi(q_{N-1}) dnum_{N-1}^T,
 *     U_i = lambda U_{i+1} + phi(q_i) dnum_i^T (u likewise with dden), then
 *     d phi(k_i) = U_i v_i + u_i,  dv_i = U_i^T phi(k_i),
 *     dk_i = J_phi(k_i)^T d phi(k_i);  dS0 = lambda U_0, dz0 = lambda u_0.
 * kpm as in orc_causal (a padded key has phi(k) = 0 and gets dk = dv = 0).
 * g [nbh][N][dv]; dS_out [nbh][F][dv] / dz_out [nbh][F] may be NULL (zero);
 * outputs dq, dk [nbh][N][dk], dv [nbh][N][dv], dS0 [nbh][F][dv], dz0
 * [nbh][F] (NULL = not written), dlam [nbh].
 * Cancellation factors (kq, kk, kv [nbh][N], NULL = not computed): for each
 * gradient row, the largest sum of absolute values of the elementary terms
 * it is made of (the recurrences above run on |.|, with |dden_i| replaced by
 * sum_d |dnum_i,d y_i,d|, the terms of dden), over the row's largest |entry|;
 * the rounding error of any evaluation order is bounded relative to the
 * former, so kappa says how far the row's own size understates it
 * (the elementwise feature maps only). */
void orc_backward(const double* q, const double* k, const double* v, const double* gy,
                  long nbh, long N, int dk, int dv, int kind, int m,
                  const double* omega, double scale, const double* lam, double eps,
                  const unsigned char* kpm, const double* S0, const double* z0,
                  const double* dS_out, const double* dz_out,
                  double* dq, double* dkx, double* dvx, double* dS0, double* dz0, double* dlam,
                  double* kq, double* kk, double* kv)
{
    const int F = feat_dim(kind, dk, m);
    const size_t FD = (size_t)F * dv;
    double* S = (double*)malloc(sizeof(double) * FD);
    double* z = (double*)malloc(sizeof(double) * (size_t)F);
    double* T = (double*)malloc(sizeof(double) * FD);
    double* t = (double*)malloc(sizeof(double) * (size_t)F);
    double* Sp = (double*)malloc(sizeof(double) * FD);
    double* zp = (double*)malloc(sizeof(double) * (size_t)F);
    double* pq = (double*)malloc(sizeof(double) * (size_t)F * (N > 0 ? N : 1));
    double* pk = (double*)malloc(sizeof(double) * (size_t)F);
    double* dp = (double*)malloc(sizeof(double) * (size_t)F);
    double* dnum = (double*)malloc(sizeof(double) * (size_t)dv * (N > 0 ? N : 1));
    double* dden = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* ddb = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* y = (double*)malloc(sizeof(double) * (size_t)dv);
    double* Sb = (double*)malloc(sizeof(double) * FD);
    double* zb = (double*)malloc(sizeof(double) * (size_t)F);
    double* xb = (double*)malloc(sizeof(double) * (size_t)(F > dv ? F : dv));
    const int want_k = kq && kk && kv && (kind == ORC_PHI_ELU1 || kind == ORC_PHI_RELU);
    for (long bh = 0; bh < nbh; ++bh) {
        const double L = lam[bh];
        const double* qr = q + (size_t)bh * N * dk;
        const double* kr = k + (size_t)bh * N * dk;
        const double* vr = v + (size_t)bh * N * dv;
        const double* gr = gy + (size_t)bh * N * dv;
        const unsigned char* mr = kpm ? kpm + (size_t)bh * N : NULL;
        if (S0) memcpy(S, S0 + (size_t)bh * FD, sizeof(double) * FD);
        else memset(S, 0, sizeof(double) * FD);
        if (z0) memcpy(z, z0 + (size_t)bh * F, sizeof(double) * (size_t)F);
        else memset(z, 0, sizeof(double) * (size_t)F);
        memset(T, 0, sizeof(double) * FD);
        memset(t, 0, sizeof(double) * (size_t)F);
        for (size_t e = 0; e < FD; ++e) Sb[e] = S0 ? fabs(S0[(size_t)bh * FD + e]) : 0.0;
        for (int f = 0; f < F; ++f) zb[f] = z0 ? fabs(z0[(size_t)bh * F + f]) : 0.0;
        double dl = 0.0;
        /* forward, token order */
        for (long i = 0; i < N; ++i) {
            memcpy(Sp, S, sizeof(double) * FD);
            memcpy(zp, z, sizeof(double) * (size_t)F);
            orc_phi(kind, kr + (size_t)i * dk, dk, m, omega, scale, pk);
            if (mr && mr[i])
                for (int f = 0; f < F; ++f) pk[f] = 0.0;
            double* pqi = pq + (size_t)i * F;
            orc_phi(kind, qr + (size_t)i * dk, dk, m, omega, scale, pqi);
            const double* vi = vr + (size_t)i * dv;
            for (int f = 0; f < F; ++f) {
                for (int d = 0; d < dv; ++d) {
                    const size_t e = (size_t)f * dv + d;
                    T[e] = L * T[e] + Sp[e];
                    S[e] = L * S[e] + pk[f] * vi[d];
                    Sb[e] = L * Sb[e] + fabs(pk[f] * vi[d]);
                }
                t[f] = L * t[f] + zp[f];
                z[f] = L * z[f] + pk[f];
                zb[f] = L * zb[f] + fabs(pk[f]);
            }
            double den = eps;
            for (int f = 0; f < F; ++f) den += pqi[f] * z[f];
            const double* gi = gr + (size_t)i * dv;
            double gy_dot = 0.0;
            for (int d = 0; d < dv; ++d) {
                double num = 0.0;
                for (int f = 0; f < F; ++f) num += pqi[f] * S[(size_t)f * dv + d];
                y[d] = num / den;
                gy_dot += gi[d] * y[d];
            }
            double* dni = dnum + (size_t)i * dv;
            for (int d = 0; d < dv; ++d) dni[d] = gi[d] / den;
            dden[i] = -gy_dot / den;
            ddb[i] = 0.0;
            for (int d = 0; d < dv; ++d) ddb[i] += fabs(dni[d] * y[d]);
            for (int f = 0; f < F; ++f) {
                double a = z[f] * dden[i], b = t[f] * dden[i];
                for (int d = 0; d < dv; ++d) {
                    a += S[(size_t)f * dv + d] * dni[d];
                    b += T[(size_t)f * dv + d] * dni[d];
                }
                dp[f] = a;
                dl += pqi[f] * b;
            }
            orc_phi_vjp(kind, qr + (size_t)i * dk, dk, m, omega, scale, dp, dq + ((size_t)bh * N + i) * dk);
            if (want_k) {
                /* |terms| of d phi(q_i) = S_i dnum_i + z_i dden_i, through |phi'| */
                for (int f = 0; f < F; ++f) {
                    double a = zb[f] * ddb[i];
                    for (int d = 0; d < dv; ++d) a += Sb[(size_t)f * dv + d] * fabs(dni[d]);
                    dp[f] = a;
                }
                orc_phi_vjp(kind, qr + (size_t)i * dk, dk, m, omega, scale, dp, xb);
                const double* dqi = dq + ((size_t)bh * N + i) * dk;
                double num = 0.0, den2 = 0.0;
                for (int f = 0; f < dk; ++f) {
                    if (fabs(xb[f]) > num) num = fabs(xb[f]);
                    if (fabs(dqi[f]) > den2) den2 = fabs(dqi[f]);
                }
                kq[(size_t)bh * N + i] = den2 > 0.0 ? num / den2 : (num > 0.0 ? INFINITY : 1.0);
            }
        }
        if (dS_out)
            for (size_t e = 0; e < FD; ++e) dl += dS_out[(size_t)bh * FD + e] * T[e];
        if (dz_out)
            for (int f = 0; f < F; ++f) dl += dz_out[(size_t)bh * F + f] * t[f];
        dlam[bh] = dl;
        /* reverse: adjoint of the state (U, u reuse S, z) */
        if (dS_out) memcpy(S, dS_out + (size_t)bh * FD, sizeof(double) * FD);
        else memset(S, 0, sizeof(double) * FD);
        if (dz_out) memcpy(z, dz_out + (size_t)bh * F, sizeof(double) * (size_t)F);
        else memset(z, 0, sizeof(double) * (size_t)F);
        for (size_t e = 0; e < FD; ++e) Sb[e] = fabs(S[e]);
        for (int f = 0; f < F; ++f) zb[f] = fabs(z[f]);
        for (long i = N - 1; i >= 0; --i) {
            const double* pqi = pq + (size_t)i * F;
            const double* dni = dnum + (size_t)i * dv;
            const double w = (i < N - 1) ? L : 1.0;
            for (int f = 0; f < F; ++f) {
                for (int d = 0; d < dv; ++d) {
                    const size_t e = (size_t)f * dv + d;
                    S[e] = w * S[e] + pqi[f] * dni[d];
                    Sb[e] = w * Sb[e] + fabs(pqi[f] * dni[d]);
                }
                z[f] = w * z[f] + pqi[f] * dden[i];
                zb[f] = w * zb[f] + fabs(pqi[f]) * ddb[i];
            }
            orc_phi(kind, kr + (size_t)i * dk, dk, m, omega, scale, pk);
            const int padded = mr && mr[i];
            if (padded)
                for (int f = 0; f < F; ++f) pk[f] = 0.0;
            const double* vi = vr + (size_t)i * dv;
            double* dvi = dvx + ((size_t)bh * N + i) * dv;
            for (int d = 0; d < dv; ++d) {
                double a = 0.0;
                for (int f = 0; f < F; ++f) a += S[(size_t)f * dv + d] * pk[f];
                dvi[d] = a;
            }
            for (int f = 0; f < F; ++f) {
                double a = z[f];
                for (int d = 0; d < dv; ++d) a += S[(size_t)f * dv + d] * vi[d];
                dp[f] = padded ? 0.0 : a;
            }
            orc_phi_vjp(kind, kr + (size_t)i * dk, dk, m, omega, scale, dp, dkx + ((size_t)bh * N + i) * dk);
            if (want_k) {
                /* dv_i = U_i^T phi(k_i): |U|^T |phi(k)| */
                double num = 0.0, den2 = 0.0;
                for (int d = 0; d < dv; ++d) {
                    double a = 0.0;
                    for (int f = 0; f < F; ++f) a += Sb[(size_t)f * dv + d] * fabs(pk[f]);
                    if (a > num) num = a;
                    if (fabs(dvi[d]) > den2) den2 = fabs(dvi[d]);
                }
                kv[(size_t)bh * N + i] = den2 > 0.0 ? num / den2 : (num > 0.0 ? INFINITY : 1.0);
                /* d phi(k_i) = U_i v_i + u_i: |U| |v| + |u|, through |phi'| */
                for (int f = 0; f < F; ++f) {
                    double a = zb[f];
                    for (int d = 0; d < dv; ++d) a += Sb[(size_t)f * dv + d] * fabs(vi[d]);
                    dp[f] = padded ? 0.0 : a;
                }
                orc_phi_vjp(kind, kr + (size_t)i * dk, dk, m, omega, scale, dp, xb);
                const double* dki = dkx + ((size_t)bh * N + i) * dk;
                num = 0.0;
                den2 = 0.0;
                for (int f = 0; f < dk; ++f) {
                    if (fabs(xb[f]) > num) num = fabs(xb[f]);
                    if (fabs(dki[f]) > den2) den2 = fabs(dki[f]);
                }
                kk[(size_t)bh * N + i] = den2 > 0.0 ? num / den2 : (num > 0.0 ? INFINITY : 1.0);
            }
        }
        /* gradient of the initial state: S_0 = lambda S_{-1} + ... */
        const double w0 = N > 0 ? L : 1.0;
        if (dS0)
            for (size_t e = 0; e < FD; ++e) dS0[(size_t)bh * FD + e] = w0 * S[e];
        if (dz0)
            for (int f = 0; f < F; ++f) dz0[(size_t)bh * F + f] = w0 * z[f];
    }
    free(S); free(z); free(T); free(t); free(Sp); free(zp); free(pq); free(pk); free(dp);
    free(dnum); free(dden); free(ddb); free(y); free(Sb); free(zb); free(xb);
}

/* Largest |a_e| over largest |r_e| of one gradient row: its cancellation
 * factor (a: the row's terms on |.|); a zero row is 1, or infinite if its
 * terms are not zero. */
static double row_kappa(const double* a, const double* r, int n)
{
    double num = 0.0, den = 0.0;
    for (int e = 0; e < n; ++e) {
        if (fabs(a[e]) > num) num = fabs(a[e]);
        if (fabs(r[e]) > den) den = fabs(r[e]);
    }
    return den > 0.0 ? num / den : (num > 0.0 ? INFINITY : 1.0);
}

/* Gradients of orc_cross (non-causal; Nq queries, Nk keys) for the loss
 * L = sum_i g_i . y_i.  With S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j)
 * over the kept keys, den_i = phi(q_i).z + eps, y_i = phi(q_i)^T S / den_i,
 * dnum_i = g_i / den_i, dden_i = -(g_i . y_i) / den_i:
 *   d phi(q_i) = S dnum_i + z dden_i,  dq_i = J_phi(q_i)^T d phi(q_i);
 *   U = sum_i phi(q_i) dnum_i^T, u = sum_i phi(q_i) dden_i (all queries);
 *   d phi(k_j) = U v_j + u,  dv_j = U^T phi(k_j),  dk_j = J_phi(k_j)^T d phi(k_j)
 * (a padded key gets dk = dv = 0).  g [nbh][Nq][dv]; outputs dq [nbh][Nq][dk],
 * dk [nbh][Nk][dk], dv [nbh][Nk][dv].  Cancellation factors kq [nbh][Nq],
 * kk, kv [nbh][Nk] (NULL = not computed; elementwise feature maps only), as
 * in orc_backward: the sums above run on |.| (|dden_i| replaced by
 * sum_d |dnum_i,d y_i,d|), and each row's largest such entry is divided by
 * the row's largest |entry|. */
void orc_cross_backward(const double* q, const double* k, const double* v, const double* gy,
                        long nbh, long Nq, long Nk, int dk, int dv, int kind, int m,
                        const double* omega, double scale, double eps, const unsigned char* kpm,
                        double* dq, double* dkx, double* dvx, double* kq, double* kk, double* kv)
{
    const int want_k = kq && kk && kv && (kind == ORC_PHI_ELU1 || kind == ORC_PHI_RELU);
    const int F = feat_dim(kind, dk, m);
    const size_t FD = (size_t)F * dv;
    double* S = (double*)malloc(sizeof(double) * FD);
    double* z = (double*)malloc(sizeof(double) * (size_t)F);
    double* U = (double*)malloc(sizeof(double) * FD);
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* p = (double*)malloc(sizeof(double) * (size_t)F);
    double* dp = (double*)malloc(sizeof(double) * (size_t)F);
    double* dn = (double*)malloc(sizeof(double) * (size_t)dv);
    double* yq = (double*)malloc(sizeof(double) * (size_t)dv);
    double* Sb = (double*)malloc(sizeof(double) * FD);  /* |.| companions (kappa) */
    double* zb = (double*)malloc(sizeof(double) * (size_t)F);
    double* Ub = (double*)malloc(sizeof(double) * FD);
    double* ub = (double*)malloc(sizeof(double) * (size_t)F);
    double* xb = (double*)malloc(sizeof(double) * (size_t)(F > dv ? F : dv));
    for (long bh = 0; bh < nbh; ++bh) {
        memset(S, 0, sizeof(double) * FD);
        memset(z, 0, sizeof(double) * (size_t)F);
        memset(U, 0, sizeof(double) * FD);
        memset(u, 0, sizeof(double) * (size_t)F);
        memset(Sb, 0, sizeof(double) * FD);
        memset(zb, 0, sizeof(double) * (size_t)F);
        memset(Ub, 0, sizeof(double) * FD);
        memset(ub, 0, sizeof(double) * (size_t)F);
        for (long j = 0; j < Nk; ++j) {
            if (kpm && kpm[(size_t)bh * Nk + j]) continue;
            orc_phi(kind, k + ((size_t)bh * Nk + j) * dk, dk, m, omega, scale, p);
            const double* vj = v + ((size_t)bh * Nk + j) * dv;
            for (int f = 0; f < F; ++f) {
                for (int d = 0; d < dv; ++d) {
                    S[(size_t)f * dv + d] += p[f] * vj[d];
                    Sb[(size_t)f * dv + d] += fabs(p[f] * vj[d]);
                }
                z[f] += p[f];
                zb[f] += fabs(p[f]);
            }
        }
        for (long i = 0; i < Nq; ++i) {
            const double* qi = q + ((size_t)bh * Nq + i) * dk;
            const double* gi = gy + ((size_t)bh * Nq + i) * dv;
            orc_phi(kind, qi, dk, m, omega, scale, p);
            double den = eps;
            for (int f = 0; f < F; ++f) den += p[f] * z[f];
            double gyd = 0.0;
            for (int d = 0; d < dv; ++d) {
                double num = 0.0;
                for (int f = 0; f < F; ++f) num += p[f] * S[(size_t)f * dv + d];
                yq[d] = num / den;
                gyd += gi[d] * yq[d];
                dn[d] = gi[d] / den;
            }
            const double dd = -gyd / den;
            double ddb = 0.0;
            for (int d = 0; d < dv; ++d) ddb += fabs(dn[d] * yq[d]);
            for (int f = 0; f < F; ++f) {
                double a = z[f] * dd;
                for (int d = 0; d < dv; ++d) {
                    a += S[(size_t)f * dv + d] * dn[d];
                    U[(size_t)f * dv + d] += p[f] * dn[d];
                    Ub[(size_t)f * dv + d] += fabs(p[f] * dn[d]);
                }
                u[f] += p[f] * dd;
                ub[f] += fabs(p[f]) * ddb;
                dp[f] = a;
            }
            double* dqi = dq + ((size_t)bh * Nq + i) * dk;
            orc_phi_vjp(kind, qi, dk, m, omega, scale, dp, dqi);
            if (want_k) {
                for (int f = 0; f < F; ++f) {
                    double a = zb[f] * ddb;
                    for (int d = 0; d < dv; ++d) a += Sb[(size_t)f * dv + d] * fabs(dn[d]);
                    dp[f] = a;
                }
                orc_phi_vjp(kind, qi, dk, m, omega, scale, dp, xb);
                kq[(size_t)bh * Nq + i] = row_kappa(xb, dqi, dk);
            }
        }
        for (long j = 0; j < Nk; ++j) {
            const double* kj = k + ((size_t)bh * Nk + j) * dk;
            const double* vj = v + ((size_t)bh * Nk + j) * dv;
            double* dvj = dvx + ((size_t)bh * Nk + j) * dv;
            const int padded = kpm && kpm[(size_t)bh * Nk + j];
            orc_phi(kind, kj, dk, m, omega, scale, p);
            for (int d = 0; d < dv; ++d) {
                double a = 0.0;
                if (!padded)
                    for (int f = 0; f < F; ++f) a += U[(size_t)f * dv + d] * p[f];
                dvj[d] = a;
            }
            for (int f = 0; f < F; ++f) {
                double a = u[f];
                for (int d = 0; d < dv; ++d) a += U[(size_t)f * dv + d] * vj[d];
                dp[f] = padded ? 0.0 : a;
            }
            double* dkj = dkx + ((size_t)bh * Nk + j) * dk;
            orc_phi_vjp(kind, kj, dk, m, omega, scale, dp, dkj);
            if (want_k) {
                /* dv_j = U^T phi(k_j): |U|^T |phi(k_j)| */
                for (int d = 0; d < dv; ++d) {
                    double a = 0.0;
                    if (!padded)
                        for (int f = 0; f < F; ++f) a += Ub[(size_t)f * dv + d] * fabs(p[f]);
                    xb[d] = a;
                }
                kv[(size_t)bh * Nk + j] = row_kappa(xb, dvj, dv);
                /* d phi(k_j) = U v_j + u: |U| |v_j| + |u|, through |phi'| */
                for (int f = 0; f < F; ++f) {
                    double a = ub[f];
                    for (int d = 0; d < dv; ++d) a += Ub[(size_t)f * dv + d] * fabs(vj[d]);
                    dp[f] = padded ? 0.0 : a;
                }
                orc_phi_vjp(kind, kj, dk, m, omega, scale, dp, xb);
                kk[(size_t)bh * Nk + j] = row_kappa(xb, dkj, dk);
            }
        }
    }
    free(S); free(z); free(U); free(u); free(p); free(dp); free(dn);
    free(yq); free(Sb); free(zb); free(Ub); free(ub); free(xb);
}
