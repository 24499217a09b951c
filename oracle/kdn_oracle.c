/*
 * kdn_oracle.c -- fp64 CPU oracle of the gated delta-rule / diagonal-Kalman
 * associative-memory recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only users of this file.  The HIP
 * library and its Python binding never load, link or call it, and the two
 * share no source: no header, no helper, no constant.
 *
 * What it computes is the plain token-by-token recurrence, in double
 * precision, in the order the pages give the steps.  No blocking, no chunking,
 * no reordering.  Pages cited (title, then the section used):
 *
 *   [TAB] "Внимание в LLM · часть 11 -- Память с поправкой" (tutorial on the
 *         delta rule): section "Сначала решить, сколько прошлого оставить"
 *         (gated state S_t = a_t S_{t-1} + w_t) and section "Записать не новое
 *         значение, а ошибку памяти" (read v^ = S^T k, compare e = v - v^,
 *         correct S += beta k e^T).
 *   [KDA] "معماری KDA: حذف تداخل حافظه با قانون دلتا در توالی‌های بلند" (Kimi
 *         Delta Attention article): section "تکامل قانون دلتا" (delta rule,
 *         beta = 1 replaces exactly) and section "از فراموشی کلی به فراموشی
 *         جزئی" (scalar retention applied to the whole state before the delta
 *         write; vector retention, one rate per key channel).
 *   [KDN] "给记忆装一个信任度探测器：Kalman Delta Networks 如何让AI知道自己
 *         "记得准不准"" (write-up of Kalman Delta Networks): section
 *         "把记忆问题重新想成一个滤波问题" (predict, then update with a gain
 *         derived from memory uncertainty and observation reliability) and
 *         section "对角近似：把矩阵压扁成一个向量" (diagonal covariance,
 *         per-channel update, mean-field projection whose mean is exact,
 *         information scaling mu of the precision increment).
 *         Isotropic KDN: section "各向同性近似：把整个头压缩成一个数" (one
 *         uncertainty scalar per head; the delta-rule form is kept and its
 *         scalar write strength is derived from the accumulated uncertainty
 *         and the observation reliability; otherwise shaped like KDA; the
 *         variance recursion is a Mobius map).
 *   [AFS] "Kalman Delta Networks: Uncertainty-aware Associative Memory"
 *         (explainer): section "Approximation 1: Diagonal KDN (Mean-Field
 *         Variational Inference)" and section "Approximation 2: Isotropic
 *         KDN (Single Scalar Uncertainty)".
 *
 * Readings of points the pages leave open (each is argued in the design
 * notes of the repository):
 *   - S is d_k x d_v and the read is v^ = S^T k.
 *   - The decay is applied before the read (Kalman predict, then update).
 *   - The output is read after the write: o_t = S_t^T q_t, with no scale.
 *   - Diagonal KDN predict: p- = a*a*p + xi (process noise xi per channel).
 *   - Gain: w = p- (.) k / s with s = r + sum_i p-_i k_i^2; this is the exact
 *     Kalman update of the mean under the diagonal prior, so the mean is exact.
 *   - Projection: the diagonal precision gains mu k_i^2 / r, i.e.
 *     p_i <- p-_i r / (r + mu p-_i k_i^2).  mu scales only the variance
 *     update, never the current write.
 *   - Degenerate values: s == 0 gives w = 0; r + mu p-_i k_i^2 == 0 leaves
 *     p_i = p-_i.
 *   - Isotropic KDN (covariance p I): the predict p I -> diag(a^2) p +
 *     diag(xi) is brought back to a multiple of I by the mean of its
 *     diagonal, p- = mean(a^2) p + mean(xi); the gain is exact under p- I,
 *     w = p- k / s with s = r + p- |k|^2 (write strength p- / s times k);
 *     the posterior precision I / p- + k k^T / r is brought back to a
 *     multiple of I by the mean of its diagonal, scaled by mu like the
 *     diagonal variant: 1/p = 1/p- + mu |k|^2 / (d_k r), i.e.
 *     p <- p- r / (r + (mu / d_k) p- |k|^2).  Degenerate values as above.
 *
 * Layouts (row-major, contiguous):
 *   q, k            [B, T, H, dk]       v, o        [B, T, H, dv]
 *   alpha           GDN: [B, T, H]      KDA/KDN:    [B, T, H, dk]
 *   beta            [B, T, H]           (not KDN)
 *   xi (proc noise) [B, T, H, dk]       r (obs noise) [B, T, H]   (KDN only)
 *   S0, S           [B, H, dk, dv]      p0, p       [B, H, dk] (isotropic: [B, H])
 *   xi and r as for diagonal KDN for the isotropic variant too.
 *
 * Variant codes: 0 DeltaNet, 1 Gated DeltaNet, 2 KDA, 3 diagonal KDN,
 * 4 isotropic KDN.
 */
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_DELTANET = 0, ORC_GATED_DELTANET = 1, ORC_KDA = 2, ORC_DIAG_KDN = 3,
       ORC_ISO_KDN = 4 };

/* One (batch, head) stream, tokens 0..T-1.  S (dk x dv) and p (dk; one value
 * for isotropic KDN) are the running state and are updated in place. */
static void run_stream(int variant, long T, long H, long dk, long dv, double mu,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta,
                       const double *xi, const double *r,
                       long b, long h, double *S, double *p, double *o,
                       double *a, double *w, double *e, double *pm)
{
    for (long t = 0; t < T; ++t) {
        const long tok = (b * T + t) * H + h;          /* index of (b,t,h) */
        const double *kt = k + tok * dk;
        const double *qt = q + tok * dk;
        const double *vt = v + tok * dv;

        /* 1. Decay vector: none, one rate for the whole state, or one rate
         *    per key channel ([TAB] gated state; [KDA] scalar -> vector). */
        for (long i = 0; i < dk; ++i) {
            if (variant == ORC_DELTANET)
                a[i] = 1.0;
            else if (variant == ORC_GATED_DELTANET)
                a[i] = alpha[tok];
            else
                a[i] = alpha[tok * dk + i];
        }

        /* 2. Write vector. */
        if (variant == ORC_DIAG_KDN) {
            /* Kalman predict of the per-channel variance ([KDN] filtering
             * section: predict tracks uncertainty under the drift). */
            for (long i = 0; i < dk; ++i)
                pm[i] = a[i] * a[i] * p[i] + xi[tok * dk + i];
            /* Innovation variance and gain under the diagonal prior ([KDN]
             * gain from uncertainty and observation reliability; diagonal
             * section: the projected mean is exact). */
            const double rt = r[tok];
            double s = rt;
            for (long i = 0; i < dk; ++i)
                s += pm[i] * kt[i] * kt[i];
            for (long i = 0; i < dk; ++i)
                w[i] = (s != 0.0) ? pm[i] * kt[i] / s : 0.0;
            /* Mean-field projection back to a diagonal: precision of channel
             * i grows by mu * k_i^2 / r ([KDN] diagonal section, information
             * scaling; [AFS] Approximation 1). */
            for (long i = 0; i < dk; ++i) {
                const double den = rt + mu * pm[i] * kt[i] * kt[i];
                p[i] = (den != 0.0) ? pm[i] * rt / den : pm[i];
            }
        } else if (variant == ORC_ISO_KDN) {
            /* One variance for the whole head ([KDN] isotropic section):
             * predict, brought back to a multiple of the identity by the mean
             * of the diagonal. */
            double a2 = 0.0, xm = 0.0, kk = 0.0;
            for (long i = 0; i < dk; ++i) {
                a2 += a[i] * a[i];
                xm += xi[tok * dk + i];
                kk += kt[i] * kt[i];
            }
            const double pmi = (a2 / (double)dk) * p[0] + xm / (double)dk;
            /* Exact gain under the isotropic prior: the delta rule with the
             * write strength pmi / s derived from the uncertainty and the
             * observation reliability. */
            const double rt = r[tok];
            const double s = rt + pmi * kk;
            for (long i = 0; i < dk; ++i)
                w[i] = (s != 0.0) ? pmi * kt[i] / s : 0.0;
            /* Precision gain averaged over the key channels, scaled by mu. */
            const double den = rt + (mu / (double)dk) * pmi * kk;
            p[0] = (den != 0.0) ? pmi * rt / den : pmi;
        } else {
            /* Delta rule write strength beta ([TAB] correct step). */
            const double bt = beta[tok];
            for (long i = 0; i < dk; ++i)
                w[i] = bt * kt[i];
        }

        /* 3. Decay the memory before the delta write ([KDA] forgetting). */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] *= a[i];

        /* 4. Read and compare: e = v - S^T k ([TAB] steps 1 and 2). */
        for (long j = 0; j < dv; ++j)
            e[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                e[j] += S[i * dv + j] * kt[i];
        for (long j = 0; j < dv; ++j)
            e[j] = vt[j] - e[j];

        /* 5. Correct: S += w e^T ([TAB] step 3). */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] += w[i] * e[j];

        /* 6. Read the output from the updated memory: o = S^T q. */
        double *ot = o + tok * dv;
        for (long j = 0; j < dv; ++j)
            ot[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                ot[j] += S[i * dv + j] * qt[i];
    }
}

/* Returns 0 on success, a negative code on a bad argument.  S0 may be NULL
 * (zero initial memory); p0 and p are used by diagonal KDN only.  S and p
 * receive the final state and may alias S0 and p0 exactly.  nthreads <= 0
 * uses the OpenMP default. */
int kdn_oracle_recurrence(int variant, long B, long T, long H, long dk, long dv,
                          double mu,
                          const double *q, const double *k, const double *v,
                          const double *alpha, const double *beta,
                          const double *xi, const double *r,
                          const double *S0, const double *p0,
                          double *o, double *S, double *p, int nthreads)
{
    if (variant < ORC_DELTANET || variant > ORC_ISO_KDN)
        return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -2;
    if (!q || !k || !v || !o || !S)
        return -3;
    if (variant != ORC_DELTANET && !alpha)
        return -4;
    const int kdn = variant == ORC_DIAG_KDN || variant == ORC_ISO_KDN;
    const long np = variant == ORC_DIAG_KDN ? dk : 1;   /* variances per stream */
    if (!kdn && !beta)
        return -5;
    if (kdn && (!xi || !r || !p0 || !p))
        return -6;

    const long BH = B * H;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        double *Sb = S + bh * dk * dv;
        double *pb = kdn ? p + bh * np : NULL;
        if (S0) {
            if (S0 + bh * dk * dv != Sb)
                memcpy(Sb, S0 + bh * dk * dv, sizeof(double) * dk * dv);
        } else {
            memset(Sb, 0, sizeof(double) * dk * dv);
        }
        if (pb && p0 + bh * np != pb)
            memcpy(pb, p0 + bh * np, sizeof(double) * np);

        double *scratch = (double *)malloc(sizeof(double) * (3 * dk + dv));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            fail = 1;
            continue;
        }
        double *a = scratch, *w = scratch + dk, *pm = scratch + 2 * dk;
        double *e = scratch + 3 * dk;
        run_stream(variant, T, H, dk, dv, mu, q, k, v, alpha, beta, xi, r,
                   b, h, Sb, pb, o, a, w, e, pm);
        free(scratch);
    }
    return fail ? -7 : 0;
}

/* Number of threads an OpenMP region started here would use. */
int kdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
