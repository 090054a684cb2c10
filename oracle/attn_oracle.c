/*
 * Float64 CPU oracle for scaled dot-product attention, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes is the plain definition, one query row at a time: each
 * matrix formula is the per-row formula applied to every row (eulerpad
 * "Attention backward", the conventions before Problem 1).  For one head
 * with Q (n x d), K (m x d), V (m x dv) and upstream gradient dO (n x dv),
 * and a scale s:
 *
 *   S_ij  = s * sum_l Q_il K_jl                 mlgrind "Forward"; eulerpad P1
 *   S_ij  = -inf for j > i when causal          mlgrind "Forward"; eulerpad P8
 *   P_i   = softmax(S_i), row max subtracted    mlgrind "Edge cases"; datatweets "Setup"
 *   O_i   = sum_j P_ij V_j                      mlgrind "Forward"; eulerpad P2
 *   LSE_i = M_i + ln Z_i  (natural log; the row statistic FlashAttention keeps
 *           in place of P, so that P_ij = exp(S_ij - LSE_i))
 *   dV_j  = sum_i P_ij dO_i                     eulerpad P2 (dV = A^T G)
 *   dP_ij = dO_i . V_j                          eulerpad P3 (dA = G V^T)
 *   D_i   = sum_j P_ij dP_ij                    eulerpad P4 (rowsum(A o dA))
 *   dS_ij = P_ij (dP_ij - D_i)                  eulerpad P4; mlgrind "Backward"
 *   dQ_i  = s * sum_j dS_ij K_j                 eulerpad P5
 *   dK_j  = s * sum_i dS_ij Q_i                 eulerpad P6
 *
 * D is taken from its definition, rowsum(dP o P).  The cheaper identity
 * rowsum(dP o P) = rowsum(dO o O) (the "Gradient of S" section of the
 * step-by-step derivation; mlgrind "Follow-up") is reported beside it as
 * D_alt so that tests can check the identity rather than assume it.
 *
 * Parity pins (what fixes this code to the pages, not to itself) live in
 * tests/test_oracle_*.py: the uniform-P worked examples of mlgrind
 * "Examples", the printed loss of the datatweets toy head, central finite
 * differences of L = sum(O o dO), closed forms, invariants, and the
 * known-wrong variants below, each of which must fail those checks.
 *
 * Layout: every tensor is contiguous [B, H, rows, cols] row-major float64.
 * Parallelism: OpenMP over (batch, head) pairs in the full routines and over
 * independent query rows in the sampled routines; neither changes what is
 * summed, only which thread sums it.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Known-wrong variants, used only as negative controls by the tests. */
enum {
    ORACLE_EXACT = 0,
    ORACLE_WRONG_DS_NO_CORRECTION = 1, /* dS = dP o P        (datatweets Exercise 1)       */
    ORACLE_WRONG_DS_DIAG_ONLY = 2,     /* dS = dP o P o (1-P) (chippytime section 3.2)      */
    ORACLE_WRONG_DV_NO_TRANSPOSE = 3,  /* dV = P dO (n == m)  (eulerpad mistake 1)          */
    ORACLE_WRONG_FLAT_JACOBIAN = 4,    /* one correction for the whole matrix (mistake 2)   */
    ORACLE_WRONG_DROP_SCALE = 5,       /* dQ, dK without s    (eulerpad mistake 3)          */
    ORACLE_WRONG_MASK_AFTER = 6,       /* zero P after an unmasked softmax (mistake 5)      */
    ORACLE_N_VARIANTS = 7
};

static double dot(const double* a, const double* b, long len) {
    double acc = 0.0;
    for (long t = 0; t < len; ++t) acc += a[t] * b[t];
    return acc;
}

/*
 * Row i of the softmax: fills S (m), returns M_i and Z_i.  Masked entries get
 * S = -inf and contribute exp(-inf) = 0 to Z (eulerpad P8).  Under the causal
 * mask key j is visible from row i when j <= i + off; off = 0 is the pages'
 * mask, where the entry j = i is always visible and M_i is finite.  A row
 * that sees no key returns M = -inf and Z = 0; callers give it all-zero
 * weights.
 */
static void score_row(const double* qi, const double* K, long i, long m, long d,
                      double scale, int causal, long off, int mask_scores, double* S,
                      double* M_out, double* Z_out) {
    double M = -INFINITY;
    for (long j = 0; j < m; ++j) {
        if (mask_scores && causal && j > i + off) {
            S[j] = -INFINITY;
        } else {
            S[j] = scale * dot(qi, K + j * d, d);
        }
        if (S[j] > M) M = S[j];
    }
    double Z = 0.0;
    if (M > -INFINITY)
        for (long j = 0; j < m; ++j) Z += exp(S[j] - M);
    *M_out = M;
    *Z_out = Z;
}

/*
 * Forward, full tensors: O [B,H,n,dv] and LSE [B,H,n].
 * Returns 0, or 1 on invalid sizes (m must be positive: a softmax over no
 * keys is undefined; causal requires n == m, mlgrind "Inputs").
 */
int oracle_attn_fwd(const double* q, const double* k, const double* v, double* o,
                    double* lse, long B, long H, long n, long m, long d, long dv,
                    double scale, int causal) {
    if (B < 0 || H < 0 || n < 0 || m <= 0 || d <= 0 || dv <= 0) return 1;
    if (causal && n != m) return 1;
    long heads = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < heads; ++bh) {
        const double* Q = q + bh * n * d;
        const double* K = k + bh * m * d;
        const double* V = v + bh * m * dv;
        double* S = (double*)malloc(sizeof(double) * (size_t)m);
        for (long i = 0; i < n; ++i) {
            double M, Z;
            score_row(Q + i * d, K, i, m, d, scale, causal, 0, 1, S, &M, &Z);
            double* oi = o + (bh * n + i) * dv;
            for (long c = 0; c < dv; ++c) oi[c] = 0.0;
            for (long j = 0; j < m; ++j) {
                double p = exp(S[j] - M) / Z;
                for (long c = 0; c < dv; ++c) oi[c] += p * V[j * dv + c];
            }
            lse[bh * n + i] = M + log(Z);
        }
        free(S);
    }
    return 0;
}

/*
 * Backward, full tensors.  P is rebuilt from Q and K here rather than kept
 * from the forward (mlgrind "Edge cases and conventions").
 *
 * Outputs (all required): dq [B,H,n,d], dk [B,H,m,d], dvv [B,H,m,dv],
 * Drow [B,H,n] = rowsum(dP o P), Drow_alt [B,H,n] = rowsum(dO o O),
 * o [B,H,n,dv], lse [B,H,n].  ds, if not NULL, receives dS [B,H,n,m] (meant
 * for tiny shapes).  `variant` selects a known-wrong formula for the
 * negative-control tests; 0 is the exact definition.
 */
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dvv, double* Drow, double* Drow_alt,
                    double* o, double* lse, double* ds, long B, long H, long n, long m,
                    long d, long dv, double scale, int causal, int variant) {
    if (B < 0 || H < 0 || n < 0 || m <= 0 || d <= 0 || dv <= 0) return 1;
    if (causal && n != m) return 1;
    if (variant < 0 || variant >= ORACLE_N_VARIANTS) return 1;
    if (variant == ORACLE_WRONG_DV_NO_TRANSPOSE && n != m) return 1;
    long heads = B * H;
    const double gscale = (variant == ORACLE_WRONG_DROP_SCALE) ? 1.0 : scale;
    const int mask_scores = (variant != ORACLE_WRONG_MASK_AFTER);

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < heads; ++bh) {
        const double* Q = q + bh * n * d;
        const double* K = k + bh * m * d;
        const double* V = v + bh * m * dv;
        const double* dO = dout + bh * n * dv;
        double* dQ = dq + bh * n * d;
        double* dK = dk + bh * m * d;
        double* dV = dvv + bh * m * dv;
        double* S = (double*)malloc(sizeof(double) * (size_t)m);
        double* P = (double*)malloc(sizeof(double) * (size_t)m);
        double* dP = (double*)malloc(sizeof(double) * (size_t)m);
        memset(dK, 0, sizeof(double) * (size_t)(m * d));
        memset(dV, 0, sizeof(double) * (size_t)(m * dv));

        /* The flattened-Jacobian mistake subtracts one total for the whole
         * matrix instead of each row's own sum; it needs that total first. */
        double flat_total = 0.0;
        if (variant == ORACLE_WRONG_FLAT_JACOBIAN) {
            for (long i = 0; i < n; ++i) {
                double M, Z;
                score_row(Q + i * d, K, i, m, d, scale, causal, 0, 1, S, &M, &Z);
                for (long j = 0; j < m; ++j)
                    flat_total += (exp(S[j] - M) / Z) * dot(dO + i * dv, V + j * dv, dv);
            }
        }

        for (long i = 0; i < n; ++i) {
            const double* qi = Q + i * d;
            const double* doi = dO + i * dv;
            double M, Z;
            score_row(qi, K, i, m, d, scale, causal, 0, mask_scores, S, &M, &Z);
            for (long j = 0; j < m; ++j) P[j] = exp(S[j] - M) / Z;
            if (!mask_scores && causal)
                for (long j = i + 1; j < m; ++j) P[j] = 0.0;
            lse[bh * n + i] = M + log(Z);

            double* oi = o + (bh * n + i) * dv;
            for (long c = 0; c < dv; ++c) oi[c] = 0.0;
            for (long j = 0; j < m; ++j)
                for (long c = 0; c < dv; ++c) oi[c] += P[j] * V[j * dv + c];

            double Di = 0.0;
            for (long j = 0; j < m; ++j) {
                dP[j] = dot(doi, V + j * dv, dv);
                Di += P[j] * dP[j];
            }
            Drow[bh * n + i] = Di;
            Drow_alt[bh * n + i] = dot(doi, oi, dv);
            double Dsub = (variant == ORACLE_WRONG_FLAT_JACOBIAN) ? flat_total : Di;

            double* dqi = dQ + i * d;
            for (long l = 0; l < d; ++l) dqi[l] = 0.0;
            for (long j = 0; j < m; ++j) {
                double dsij;
                switch (variant) {
                case ORACLE_WRONG_DS_NO_CORRECTION: dsij = dP[j] * P[j]; break;
                case ORACLE_WRONG_DS_DIAG_ONLY: dsij = dP[j] * P[j] * (1.0 - P[j]); break;
                default: dsij = P[j] * (dP[j] - Dsub); break;
                }
                if (ds) ds[(bh * n + i) * m + j] = dsij;
                for (long l = 0; l < d; ++l) {
                    dqi[l] += gscale * dsij * K[j * d + l];
                    dK[j * d + l] += gscale * dsij * qi[l];
                }
                if (variant == ORACLE_WRONG_DV_NO_TRANSPOSE) {
                    /* row i of P dO, written where the gradient of V_i goes */
                    for (long c = 0; c < dv; ++c) dV[i * dv + c] += P[j] * dO[j * dv + c];
                } else {
                    for (long c = 0; c < dv; ++c) dV[j * dv + c] += P[j] * doi[c];
                }
            }
        }
        free(S);
        free(P);
        free(dP);
    }
    return 0;
}

/*
 * Masks beyond causal n == m.  The pages define only the causal mask with
 * n == m (mlgrind "Inputs") and name padding masks in passing; this routine
 * extends the same row definition with the readings below.
 *
 *  - Per-batch lengths: batch b uses query rows i < nq[b] and key rows
 *    j < nk[b] of its n and m slots (nq or nk NULL means n or m for every
 *    b; values are clamped into [0, n] and [0, m]); the rest is padding.
 *  - mask 0: every key j < nk[b] is visible; mask 1 (causal, top-left):
 *    j <= i; mask 2 (causal, bottom-right, the last query row sees the last
 *    key): j <= i + nk[b] - nq[b].  With nq[b] == nk[b] masks 1 and 2 are
 *    the pages' causal mask.
 *  - A row that sees no key (nk[b] == 0, or mask 2 with i < nq[b] - nk[b])
 *    takes all-zero weights: O_i = 0, LSE_i = -inf, D_i = 0, dQ_i = 0.
 *    Padded query rows are written the same way; padded key rows get
 *    dK_j = dV_j = 0.
 *
 * Outputs as in oracle_attn_bwd (no dS, no variants).
 */
int oracle_attn_bwd_masked(const double* q, const double* k, const double* v,
                           const double* dout, double* dq, double* dk, double* dvv,
                           double* Drow, double* o, double* lse, long B, long H, long n,
                           long m, long d, long dv, double scale, int mask, const long* nq,
                           const long* nk) {
    if (B < 0 || H < 0 || n < 0 || m < 0 || d <= 0 || dv <= 0) return 1;
    if (mask < 0 || mask > 2) return 1;
    long heads = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < heads; ++bh) {
        const long b = H > 0 ? bh / H : 0;
        long nb = nq ? nq[b] : n, mb = nk ? nk[b] : m;
        nb = nb < 0 ? 0 : (nb > n ? n : nb);
        mb = mb < 0 ? 0 : (mb > m ? m : mb);
        const long off = (mask == 2) ? mb - nb : 0;
        const double* Q = q + bh * n * d;
        const double* K = k + bh * m * d;
        const double* V = v + bh * m * dv;
        const double* dO = dout + bh * n * dv;
        double* dQ = dq + bh * n * d;
        double* dK = dk + bh * m * d;
        double* dV = dvv + bh * m * dv;
        double* S = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
        double* P = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
        double* dP = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
        memset(dQ, 0, sizeof(double) * (size_t)(n * d));
        memset(dK, 0, sizeof(double) * (size_t)(m * d));
        memset(dV, 0, sizeof(double) * (size_t)(m * dv));
        memset(o + bh * n * dv, 0, sizeof(double) * (size_t)(n * dv));
        for (long i = 0; i < n; ++i) {
            lse[bh * n + i] = -INFINITY;
            Drow[bh * n + i] = 0.0;
        }
        for (long i = 0; i < nb; ++i) {
            const double* qi = Q + i * d;
            const double* doi = dO + i * dv;
            double M = -INFINITY, Z = 0.0;
            if (mb > 0) score_row(qi, K, i, mb, d, scale, mask != 0, off, 1, S, &M, &Z);
            if (Z == 0.0) continue;          /* no visible key: all-zero weights */
            for (long j = 0; j < mb; ++j) P[j] = exp(S[j] - M) / Z;
            lse[bh * n + i] = M + log(Z);
            double* oi = o + (bh * n + i) * dv;
            for (long j = 0; j < mb; ++j)
                for (long c = 0; c < dv; ++c) oi[c] += P[j] * V[j * dv + c];
            double Di = 0.0;
            for (long j = 0; j < mb; ++j) {
                dP[j] = dot(doi, V + j * dv, dv);
                Di += P[j] * dP[j];
            }
            Drow[bh * n + i] = Di;
            double* dqi = dQ + i * d;
            for (long j = 0; j < mb; ++j) {
                const double dsij = P[j] * (dP[j] - Di);
                for (long l = 0; l < d; ++l) {
                    dqi[l] += scale * dsij * K[j * d + l];
                    dK[j * d + l] += scale * dsij * qi[l];
                }
                for (long c = 0; c < dv; ++c) dV[j * dv + c] += P[j] * doi[c];
            }
        }
        free(S);
        free(P);
        free(dP);
    }
    return 0;
}

/*
 * Sampled routines for one head at sizes where the full oracle is too slow.
 * They evaluate the same definition for chosen query rows or key rows only,
 * with the causal offset `off` of the masked routine below (0 for the
 * pages' mask).
 *
 * oracle_attn_rows: for each listed query row i, O_i, LSE_i, D_i and dQ_i.
 * A query row's outputs depend on that row alone, so each is exact.
 */
int oracle_attn_rows(const double* Q, const double* K, const double* V, const double* dO,
                     long n, long m, long d, long dv, double scale, int causal, long off,
                     const long* rows, long nrows, double* o_rows, double* lse_rows,
                     double* D_rows, double* dq_rows) {
    if (n <= 0 || m <= 0 || d <= 0 || dv <= 0 || nrows < 0) return 1;
    for (long r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= n) return 1;
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)m);
        double* P = (double*)malloc(sizeof(double) * (size_t)m);
        double* dP = (double*)malloc(sizeof(double) * (size_t)m);
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < nrows; ++r) {
            long i = rows[r];
            const double* qi = Q + i * d;
            const double* doi = dO + i * dv;
            double M, Z;
            score_row(qi, K, i, m, d, scale, causal, off, 1, S, &M, &Z);
            double Di = 0.0;
            double* oi = o_rows + r * dv;
            for (long c = 0; c < dv; ++c) oi[c] = 0.0;
            for (long j = 0; j < m; ++j) {
                P[j] = Z > 0.0 ? exp(S[j] - M) / Z : 0.0;
                dP[j] = dot(doi, V + j * dv, dv);
                Di += P[j] * dP[j];
                for (long c = 0; c < dv; ++c) oi[c] += P[j] * V[j * dv + c];
            }
            lse_rows[r] = Z > 0.0 ? M + log(Z) : -INFINITY;
            D_rows[r] = Di;
            double* dqi = dq_rows + r * d;
            for (long l = 0; l < d; ++l) dqi[l] = 0.0;
            for (long j = 0; j < m; ++j) {
                double dsij = P[j] * (dP[j] - Di);
                for (long l = 0; l < d; ++l) dqi[l] += scale * dsij * K[j * d + l];
            }
        }
        free(S);
        free(P);
        free(dP);
    }
    return 0;
}

/*
 * oracle_attn_cols: for each listed key row j, dK_j and dV_j.  These sum over
 * every query row, so the row statistics M_i, Z_i and D_i of all n rows are
 * computed first (each from its own row only), then each listed column is
 * summed over i in increasing order.  Under the causal mask a row i < j - off
 * has P_ij = 0 exactly (eulerpad P8), so such terms are zero and are not
 * added; neither are rows that see no key at all.
 */
int oracle_attn_cols(const double* Q, const double* K, const double* V, const double* dO,
                     long n, long m, long d, long dv, double scale, int causal, long off,
                     const long* cols, long ncols, double* dk_cols, double* dv_cols) {
    if (n < 0 || m <= 0 || d <= 0 || dv <= 0 || ncols < 0) return 1;
    for (long c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= m) return 1;
    double* Mrow = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* Zrow = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* Drow = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)m);
#pragma omp for schedule(dynamic, 16)
        for (long i = 0; i < n; ++i) {
            double M, Z;
            score_row(Q + i * d, K, i, m, d, scale, causal, off, 1, S, &M, &Z);
            double Di = 0.0;
            for (long j = 0; j < m && Z > 0.0; ++j) {
                double p = exp(S[j] - M) / Z;
                if (p != 0.0) Di += p * dot(dO + i * dv, V + j * dv, dv);
            }
            Mrow[i] = M;
            Zrow[i] = Z;
            Drow[i] = Di;
        }
        free(S);
#pragma omp for schedule(dynamic, 1)
        for (long c = 0; c < ncols; ++c) {
            long j = cols[c];
            double* dkj = dk_cols + c * d;
            double* dvj = dv_cols + c * dv;
            for (long l = 0; l < d; ++l) dkj[l] = 0.0;
            for (long t = 0; t < dv; ++t) dvj[t] = 0.0;
            for (long i = (causal ? (j - off > 0 ? j - off : 0) : 0); i < n; ++i) {
                if (Zrow[i] == 0.0) continue;   /* a row that sees no key */
                double sij = scale * dot(Q + i * d, K + j * d, d);
                double p = exp(sij - Mrow[i]) / Zrow[i];
                double dpij = dot(dO + i * dv, V + j * dv, dv);
                double dsij = p * (dpij - Drow[i]);
                for (long l = 0; l < d; ++l) dkj[l] += scale * dsij * Q[i * d + l];
                for (long t = 0; t < dv; ++t) dvj[t] += p * dO[i * dv + t];
            }
        }
    }
    free(Mrow);
    free(Zrow);
    free(Drow);
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
