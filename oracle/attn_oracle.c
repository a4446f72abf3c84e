/*
 * attn_oracle.c -- fp64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * What it computes, per attention head, with Q, K, V, dO given as row-major
 * N x d arrays of doubles (the caller converts bf16/fp32 inputs exactly):
 *
 *   S = scale * Q K^T                   "IO-4 FlashAttention", problem setup:
 *                                        Attention(Q,K,V) = softmax(QK^T/sqrt(d_k)) V;
 *                                        "Flash Attention-3" blog, code example
 *                                        (scale = d^-0.5, softmax over the last dim)
 *   causal: S_ij = -inf for key j > query i   (the plainest reading; not on the pages)
 *   block mask (optional): S_ij = -inf where entry (i / block, j / block) of a
 *     T x T byte mask is zero, T = ceil(N / block)
 *                                        FlashAttention-2 review, 'sparse/hybrid'
 *                                        answer, section 3 (1) (Sparse FlashAttention:
 *                                        only the important blocks are computed)
 *   a row with no kept key: P_i = 0, O_i = 0, LSE_i = log(0) = -inf, and it
 *   adds nothing to any gradient (the empty sum; the pages never meet the case)
 *   P = softmax(S) row-wise, O = P V     FlashAttention-2 review, "core algorithm"
 *                                        answer, section 1 (basic operation)
 *   LSE_i = m_i + ln(l_i)                the saved row statistic (m, l) of the same
 *                                        answer, section 2 (3) Backward Pass, item 1,
 *                                        folded into one number
 *   dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P o (dP - D)
 *   dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q
 *                                        same answer, section 2 (3) Backward Pass,
 *                                        item 2, read as the softmax Jacobian with the
 *                                        chain-rule scale (the printed dS is garbled)
 *
 * and a second forward that follows the tiled online recurrence of the same
 * answer, section 2 (2) Forward Pass, item 2, and "IO-4 FlashAttention",
 * section 4 (Online Softmax): running max m and running sum l per row, with
 * the old sum and the old output rescaled by exp(m_old - m_new), and one final
 * division by l ("adjust only at the final stage", FlashAttention-2 review,
 * strengths answer, "non-matmul operations").
 *
 * The naive functions keep the N x N matrices S, P, dP, dS explicitly
 * ("Standard Attention memory flow", IO-4 note section 1).  Rows are spread
 * over OpenMP threads; nothing is blocked, fused or reordered beyond that.
 *
 * Error behaviour: every function returns 0 on success, -1 on a bad argument
 * and -2 when a scratch allocation fails.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* The keys each query attends to. */
typedef struct {
    int causal;
    const unsigned char* bmask;   /* NULL: no block mask */
    long block, nblk;             /* block edge, blocks per side */
} keyset;

static keyset make_keyset(long N, int causal, const unsigned char* bmask, long block)
{
    keyset ks = {causal, bmask, block, bmask ? (N + block - 1) / block : 0};
    return ks;
}

static int allowed(const keyset* ks, long i, long j)
{
    if (ks->causal && j > i) return 0;
    return !ks->bmask || ks->bmask[(i / ks->block) * ks->nblk + j / ks->block] != 0;
}

static double dot(const double* a, const double* b, long d)
{
    double s = 0.0;
    for (long k = 0; k < d; ++k) s += a[k] * b[k];
    return s;
}

static int bad_args(long N, long d, double scale, int causal, const unsigned char* bmask, long block)
{
    return N < 1 || d < 1 || !isfinite(scale) || (causal != 0 && causal != 1) || (bmask && block < 1);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Naive forward with explicit S and P (N x N).  P_out (optional, N x N)
 * receives P.  O: N x d, LSE: N. */
int oracle_fwd(const double* Q, const double* K, const double* V, long N, long d,
               double scale, int causal, const unsigned char* bmask, long block,
               double* O, double* LSE, double* P_out)
{
    if (!Q || !K || !V || !O || !LSE || bad_args(N, d, scale, causal, bmask, block)) return -1;
    const keyset ks = make_keyset(N, causal, bmask, block);
    double* S = (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
    double* P = P_out ? P_out : (double*)malloc(sizeof(double) * (size_t)N * (size_t)N);
    if (!S || !P) { free(S); if (!P_out) free(P); return -2; }

    /* S = scale * Q K^T, masked entries -inf */
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < N; ++i)
        for (long j = 0; j < N; ++j)
            S[i * N + j] = allowed(&ks, i, j) ? scale * dot(Q + i * d, K + j * d, d) : -INFINITY;

    /* P = softmax(S) row-wise; LSE = m + ln l */
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < N; ++i) {
        const double* s = S + i * N;
        double m = -INFINITY;
        for (long j = 0; j < N; ++j) if (s[j] > m) m = s[j];
        double l = 0.0;
        for (long j = 0; j < N; ++j) l += (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        for (long j = 0; j < N; ++j) P[i * N + j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) / l;
        LSE[i] = m + log(l);
    }

    /* O = P V */
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < N; ++i) {
        double* o = O + i * d;
        for (long k = 0; k < d; ++k) o[k] = 0.0;
        for (long j = 0; j < N; ++j) {
            double p = P[i * N + j];
            if (p == 0.0) continue;
            for (long k = 0; k < d; ++k) o[k] += p * V[j * d + k];
        }
    }
    free(S);
    if (!P_out) free(P);
    return 0;
}

/* Naive backward with explicit S, P, dP, dS.  Recomputes the forward from Q, K,
 * V (it takes nothing from any forward).  D_out (optional, N) receives
 * D_i = sum_j P_ij dP_ij and D2_out (optional, N) receives the same quantity as
 * sum_k dO_ik O_ik, so that a caller can check the two are equal. */
int oracle_bwd(const double* Q, const double* K, const double* V, const double* dO,
               long N, long d, double scale, int causal, const unsigned char* bmask, long block,
               double* dQ, double* dK, double* dV, double* D_out, double* D2_out)
{
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV || bad_args(N, d, scale, causal, bmask, block)) return -1;
    size_t nn = (size_t)N * (size_t)N;
    double* P = (double*)malloc(sizeof(double) * nn);
    double* dS = (double*)malloc(sizeof(double) * nn);
    double* O = (double*)malloc(sizeof(double) * (size_t)N * (size_t)d);
    double* LSE = (double*)malloc(sizeof(double) * (size_t)N);
    double* D = (double*)malloc(sizeof(double) * (size_t)N);
    int rc = -2;
    if (!P || !dS || !O || !LSE || !D) goto out;
    rc = oracle_fwd(Q, K, V, N, d, scale, causal, bmask, block, O, LSE, P);
    if (rc) goto out;

    /* dP = dO V^T (stored in dS for now), D_i = sum_j P_ij dP_ij */
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < N; ++i) {
        double acc = 0.0;
        for (long j = 0; j < N; ++j) {
            double dp = dot(dO + i * d, V + j * d, d);
            dS[i * N + j] = dp;
            acc += P[i * N + j] * dp;
        }
        D[i] = acc;
        if (D_out) D_out[i] = acc;
        if (D2_out) D2_out[i] = dot(dO + i * d, O + i * d, d);
    }
    /* dS = P o (dP - D) */
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < N; ++i)
        for (long j = 0; j < N; ++j)
            dS[i * N + j] = P[i * N + j] * (dS[i * N + j] - D[i]);

    /* dQ = scale dS K */
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < N; ++i) {
        double* g = dQ + i * d;
        for (long k = 0; k < d; ++k) g[k] = 0.0;
        for (long j = 0; j < N; ++j) {
            double s = dS[i * N + j];
            if (s == 0.0) continue;
            for (long k = 0; k < d; ++k) g[k] += s * K[j * d + k];
        }
        for (long k = 0; k < d; ++k) g[k] *= scale;
    }
    /* dK = scale dS^T Q, dV = P^T dO */
#pragma omp parallel for schedule(dynamic, 4)
    for (long j = 0; j < N; ++j) {
        double* gk = dK + j * d;
        double* gv = dV + j * d;
        for (long k = 0; k < d; ++k) { gk[k] = 0.0; gv[k] = 0.0; }
        for (long i = 0; i < N; ++i) {
            double s = dS[i * N + j], p = P[i * N + j];
            for (long k = 0; k < d; ++k) {
                gk[k] += s * Q[i * d + k];
                gv[k] += p * dO[i * d + k];
            }
        }
        for (long k = 0; k < d; ++k) gk[k] *= scale;
    }
    rc = 0;
out:
    free(P); free(dS); free(O); free(LSE); free(D);
    return rc;
}

/* Forward by the tiled online recurrence: Q split into row blocks of Br,
 * K and V into column blocks of Bc.  For each row block and each column block
 * in order:  m' = max(m, rowmax S_blk);  alpha = exp(m - m');
 * l = alpha l + rowsum exp(S_blk - m');  acc = alpha acc + exp(S_blk - m') V_blk;
 * m = m'.  At the end O = acc / l and LSE = m + ln l. */
int oracle_fwd_online(const double* Q, const double* K, const double* V, long N, long d,
                      double scale, int causal, const unsigned char* bmask, long block,
                      long Br, long Bc, double* O, double* LSE)
{
    if (!Q || !K || !V || !O || !LSE || bad_args(N, d, scale, causal, bmask, block) || Br < 1 || Bc < 1)
        return -1;
    const keyset ks = make_keyset(N, causal, bmask, block);
    long Tr = (N + Br - 1) / Br;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bi = 0; bi < Tr; ++bi) {
        long r0 = bi * Br, r1 = r0 + Br < N ? r0 + Br : N, nr = r1 - r0;
        double* m = (double*)malloc(sizeof(double) * (size_t)nr);
        double* l = (double*)malloc(sizeof(double) * (size_t)nr);
        double* acc = (double*)malloc(sizeof(double) * (size_t)nr * (size_t)d);
        double* Sb = (double*)malloc(sizeof(double) * (size_t)nr * (size_t)Bc);
        if (!m || !l || !acc || !Sb) {
#pragma omp critical
            rc = -2;
            free(m); free(l); free(acc); free(Sb);
            continue;
        }
        for (long r = 0; r < nr; ++r) { m[r] = -INFINITY; l[r] = 0.0; }
        for (long x = 0; x < nr * d; ++x) acc[x] = 0.0;
        for (long c0 = 0; c0 < N; c0 += Bc) {
            long c1 = c0 + Bc < N ? c0 + Bc : N, nc = c1 - c0;
            for (long r = 0; r < nr; ++r) {
                long i = r0 + r;
                double* s = Sb + r * Bc;
                double rowmax = -INFINITY;
                for (long c = 0; c < nc; ++c) {
                    long j = c0 + c;
                    s[c] = allowed(&ks, i, j) ? scale * dot(Q + i * d, K + j * d, d) : -INFINITY;
                    if (s[c] > rowmax) rowmax = s[c];
                }
                double mnew = m[r] > rowmax ? m[r] : rowmax;
                if (mnew == -INFINITY) continue;     /* whole block masked, nothing seen yet */
                double alpha = (m[r] == -INFINITY) ? 0.0 : exp(m[r] - mnew);
                double rowsum = 0.0;
                double* a = acc + r * d;
                for (long k = 0; k < d; ++k) a[k] *= alpha;
                for (long c = 0; c < nc; ++c) {
                    double p = (s[c] == -INFINITY) ? 0.0 : exp(s[c] - mnew);
                    rowsum += p;
                    for (long k = 0; k < d; ++k) a[k] += p * V[(c0 + c) * d + k];
                }
                l[r] = alpha * l[r] + rowsum;
                m[r] = mnew;
            }
        }
        for (long r = 0; r < nr; ++r) {
            /* a row that kept no key stays at acc = 0, l = 0: O = 0 */
            for (long k = 0; k < d; ++k) O[(r0 + r) * d + k] = l[r] > 0.0 ? acc[r * d + k] / l[r] : 0.0;
            LSE[r0 + r] = m[r] + log(l[r]);
        }
        free(m); free(l); free(acc); free(Sb);
    }
    return rc;
}

/* The definition evaluated for selected query rows only (no N x N storage):
 * O, LSE and dQ of rows[0..nrows).  O_rows, dQ_rows: nrows x d; LSE_rows: nrows.
 * dO and dQ_rows may both be NULL to skip the gradient. */
int oracle_rows(const double* Q, const double* K, const double* V, const double* dO,
                long N, long d, double scale, int causal, const unsigned char* bmask, long block,
                const long* rows, long nrows, double* O_rows, double* LSE_rows, double* dQ_rows)
{
    if (!Q || !K || !V || !rows || !O_rows || !LSE_rows || bad_args(N, d, scale, causal, bmask, block)) return -1;
    const keyset ks = make_keyset(N, causal, bmask, block);
    if ((dO == NULL) != (dQ_rows == NULL)) return -1;
    for (long t = 0; t < nrows; ++t) if (rows[t] < 0 || rows[t] >= N) return -1;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long t = 0; t < nrows; ++t) {
        long i = rows[t];
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        if (!s) {
#pragma omp critical
            rc = -2;
            continue;
        }
        double m = -INFINITY;
        for (long j = 0; j < N; ++j) {
            s[j] = allowed(&ks, i, j) ? scale * dot(Q + i * d, K + j * d, d) : -INFINITY;
            if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (long j = 0; j < N; ++j) l += (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        double* o = O_rows + t * d;
        for (long k = 0; k < d; ++k) o[k] = 0.0;
        for (long j = 0; j < N; ++j) {
            s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m) / l;       /* s now holds P_i. */
            for (long k = 0; k < d; ++k) o[k] += s[j] * V[j * d + k];
        }
        LSE_rows[t] = m + log(l);
        if (dQ_rows) {
            const double* g = dO + i * d;
            double D = dot(g, o, d);                                     /* D_i = dO_i . O_i */
            double* dq = dQ_rows + t * d;
            for (long k = 0; k < d; ++k) dq[k] = 0.0;
            for (long j = 0; j < N; ++j) {
                if (s[j] == 0.0) continue;
                double ds = s[j] * (dot(g, V + j * d, d) - D);
                for (long k = 0; k < d; ++k) dq[k] += ds * K[j * d + k];
            }
            for (long k = 0; k < d; ++k) dq[k] *= scale;
        }
        free(s);
    }
    return rc;
}

/* The definition evaluated for selected key columns: dK and dV of
 * cols[0..ncols).  Every query row's LSE_i and D_i = dO_i . O_i is computed
 * first (row by row, as in oracle_rows), then P_ij = exp(S_ij - LSE_i). */
int oracle_cols(const double* Q, const double* K, const double* V, const double* dO,
                long N, long d, double scale, int causal, const unsigned char* bmask, long block,
                const long* cols, long ncols, double* dK_cols, double* dV_cols)
{
    if (!Q || !K || !V || !dO || !cols || !dK_cols || !dV_cols || bad_args(N, d, scale, causal, bmask, block))
        return -1;
    const keyset ks = make_keyset(N, causal, bmask, block);
    for (long t = 0; t < ncols; ++t) if (cols[t] < 0 || cols[t] >= N) return -1;
    double* LSE = (double*)malloc(sizeof(double) * (size_t)N);
    double* D = (double*)malloc(sizeof(double) * (size_t)N);
    int rc = 0;
    if (!LSE || !D) { free(LSE); free(D); return -2; }
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = 0; i < N; ++i) {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N + d));
        if (!s) {
#pragma omp critical
            rc = -2;
            continue;
        }
        double* o = s + N;
        double m = -INFINITY;
        for (long j = 0; j < N; ++j) {
            s[j] = allowed(&ks, i, j) ? scale * dot(Q + i * d, K + j * d, d) : -INFINITY;
            if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (long j = 0; j < N; ++j) l += (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
        for (long k = 0; k < d; ++k) o[k] = 0.0;
        for (long j = 0; j < N; ++j) {
            if (s[j] == -INFINITY) continue;
            double p = exp(s[j] - m) / l;
            for (long k = 0; k < d; ++k) o[k] += p * V[j * d + k];
        }
        LSE[i] = m + log(l);
        D[i] = dot(dO + i * d, o, d);
        free(s);
    }
    if (rc) { free(LSE); free(D); return rc; }
#pragma omp parallel for schedule(dynamic, 1)
    for (long t = 0; t < ncols; ++t) {
        long j = cols[t];
        double* gk = dK_cols + t * d;
        double* gv = dV_cols + t * d;
        for (long k = 0; k < d; ++k) { gk[k] = 0.0; gv[k] = 0.0; }
        for (long i = 0; i < N; ++i) {
            if (!allowed(&ks, i, j)) continue;
            double p = exp(scale * dot(Q + i * d, K + j * d, d) - LSE[i]);
            double ds = p * (dot(dO + i * d, V + j * d, d) - D[i]);
            for (long k = 0; k < d; ++k) {
                gv[k] += p * dO[i * d + k];
                gk[k] += ds * Q[i * d + k];
            }
        }
        for (long k = 0; k < d; ++k) gk[k] *= scale;
    }
    free(LSE); free(D);
    return 0;
}
