/*
 * oracle.c -- plain fp64 CPU reference for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code with the GPU kernels.
 *
 * What it computes (per batch b, head h and query row i), all in double:
 *   s_ij   = scale * sum_c q[i][c] * k[j][c]           for j in Vis(i)
 *   m_i    = max_{j in Vis(i)} s_ij                     (pass 1)
 *   l_i    = sum_{j in Vis(i)} exp(s_ij - m_i)           (pass 2)
 *   o_i    = sum_{j in Vis(i)} exp(s_ij - m_i) * v[j] / l_i
 *   lse_i  = m_i + ln(l_i)
 * with Vis(i) = { 0 <= j < Nk : !causal || j <= i }.
 *
 * Sources (pages cited by site: [nanhubrain] = nanhubrain.csdn.net, FlashAttention
 * in CANN ops-transformer; [pwwt] = www.pwwt.cn/news/2518640; [ascendai] =
 * ascendai.csdn.net, efficient attention in CANN ops-nn):
 *   - [nanhubrain] section "exact source of the quadratic memory": S = Q K^T /
 *     sqrt(d_k), P = softmax(S), O = P V;
 *   - [nanhubrain] section "online softmax mathematics": softmax with the row
 *     maximum subtracted before the exponential;
 *   - [nanhubrain] section "tiling skeleton": the per-row statistics (row max,
 *     row sum) that the tiled forward returns next to O;
 *   - [ascendai] section 6.1 (complete example): the causal variant sets the
 *     strict upper triangle (triu, diagonal 1) to -inf before the softmax, so
 *     key j is visible to query i iff j <= i (top-left alignment);
 *   - [pwwt] section "standard vs IO-aware": the naive matmul-softmax-matmul.
 *
 * The log-sum-exp output is not on the pages; it is the one number per row
 * from which [nanhubrain] section "backward recomputation" rebuilds P as
 * exp(S - m) / l, i.e. lse = m + ln l.
 *
 * Inputs are float32 arrays (exactly the values the GPU receives: bf16 inputs
 * widen to float32 without rounding); every product, sum, exp and log is done
 * in double.  Q, K, V are addressed through element strides
 * (batch, head, row); the head dimension is contiguous.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* One query row: two-pass softmax attention in double.  `s` is scratch of
 * Nk doubles.  Returns the number of visible keys (0 = no visible key). */
static int one_row(const float* qi, const float* kbh, const float* vbh,
                   int64_t k_sn, int64_t v_sn, int Nk, int d,
                   double scale, int causal, int i,
                   double* s, double* out_o, double* out_lse)
{
    int nvis = Nk;
    if (causal && i + 1 < nvis) nvis = i + 1;
    if (nvis <= 0) return 0;

    /* scores */
    for (int j = 0; j < nvis; ++j) {
        const float* kj = kbh + (int64_t)j * k_sn;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += (double)qi[c] * (double)kj[c];
        s[j] = scale * dot;
    }
    /* pass 1: row max */
    double m = s[0];
    for (int j = 1; j < nvis; ++j)
        if (s[j] > m) m = s[j];
    /* pass 2: exponentials, their sum, and the weighted sum of value rows */
    double l = 0.0;
    for (int c = 0; c < d; ++c) out_o[c] = 0.0;
    for (int j = 0; j < nvis; ++j) {
        double p = exp(s[j] - m);
        l += p;
        const float* vj = vbh + (int64_t)j * v_sn;
        for (int c = 0; c < d; ++c) out_o[c] += p * (double)vj[c];
    }
    for (int c = 0; c < d; ++c) out_o[c] /= l;
    *out_lse = m + log(l);
    return nvis;
}

/*
 * oracle_attn_fwd: O [B,H,R,d] and LSE [B,H,R] in double, where the R rows
 * are `rows[0..n_rows)` (query indices, each in [0,Nq)) or all Nq rows when
 * rows == NULL.  n_threads <= 0 means the OpenMP default.
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure,
 * -3 if some row has no visible key.
 */
int oracle_attn_fwd(const float* q, const float* k, const float* v,
                    int64_t q_sb, int64_t q_sh, int64_t q_sn,
                    int64_t k_sb, int64_t k_sh, int64_t k_sn,
                    int64_t v_sb, int64_t v_sh, int64_t v_sn,
                    int B, int H, int Nq, int Nk, int d,
                    double scale, int causal,
                    const int32_t* rows, int n_rows,
                    double* o, double* lse, int n_threads)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return -1;
    int R = rows ? n_rows : Nq;
    if (R < 1) return -1;
    if (rows)
        for (int r = 0; r < R; ++r)
            if (rows[r] < 0 || rows[r] >= Nq) return -1;
    if (n_threads <= 0) n_threads = omp_get_max_threads();

    int status = 0;
    int64_t total = (int64_t)B * H * R;
#pragma omp parallel num_threads(n_threads)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
        if (!s) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < total; ++t) {
            if (!s) continue;
            int64_t bh = t / R;
            int r = (int)(t % R);
            int b = (int)(bh / H), h = (int)(bh % H);
            int i = rows ? rows[r] : r;
            const float* qi = q + b * q_sb + h * q_sh + (int64_t)i * q_sn;
            const float* kbh = k + b * k_sb + h * k_sh;
            const float* vbh = v + b * v_sb + h * v_sh;
            int nvis = one_row(qi, kbh, vbh, k_sn, v_sn, Nk, d, scale, causal, i,
                               s, o + t * d, lse + t);
            if (nvis == 0) {
#pragma omp atomic write
                status = -3;
            }
        }
        free(s);
    }
    return status;
}

/*
 * oracle_attn_probs: the full probability matrix P [Nq, Nk] of one (b, h),
 * P_ij = exp(s_ij - m_i) / l_i on visible keys and 0 on masked ones.  For
 * small shapes only (the normalisation checks).  Same return codes.
 */
int oracle_attn_probs(const float* q, const float* k,
                      int64_t q_sn, int64_t k_sn,
                      int Nq, int Nk, int d, double scale, int causal,
                      double* p)
{
    if (!q || !k || !p || Nq < 1 || Nk < 1 || d < 1) return -1;
    for (int i = 0; i < Nq; ++i) {
        double* pi = p + (int64_t)i * Nk;
        int nvis = Nk;
        if (causal && i + 1 < nvis) nvis = i + 1;
        for (int j = 0; j < Nk; ++j) pi[j] = 0.0;
        const float* qi = q + (int64_t)i * q_sn;
        for (int j = 0; j < nvis; ++j) {
            const float* kj = k + (int64_t)j * k_sn;
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += (double)qi[c] * (double)kj[c];
            pi[j] = scale * dot;
        }
        double m = pi[0];
        for (int j = 1; j < nvis; ++j)
            if (pi[j] > m) m = pi[j];
        double l = 0.0;
        for (int j = 0; j < nvis; ++j) {
            pi[j] = exp(pi[j] - m);
            l += pi[j];
        }
        for (int j = 0; j < nvis; ++j) pi[j] /= l;
    }
    return 0;
}

/* Threads an OpenMP parallel region would use by default. */
int oracle_max_threads(void) { return omp_get_max_threads(); }
