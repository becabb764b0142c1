/*
 * oracle.c -- plain fp64 CPU reference for the attention forward pass and its
 * gradients (the backward pass, near the end of the file).
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

/* The forward over R rows per (b, h): rows[r] (shared by every head) or,
 * with rows_per_head, rows[bh * R + r] for head bh = b * H + h; all Nq rows
 * when rows == NULL. */
static int attn_fwd_rows(const float* q, const float* k, const float* v,
                         int64_t q_sb, int64_t q_sh, int64_t q_sn,
                         int64_t k_sb, int64_t k_sh, int64_t k_sn,
                         int64_t v_sb, int64_t v_sh, int64_t v_sn,
                         int B, int H, int Nq, int Nk, int d,
                         double scale, int causal,
                         const int32_t* rows, int n_rows, int rows_per_head,
                         double* o, double* lse, int n_threads)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return -1;
    int R = rows ? n_rows : Nq;
    if (R < 1) return -1;
    if (rows) {
        const int64_t n_entries = rows_per_head ? (int64_t)B * H * R : R;
        for (int64_t r = 0; r < n_entries; ++r)
            if (rows[r] < 0 || rows[r] >= Nq) return -1;
    }
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
            int i = rows ? rows[(rows_per_head ? bh * R : 0) + r] : r;
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
    return attn_fwd_rows(q, k, v, q_sb, q_sh, q_sn, k_sb, k_sh, k_sn, v_sb, v_sh, v_sn,
                         B, H, Nq, Nk, d, scale, causal, rows, n_rows, 0, o, lse, n_threads);
}

/*
 * oracle_attn_fwd_rowtab: as oracle_attn_fwd, with a row table of its own
 * for every (b, h): rows [B*H][n_rows], entry [b*H + h][r] is the query
 * index of output row r of head (b, h).
 */
int oracle_attn_fwd_rowtab(const float* q, const float* k, const float* v,
                           int64_t q_sb, int64_t q_sh, int64_t q_sn,
                           int64_t k_sb, int64_t k_sh, int64_t k_sn,
                           int64_t v_sb, int64_t v_sh, int64_t v_sn,
                           int B, int H, int Nq, int Nk, int d,
                           double scale, int causal,
                           const int32_t* rows, int n_rows,
                           double* o, double* lse, int n_threads)
{
    if (!rows) return -1;
    return attn_fwd_rows(q, k, v, q_sb, q_sh, q_sn, k_sb, k_sh, k_sn, v_sb, v_sh, v_sn,
                         B, H, Nq, Nk, d, scale, causal, rows, n_rows, 1, o, lse, n_threads);
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

/* ------------------------------------------------------------------------
 * Backward pass (gradients of a loss L through O), in double.
 *
 * For one (b, h), with P the forward's probabilities and dO = dL/dO:
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij          (the whole visible row)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * over visible pairs only (masked pairs have P = 0 and carry no gradient).
 *
 * [nanhubrain] section "backward recomputation" rebuilds P from the row
 * statistics and accumulates dV += P^T dO, dP = dO V^T,
 * dS = P * (dP - rowsum(P * dP)), dQ += dS K, dK += dS^T Q block by block.
 * Its row term is summed over one key block only; the derivative of the
 * softmax needs it over the whole row (D_i above, which also equals
 * dO_i . O_i), and that is what is computed here.  The score scale
 * (S = scale * Q K^T) enters dQ and dK by the chain rule; the listing's
 * 1/sqrt(d) is that scale.
 * ---------------------------------------------------------------------- */

/* Row pass for query i of one (b, h): P_ij into p[], dP_ij into g[] (visible
 * j only), the row's log-sum-exp and D_i.  Returns the visible count. */
static int grad_row(const float* qi, const float* gi, const float* kbh, const float* vbh,
                    int64_t k_sn, int Nk, int d, double scale, int causal, int i,
                    double* p, double* g, double* lse_i, double* D_i)
{
    int vis = Nk;
    if (causal && i + 1 < vis) vis = i + 1;
    double top = -INFINITY;
    for (int j = 0; j < vis; ++j) {
        const float* kj = kbh + (int64_t)j * k_sn;
        const float* vj = vbh + (int64_t)j * k_sn;
        double a = 0.0, b = 0.0;
        for (int c = 0; c < d; ++c) {
            a += (double)qi[c] * (double)kj[c];
            b += (double)gi[c] * (double)vj[c];
        }
        p[j] = scale * a;
        g[j] = b;
        if (p[j] > top) top = p[j];
    }
    double z = 0.0;
    for (int j = 0; j < vis; ++j) z += exp(p[j] - top);
    const double lse = top + log(z);
    double D = 0.0;
    for (int j = 0; j < vis; ++j) {
        p[j] = exp(p[j] - lse);
        D += p[j] * g[j];
    }
    *lse_i = lse;
    *D_i = D;
    return vis;
}

/*
 * oracle_attn_bwd: dQ [B,H,RQ,d], dK and dV [B,H,RK,d] in double, where the
 * RQ query rows are qrows[0..n_qrows) (all Nq when qrows == NULL) and the RK
 * key rows krows[0..n_krows) (all Nk when krows == NULL).  dq == NULL skips
 * dQ; dk == NULL or dv == NULL skips dK and dV.  dO uses Q's strides, V uses
 * K's.  Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int oracle_attn_bwd(const float* q, const float* k, const float* v, const float* dout,
                    int64_t q_sb, int64_t q_sh, int64_t q_sn,
                    int64_t k_sb, int64_t k_sh, int64_t k_sn,
                    int B, int H, int Nq, int Nk, int d,
                    double scale, int causal,
                    const int32_t* qrows, int n_qrows, const int32_t* krows, int n_krows,
                    double* dq, double* dk, double* dv, int n_threads)
{
    if (!q || !k || !v || !dout) return -1;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return -1;
    const int RQ = qrows ? n_qrows : Nq, RK = krows ? n_krows : Nk;
    if (RQ < 0 || RK < 0) return -1;
    for (int r = 0; qrows && r < RQ; ++r)
        if (qrows[r] < 0 || qrows[r] >= Nq) return -1;
    for (int r = 0; krows && r < RK; ++r)
        if (krows[r] < 0 || krows[r] >= Nk) return -1;
    const int want_kv = dk && dv;
    if (n_threads <= 0) n_threads = omp_get_max_threads();

    double* stat = (double*)malloc(sizeof(double) * 2 * (size_t)Nq);
    if (!stat) return -2;
    double* lse = stat;
    double* Dr = stat + Nq;
    int status = 0;

    for (int bh = 0; bh < B * H && status == 0; ++bh) {
        const int b = bh / H, h = bh % H;
        const int64_t qoff = (int64_t)b * q_sb + (int64_t)h * q_sh;
        const int64_t koff = (int64_t)b * k_sb + (int64_t)h * k_sh;
        const float* qbh = q + qoff;
        const float* gbh = dout + qoff;
        const float* kbh = k + koff;
        const float* vbh = v + koff;

        /* pass 1: row statistics (lse_i, D_i) of every query; pass 2: dQ of
         * the requested rows, from the same row pass */
#pragma omp parallel num_threads(n_threads)
        {
            double* p = (double*)malloc(sizeof(double) * 2 * (size_t)Nk);
            if (!p) {
#pragma omp atomic write
                status = -2;
            }
#pragma omp for schedule(dynamic, 8)
            for (int i = 0; i < Nq; ++i) {
                if (!p) continue;
                grad_row(qbh + (int64_t)i * q_sn, gbh + (int64_t)i * q_sn, kbh, vbh, k_sn, Nk, d,
                         scale, causal, i, p, p + Nk, &lse[i], &Dr[i]);
            }
            if (dq) {
#pragma omp for schedule(dynamic, 4)
                for (int r = 0; r < RQ; ++r) {
                    if (!p) continue;
                    const int i = qrows ? qrows[r] : r;
                    double unused_lse, Di;
                    const int vis = grad_row(qbh + (int64_t)i * q_sn, gbh + (int64_t)i * q_sn, kbh, vbh,
                                             k_sn, Nk, d, scale, causal, i, p, p + Nk, &unused_lse, &Di);
                    double* out = dq + ((int64_t)bh * RQ + r) * d;
                    for (int c = 0; c < d; ++c) out[c] = 0.0;
                    for (int j = 0; j < vis; ++j) {
                        const double ds = p[j] * (p[Nk + j] - Di);
                        const float* kj = kbh + (int64_t)j * k_sn;
                        for (int c = 0; c < d; ++c) out[c] += ds * (double)kj[c];
                    }
                    for (int c = 0; c < d; ++c) out[c] *= scale;
                }
            }
            free(p);
        }
        if (status != 0 || !want_kv) continue;

        /* pass 3: dK and dV of the requested key rows, one column at a time,
         * from the row statistics of pass 1 */
#pragma omp parallel for num_threads(n_threads) schedule(dynamic, 4)
        for (int r = 0; r < RK; ++r) {
            const int j = krows ? krows[r] : r;
            const float* kj = kbh + (int64_t)j * k_sn;
            const float* vj = vbh + (int64_t)j * k_sn;
            double* gk = dk + ((int64_t)bh * RK + r) * d;
            double* gv = dv + ((int64_t)bh * RK + r) * d;
            for (int c = 0; c < d; ++c) gk[c] = gv[c] = 0.0;
            for (int i = causal ? j : 0; i < Nq; ++i) {
                const float* qi = qbh + (int64_t)i * q_sn;
                const float* gi = gbh + (int64_t)i * q_sn;
                double a = 0.0, e = 0.0;
                for (int c = 0; c < d; ++c) {
                    a += (double)qi[c] * (double)kj[c];
                    e += (double)gi[c] * (double)vj[c];
                }
                const double pij = exp(scale * a - lse[i]);
                const double ds = pij * (e - Dr[i]);
                for (int c = 0; c < d; ++c) {
                    gv[c] += pij * (double)gi[c];
                    gk[c] += ds * (double)qi[c];
                }
            }
            for (int c = 0; c < d; ++c) gk[c] *= scale;
        }
    }
    free(stat);
    return status;
}

/* ------------------------------------------------------------------------
 * Extended forward: grouped key/value heads and a band of visible keys, in
 * double.
 *
 * Visible keys of query i: lo_i <= j <= hi_i with
 *   lo_i = max(0, i - window_left)            (window_left < 0: lo_i = 0)
 *   hi_i = min(Nk - 1, i + window_right)      (window_right < 0: Nk - 1)
 * and, if causal, hi_i <= i as well.  This is the band of [pwwt] "standard vs
 * IO-aware" (`pre_tokens` keys before the query, `next_tokens` after it;
 * causal = next_tokens 0).  Query head h reads key/value head h / (H / Hkv):
 * the grouped (GQA) and multi-query (MQA, Hkv = 1) head maps of [nanhubrain]
 * "GatherPAKVCache" (only the needed KV heads are read).  A row with no
 * visible key has an empty softmax: O = 0 and LSE = -inf (the log of an
 * empty sum).
 * ---------------------------------------------------------------------- */

/* One query row over keys [lo, hi] (lo <= hi): scores, max, exp-sum, weighted
 * sum of value rows, all in double; `s` is scratch of Nk doubles. */
static void band_row(const float* qi, const float* kbh, const float* vbh, int64_t kv_sn,
                     int lo, int hi, int d, double scale, double* s, double* out_o, double* out_lse)
{
    double top = -INFINITY;
    for (int j = lo; j <= hi; ++j) {
        const float* kj = kbh + (int64_t)j * kv_sn;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)qi[c] * (double)kj[c];
        s[j] = scale * acc;
        if (s[j] > top) top = s[j];
    }
    double z = 0.0;
    for (int c = 0; c < d; ++c) out_o[c] = 0.0;
    for (int j = lo; j <= hi; ++j) {
        const double w = exp(s[j] - top);
        z += w;
        const float* vrow = vbh + (int64_t)j * kv_sn;
        for (int c = 0; c < d; ++c) out_o[c] += w * (double)vrow[c];
    }
    for (int c = 0; c < d; ++c) out_o[c] /= z;
    *out_lse = top + log(z);
}

/*
 * oracle_attn_fwd_ex: O [B,H,R,d] and LSE [B,H,R] in double for queries with H
 * heads and keys/values with Hkv heads (H % Hkv == 0; K/V strides describe the
 * Hkv-head tensors), under the band (window_left, window_right; negative =
 * unbounded) and the causal flag.  Rows as in oracle_attn_fwd.  Returns 0, -1
 * on bad arguments, -2 on allocation failure.
 */
int oracle_attn_fwd_ex(const float* q, const float* k, const float* v,
                       int64_t q_sb, int64_t q_sh, int64_t q_sn,
                       int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                       int B, int H, int Hkv, int Nq, int Nk, int d,
                       double scale, int causal, int window_left, int window_right,
                       const int32_t* rows, int n_rows,
                       double* o, double* lse, int n_threads)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || Nq < 1 || Nk < 1 || d < 1) return -1;
    const int R = rows ? n_rows : Nq;
    if (R < 1) return -1;
    for (int r = 0; rows && r < R; ++r)
        if (rows[r] < 0 || rows[r] >= Nq) return -1;
    if (n_threads <= 0) n_threads = omp_get_max_threads();
    const int group = H / Hkv;

    int status = 0;
    const int64_t total = (int64_t)B * H * R;
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
            const int64_t bh = t / R;
            const int r = (int)(t % R);
            const int b = (int)(bh / H), h = (int)(bh % H), hk = h / group;
            const int i = rows == NULL ? r : rows[r];
            int lo = 0, hi = Nk - 1;
            if (window_left >= 0 && i - window_left > lo) lo = i - window_left;
            if (window_right >= 0 && (int64_t)i + window_right < hi) hi = i + window_right;
            if (causal && i < hi) hi = i;
            double* out_o = o + t * d;
            if (lo > hi) {
                for (int c = 0; c < d; ++c) out_o[c] = 0.0;
                lse[t] = -INFINITY;
                continue;
            }
            const float* qi = q + (int64_t)b * q_sb + (int64_t)h * q_sh + (int64_t)i * q_sn;
            const int64_t kvoff = (int64_t)b * kv_sb + (int64_t)hk * kv_sh;
            band_row(qi, k + kvoff, v + kvoff, kv_sn, lo, hi, d, scale, s, out_o, lse + t);
        }
        free(s);
    }
    return status;
}

/* ------------------------------------------------------------------------
 * Extended backward: the gradients of oracle_attn_bwd under grouped
 * key/value heads and the band of oracle_attn_fwd_ex, in double.
 *
 * Row i of query head h sees keys lo_i..hi_i of key/value head
 * hk = h / (H / Hkv) (the band and causal flag as in oracle_attn_fwd_ex).
 * Over that set, P, dP, D_i and dS are those of oracle_attn_bwd.  K and V
 * of head hk enter the softmax of every query head of its group, so dK_j and
 * dV_j of head hk are the sums of the per-head terms over those query heads
 * (the chain rule through the shared rows).  A row with no visible key has
 * an empty softmax: it has no gradient of its own (dQ_i = 0) and passes none
 * to any key.
 * ---------------------------------------------------------------------- */

/* Visible keys [*lo, *hi] of query i; returns 0 when there are none. */
static int visible_keys(int i, int Nk, int causal, int window_left, int window_right, int* lo, int* hi)
{
    int a = 0, z = Nk - 1;
    if (window_left >= 0 && (int64_t)i - window_left > a) a = i - window_left;
    if (window_right >= 0 && (int64_t)i + window_right < z) z = i + window_right;
    if (causal && i < z) z = i;
    *lo = a;
    *hi = z;
    return a <= z;
}

/* Statistics of one row over keys [lo, hi]: the log-sum-exp of the scaled
 * scores and D = sum_j P_j (dO . v_j), in double.  sc and dp are scratch of
 * Nk doubles (the scaled scores and dO . v_j of the row). */
static void band_grad_stats(const float* qi, const float* gi, const float* kbh, const float* vbh,
                            int64_t kv_sn, int lo, int hi, int d, double scale, double* sc, double* dp,
                            double* out_lse, double* out_D)
{
    double top = -INFINITY;
    for (int j = lo; j <= hi; ++j) {
        const float* krow = kbh + (int64_t)j * kv_sn;
        const float* vj = vbh + (int64_t)j * kv_sn;
        double dot = 0.0, dpv = 0.0;
        for (int c = 0; c < d; ++c) {
            dot += (double)qi[c] * (double)krow[c];
            dpv += (double)gi[c] * (double)vj[c];
        }
        sc[j] = scale * dot;
        dp[j] = dpv;
        if (sc[j] > top) top = sc[j];
    }
    double z = 0.0;
    for (int j = lo; j <= hi; ++j) z += exp(sc[j] - top);
    const double l = top + log(z);
    double D = 0.0;
    for (int j = lo; j <= hi; ++j) D += exp(sc[j] - l) * dp[j];
    *out_lse = l;
    *out_D = D;
}

/*
 * oracle_attn_bwd_ex: dQ [B,H,RQ,d], dK and dV [B,Hkv,RK,d] in double; Q and
 * dO have H heads (strides q_*), K and V Hkv heads (strides kv_*); rows as in
 * oracle_attn_bwd.  Only the row statistics that a requested output needs are
 * computed.  Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int oracle_attn_bwd_ex(const float* q, const float* k, const float* v, const float* dout,
                       int64_t q_sb, int64_t q_sh, int64_t q_sn,
                       int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                       int B, int H, int Hkv, int Nq, int Nk, int d,
                       double scale, int causal, int window_left, int window_right,
                       const int32_t* qrows, int n_qrows, const int32_t* krows, int n_krows,
                       double* dq, double* dk, double* dv, int n_threads)
{
    if (!q || !k || !v || !dout) return -1;
    if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || Nq < 1 || Nk < 1 || d < 1) return -1;
    const int RQ = qrows ? n_qrows : Nq, RK = krows ? n_krows : Nk;
    if (RQ < 0 || RK < 0) return -1;
    for (int r = 0; qrows && r < RQ; ++r)
        if (qrows[r] < 0 || qrows[r] >= Nq) return -1;
    for (int r = 0; krows && r < RK; ++r)
        if (krows[r] < 0 || krows[r] >= Nk) return -1;
    const int grads_kv = dk != NULL && dv != NULL;
    if (n_threads <= 0) n_threads = omp_get_max_threads();
    const int group = H / Hkv;

    /* requested keys as a prefix count over key positions: row i reaches a
     * requested key iff the count rises within [lo_i, hi_i] */
    int* kcount = (int*)calloc((size_t)Nk + 1, sizeof(int));
    double* row_lse = (double*)malloc(sizeof(double) * (size_t)group * Nq);
    double* row_D = (double*)malloc(sizeof(double) * (size_t)group * Nq);
    char* need = (char*)malloc((size_t)Nq);
    if (!kcount || !row_lse || !row_D || !need) {
        free(kcount); free(row_lse); free(row_D); free(need);
        return -2;
    }
    for (int r = 0; grads_kv && r < RK; ++r) kcount[(krows ? krows[r] : r) + 1] = 1;
    for (int j = 0; j < Nk; ++j) kcount[j + 1] += kcount[j];
    for (int i = 0; i < Nq; ++i) {
        int lo, hi;
        need[i] = visible_keys(i, Nk, causal, window_left, window_right, &lo, &hi) &&
                  kcount[hi + 1] - kcount[lo] > 0;
    }
    for (int r = 0; dq && r < RQ; ++r) need[qrows ? qrows[r] : r] = 1;

    for (int bk = 0; bk < B * Hkv; ++bk) {
        const int b = bk / Hkv, hk = bk % Hkv;
        const int64_t kvoff = (int64_t)b * kv_sb + (int64_t)hk * kv_sh;
        const float* kbh = k + kvoff;
        const float* vbh = v + kvoff;

        /* pass 1: statistics of the needed rows of the group's query heads */
        int oom = 0;
#pragma omp parallel num_threads(n_threads)
        {
            double* scratch = (double*)malloc(sizeof(double) * 2 * (size_t)Nk);
            if (!scratch) {
#pragma omp atomic write
                oom = 1;
            }
#pragma omp for schedule(dynamic, 8)
            for (int64_t t = 0; t < (int64_t)group * Nq; ++t) {
                const int g = (int)(t / Nq), i = (int)(t % Nq);
                int lo, hi;
                row_lse[t] = -INFINITY;
                row_D[t] = 0.0;
                if (!scratch || !need[i] || !visible_keys(i, Nk, causal, window_left, window_right, &lo, &hi))
                    continue;
                const int64_t qo = (int64_t)b * q_sb + (int64_t)(hk * group + g) * q_sh + (int64_t)i * q_sn;
                band_grad_stats(q + qo, dout + qo, kbh, vbh, kv_sn, lo, hi, d, scale, scratch, scratch + Nk,
                                &row_lse[t], &row_D[t]);
            }
            free(scratch);
        }
        if (oom) {
            free(kcount); free(row_lse); free(row_D); free(need);
            return -2;
        }

        /* pass 2: dQ of the requested rows of each query head of the group */
        if (dq) {
#pragma omp parallel for num_threads(n_threads) schedule(dynamic, 4)
            for (int64_t t = 0; t < (int64_t)group * RQ; ++t) {
                const int g = (int)(t / RQ), r = (int)(t % RQ);
                const int h = hk * group + g;
                const int i = qrows ? qrows[r] : r;
                double* out = dq + (((int64_t)b * H + h) * RQ + r) * d;
                for (int c = 0; c < d; ++c) out[c] = 0.0;
                int lo, hi;
                if (!visible_keys(i, Nk, causal, window_left, window_right, &lo, &hi)) continue;
                const int64_t qo = (int64_t)b * q_sb + (int64_t)h * q_sh + (int64_t)i * q_sn;
                const float* qi = q + qo;
                const float* gi = dout + qo;
                const double l = row_lse[(int64_t)g * Nq + i], Di = row_D[(int64_t)g * Nq + i];
                for (int j = lo; j <= hi; ++j) {
                    const float* krow = kbh + (int64_t)j * kv_sn;
                    const float* vj = vbh + (int64_t)j * kv_sn;
                    double dot = 0.0, dpv = 0.0;
                    for (int c = 0; c < d; ++c) {
                        dot += (double)qi[c] * (double)krow[c];
                        dpv += (double)gi[c] * (double)vj[c];
                    }
                    const double dsij = exp(scale * dot - l) * (dpv - Di);
                    for (int c = 0; c < d; ++c) out[c] += dsij * (double)krow[c];
                }
                for (int c = 0; c < d; ++c) out[c] = scale * out[c];
            }
        }
        if (!grads_kv) continue;

        /* pass 3: dK and dV of the requested keys, summed over the group's
         * query heads and the queries that see the key */
#pragma omp parallel for num_threads(n_threads) schedule(dynamic, 4)
        for (int r = 0; r < RK; ++r) {
            const int j = krows ? krows[r] : r;
            const float* krow = kbh + (int64_t)j * kv_sn;
            const float* vj = vbh + (int64_t)j * kv_sn;
            double* ok = dk + ((int64_t)bk * RK + r) * d;
            double* ov = dv + ((int64_t)bk * RK + r) * d;
            for (int c = 0; c < d; ++c) ok[c] = ov[c] = 0.0;
            for (int g = 0; g < group; ++g) {
                const int h = hk * group + g;
                for (int i = 0; i < Nq; ++i) {
                    int lo, hi;
                    if (!visible_keys(i, Nk, causal, window_left, window_right, &lo, &hi) || j < lo || j > hi)
                        continue;
                    const int64_t qo = (int64_t)b * q_sb + (int64_t)h * q_sh + (int64_t)i * q_sn;
                    const float* qi = q + qo;
                    const float* gi = dout + qo;
                    double dot = 0.0, dpv = 0.0;
                    for (int c = 0; c < d; ++c) {
                        dot += (double)qi[c] * (double)krow[c];
                        dpv += (double)gi[c] * (double)vj[c];
                    }
                    const double pij = exp(scale * dot - row_lse[(int64_t)g * Nq + i]);
                    const double dsij = pij * (dpv - row_D[(int64_t)g * Nq + i]);
                    for (int c = 0; c < d; ++c) {
                        ov[c] += pij * (double)gi[c];
                        ok[c] += dsij * (double)qi[c];
                    }
                }
            }
            for (int c = 0; c < d; ++c) ok[c] *= scale;
        }
    }
    free(kcount);
    free(row_lse);
    free(row_D);
    free(need);
    return 0;
}
