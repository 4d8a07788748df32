/*
 * oracle_attn.c -- float64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU product path
 * never calls it and shares no code with it.
 *
 * What it computes (plain definition, no tiling, no fusion):
 *   For every batch b, query head h, query row i, with kv head
 *   g = h / (H / H_kv) and visible key set V_i = { j < T : !causal or j <= i },
 *     s_ij = scale * sum_d q[b,i,h,d] * k[b,j,g,d]
 *     m_i  = max_{j in V_i} s_ij
 *     Z_i  = sum_{j in V_i} exp(s_ij - m_i)
 *     O[b,i,h,:] = sum_{j in V_i} (exp(s_ij - m_i) / Z_i) * v[b,j,g,:]
 *     L[b,h,i]   = m_i + ln Z_i
 *
 * Sources (pages, by title and section):
 *  - yelogs.com Flash Attention2-in-Triton article, section
 *    "問題的根源：傳統注意力機制的痛點" (the ScaledDotProductAttention module:
 *    dot product, division by sqrt(d), masked_fill of masked positions, softmax,
 *    weighted sum of V). Masked keys are excluded from the row, which gives the
 *    same values as the module's -1e9 fill.
 *  - same article, "核心思想：分塊計算與在線更新" (traditional_softmax:
 *    subtract the row max, exponentiate, normalise) -- the two-pass form here.
 *  - same article, "因果掩碼的高效實現" (query position >= key position is
 *    visible, diagonal included).
 *  - same article, "核心 Kernel 實現" epilogue (the stored per-row statistic is
 *    the running max plus the natural log of the normaliser; eps taken as 0).
 *  - same article, "多查詢注意力（MQA）" (one kv head shared by all query heads);
 *    groups for 1 < H_kv < H are contiguous runs of H/H_kv query heads.
 *  - "Flash Attention Memory Optimization Explained" (lzwjava.github.io),
 *    "What is Flash Attention?": the four naive steps Q@K^T, scale and mask,
 *    softmax, weighted sum with V.
 *
 * Memory layout (row-major):
 *   q, o : [B, T, H,    D]     k, v : [B, T, H_kv, D]     lse : [B, H, T]
 *
 * oracle_attn_online_f64 follows the online-softmax recurrence of the same
 * article ("Softmax 的在線計算": running max m, normaliser l rescaled by
 * exp(m_old - m_new)), over key chunks of a caller-chosen size. It exists so a
 * test can show the recurrence reaches the two-pass result.
 *
 * oracle_attn_range_f64 is the definition above with the visible set cut to a
 * key range [lo, hi): output normalised over those keys only, L = ln of their
 * sum of exp(s); an empty range gives O = 0, L = -inf. oracle_lse_combine_f64
 * merges such partials over disjoint ranges: L = ln sum_s exp(L_s) (the max
 * is subtracted before exponentiating), O = sum_s exp(L_s - L) O_s -- the
 * same rescale-and-add the online recurrence applies between two chunks, with
 * each chunk's own normaliser folded into exp(L_s).
 *
 * oracle_attn_masked_f64 is the definition with the visible set cut by the
 * sparse patterns of the same article ("Flash Attention2 的變體", sparse
 * attention support): sliding window, key j visible to query i iff
 * |i - j| <= window; local-global, iff |i - j| <= window or j is one of the
 * global tokens. The causal flag, when set, also applies (j <= i). Each row's
 * visible keys are listed explicitly and the row is the plain two-pass
 * softmax over them; a row with no visible key (possible only when no
 * window contains the row itself, i.e. never for window >= 0) gets O = 0,
 * L = -inf.
 *
 * oracle_attn_decode_f64 is the definition for T_q query rows against T_k
 * keys and values (a key/value cache), the decoding case that "Flash
 * Attention Memory Optimization Explained", "Why It Matters", names
 * (FlashDecoding for inference). The query rows are the last T_q positions of
 * the T_k-long sequence: query i sits at position T_k - T_q + i, and under the
 * causal mask sees keys j <= T_k - T_q + i ("因果掩碼的高效實現": key position
 * <= query position). A row with no visible key (possible when T_q > T_k)
 * gets O = 0, L = -inf. Layout: q, o [B, T_q, H, D]; k, v [B, T_k, H_kv, D];
 * lse [B, H, T_q]. With T_q = T_k it is oracle_attn_f64.
 *
 * oracle_attn_bwd_f64 is the gradient of that definition, for a loss whose
 * gradient with respect to O is dO (L is treated as an auxiliary output that
 * the loss does not use). "Flash Attention Memory Optimization Explained",
 * "Key Mechanisms" (backward checkpointing: the backward pass recomputes the
 * forward's intermediates instead of reading them back) says what the method
 * keeps, not the formulas; those are the chain rule applied to the four naive
 * steps, written out here with every intermediate recomputed from q, k, v:
 *     P_ij  = exp(s_ij - m_i) / Z_i                     (two-pass, as above)
 *     dV_j += P_ij dO_i                  dP_ij = dO_i . v_j
 *     dS_ij = P_ij (dP_ij - sum_{k in V_i} P_ik dP_ik)  (softmax Jacobian)
 *     dQ_i  = scale sum_j dS_ij k_j      dK_j += scale dS_ij q_i
 * with dK and dV of a kv head summed over the query heads that share it. It
 * uses neither L nor the identity sum_k P_ik dP_ik = dO_i . O_i.
 * oracle_attn_bwd_masked_f64 is the same over the visible sets of the
 * sliding-window / local-global masks.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math, no BLAS).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static size_t qidx(int b, int t, int h, int H, int T, int D) {
    return (((size_t)b * T + t) * H + h) * (size_t)D;
}

/* One query row, two-pass softmax. s is caller scratch of length T. */
static void attn_row(const double *q, const double *k, const double *v,
                     double *o_row, double *lse_out,
                     int H, int H_kv, int T, int D, int causal, double scale,
                     int b, int h, int i, double *s) {
    const int group = H / H_kv;
    const int g = h / group;
    const int nvis = causal ? i + 1 : T;
    const double *qi = q + qidx(b, i, h, H, T, D);

    /* pass 1: scores and their max */
    double m = -INFINITY;
    for (int j = 0; j < nvis; ++j) {
        const double *kj = k + qidx(b, j, g, H_kv, T, D);
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    /* pass 2: exponentials and normaliser */
    double z = 0.0;
    for (int j = 0; j < nvis; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    /* weighted sum of V with the normalised weights */
    for (int d = 0; d < D; ++d) o_row[d] = 0.0;
    for (int j = 0; j < nvis; ++j) {
        const double w = s[j] / z;
        const double *vj = v + qidx(b, j, g, H_kv, T, D);
        for (int d = 0; d < D; ++d) o_row[d] += w * vj[d];
    }
    *lse_out = m + log(z);
}

static int bad_args(int B, int H, int H_kv, int T, int D) {
    return B < 1 || H < 1 || H_kv < 1 || T < 1 || D < 1 || (H % H_kv) != 0;
}

/* Full attention. Returns 0 on success, -1 on bad shape, -2 on no memory. */
int oracle_attn_f64(const double *q, const double *k, const double *v,
                    double *o, double *lse,
                    int B, int H, int H_kv, int T, int D, int causal, double scale) {
    if (bad_args(B, H, H_kv, T, D)) return -1;
    const long long nrows = (long long)B * H * T;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long long r = 0; r < nrows; ++r) {
                /* r enumerates (b, h, i) with i fastest */
                const int i = (int)(r % T);
                const int h = (int)((r / T) % H);
                const int b = (int)(r / ((long long)T * H));
                attn_row(q, k, v, o + qidx(b, i, h, H, T, D),
                         lse + ((size_t)b * H + h) * T + i,
                         H, H_kv, T, D, causal, scale, b, h, i, s);
            }
            free(s);
        }
    }
    return fail ? -2 : 0;
}

/* Selected rows only. rows[r] = (b*H + h)*T + i. o_rows is [nrows, D],
 * lse_rows is [nrows]. Returns -3 if a row index is out of range. */
int oracle_attn_rows_f64(const double *q, const double *k, const double *v,
                         const int64_t *rows, long long nrows,
                         double *o_rows, double *lse_rows,
                         int B, int H, int H_kv, int T, int D, int causal,
                         double scale) {
    if (bad_args(B, H, H_kv, T, D)) return -1;
    const long long total = (long long)B * H * T;
    for (long long r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -3;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (long long r = 0; r < nrows; ++r) {
                const long long id = rows[r];
                const int i = (int)(id % T);
                const int h = (int)((id / T) % H);
                const int b = (int)(id / ((long long)T * H));
                attn_row(q, k, v, o_rows + (size_t)r * D, lse_rows + r,
                         H, H_kv, T, D, causal, scale, b, h, i, s);
            }
            free(s);
        }
    }
    return fail ? -2 : 0;
}

/* Online-softmax recurrence over key chunks of `chunk` keys, per row:
 *   m_new = max(m, max_j s_j) ; a = exp(m - m_new) ; p_j = exp(s_j - m_new)
 *   l = a*l + sum_j p_j ; acc = a*acc + sum_j p_j v_j ; m = m_new
 * then O = acc / l and L = m + ln l. Initial state m = -inf, l = 0, acc = 0. */
int oracle_attn_online_f64(const double *q, const double *k, const double *v,
                           double *o, double *lse,
                           int B, int H, int H_kv, int T, int D, int causal,
                           double scale, int chunk) {
    if (bad_args(B, H, H_kv, T, D) || chunk < 1) return -1;
    const int group = H / H_kv;
    const long long nrows = (long long)B * H * T;
    int fail = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        double *p = (double *)malloc(sizeof(double) * (size_t)chunk);
        if (!acc || !p) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long long r = 0; r < nrows; ++r) {
                const int i = (int)(r % T);
                const int h = (int)((r / T) % H);
                const int b = (int)(r / ((long long)T * H));
                const int g = h / group;
                const int nvis = causal ? i + 1 : T;
                const double *qi = q + qidx(b, i, h, H, T, D);
                double m = -INFINITY, l = 0.0;
                for (int d = 0; d < D; ++d) acc[d] = 0.0;
                for (int j0 = 0; j0 < nvis; j0 += chunk) {
                    const int n = (nvis - j0 < chunk) ? nvis - j0 : chunk;
                    double cmax = -INFINITY;
                    for (int t = 0; t < n; ++t) {
                        const double *kj = k + qidx(b, j0 + t, g, H_kv, T, D);
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
                        p[t] = scale * dot;
                        if (p[t] > cmax) cmax = p[t];
                    }
                    const double m_new = (cmax > m) ? cmax : m;
                    /* exp(-inf - finite) = 0: the empty initial state drops out */
                    const double a = exp(m - m_new);
                    double psum = 0.0;
                    for (int t = 0; t < n; ++t) {
                        p[t] = exp(p[t] - m_new);
                        psum += p[t];
                    }
                    l = a * l + psum;
                    for (int d = 0; d < D; ++d) acc[d] *= a;
                    for (int t = 0; t < n; ++t) {
                        const double *vj = v + qidx(b, j0 + t, g, H_kv, T, D);
                        for (int d = 0; d < D; ++d) acc[d] += p[t] * vj[d];
                    }
                    m = m_new;
                }
                double *orow = o + qidx(b, i, h, H, T, D);
                for (int d = 0; d < D; ++d) orow[d] = acc[d] / l;
                lse[((size_t)b * H + h) * T + i] = m + log(l);
            }
        }
        free(acc);
        free(p);
    }
    return fail ? -2 : 0;
}

/* Attention over keys [key_lo, key_hi) only. o_part [B, H, T, D] and
 * lse_part [B, H, T] (row (b*H + h)*T + i). Returns 0, or -1 on bad shape. */
int oracle_attn_range_f64(const double *q, const double *k, const double *v,
                          double *o_part, double *lse_part,
                          int B, int H, int H_kv, int T, int D, int causal, double scale,
                          int key_lo, int key_hi) {
    if (bad_args(B, H, H_kv, T, D)) return -1;
    const long long nrows = (long long)B * H * T;
    const int group = H / H_kv;
#pragma omp parallel for schedule(dynamic, 16)
    for (long long r = 0; r < nrows; ++r) {
        const int i = (int)(r % T);
        const int h = (int)((r / T) % H);
        const int b = (int)(r / ((long long)T * H));
        const int g = h / group;
        const int nvis = causal ? i + 1 : T;
        const int lo = key_lo < 0 ? 0 : key_lo;
        const int hi = key_hi < nvis ? key_hi : nvis;
        const double *qi = q + qidx(b, i, h, H, T, D);
        double *orow = o_part + (size_t)r * D;
        for (int d = 0; d < D; ++d) orow[d] = 0.0;
        if (lo >= hi) {
            lse_part[r] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int j = lo; j < hi; ++j) {
            const double *kj = k + qidx(b, j, g, H_kv, T, D);
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
            if (scale * dot > m) m = scale * dot;
        }
        double z = 0.0;
        for (int j = lo; j < hi; ++j) {
            const double *kj = k + qidx(b, j, g, H_kv, T, D);
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
            const double w = exp(scale * dot - m);
            z += w;
            const double *vj = v + qidx(b, j, g, H_kv, T, D);
            for (int d = 0; d < D; ++d) orow[d] += w * vj[d];
        }
        for (int d = 0; d < D; ++d) orow[d] /= z;
        lse_part[r] = m + log(z);
    }
    return 0;
}

/* Merge n partials: o_parts [n][rows][D], lse_parts [n][rows] -> o [rows][D],
 * lse [rows]. Rows whose parts are all empty get o = 0, lse = -inf. */
int oracle_lse_combine_f64(const double *o_parts, const double *lse_parts, int n,
                           long long rows, int D, double *o, double *lse) {
    if (n < 1 || rows < 0 || D < 1) return -1;
#pragma omp parallel for schedule(static)
    for (long long r = 0; r < rows; ++r) {
        double m = -INFINITY;
        for (int s = 0; s < n; ++s)
            if (lse_parts[(size_t)s * rows + r] > m) m = lse_parts[(size_t)s * rows + r];
        double *orow = o + (size_t)r * D;
        for (int d = 0; d < D; ++d) orow[d] = 0.0;
        if (m == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (int s = 0; s < n; ++s) z += exp(lse_parts[(size_t)s * rows + r] - m);
        const double L = m + log(z);
        for (int s = 0; s < n; ++s) {
            const double w = exp(lse_parts[(size_t)s * rows + r] - L);
            const double *op = o_parts + ((size_t)s * rows + r) * D;
            for (int d = 0; d < D; ++d) orow[d] += w * op[d];
        }
        lse[r] = L;
    }
    return 0;
}

/* Attention under the sliding-window / local-global mask. is_global: T bytes,
 * nonzero for the global tokens (NULL: none). window >= 0. */
int oracle_attn_masked_f64(const double *q, const double *k, const double *v,
                           double *o, double *lse,
                           int B, int H, int H_kv, int T, int D, int causal, double scale,
                           int window, const unsigned char *is_global) {
    if (bad_args(B, H, H_kv, T, D) || window < 0) return -1;
    const long long nrows = (long long)B * H * T;
    const int group = H / H_kv;
    int fail = 0;
#pragma omp parallel
    {
        int *vis = (int *)malloc(sizeof(int) * (size_t)T);
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        if (!vis || !s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long long r = 0; r < nrows; ++r) {
                const int i = (int)(r % T);
                const int h = (int)((r / T) % H);
                const int b = (int)(r / ((long long)T * H));
                const int g = h / group;
                /* the visible set of row i, from the mask predicates */
                int n = 0;
                for (int j = 0; j < T; ++j) {
                    const int local = (i - j <= window) && (j - i <= window);
                    const int glob = is_global && is_global[j];
                    const int causal_ok = !causal || j <= i;
                    if ((local || glob) && causal_ok) vis[n++] = j;
                }
                const double *qi = q + qidx(b, i, h, H, T, D);
                double *orow = o + qidx(b, i, h, H, T, D);
                double *lrow = lse + ((size_t)b * H + h) * T + i;
                for (int d = 0; d < D; ++d) orow[d] = 0.0;
                if (n == 0) {
                    *lrow = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (int t = 0; t < n; ++t) {
                    const double *kj = k + qidx(b, vis[t], g, H_kv, T, D);
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
                    s[t] = scale * dot;
                    if (s[t] > m) m = s[t];
                }
                double z = 0.0;
                for (int t = 0; t < n; ++t) {
                    s[t] = exp(s[t] - m);
                    z += s[t];
                }
                for (int t = 0; t < n; ++t) {
                    const double *vj = v + qidx(b, vis[t], g, H_kv, T, D);
                    const double w = s[t] / z;
                    for (int d = 0; d < D; ++d) orow[d] += w * vj[d];
                }
                *lrow = m + log(z);
            }
        }
        free(vis);
        free(s);
    }
    return fail ? -2 : 0;
}

/* Gradients of attention over each row's visible keys: j <= i when causal
 * and, when window >= 0, |i - j| <= window or is_global[j] (is_global may be
 * NULL). dout, dq: [B, T, H, D]; dk, dv: [B, T, H_kv, D] (overwritten).
 * Parallel over (batch, kv head); each task owns the dk/dv rows of its kv
 * head, so no two tasks write the same element. A row with no visible key
 * (impossible for window >= 0) contributes nothing. */
static int attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv, int B, int H, int H_kv, int T, int D,
                    int causal, double scale, int window, const unsigned char *is_global) {
    if (bad_args(B, H, H_kv, T, D)) return -1;
    const int group = H / H_kv;
    int fail = 0;
#pragma omp parallel
    {
        int *vis = (int *)malloc(sizeof(int) * (size_t)T);
        double *p = (double *)malloc(sizeof(double) * (size_t)T);
        double *dp = (double *)malloc(sizeof(double) * (size_t)T);
        if (!vis || !p || !dp) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long long task = 0; task < (long long)B * H_kv; ++task) {
                const int b = (int)(task / H_kv), g = (int)(task % H_kv);
                for (int j = 0; j < T; ++j)
                    for (int d = 0; d < D; ++d) {
                        dk[qidx(b, j, g, H_kv, T, D) + d] = 0.0;
                        dv[qidx(b, j, g, H_kv, T, D) + d] = 0.0;
                    }
                for (int h = g * group; h < (g + 1) * group; ++h)
                    for (int i = 0; i < T; ++i) {
                        /* the visible keys of row i */
                        int n = 0;
                        for (int j = 0; j < T; ++j) {
                            const int causal_ok = !causal || j <= i;
                            const int local = window < 0 ||
                                              ((i - j <= window) && (j - i <= window));
                            const int glob = window >= 0 && is_global && is_global[j];
                            if (causal_ok && (local || glob)) vis[n++] = j;
                        }
                        const double *qi = q + qidx(b, i, h, H, T, D);
                        const double *doi = dout + qidx(b, i, h, H, T, D);
                        double *dqi = dq + qidx(b, i, h, H, T, D);
                        for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                        if (n == 0) continue;
                        /* forward recomputed: scores, max, normaliser, P */
                        double m = -INFINITY;
                        for (int t = 0; t < n; ++t) {
                            const double *kj = k + qidx(b, vis[t], g, H_kv, T, D);
                            double dot = 0.0;
                            for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
                            p[t] = scale * dot;
                            if (p[t] > m) m = p[t];
                        }
                        double z = 0.0;
                        for (int t = 0; t < n; ++t) {
                            p[t] = exp(p[t] - m);
                            z += p[t];
                        }
                        for (int t = 0; t < n; ++t) p[t] /= z;
                        /* dP and the softmax Jacobian's row term */
                        double rowdot = 0.0;
                        for (int t = 0; t < n; ++t) {
                            const double *vj = v + qidx(b, vis[t], g, H_kv, T, D);
                            double dot = 0.0;
                            for (int d = 0; d < D; ++d) dot += doi[d] * vj[d];
                            dp[t] = dot;
                            rowdot += p[t] * dot;
                        }
                        for (int t = 0; t < n; ++t) {
                            const double ds = p[t] * (dp[t] - rowdot);
                            const double *kj = k + qidx(b, vis[t], g, H_kv, T, D);
                            double *dkj = dk + qidx(b, vis[t], g, H_kv, T, D);
                            double *dvj = dv + qidx(b, vis[t], g, H_kv, T, D);
                            for (int d = 0; d < D; ++d) {
                                dqi[d] += scale * ds * kj[d];
                                dkj[d] += scale * ds * qi[d];
                                dvj[d] += p[t] * doi[d];
                            }
                        }
                    }
            }
        }
        free(vis);
        free(p);
        free(dp);
    }
    return fail ? -2 : 0;
}

/* Gradients of full attention (causal or not). */
int oracle_attn_bwd_f64(const double *q, const double *k, const double *v, const double *dout,
                        double *dq, double *dk, double *dv,
                        int B, int H, int H_kv, int T, int D, int causal, double scale) {
    return attn_bwd(q, k, v, dout, dq, dk, dv, B, H, H_kv, T, D, causal, scale, -1, NULL);
}

/* Gradients of the sliding-window / local-global attention of
 * oracle_attn_masked_f64 (window >= 0). */
int oracle_attn_bwd_masked_f64(const double *q, const double *k, const double *v,
                               const double *dout, double *dq, double *dk, double *dv,
                               int B, int H, int H_kv, int T, int D, int causal, double scale,
                               int window, const unsigned char *is_global) {
    if (window < 0) return -1;
    return attn_bwd(q, k, v, dout, dq, dk, dv, B, H, H_kv, T, D, causal, scale, window,
                    is_global);
}

/* dQ of selected rows, flat ids (b*H + h)*T + i, for the plain (maskless or
 * causal) attention: the row's forward recomputed (scores, max, normaliser,
 * weights P), dP_j = dO_i . v_j, Delta_i = sum_j P_j dP_j, and
 * dQ_i = scale * sum_j P_j (dP_j - Delta_i) k_j, keys in ascending order --
 * the dQ part of the full backward above, one row at a time. */
int oracle_attn_bwd_dq_rows_f64(const double *q, const double *k, const double *v,
                                const double *dout, const int64_t *rows, long long nrows,
                                double *dq_rows, int B, int H, int H_kv, int T, int D,
                                int causal, double scale) {
    if (bad_args(B, H, H_kv, T, D)) return -1;
    const long long total = (long long)B * H * T;
    for (long long r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -3;
    const int group = H / H_kv;
    int fail = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)T);
        double *dp = (double *)malloc(sizeof(double) * (size_t)T);
        if (!p || !dp) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long long r = 0; r < nrows; ++r) {
                const long long id = rows[r];
                const int i = (int)(id % T);
                const int h = (int)((id / T) % H);
                const int b = (int)(id / ((long long)T * H));
                const int g = h / group;
                const int n = causal ? i + 1 : T;   /* visible keys 0 .. n-1 */
                const double *qi = q + qidx(b, i, h, H, T, D);
                const double *doi = dout + qidx(b, i, h, H, T, D);
                double *dqi = dq_rows + (size_t)r * D;
                for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                double m = -INFINITY;
                for (int j = 0; j < n; ++j) {
                    const double *kj = k + qidx(b, j, g, H_kv, T, D);
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
                    p[j] = scale * dot;
                    if (p[j] > m) m = p[j];
                }
                double z = 0.0;
                for (int j = 0; j < n; ++j) {
                    p[j] = exp(p[j] - m);
                    z += p[j];
                }
                for (int j = 0; j < n; ++j) p[j] /= z;
                double rowdot = 0.0;
                for (int j = 0; j < n; ++j) {
                    const double *vj = v + qidx(b, j, g, H_kv, T, D);
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += doi[d] * vj[d];
                    dp[j] = dot;
                    rowdot += p[j] * dot;
                }
                for (int j = 0; j < n; ++j) {
                    const double ds = p[j] * (dp[j] - rowdot);
                    const double *kj = k + qidx(b, j, g, H_kv, T, D);
                    for (int d = 0; d < D; ++d) dqi[d] += scale * ds * kj[d];
                }
            }
        }
        free(p);
        free(dp);
    }
    return fail ? -2 : 0;
}

/* Decode-shaped attention: T_q query rows at positions T_k - T_q + i against
 * T_k keys. Returns 0, -1 on bad shape, -2 on no memory. */
int oracle_attn_decode_f64(const double *q, const double *k, const double *v, double *o,
                           double *lse, int B, int H, int H_kv, int Tq, int Tk, int D,
                           int causal, double scale) {
    if (B < 1 || H < 1 || H_kv < 1 || Tq < 1 || Tk < 1 || D < 1 || (H % H_kv) != 0) return -1;
    const int group = H / H_kv;
    const long long nrows = (long long)B * H * Tq;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Tk);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (long long r = 0; r < nrows; ++r) {
            if (!s) continue;
            const int i = (int)(r % Tq);
            const int h = (int)((r / Tq) % H);
            const int b = (int)(r / ((long long)Tq * H));
            const int g = h / group;
            /* keys 0 .. last are visible */
            long long last = causal ? (long long)Tk - Tq + i : (long long)Tk - 1;
            if (last > Tk - 1) last = Tk - 1;
            double *orow = o + qidx(b, i, h, H, Tq, D);
            double *lrow = lse + ((size_t)b * H + h) * Tq + i;
            if (last < 0) {
                for (int d = 0; d < D; ++d) orow[d] = 0.0;
                *lrow = -INFINITY;
                continue;
            }
            const int nvis = (int)last + 1;
            const double *qi = q + qidx(b, i, h, H, Tq, D);
            double m = -INFINITY;
            for (int j = 0; j < nvis; ++j) {
                const double *kj = k + qidx(b, j, g, H_kv, Tk, D);
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            double z = 0.0;
            for (int j = 0; j < nvis; ++j) {
                s[j] = exp(s[j] - m);
                z += s[j];
            }
            for (int d = 0; d < D; ++d) orow[d] = 0.0;
            for (int j = 0; j < nvis; ++j) {
                const double w = s[j] / z;
                const double *vj = v + qidx(b, j, g, H_kv, Tk, D);
                for (int d = 0; d < D; ++d) orow[d] += w * vj[d];
            }
            *lrow = m + log(z);
        }
        free(s);
    }
    return fail ? -2 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the oracle's loops use from now on (n >= 1). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
