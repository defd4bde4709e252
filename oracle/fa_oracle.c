/*
 * CPU oracle for exact scaled-dot-product attention (forward and gradients).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or helper with the GPU library, and it never sees a
 * value produced by the GPU library except to compare against it.
 *
 * Everything is computed in IEEE double precision with libm exp/log, in the
 * plain order the method's definition gives, with no blocking or fusion
 * beyond what each function's cited passage states.
 *
 * Sources (pages of the reference; sections as numbered on each page):
 *  - "Flash Attention 原理与实践" (bjdmk.com.cn), section 1.3: standard
 *    attention S = QK^T, P = softmax(S), O = PV; section 2.2: the online
 *    softmax identity; section 2.3: the v1 loop order (KV outer, Q inner,
 *    O/l/m written back after every step).
 *  - "FlashAttention算子优化" (viperekura.xyz), section 1: the three-pass
 *    softmax (row max, exp-sum, normalise); section 2: the fused forward in
 *    v2 loop order (one Q block, KV blocks inside, division by l after the
 *    KV loop), scale = 1/sqrt(d) applied to S before the max.
 *  - "FlashAttention 与显存" (world.lapla.si plate F51), plate 04 (standard
 *    method), plate 08 (merge rule m_new = max(m, m~),
 *    l_new = e^(m - m_new) l + e^(m~ - m_new) l~, result equal to the
 *    full-row softmax up to rounding), plate 09 (only O and per-row
 *    statistics are kept).
 *
 * Readings where the pages are silent (each restated in the design notes):
 *  - causal masking is top-left aligned: key j is visible to query i iff
 *    j <= i (also when n_q != n_kv);
 *  - LSE_i = m_i + ln(l_i) in natural-log units of the scaled scores;
 *  - a key block with no visible key for a row is skipped for that row (the
 *    merge would otherwise form e^(-inf - (-inf)));
 *  - ragged tails: block counts use the ceiling and the last block is
 *    shorter (the floor in the v1 listing would drop the tail).
 *
 * Status codes: 0 ok, 1 bad argument, 2 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads a parallel region of this library uses. */
int fa_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of threads later parallel regions of the calling thread
 * use (n >= 1); returns the previous value.  Used to time the oracle on one
 * core beside its multi-core run. */
int fa_oracle_set_num_threads(int n)
{
    const int prev = fa_oracle_num_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}

/* Number of keys row i may attend to. */
static int64_t visible_keys(int64_t i, int64_t n_kv, int causal)
{
    if (!causal) return n_kv;
    return (i + 1 < n_kv) ? i + 1 : n_kv;
}

/* s = scale * <q_i, k_j>, plain sequential dot product. */
static double score(const double *qi, const double *kj, int64_t d, double scale)
{
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c) acc += qi[c] * kj[c];
    return scale * acc;
}

/*
 * Standard attention for selected rows of one (batch, head) slice, in the
 * three passes of the softmax ("FlashAttention算子优化" section 1; standard
 * method of plate 04 and section 1.3 of the first page):
 *   pass 1: s_j = scale * q_i . k_j for visible j, m = max_j s_j
 *   pass 2: l = sum_j exp(s_j - m)
 *   pass 3: P_ij = exp(s_j - m) / l, O_i = sum_j P_ij v_j
 *   LSE_i = m + ln l
 * q: [n_q, d], k, v: [n_kv, d], row-major.  rows: row indices into q (NULL =
 * all n_q rows, then n_rows must equal n_q).  o: [n_rows, d], lse: [n_rows],
 * p: optional [n_rows, n_kv] probabilities (masked entries 0).
 */
int fa_oracle_naive(const double *q, const double *k, const double *v,
                    int64_t n_q, int64_t n_kv, int64_t d, double scale, int causal,
                    const int64_t *rows, int64_t n_rows,
                    double *o, double *lse, double *p)
{
    if (!q || !k || !v || !o || !lse || n_q < 0 || n_kv < 1 || d < 1 || n_rows < 0) return 1;
    if (!rows && n_rows != n_q) return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= n_q) return 1;
    }
    int status = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)n_kv * sizeof(double));
        if (!s) {
#pragma omp atomic write
            status = 2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            int64_t i = rows ? rows[r] : r;
            const double *qi = q + i * d;
            int64_t nv = visible_keys(i, n_kv, causal);
            /* pass 1 */
            double m = -INFINITY;
            for (int64_t j = 0; j < nv; ++j) {
                s[j] = score(qi, k + j * d, d, scale);
                if (s[j] > m) m = s[j];
            }
            /* pass 2 */
            double l = 0.0;
            for (int64_t j = 0; j < nv; ++j) l += exp(s[j] - m);
            /* pass 3 */
            double *oi = o + r * d;
            for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
            for (int64_t j = 0; j < nv; ++j) {
                double pij = exp(s[j] - m) / l;
                if (p) p[r * n_kv + j] = pij;
                const double *vj = v + j * d;
                for (int64_t c = 0; c < d; ++c) oi[c] += pij * vj[c];
            }
            if (p)
                for (int64_t j = nv; j < n_kv; ++j) p[r * n_kv + j] = 0.0;
            lse[r] = m + log(l);
        }
        free(s);
    }
    return status;
}

/* Checks that cuts is 0 = c_0 < c_1 < ... < c_{n-1} = total. */
static int valid_cuts(const int64_t *cuts, int64_t n, int64_t total)
{
    if (!cuts || n < 2 || cuts[0] != 0 || cuts[n - 1] != total) return 0;
    for (int64_t t = 1; t < n; ++t)
        if (cuts[t] <= cuts[t - 1]) return 0;
    return 1;
}

/*
 * Blockwise forward in v2 loop order ("FlashAttention算子优化" section 2):
 * for each query block, a running (m, l, O_acc) per row starts at
 * (-inf, 0, 0); each key block contributes its own block max m~, block
 * probabilities P~ = exp(s - m~), block sum l~ = sum P~ and block product
 * P~ V; they are merged with the rule of plate 08:
 *   m_new = max(m, m~)
 *   l     = e^(m - m_new) l + e^(m~ - m_new) l~
 *   O_acc = e^(m - m_new) O_acc + e^(m~ - m_new) (P~ V)
 * and O = O_acc / l only after the last key block (v2 defers the division).
 * The query partition is q_cuts, the key partition kv_cuts (boundaries, both
 * starting at 0 and ending at n_q / n_kv).  Rows of a query block are
 * independent, so each row is carried through the key blocks on its own.
 * o: [n_q, d], lse: [n_q].
 */
int fa_oracle_blockwise(const double *q, const double *k, const double *v,
                        int64_t n_q, int64_t n_kv, int64_t d, double scale, int causal,
                        const int64_t *q_cuts, int64_t n_qcuts,
                        const int64_t *kv_cuts, int64_t n_kvcuts,
                        double *o, double *lse)
{
    if (!q || !k || !v || !o || !lse || n_q < 1 || n_kv < 1 || d < 1) return 1;
    if (!valid_cuts(q_cuts, n_qcuts, n_q) || !valid_cuts(kv_cuts, n_kvcuts, n_kv)) return 1;
    int status = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)n_kv * sizeof(double));
        double *pv = (double *)malloc((size_t)d * sizeof(double));
        if (!s || !pv) {
#pragma omp atomic write
            status = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t qb = 0; qb < n_qcuts - 1; ++qb) {
            if (!s || !pv) continue;
            for (int64_t i = q_cuts[qb]; i < q_cuts[qb + 1]; ++i) {
                const double *qi = q + i * d;
                int64_t nv = visible_keys(i, n_kv, causal);
                double m = -INFINITY, l = 0.0;
                double *acc = o + i * d;
                for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
                for (int64_t kb = 0; kb < n_kvcuts - 1; ++kb) {
                    int64_t a = kv_cuts[kb];
                    int64_t b = kv_cuts[kb + 1] < nv ? kv_cuts[kb + 1] : nv;
                    if (b <= a) continue; /* no visible key in this block */
                    /* block scores and block max m~ */
                    double mt = -INFINITY;
                    for (int64_t j = a; j < b; ++j) {
                        s[j] = score(qi, k + j * d, d, scale);
                        if (s[j] > mt) mt = s[j];
                    }
                    /* P~ = exp(s - m~), l~ = sum P~, P~ V */
                    double lt = 0.0;
                    for (int64_t c = 0; c < d; ++c) pv[c] = 0.0;
                    for (int64_t j = a; j < b; ++j) {
                        double pj = exp(s[j] - mt);
                        lt += pj;
                        const double *vj = v + j * d;
                        for (int64_t c = 0; c < d; ++c) pv[c] += pj * vj[c];
                    }
                    /* merge (plate 08) */
                    double m_new = m > mt ? m : mt;
                    double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
                    double beta = exp(mt - m_new);
                    l = alpha * l + beta * lt;
                    for (int64_t c = 0; c < d; ++c) acc[c] = alpha * acc[c] + beta * pv[c];
                    m = m_new;
                }
                for (int64_t c = 0; c < d; ++c) acc[c] /= l;
                lse[i] = m + log(l);
            }
        }
        free(s);
        free(pv);
    }
    return status;
}

/*
 * Blockwise forward in v1 loop order ("Flash Attention 原理与实践" section
 * 2.3): key blocks outside, query blocks inside; after every step the
 * normalised output O, the sum l and the max m of each row are written back,
 * and the step's update is
 *   O_new = (l e^(m - m_new) O + e^(m~ - m_new) P~ V) / l_new.
 * Block counts use the ceiling (the listing's floor would drop a ragged
 * tail).  o: [n_q, d], lse: [n_q]; m_buf, l_buf: scratch [n_q] each.
 */
int fa_oracle_blockwise_v1(const double *q, const double *k, const double *v,
                           int64_t n_q, int64_t n_kv, int64_t d, double scale, int causal,
                           const int64_t *q_cuts, int64_t n_qcuts,
                           const int64_t *kv_cuts, int64_t n_kvcuts,
                           double *o, double *lse)
{
    if (!q || !k || !v || !o || !lse || n_q < 1 || n_kv < 1 || d < 1) return 1;
    if (!valid_cuts(q_cuts, n_qcuts, n_q) || !valid_cuts(kv_cuts, n_kvcuts, n_kv)) return 1;
    double *m_buf = (double *)malloc((size_t)n_q * sizeof(double));
    double *l_buf = (double *)malloc((size_t)n_q * sizeof(double));
    double *s = (double *)malloc((size_t)n_kv * sizeof(double));
    double *pv = (double *)malloc((size_t)d * sizeof(double));
    if (!m_buf || !l_buf || !s || !pv) {
        free(m_buf); free(l_buf); free(s); free(pv);
        return 2;
    }
    for (int64_t i = 0; i < n_q; ++i) {
        m_buf[i] = -INFINITY;
        l_buf[i] = 0.0;
        for (int64_t c = 0; c < d; ++c) o[i * d + c] = 0.0;
    }
    for (int64_t kb = 0; kb < n_kvcuts - 1; ++kb) {
        for (int64_t qb = 0; qb < n_qcuts - 1; ++qb) {
            for (int64_t i = q_cuts[qb]; i < q_cuts[qb + 1]; ++i) {
                const double *qi = q + i * d;
                int64_t nv = visible_keys(i, n_kv, causal);
                int64_t a = kv_cuts[kb];
                int64_t b = kv_cuts[kb + 1] < nv ? kv_cuts[kb + 1] : nv;
                if (b <= a) continue;
                double mt = -INFINITY;
                for (int64_t j = a; j < b; ++j) {
                    s[j] = score(qi, k + j * d, d, scale);
                    if (s[j] > mt) mt = s[j];
                }
                double lt = 0.0;
                for (int64_t c = 0; c < d; ++c) pv[c] = 0.0;
                for (int64_t j = a; j < b; ++j) {
                    double pj = exp(s[j] - mt);
                    lt += pj;
                    for (int64_t c = 0; c < d; ++c) pv[c] += pj * v[j * d + c];
                }
                double mi = m_buf[i], li = l_buf[i];
                double m_new = mi > mt ? mi : mt;
                double old_w = (mi == -INFINITY) ? 0.0 : li * exp(mi - m_new);
                double new_w = exp(mt - m_new);
                double l_new = old_w + new_w * lt;
                double *oi = o + i * d;
                for (int64_t c = 0; c < d; ++c) oi[c] = (old_w * oi[c] + new_w * pv[c]) / l_new;
                m_buf[i] = m_new;
                l_buf[i] = l_new;
            }
        }
    }
    for (int64_t i = 0; i < n_q; ++i) lse[i] = m_buf[i] + log(l_buf[i]);
    free(m_buf); free(l_buf); free(s); free(pv);
    return 0;
}

/*
 * Merge of partial results computed over a partition of the key range (the
 * final step of Flash-Decoding, "Flash Attention 原理与实践" section 5.1):
 * the merge rule of plate 08 applied to whole chunks.  With L_s the LSE and
 * O_s the normalised output of chunk s for one row,
 *   L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s
 * (computed against M = max_s L_s).  A chunk with no visible key has
 * L_s = -inf and weight 0; a row with no visible key in any chunk is an error.
 * o_parts: [n_parts, n_rows, d], lse_parts: [n_parts, n_rows]; o: [n_rows, d],
 * lse: [n_rows].
 */
int fa_oracle_merge(const double *o_parts, const double *lse_parts, int64_t n_parts,
                    int64_t n_rows, int64_t d, double *o, double *lse)
{
    if (!o_parts || !lse_parts || !o || !lse || n_parts < 1 || n_rows < 0 || d < 1) return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        double m = -INFINITY;
        for (int64_t s = 0; s < n_parts; ++s)
            if (lse_parts[s * n_rows + r] > m) m = lse_parts[s * n_rows + r];
        if (m == -INFINITY) return 1;
        double den = 0.0;
        for (int64_t c = 0; c < d; ++c) o[r * d + c] = 0.0;
        for (int64_t s = 0; s < n_parts; ++s) {
            const double ls = lse_parts[s * n_rows + r];
            if (ls == -INFINITY) continue;
            const double w = exp(ls - m);
            den += w;
            for (int64_t c = 0; c < d; ++c) o[r * d + c] += w * o_parts[(s * n_rows + r) * d + c];
        }
        for (int64_t c = 0; c < d; ++c) o[r * d + c] /= den;
        lse[r] = m + log(den);
    }
    return 0;
}

/*
 * Gradients of standard attention for one (batch, head) slice (the backward
 * pass of "FlashAttention 与显存" plate 09, which keeps only O and per-row
 * statistics and recomputes the rest).  The pages give no derivative
 * formulas; these are the textbook ones for O = softmax(S) V with
 * S = scale * Q K^T (rows masked as in the forward):
 *   P_ij  = exp(s_ij - m_i) / l_i            (the forward's probabilities)
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij                  (softmax Jacobian term)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j
 *   dK_j  = scale sum_i dS_ij q_i
 * for visible (i, j) only.  Computed in three plain passes:
 *   pass 1, every row i: s_ij, m_i, l_i, P_ij, dP_ij, D_i (kept: m, l, D);
 *   pass 2, selected rows: dQ_i (s_ij, dP_ij recomputed);
 *   pass 3, selected keys: dV_j and dK_j over the rows that see key j.
 * q, dout: [n_q, d]; k, v: [n_kv, d].  rows/keys: indices of the rows of dq
 * and keys of dk/dv to produce (NULL: all, then n_rows = n_q, n_keys = n_kv).
 * dq: [n_rows, d]; dk, dv: [n_keys, d].  Any of dq, dk, dv may be NULL.
 */
int fa_oracle_backward(const double *q, const double *k, const double *v, const double *dout,
                       int64_t n_q, int64_t n_kv, int64_t d, double scale, int causal,
                       const int64_t *rows, int64_t n_rows, const int64_t *keys, int64_t n_keys,
                       double *dq, double *dk, double *dv)
{
    if (!q || !k || !v || !dout || n_q < 0 || n_kv < 1 || d < 1 || n_rows < 0 || n_keys < 0) return 1;
    if ((!rows && n_rows != n_q) || (!keys && n_keys != n_kv)) return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= n_q) return 1;
    }
    for (int64_t r = 0; r < n_keys; ++r) {
        int64_t j = keys ? keys[r] : r;
        if (j < 0 || j >= n_kv) return 1;
    }
    double *m = (double *)malloc((size_t)(n_q ? n_q : 1) * sizeof(double));
    double *l = (double *)malloc((size_t)(n_q ? n_q : 1) * sizeof(double));
    double *D = (double *)malloc((size_t)(n_q ? n_q : 1) * sizeof(double));
    if (!m || !l || !D) {
        free(m); free(l); free(D);
        return 2;
    }
    int status = 0;
    /* pass 1: row statistics */
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)n_kv * sizeof(double));
        if (!s) {
#pragma omp atomic write
            status = 2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_q; ++i) {
            if (!s) continue;
            const int64_t nv = visible_keys(i, n_kv, causal);
            double mi = -INFINITY;
            for (int64_t j = 0; j < nv; ++j) {
                s[j] = score(q + i * d, k + j * d, d, scale);
                if (s[j] > mi) mi = s[j];
            }
            double li = 0.0;
            for (int64_t j = 0; j < nv; ++j) li += exp(s[j] - mi);
            double Di = 0.0;
            for (int64_t j = 0; j < nv; ++j) {
                const double pij = exp(s[j] - mi) / li;
                double dpij = 0.0;
                for (int64_t c = 0; c < d; ++c) dpij += dout[i * d + c] * v[j * d + c];
                Di += pij * dpij;
            }
            m[i] = mi;
            l[i] = li;
            D[i] = Di;
        }
        free(s);
    }
    /* pass 2: dQ of the selected rows */
    if (!status && dq) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t i = rows ? rows[r] : r;
            const int64_t nv = visible_keys(i, n_kv, causal);
            double *dqi = dq + r * d;
            for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
            for (int64_t j = 0; j < nv; ++j) {
                const double pij = exp(score(q + i * d, k + j * d, d, scale) - m[i]) / l[i];
                double dpij = 0.0;
                for (int64_t c = 0; c < d; ++c) dpij += dout[i * d + c] * v[j * d + c];
                const double dsij = pij * (dpij - D[i]);
                for (int64_t c = 0; c < d; ++c) dqi[c] += dsij * k[j * d + c];
            }
            for (int64_t c = 0; c < d; ++c) dqi[c] *= scale;
        }
    }
    /* pass 3: dK and dV of the selected keys */
    if (!status && (dk || dv)) {
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_keys; ++r) {
            const int64_t j = keys ? keys[r] : r;
            double *dkj = dk ? dk + r * d : NULL;
            double *dvj = dv ? dv + r * d : NULL;
            for (int64_t c = 0; c < d; ++c) {
                if (dkj) dkj[c] = 0.0;
                if (dvj) dvj[c] = 0.0;
            }
            for (int64_t i = 0; i < n_q; ++i) {
                if (j >= visible_keys(i, n_kv, causal)) continue;
                const double pij = exp(score(q + i * d, k + j * d, d, scale) - m[i]) / l[i];
                double dpij = 0.0;
                for (int64_t c = 0; c < d; ++c) dpij += dout[i * d + c] * v[j * d + c];
                const double dsij = pij * (dpij - D[i]);
                for (int64_t c = 0; c < d; ++c) {
                    if (dvj) dvj[c] += pij * dout[i * d + c];
                    if (dkj) dkj[c] += dsij * q[i * d + c];
                }
            }
            if (dkj)
                for (int64_t c = 0; c < d; ++c) dkj[c] *= scale;
        }
    }
    free(m); free(l); free(D);
    return status;
}

/*
 * Dropout (a training-time feature "FlashAttention 与显存" plates 07 and 09
 * name for the fused kernel, with the random state replayed in the backward
 * pass).  The pages specify no generator; this one is Philox4x32-10
 * (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3", SC 2011), written from that paper's definition: 10 rounds of
 *   (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2   (32x32 -> 64-bit products)
 *   c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
 * with M0 = 0xD2511F53, M1 = 0xCD9E8D57, and the key bumped by the Weyl
 * constants (0x9E3779B9, 0xBB67AE85) after every round.
 */
void fa_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * Dropout threshold: p is quantised to p8 / 256, p8 = floor(p * 256 + 1/2)
 * clamped to [0, 255]; 0 means no dropout.
 */
int fa_oracle_dropout_p8(double p)
{
    double x = floor(p * 256.0 + 0.5);
    if (x < 0.0) x = 0.0;
    if (x > 255.0) x = 255.0;
    return (int)x;
}

/*
 * Keep mask of one (batch, head) slice, bh = b * H + h: element (i, j) is
 * kept iff byte 4 (i mod 4) + (j mod 4) of Philox4x32-10 with counter
 * (j / 4, i / 4, bh, offset mod 2^32) and key (seed mod 2^32, seed / 2^32)
 * is >= p8 (byte b of the output is bits 8 (b mod 4) .. +7 of word b / 4).
 * mask: [n_q, n_kv] bytes, 1 = kept.
 */
int fa_oracle_dropout_mask(uint64_t seed, uint64_t offset, int64_t bh, int64_t n_q, int64_t n_kv,
                           int p8, uint8_t *mask)
{
    if (!mask || n_q < 0 || n_kv < 0 || bh < 0 || p8 < 0 || p8 > 255) return 1;
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int64_t i = 0; i < n_q; ++i)
        for (int64_t j = 0; j < n_kv; ++j) {
            const uint32_t ctr[4] = {(uint32_t)(j / 4), (uint32_t)(i / 4), (uint32_t)bh, (uint32_t)offset};
            uint32_t out[4];
            fa_oracle_philox4x32_10(ctr, key, out);
            const unsigned byte = (out[i % 4] >> (8 * (j % 4))) & 0xFFu;
            mask[i * n_kv + j] = byte >= (unsigned)p8 ? 1 : 0;
        }
    return 0;
}

/*
 * Attention with dropout for one (batch, head) slice: P as in
 * fa_oracle_naive (three passes over the visible keys), then
 *   O_i = rescale * sum_j P_ij keep_ij v_j,   LSE_i = m_i + ln l_i
 * (the LSE is that of the scores, before dropout).  keep: [n_q, n_kv]
 * bytes; rescale = 1 / (1 - p8 / 256) is passed in.  rows: optional
 * indices of the rows to compute (NULL: all n_q; then n_rows = n_q); row r
 * of o / lse is query rows[r].
 */
int fa_oracle_attention_dropout(const double *q, const double *k, const double *v, int64_t n_q,
                                int64_t n_kv, int64_t d, double scale, int causal,
                                const int64_t *rows, int64_t n_rows,
                                const uint8_t *keep, double rescale, double *o, double *lse)
{
    if (!q || !k || !v || !keep || !o || !lse || n_q < 0 || n_kv < 1 || d < 1 || n_rows < 0) return 1;
    if (!rows && n_rows != n_q) return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= n_q) return 1;
    }
    int status = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)n_kv * sizeof(double));
        if (!s) {
#pragma omp atomic write
            status = 2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            const int64_t i = rows ? rows[r] : r;
            const int64_t nv = visible_keys(i, n_kv, causal);
            double m = -INFINITY;
            for (int64_t j = 0; j < nv; ++j) {
                s[j] = score(q + i * d, k + j * d, d, scale);
                if (s[j] > m) m = s[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < nv; ++j) l = l + exp(s[j] - m);
            double *oi = o + r * d;
            for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
            for (int64_t j = 0; j < nv; ++j) {
                if (!keep[i * n_kv + j]) continue;
                const double zij = rescale * exp(s[j] - m) / l;
                for (int64_t c = 0; c < d; ++c) oi[c] += zij * v[j * d + c];
            }
            lse[r] = log(l) + m;
        }
        free(s);
    }
    return status;
}

/*
 * Gradients of fa_oracle_attention_dropout for one slice (textbook, as
 * fa_oracle_backward, with Z_ij = rescale * keep_ij):
 *   dV_j = sum_i P_ij Z_ij dO_i,   dP_ij = Z_ij (dO_i . v_j),
 *   D_i = sum_j P_ij dP_ij,        dS_ij = P_ij (dP_ij - D_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
 * Whole slices: dq [n_q, d], dk, dv [n_kv, d].
 */
int fa_oracle_backward_dropout(const double *q, const double *k, const double *v, const double *dout,
                               int64_t n_q, int64_t n_kv, int64_t d, double scale, int causal,
                               const uint8_t *keep, double rescale, double *dq, double *dk, double *dv)
{
    if (!q || !k || !v || !dout || !keep || !dq || !dk || !dv || n_q < 0 || n_kv < 1 || d < 1) return 1;
    double *P = (double *)calloc((size_t)(n_q ? n_q : 1) * (size_t)n_kv, sizeof(double));
    double *dS = (double *)calloc((size_t)(n_q ? n_q : 1) * (size_t)n_kv, sizeof(double));
    if (!P || !dS) {
        free(P); free(dS);
        return 2;
    }
    /* per row: P, dP, D, dS and dQ */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_q; ++i) {
        const int64_t nv = visible_keys(i, n_kv, causal);
        double m = -INFINITY;
        for (int64_t j = 0; j < nv; ++j) {
            P[i * n_kv + j] = score(q + i * d, k + j * d, d, scale);
            if (P[i * n_kv + j] > m) m = P[i * n_kv + j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nv; ++j) l += exp(P[i * n_kv + j] - m);
        for (int64_t j = 0; j < nv; ++j) P[i * n_kv + j] = exp(P[i * n_kv + j] - m) / l;
        double Di = 0.0;
        for (int64_t j = 0; j < nv; ++j) {
            double dpt = 0.0;
            for (int64_t c = 0; c < d; ++c) dpt += dout[i * d + c] * v[j * d + c];
            const double dpij = keep[i * n_kv + j] ? rescale * dpt : 0.0;
            dS[i * n_kv + j] = dpij;
            Di += P[i * n_kv + j] * dpij;
        }
        for (int64_t c = 0; c < d; ++c) dq[i * d + c] = 0.0;
        for (int64_t j = 0; j < nv; ++j) {
            dS[i * n_kv + j] = P[i * n_kv + j] * (dS[i * n_kv + j] - Di);
            for (int64_t c = 0; c < d; ++c) dq[i * d + c] += dS[i * n_kv + j] * k[j * d + c];
        }
        for (int64_t c = 0; c < d; ++c) dq[i * d + c] *= scale;
    }
    /* per key: dV and dK (P and dS are zero where key j is not visible) */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < n_kv; ++j) {
        for (int64_t c = 0; c < d; ++c) {
            dk[j * d + c] = 0.0;
            dv[j * d + c] = 0.0;
        }
        for (int64_t i = 0; i < n_q; ++i) {
            const double zij = keep[i * n_kv + j] ? rescale * P[i * n_kv + j] : 0.0;
            for (int64_t c = 0; c < d; ++c) {
                dv[j * d + c] += zij * dout[i * d + c];
                dk[j * d + c] += dS[i * n_kv + j] * q[i * d + c];
            }
        }
        for (int64_t c = 0; c < d; ++c) dk[j * d + c] *= scale;
    }
    free(P); free(dS);
    return 0;
}

/*
 * OCP 8-bit floating point E4M3 ("fn" variant) to double: 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
 * subnormals m * 2^-9; the all-ones pattern S.1111.111 is NaN and there are no
 * infinities; largest finite magnitude 1.75 * 2^8 = 448.
 */
double fa_oracle_e4m3_to_double(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double mag;
    if (e == 0xF && mant == 0x7) return NAN;
    if (e == 0) mag = ldexp((double)mant, -9);
    else mag = ldexp(1.0 + mant / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Decodes n E4M3 codes and multiplies each by descale (the product of two
 * doubles with 4 and 24 significant bits is exact). */
int fa_oracle_dequant_e4m3(const uint8_t *codes, int64_t n, double descale, double *out)
{
    if ((!codes || !out) && n > 0) return 1;
    for (int64_t t = 0; t < n; ++t) out[t] = fa_oracle_e4m3_to_double(codes[t]) * descale;
    return 0;
}
