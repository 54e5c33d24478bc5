/*
 * mha_oracle.c -- CPU fp64 oracle for multi-head scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library; it is the plain definition of the
 * operation, written out step by step, slow on purpose.
 *
 * What it computes, per batch b, head t and query row i:
 *
 *   1. scores   s_ij = scale * sum_c Q[b,t,i,c] * K[b,t,j,c]   for every key j
 *        ("Transformer: 详解" §4.1, the energy / scaling steps;
 *         "序列建模架构的演进与变革（二）" §4.3 steps 2-3 and §4.9 step ①;
 *         hugogu wiki "Transformer", self-attention steps 2-3, which fixes
 *         Q in R^{n x d_k}, K in R^{m x d_k}, V in R^{m x d_v}).
 *   2. mask     s_ij = -inf unless  j < L_b  and  (not causal or j <= i)
 *        key padding: "Transformer: 详解" §3.4 (keep-mask over the key axis,
 *        broadcast over heads and queries); causal: "Transformer: 详解" §5.3
 *        (Mask_ij = 0 for j <= i, -inf for j > i) and "第2章：完整的
 *        Transformer 架构" §6; the two are combined with AND ("Transformer:
 *        详解" §5.3, tgt_mask = pad_mask & subsequent_mask).
 *   3. softmax  a_ij = exp(s_ij - M_i) / sum_k exp(s_ik - M_i),  M_i = max_k s_ik
 *        ("序列建模架构的演进与变革（二）" §4.3 step 4; subtracting the row
 *        maximum leaves the real-valued result unchanged).  A row with no
 *        valid key (M_i = -inf) gets all-zero weights and a zero output: the
 *        pages leave this case open and this is the reading adopted.
 *   4. output   O[b,t,i,:] = sum_j a_ij * V[b,t,j,:]   summed over the m keys
 *        ("序列建模架构的演进与变革（二）" §4.3 step 5).
 *
 * The extended entry points (mha_oracle_ex_f64, mha_oracle_ex_rows_f64) add
 * the variants that sit next to the core on the pages, each still as its
 * plain definition:
 *
 *   - grouped / multi-query attention: Hkv key/value heads shared by groups
 *     of H/Hkv consecutive query heads; query head t reads K/V head
 *     t / (H/Hkv) (hugogu wiki "Transformer", attention-optimisation table, and
 *     "序列建模架构的演进与变革（二）" §3.8:
 *     GQA reduces the number of K/V heads, MQA shares one K/V head among
 *     all queries);
 *   - ALiBi: the scaled score gets -slope_t * |p_i - j| added before the
 *     softmax, with a per-head slope and p_i the query's position
 *     ("第2章：完整的 Transformer 架构" §5.3);
 *   - causal alignment: top-left (key j visible to query i when j <= i, the
 *     decoder mask of "Transformer: 详解" §5.3) or bottom-right (query i is
 *     the token at position p_i = i + L_b - n of a sequence whose first L_b
 *     keys are filled, as in incremental decoding with a key/value cache,
 *     hugogu wiki "Transformer", KV-cache section); without a causal mask
 *     p_i = i;
 *   - the natural-log log-sum-exp of each row's valid scores (-inf for a
 *     row with no valid key): A_ij = exp(s_ij - lse_i), which is what a
 *     second pass needs to return the weights.
 *
 * Layouts: Q [B,H,n,dk], K [B,H,m,dk], V [B,H,m,dv], O [B,H,n,dv], all
 * row-major contiguous float64 (K and V have Hkv heads in the extended
 * entry points).  key_lens: int32[B] or NULL (= all m keys);
 * each length is clamped to [0, m].  Build: -O2, no fast-math, no FP
 * contraction; OpenMP over rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int64_t clamp_len(const int32_t *key_lens, int64_t b, int64_t m)
{
    if (key_lens == NULL) return m;
    int64_t L = key_lens[b];
    if (L < 0) L = 0;
    if (L > m) L = m;
    return L;
}

/* What one query row sees: the valid-key count of its sequence, the mask
 * mode (0 none, 1 causal top-left, 2 causal bottom-right), its position p
 * (i, or i + L - n for mode 2) and the ALiBi slope of its head (0 = none). */
typedef struct {
    int64_t L;
    int mode;
    int64_t pos;
    double slope;
} row_view;

static int key_visible(const row_view *rv, int64_t j)
{
    return j < rv->L && (rv->mode == 0 || j <= rv->pos);
}

/*
 * One query row: steps 1-4 above.  s_row and a_row are caller-provided rows
 * of length m that receive the masked scores and the weights; o_row has dv
 * entries.  *lse receives the log-sum-exp of the valid scores (-inf when
 * there is none).  Returns the number of valid keys in the row.
 */
static int64_t attend_row(const double *q, const double *Kh, const double *Vh,
                          int64_t m, int64_t dk, int64_t dv,
                          const row_view *rv, double scale,
                          double *s_row, double *a_row, double *o_row,
                          double *lse)
{
    int64_t nvalid = 0;
    /* step 1 + step 2: explicit score row, invalid keys set to -inf */
    for (int64_t j = 0; j < m; ++j) {
        if (!key_visible(rv, j)) {
            s_row[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        const double *k = Kh + j * dk;
        for (int64_t c = 0; c < dk; ++c) dot += q[c] * k[c];
        double dist = (double)(rv->pos - j);
        if (dist < 0) dist = -dist;
        s_row[j] = scale * dot - rv->slope * dist;
        ++nvalid;
    }
    /* step 3: row softmax with max subtraction */
    double M = -INFINITY;
    for (int64_t j = 0; j < m; ++j)
        if (s_row[j] > M) M = s_row[j];
    if (M == -INFINITY) {
        for (int64_t j = 0; j < m; ++j) a_row[j] = 0.0;
        for (int64_t c = 0; c < dv; ++c) o_row[c] = 0.0;
        *lse = -INFINITY;
        return 0;
    }
    double Z = 0.0;
    for (int64_t j = 0; j < m; ++j) {
        double e = (s_row[j] == -INFINITY) ? 0.0 : exp(s_row[j] - M);
        a_row[j] = e;
        Z += e;
    }
    for (int64_t j = 0; j < m; ++j) a_row[j] /= Z;
    *lse = M + log(Z);
    /* step 4: weighted sum of value rows */
    for (int64_t c = 0; c < dv; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < m; ++j) {
        double a = a_row[j];
        if (a == 0.0) continue;
        const double *v = Vh + j * dv;
        for (int64_t c = 0; c < dv; ++c) o_row[c] += a * v[c];
    }
    return nvalid;
}

static row_view view_of(const int32_t *key_lens, int mode, const double *slopes,
                        int64_t b, int64_t t, int64_t i, int64_t n, int64_t m)
{
    row_view rv;
    rv.L = clamp_len(key_lens, b, m);
    rv.mode = mode;
    rv.pos = (mode == 2) ? i + rv.L - n : i;
    rv.slope = slopes ? slopes[t] : 0.0;
    return rv;
}

/* Per-thread score and weight rows for the loops below. */
static int thread_count(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int thread_id(void)
{
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

static int shapes_ok(int64_t B, int64_t H, int64_t Hkv, int64_t n, int64_t m,
                     int64_t dk, int64_t dv, int mode)
{
    if (B < 0 || H < 0 || n < 0 || m < 0 || dk < 0 || dv < 0) return 0;
    if (Hkv <= 0 || H % Hkv != 0) return H == 0 && Hkv == 0;
    return mode >= 0 && mode <= 2;
}

/*
 * Full extended oracle: every row of every (b, t).  K and V have Hkv heads;
 * mode is the mask mode above; slopes is double[H] or NULL.  LSE_out
 * ([B,H,n]), S_out and A_out ([B,H,n,m]) are optional.
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int mha_oracle_ex_f64(const double *Q, const double *K, const double *V,
                      const int32_t *key_lens, int mode, const double *slopes,
                      double scale, int64_t B, int64_t H, int64_t Hkv,
                      int64_t n, int64_t m, int64_t dk, int64_t dv,
                      double *O, double *LSE_out, double *S_out, double *A_out)
{
    if (!shapes_ok(B, H, Hkv, n, m, dk, dv, mode)) return -1;
    const int64_t rows = B * H * n;
    const int64_t group = Hkv > 0 ? H / Hkv : 1;
    const int nt = thread_count();
    const size_t mm = (size_t)(m > 0 ? m : 1);
    double *pool = (double *)malloc(sizeof(double) * mm * 2 * (size_t)nt);
    if (pool == NULL) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t i = r % n;
        const int64_t bt = r / n;
        const int64_t b = bt / H, t = bt % H;
        const int64_t bkv = b * Hkv + t / group;
        double *mine = pool + (size_t)thread_id() * 2 * mm;
        double *s_row = S_out ? S_out + r * m : mine;
        double *a_row = A_out ? A_out + r * m : mine + mm;
        const row_view rv = view_of(key_lens, mode, slopes, b, t, i, n, m);
        double lse;
        attend_row(Q + r * dk, K + bkv * m * dk, V + bkv * m * dv, m, dk, dv,
                   &rv, scale, s_row, a_row, O + r * dv, &lse);
        if (LSE_out) LSE_out[r] = lse;
    }
    free(pool);
    return 0;
}

/*
 * Sampled rows of the extended oracle: the rows named in idx, an int64
 * array of nrows triples (b, t, i).  O_rows receives nrows x dv values and
 * LSE_rows (optional) nrows values.  Used where the full problem is too
 * large to evaluate on the CPU in the time a test may take.  Returns 0, or
 * -1 on a bad argument, a bad index or allocation failure.
 */
int mha_oracle_ex_rows_f64(const double *Q, const double *K, const double *V,
                           const int32_t *key_lens, int mode, const double *slopes,
                           double scale, int64_t B, int64_t H, int64_t Hkv,
                           int64_t n, int64_t m, int64_t dk, int64_t dv,
                           const int64_t *idx, int64_t nrows, double *O_rows,
                           double *LSE_rows)
{
    if (!shapes_ok(B, H, Hkv, n, m, dk, dv, mode)) return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t b = idx[3 * r], t = idx[3 * r + 1], i = idx[3 * r + 2];
        if (b < 0 || b >= B || t < 0 || t >= H || i < 0 || i >= n) return -1;
    }
    const int64_t group = Hkv > 0 ? H / Hkv : 1;
    const int nt = thread_count();
    const size_t mm = (size_t)(m > 0 ? m : 1);
    double *pool = (double *)malloc(sizeof(double) * mm * 2 * (size_t)nt);
    if (pool == NULL) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = idx[3 * r], t = idx[3 * r + 1], i = idx[3 * r + 2];
        const int64_t bt = b * H + t;
        const int64_t bkv = b * Hkv + t / group;
        double *mine = pool + (size_t)thread_id() * 2 * mm;
        const row_view rv = view_of(key_lens, mode, slopes, b, t, i, n, m);
        double lse;
        attend_row(Q + (bt * n + i) * dk, K + bkv * m * dk, V + bkv * m * dv,
                   m, dk, dv, &rv, scale, mine, mine + mm, O_rows + r * dv,
                   &lse);
        if (LSE_rows) LSE_rows[r] = lse;
    }
    free(pool);
    return 0;
}

/*
 * The core operation of the benchmark workloads: H K/V heads, the causal
 * mask top-left (which needs n == m here), no ALiBi.  S_out and A_out, when
 * not NULL, receive the masked score matrix and the weights, [B,H,n,m].
 */
int mha_oracle_f64(const double *Q, const double *K, const double *V,
                   const int32_t *key_lens, int causal, double scale,
                   int64_t B, int64_t H, int64_t n, int64_t m,
                   int64_t dk, int64_t dv,
                   double *O, double *S_out, double *A_out)
{
    if (causal && n != m) return -1;
    return mha_oracle_ex_f64(Q, K, V, key_lens, causal ? 1 : 0, NULL, scale, B,
                             H, H, n, m, dk, dv, O, NULL, S_out, A_out);
}

/* Sampled rows of the core operation (see mha_oracle_f64). */
int mha_oracle_rows_f64(const double *Q, const double *K, const double *V,
                        const int32_t *key_lens, int causal, double scale,
                        int64_t B, int64_t H, int64_t n, int64_t m,
                        int64_t dk, int64_t dv,
                        const int64_t *idx, int64_t nrows, double *O_rows)
{
    if (causal && n != m) return -1;
    return mha_oracle_ex_rows_f64(Q, K, V, key_lens, causal ? 1 : 0, NULL,
                                  scale, B, H, H, n, m, dk, dv, idx, nrows,
                                  O_rows, NULL);
}

/* Threads the OpenMP runtime will use for the calls above. */
int mha_oracle_threads(void)
{
    return thread_count();
}
