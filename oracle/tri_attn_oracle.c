/*
 * oracle/tri_attn_oracle.c -- THE ORACLE: a plain, slow, fp64 CPU reference for
 * pair-biased triangle attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or run this code.  It shares nothing with the HIP path
 * (no kernels, headers, helpers, tables or constants) and the product never calls it.
 *
 * What it computes (per batch b, query row i, query column j and head h):
 *
 *   s_k = (1/sqrt(D)) * sum_d q[b,i,j,h,d] * k[b,i,k,h,d] + bias[b,h,j,k] + mask[b,k]
 *   out[b,i,j,h,:] = sum_k softmax_k(s)_k * v[b,i,k,h,:]
 *
 * Sources:
 *   - "Fold-CP: A Context Parallelism Framework for Biomolecular Modeling", Table 1
 *     (triangle attention, serial time B*H*N^3*D and space B*H*N^2*D: N^2 query
 *     positions (i,j) against N keys per head, score tensor never stored) and
 *     Figure 2(a) (the bias is the "triangular" one, indexed by the third edge (j,k)
 *     and so shared by every row i; keys, values and bias travel round a ring and
 *     the partial results are joined by a tiled-softmax merge).
 *   - Table 1's caption: every ring pattern takes P steps; each step contributes one
 *     contiguous key tile, so the key axis is cut into T tiles processed in order.
 *   - The merge is the online-normaliser rule of "Online normalizer calculation for
 *     softmax" (listed among Design-CP's prior work): a tile's state (m_t, l_t, a_t)
 *     joins the running state (m, l, a) as
 *        M = max(m, m_t),  l = e^(m-M) l + e^(m_t-M) l_t,  a = e^(m-M) a + e^(m_t-M) a_t.
 * Readings where the pages are silent: 1/sqrt(D) scales q.k only; the mask is an
 * additive [B,N] term over the key index; a tile whose keys are all -inf is the
 * identity of the merge; a row with no finite score gives out = 0 and lse = -inf.
 *
 * Ending-node orientation (oracle_tri_attn_ending): Figure 2(a) transposes the pair
 * tensor across its axes before the ring; read plainly, the same attention then runs
 * along columns with the triangular bias transposed:
 *
 *   s_k = (1/sqrt(D)) * sum_d q[b,i,j,h,d] * k[b,k,j,h,d] + bias[b,h,k,i] + mask[b,k]
 *   out[b,i,j,h,:] = sum_k softmax_k(s)_k * v[b,k,j,h,:]
 *
 * Split tiles (oracle_tile_state): one ring step's own softmax state over a key range,
 * (m_t, l_t, a_t) above with m_t the range's maximum score, unnormalised -- the
 * quantity a rank holds between the ring steps of Figure 2(a).
 *
 * Backward (oracle_tri_attn_bwd): Fold-CP trains through its context-parallel modules;
 * the pages give no formula for the gradients, so the oracle takes the plain derivative
 * of the definition (stated where the function is defined).
 *
 * All arithmetic is IEEE double, libm exp/log/sqrt, no fast-math and no contraction
 * (built with -ffp-contract=off).  Inputs are widened exactly: binary32 as is,
 * bfloat16 as the upper half of a binary32.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_DTYPE_FP32 0
#define ORACLE_DTYPE_BF16 1

#define ORACLE_OK 0
#define ORACLE_ERR_ARG -1
#define ORACLE_ERR_NOMEM -2

/* Exact widening of one stored element to double. */
static double widen(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_DTYPE_FP32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}

/* Near-equal contiguous key tiles: the first N mod T tiles hold ceil(N/T) keys,
 * the rest floor(N/T).  starts[] receives T+1 entries (starts[T] == N). */
void oracle_even_tiles(int64_t N, int64_t T, int64_t *starts)
{
    for (int64_t t = 0; t <= T; ++t)
        starts[t] = t * (N / T) + (t < N % T ? t : N % T);
}

/*
 * Shared body.  ending == 0: starting node (rows i in [0, I)); ending == 1: ending node
 * (I == N).  The tiles tile_start[0] < ... < tile_start[T] cover the keys taken into
 * account (all N keys for a forward; one range for a state).  state == 0: out and lse
 * receive the normalised result; state == 1: out receives the unnormalised accumulator
 * a and lse the pair (m, l) as [.., H, 2], the merged state of the tiles with m the
 * running maximum (m = -inf, l = 0, a = 0 when no score is finite).
 */
static int tri_attn_impl(const void *q, const void *k, const void *v, const void *bias,
                         const float *mask, int dtype,
                         int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                         const int64_t *tile_start, int64_t T, int64_t first_tile,
                         const int64_t *rows, int64_t n_rows,
                         double *out, double *lse, int ending, int state)
{
    if (!q || !k || !v || !bias || !out || !tile_start)
        return ORACLE_ERR_ARG;
    if (B < 1 || H < 1 || I < 1 || N < 1 || D < 1 || I > N || T < 1 || T > N)
        return ORACLE_ERR_ARG;
    if (ending && I != N)
        return ORACLE_ERR_ARG;
    if (state && !lse)
        return ORACLE_ERR_ARG;
    if (dtype != ORACLE_DTYPE_FP32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_ERR_ARG;
    if (tile_start[0] < 0 || tile_start[T] > N || first_tile < 0 || first_tile >= T)
        return ORACLE_ERR_ARG;
    if (!state && (tile_start[0] != 0 || tile_start[T] != N))
        return ORACLE_ERR_ARG;
    int64_t widest = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (tile_start[t + 1] <= tile_start[t])
            return ORACLE_ERR_ARG;
        if (tile_start[t + 1] - tile_start[t] > widest)
            widest = tile_start[t + 1] - tile_start[t];
    }
    const int64_t total = rows ? n_rows : B * I * N;
    if (rows) {
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= B * I * N)
                return ORACLE_ERR_ARG;
    }
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)widest * sizeof(double));
        double *a = (double *)malloc((size_t)D * sizeof(double));
        double *a_t = (double *)malloc((size_t)D * sizeof(double));
        const int ok = s && a && a_t;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < total; ++r) {
            if (!ok)
                continue;
            const int64_t flat = rows ? rows[r] : r;
            const int64_t j = flat % N;
            const int64_t bi = flat / N;        /* b*I + i */
            const int64_t b = bi / I, i = bi % I;
            for (int64_t h = 0; h < H; ++h) {
                const int64_t q_off = ((bi * N + j) * H + h) * D;
                double m = -INFINITY, l = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    a[d] = 0.0;
                for (int64_t step = 0; step < T; ++step) {
                    const int64_t t = (first_tile + step) % T;
                    const int64_t k0 = tile_start[t], k1 = tile_start[t + 1];
                    /* scores of this key tile and their maximum */
                    double m_t = -INFINITY;
                    for (int64_t kk = k0; kk < k1; ++kk) {
                        /* starting node: key (i, kk), bias[b,h,j,kk];
                         * ending node:   key (kk, j), bias[b,h,kk,i] */
                        const int64_t k_off = ending ? (((b * N + kk) * N + j) * H + h) * D
                                                     : ((bi * N + kk) * H + h) * D;
                        const int64_t b_off = ending ? ((b * H + h) * N + kk) * N + i
                                                     : ((b * H + h) * N + j) * N + kk;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dot += widen(q, q_off + d, dtype) * widen(k, k_off + d, dtype);
                        double sc = dot * inv_sqrt_d + widen(bias, b_off, dtype);
                        if (mask)
                            sc += (double)mask[b * N + kk];
                        s[kk - k0] = sc;
                        if (sc > m_t)
                            m_t = sc;
                    }
                    if (m_t == -INFINITY)
                        continue;   /* every key of the tile dropped: identity of the merge */
                    /* the tile's own softmax state relative to its maximum */
                    double l_t = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        a_t[d] = 0.0;
                    for (int64_t kk = k0; kk < k1; ++kk) {
                        const double w = exp(s[kk - k0] - m_t);
                        const int64_t v_off = ending ? (((b * N + kk) * N + j) * H + h) * D
                                                     : ((bi * N + kk) * H + h) * D;
                        l_t += w;
                        for (int64_t d = 0; d < D; ++d)
                            a_t[d] += w * widen(v, v_off + d, dtype);
                    }
                    /* merge the tile into the running state */
                    const double M = m > m_t ? m : m_t;
                    const double alpha = (m == -INFINITY) ? 0.0 : exp(m - M);
                    const double beta = exp(m_t - M);
                    l = alpha * l + beta * l_t;
                    for (int64_t d = 0; d < D; ++d)
                        a[d] = alpha * a[d] + beta * a_t[d];
                    m = M;
                }
                double *o = out + (r * H + h) * D;
                if (state) {
                    for (int64_t d = 0; d < D; ++d)
                        o[d] = a[d];
                    lse[(r * H + h) * 2] = m;
                    lse[(r * H + h) * 2 + 1] = l;
                    continue;
                }
                for (int64_t d = 0; d < D; ++d)
                    o[d] = (l > 0.0) ? a[d] / l : 0.0;
                if (lse)
                    lse[r * H + h] = (l > 0.0) ? m + log(l) : -INFINITY;
            }
        }
        free(s);
        free(a);
        free(a_t);
    }
    return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * Starting-node triangle attention.
 * q, k, v:   [B, I, N, H, D] of dtype;  bias: [B, H, N, N] of dtype;
 * mask:      [B, N] binary32 additive, or NULL;
 * tile_start: T+1 increasing key offsets, tile_start[0] = 0, tile_start[T] = N;
 * first_tile: the ring step that runs first (tiles taken first_tile, first_tile+1, ... mod T);
 * rows:      n_rows flat row indices (b*I + i)*N + j, or NULL for all B*I*N rows in order;
 * out:       [n_rows, H, D] doubles;  lse: [n_rows, H] doubles (log-sum-exp of the scores), or NULL.
 * Returns 0, or a negative code for bad arguments / no memory.
 */
int oracle_tri_attn(const void *q, const void *k, const void *v, const void *bias,
                    const float *mask, int dtype,
                    int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                    const int64_t *tile_start, int64_t T, int64_t first_tile,
                    const int64_t *rows, int64_t n_rows,
                    double *out, double *lse)
{
    return tri_attn_impl(q, k, v, bias, mask, dtype, B, H, I, N, D, tile_start, T, first_tile,
                         rows, n_rows, out, lse, 0, 0);
}

/*
 * Ending-node triangle attention; q, k, v [B, N, N, H, D], flat rows (b*N + i)*N + j,
 * everything else as oracle_tri_attn.
 */
int oracle_tri_attn_ending(const void *q, const void *k, const void *v, const void *bias,
                           const float *mask, int dtype,
                           int64_t B, int64_t H, int64_t N, int64_t D,
                           const int64_t *tile_start, int64_t T, int64_t first_tile,
                           const int64_t *rows, int64_t n_rows,
                           double *out, double *lse)
{
    return tri_attn_impl(q, k, v, bias, mask, dtype, B, H, N, N, D, tile_start, T, first_tile,
                         rows, n_rows, out, lse, 1, 0);
}

/*
 * Softmax state of the keys [key_begin, key_end) as one tile, for either orientation
 * (ending = 0 or 1): acc [n_rows, H, D] receives a_t, ml [n_rows, H, 2] the pair
 * (m_t, l_t); m_t is the range's maximum score.
 */
int oracle_tile_state(const void *q, const void *k, const void *v, const void *bias,
                      const float *mask, int dtype,
                      int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                      int64_t key_begin, int64_t key_end, int ending,
                      const int64_t *rows, int64_t n_rows,
                      double *acc, double *ml)
{
    if (key_begin < 0 || key_end > N || key_begin >= key_end)
        return ORACLE_ERR_ARG;
    const int64_t range[2] = {key_begin, key_end};
    return tri_attn_impl(q, k, v, bias, mask, dtype, B, H, I, N, D, range, 1, 0,
                         rows, n_rows, acc, ml, ending != 0, 1);
}

/*
 * Backward of starting-node triangle attention: the derivative of the definition above
 * (softmax attention with an additive bias) with respect to q, k, v and the triangular
 * bias, for an upstream gradient dout [B, I, N, H, D] (binary32).  The tiling of the key
 * axis does not enter: the forward result it produces is the definition's.  Per (b,i,j,h):
 *
 *   p_k   = softmax_k(s)_k,          o = sum_k p_k v_k
 *   dp_k  = dout . v_k,              delta = sum_k p_k dp_k  (= dout . o)
 *   ds_k  = p_k (dp_k - delta)
 *   dq_j += sum_k ds_k k_k / sqrt(D);   dk_k += ds_k q_j / sqrt(D);   dv_k += p_k dout_j
 *   dbias[b,h,j,k] += ds_k              (summed over every row i: the bias is shared)
 *
 * A key with mask -inf has p_k = 0 and receives nothing; a row with no finite score
 * contributes nothing.  dq, dk, dv [B, I, N, H, D] and dbias [B, H, N, N] are doubles,
 * overwritten.  One OpenMP task per (b, h), so every sum over rows runs in one thread
 * in row order.
 */
int oracle_tri_attn_bwd(const void *q, const void *k, const void *v, const void *bias,
                        const float *mask, const float *dout, int dtype,
                        int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                        double *dq, double *dk, double *dv, double *dbias)
{
    if (!q || !k || !v || !bias || !dout || !dq || !dk || !dv || !dbias)
        return ORACLE_ERR_ARG;
    if (B < 1 || H < 1 || I < 1 || N < 1 || D < 1 || I > N)
        return ORACLE_ERR_ARG;
    if (dtype != ORACLE_DTYPE_FP32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_ERR_ARG;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    const int64_t n_elem = B * I * N * H * D;
    for (int64_t e = 0; e < n_elem; ++e)
        dq[e] = dk[e] = dv[e] = 0.0;
    for (int64_t e = 0; e < B * H * N * N; ++e)
        dbias[e] = 0.0;
    int failed = 0;

#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)N * sizeof(double));
        double *dp = (double *)malloc((size_t)N * sizeof(double));
        const int ok = p && dp;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (!ok)
                continue;
            const int64_t b = bh / H, h = bh % H;
            for (int64_t i = 0; i < I; ++i) {
                const int64_t line = (b * I + i) * N;     /* flat (b, i, j=0) */
                for (int64_t j = 0; j < N; ++j) {
                    const int64_t q_off = ((line + j) * H + h) * D;
                    /* scores and their maximum */
                    double mx = -INFINITY;
                    for (int64_t kk = 0; kk < N; ++kk) {
                        const int64_t k_off = ((line + kk) * H + h) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dot += widen(q, q_off + d, dtype) * widen(k, k_off + d, dtype);
                        double sc = dot * inv_sqrt_d + widen(bias, ((b * H + h) * N + j) * N + kk, dtype);
                        if (mask)
                            sc += (double)mask[b * N + kk];
                        p[kk] = sc;
                        if (sc > mx)
                            mx = sc;
                    }
                    if (mx == -INFINITY)
                        continue;   /* no finite score: the row has no gradient */
                    double l = 0.0;
                    for (int64_t kk = 0; kk < N; ++kk) {
                        p[kk] = exp(p[kk] - mx);
                        l += p[kk];
                    }
                    double delta = 0.0;
                    for (int64_t kk = 0; kk < N; ++kk) {
                        p[kk] /= l;
                        const int64_t v_off = ((line + kk) * H + h) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dot += (double)dout[q_off + d] * widen(v, v_off + d, dtype);
                        dp[kk] = dot;
                        delta += p[kk] * dot;
                    }
                    for (int64_t kk = 0; kk < N; ++kk) {
                        const double ds = p[kk] * (dp[kk] - delta);
                        const int64_t kv_off = ((line + kk) * H + h) * D;
                        for (int64_t d = 0; d < D; ++d) {
                            dq[q_off + d] += ds * widen(k, kv_off + d, dtype) * inv_sqrt_d;
                            dk[kv_off + d] += ds * widen(q, q_off + d, dtype) * inv_sqrt_d;
                            dv[kv_off + d] += p[kk] * (double)dout[q_off + d];
                        }
                        dbias[((b * H + h) * N + j) * N + kk] += ds;
                    }
                }
            }
        }
        free(p);
        free(dp);
    }
    return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * dbias of selected query columns: dbias[b, h, j, k] = sum over every row i of ds_k for the
 * query (b, i, j, h), with p, dp, delta and ds as written above oracle_tri_attn_bwd, for j
 * in cols[0 .. n_cols-1] only (so that a column sum over all N rows of a large problem
 * costs O(I N D) per column instead of the whole backward).  out [B, H, n_cols, N] doubles,
 * overwritten.  One OpenMP task per (b, h, column); each sum over rows runs in one thread
 * in row order.  A row whose query has no finite score contributes nothing.
 */
int oracle_tri_attn_dbias_cols(const void *q, const void *k, const void *v, const void *bias,
                               const float *mask, const float *dout, int dtype,
                               int64_t B, int64_t H, int64_t I, int64_t N, int64_t D,
                               const int64_t *cols, int64_t n_cols, double *out)
{
    if (!q || !k || !v || !bias || !dout || !cols || !out || n_cols < 1)
        return ORACLE_ERR_ARG;
    if (B < 1 || H < 1 || I < 1 || N < 1 || D < 1 || I > N)
        return ORACLE_ERR_ARG;
    if (dtype != ORACLE_DTYPE_FP32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_ERR_ARG;
    for (int64_t c = 0; c < n_cols; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return ORACLE_ERR_ARG;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int64_t e = 0; e < B * H * n_cols * N; ++e)
        out[e] = 0.0;
    int failed = 0;

#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)N * sizeof(double));
        double *dp = (double *)malloc((size_t)N * sizeof(double));
        const int ok = p && dp;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < B * H * n_cols; ++t) {
            if (!ok)
                continue;
            const int64_t c = t % n_cols, bh = t / n_cols, b = bh / H, h = bh % H, j = cols[c];
            double *row = out + t * N;
            for (int64_t i = 0; i < I; ++i) {
                const int64_t line = (b * I + i) * N;     /* flat (b, i, j=0) */
                const int64_t q_off = ((line + j) * H + h) * D;
                double mx = -INFINITY;
                for (int64_t kk = 0; kk < N; ++kk) {
                    const int64_t k_off = ((line + kk) * H + h) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        dot += widen(q, q_off + d, dtype) * widen(k, k_off + d, dtype);
                    double sc = dot * inv_sqrt_d + widen(bias, ((b * H + h) * N + j) * N + kk, dtype);
                    if (mask)
                        sc += (double)mask[b * N + kk];
                    p[kk] = sc;
                    if (sc > mx)
                        mx = sc;
                }
                if (mx == -INFINITY)
                    continue;
                double l = 0.0;
                for (int64_t kk = 0; kk < N; ++kk) {
                    p[kk] = exp(p[kk] - mx);
                    l += p[kk];
                }
                double delta = 0.0;
                for (int64_t kk = 0; kk < N; ++kk) {
                    p[kk] /= l;
                    const int64_t v_off = ((line + kk) * H + h) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        dot += (double)dout[q_off + d] * widen(v, v_off + d, dtype);
                    dp[kk] = dot;
                    delta += p[kk] * dot;
                }
                for (int64_t kk = 0; kk < N; ++kk)
                    row[kk] += p[kk] * (dp[kk] - delta);
            }
        }
        free(p);
        free(dp);
    }
    return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}
