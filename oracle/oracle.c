/*
 * Attention oracle (forward and backward): TEST INFRASTRUCTURE, not part of
 * the product.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. It shares no code, header or constant with the HIP
 * path, and the HIP path never calls it.
 *
 * Everything is plain fp64 C, built without fast-math, so a reader can check
 * each function against the passage it cites:
 *
 *   [P1] "FlashAttention: The GPU Memory Hack That Changed Everything"
 *        (ai.branddocks.com, episode 75)
 *   [P2] "Flash Attention Optimization" chapter (aicomputerinstitute.com)
 *
 * Conventions (readings of points the pages leave open):
 *   - tensors are contiguous [B][H][N][d], one (b, h) pair = one "head";
 *   - scores carry an explicit `scale` (the pages use 1/sqrt(d));
 *   - causal means key j is visible to query i iff j <= i (square
 *     self-attention), so every row sees at least key 0;
 *   - lse is the natural-log log-sum-exp of the scaled, masked scores,
 *     lse_i = m_i + ln(l_i).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Direct softmax-weighted sum for one query row: subtract the global max,
 * exponentiate, normalize, then weight the values.
 * [P2, "Worked example: online softmax by hand", the direct computation]
 * [P2, "Attention is not slow because of arithmetic": P = softmax(S), O = P V]
 *
 * s: n scores; v: n value vectors of length dv (row-major [n][dv]);
 * out: dv outputs; lse (may be NULL): m + ln(sum).
 * Scores equal to -INFINITY (masked keys) get weight 0; at least one score
 * must be finite.
 */
int oracle_softmax_row(const double *s, const double *v, long n, long dv,
                       double *out, double *lse)
{
    if (!s || !v || !out || n < 1 || dv < 1)
        return ORACLE_ERR_ARG;
    double m = -INFINITY;
    for (long j = 0; j < n; ++j)
        if (s[j] > m)
            m = s[j];
    if (!(m > -INFINITY))
        return ORACLE_ERR_ARG;
    double *p = (double *)malloc((size_t)n * sizeof(double));
    if (!p)
        return ORACLE_ERR_NOMEM;
    double sum = 0.0;
    for (long j = 0; j < n; ++j) {
        p[j] = exp(s[j] - m);
        sum += p[j];
    }
    for (long j = 0; j < n; ++j)
        p[j] /= sum;
    for (long t = 0; t < dv; ++t)
        out[t] = 0.0;
    for (long j = 0; j < n; ++j)
        for (long t = 0; t < dv; ++t)
            out[t] += p[j] * v[j * dv + t];
    if (lse)
        *lse = m + log(sum);
    free(p);
    return ORACLE_OK;
}

/*
 * Partial softmax state of one row over a subset of its keys:
 *   m   = the largest score in the subset (the exponent offset),
 *   l   = sum over the subset of exp(s_j - m),
 *   acc = sum over the subset of exp(s_j - m) * v_j   (dv values).
 * The empty subset (or one whose scores are all -inf) is m = -inf, l = 0,
 * acc = 0. Two states of disjoint subsets combine into the state of their
 * union by moving both to the common offset max(m_a, m_b); the combination
 * is associative and commutative, so any blocking of a row gives the same
 * state up to rounding.
 * [P2, "The fix: tile the computation, never materialize the full matrix":
 *  the per-block max, sum and weighted sum, and the combination of a running
 *  result with a new block through two correction factors]
 */
typedef struct {
    double m;
    double l;
    double *acc;
} row_state;

/* State of keys [lo, hi) of a row, computed from its own max. */
static void state_of_keys(const double *s, const double *v, long lo, long hi,
                          long dv, row_state *st)
{
    st->m = -INFINITY;
    for (long j = lo; j < hi; ++j)
        st->m = s[j] > st->m ? s[j] : st->m;
    st->l = 0.0;
    for (long t = 0; t < dv; ++t)
        st->acc[t] = 0.0;
    if (!(st->m > -INFINITY))
        return; /* every key of the subset masked: the empty state */
    for (long j = lo; j < hi; ++j) {
        const double w = exp(s[j] - st->m);
        st->l += w;
        for (long t = 0; t < dv; ++t)
            st->acc[t] += w * v[j * dv + t];
    }
}

/* *a becomes the state of the union of a's and b's (disjoint) subsets. */
static void state_combine(row_state *a, const row_state *b, long dv)
{
    if (!(b->l > 0.0))
        return; /* b is empty */
    if (!(a->l > 0.0)) {
        a->m = b->m;
        a->l = b->l;
        for (long t = 0; t < dv; ++t)
            a->acc[t] = b->acc[t];
        return;
    }
    const double offset = a->m > b->m ? a->m : b->m;
    const double fa = exp(a->m - offset), fb = exp(b->m - offset);
    a->l = a->l * fa + b->l * fb;
    for (long t = 0; t < dv; ++t)
        a->acc[t] = a->acc[t] * fa + b->acc[t] * fb;
    a->m = offset;
}

/*
 * Online softmax of one row in block-local form: the row is cut into blocks
 * of `block` consecutive keys, each block's state is computed on its own
 * (state_of_keys) and combined into the running state (state_combine) in
 * key order; the output is acc / l of the final state.
 * [P2, "The fix: tile the computation, never materialize the full matrix"]
 * [P2, "Tracing the algorithm as code"]
 *
 * Reading for a case the pages do not cover: a block whose scores are all
 * -inf (all masked) is the empty state and changes nothing, instead of
 * producing exp(-inf + inf).
 * m_out / l_out (may be NULL) receive the final state's offset and sum.
 */
int oracle_online_row_two_scale(const double *s, const double *v, long n,
                                long dv, long block, double *out,
                                double *m_out, double *l_out)
{
    if (!s || !v || !out || n < 1 || dv < 1 || block < 1)
        return ORACLE_ERR_ARG;
    row_state run = {-INFINITY, 0.0, (double *)calloc((size_t)dv, sizeof(double))};
    row_state part = {-INFINITY, 0.0, (double *)calloc((size_t)dv, sizeof(double))};
    if (!run.acc || !part.acc) {
        free(run.acc);
        free(part.acc);
        return ORACLE_ERR_NOMEM;
    }
    for (long lo = 0; lo < n; lo += block) {
        const long hi = lo + block < n ? lo + block : n;
        state_of_keys(s, v, lo, hi, dv, &part);
        state_combine(&run, &part, dv);
    }
    int rc = ORACLE_OK;
    if (!(run.l > 0.0))
        rc = ORACLE_ERR_ARG; /* every score was -inf */
    else
        for (long t = 0; t < dv; ++t)
            out[t] = run.acc[t] / run.l;
    if (m_out)
        *m_out = run.m;
    if (l_out)
        *l_out = run.l;
    free(run.acc);
    free(part.acc);
    return rc;
}

/*
 * Online softmax, single running-max form, for one row.
 * [P1, "FlashAttention: IO-Aware Tiling" / "The Tiling Strategy", the
 *  pseudocode's inner loop, and "The Online Softmax Trick"]
 *
 * Per block: block max, new running max m_new = max(m, block max);
 * l = l*exp(m - m_new) + sum(exp(s - m_new));
 * O = O*exp(m - m_new) + sum(exp(s - m_new) * v); m = m_new.
 * After the last block the output is O / l.
 * Reading: a block with every score -inf leaves m unchanged and adds 0
 * (exp(-inf - m) = 0); if m is still -inf there, the block is skipped.
 */
int oracle_online_row_single_max(const double *s, const double *v, long n,
                                 long dv, long block, double *out,
                                 double *m_out, double *l_out)
{
    if (!s || !v || !out || n < 1 || dv < 1 || block < 1)
        return ORACLE_ERR_ARG;
    double *o = (double *)calloc((size_t)dv, sizeof(double));
    if (!o)
        return ORACLE_ERR_NOMEM;
    double m = -INFINITY, l = 0.0;
    for (long start = 0; start < n; start += block) {
        long end = start + block < n ? start + block : n;
        double m_blk = -INFINITY;
        for (long j = start; j < end; ++j)
            if (s[j] > m_blk)
                m_blk = s[j];
        double m_new = m > m_blk ? m : m_blk;
        if (!(m_new > -INFINITY))
            continue; /* nothing visible yet */
        double corr = exp(m - m_new);
        double sum = 0.0;
        for (long j = start; j < end; ++j)
            sum += exp(s[j] - m_new);
        l = l * corr + sum;
        for (long t = 0; t < dv; ++t) {
            double pv = 0.0;
            for (long j = start; j < end; ++j)
                pv += exp(s[j] - m_new) * v[j * dv + t];
            o[t] = o[t] * corr + pv;
        }
        m = m_new;
    }
    int rc = ORACLE_OK;
    if (!(l > 0.0))
        rc = ORACLE_ERR_ARG;
    else
        for (long t = 0; t < dv; ++t)
            out[t] = o[t] / l;
    if (m_out)
        *m_out = m;
    if (l_out)
        *l_out = l;
    free(o);
    return rc;
}

/*
 * One query row of standard attention, materializing that row of S and P.
 * S[j] = scale * sum_t Q[i][t] K[j][t]; causal: S[j] = -inf for j > i;
 * P[j] = exp(S[j] - max S) / sum_j exp(S[j] - max S); O[i] = sum_j P[j] V[j];
 * lse_i = max S + ln(sum_j exp(S[j] - max S)).
 * [P1, "Standard Attention: The Memory-Wasteful Way", steps 1-3]
 * [P2, "Attention is not slow because of arithmetic": S = QK^T/sqrt(d),
 *  P = softmax(S) row-wise, O = P V]
 * [P1, "Integration": is_causal=True]
 */
static void attention_row(const double *q, const double *k, const double *v,
                          long N, long d, double scale, int causal, long i,
                          double *S, double *P, double *o_row, double *lse)
{
    const double *qi = q + i * d;
    /* step 1: one row of S = scale * Q K^T */
    for (long j = 0; j < N; ++j) {
        const double *kj = k + j * d;
        double dot = 0.0;
        for (long t = 0; t < d; ++t)
            dot += qi[t] * kj[t];
        S[j] = scale * dot;
    }
    /* causal mask: keys after the query are invisible */
    if (causal)
        for (long j = i + 1; j < N; ++j)
            S[j] = -INFINITY;
    /* step 2: row softmax with the global row max subtracted */
    double m = -INFINITY;
    for (long j = 0; j < N; ++j)
        if (S[j] > m)
            m = S[j];
    double l = 0.0;
    for (long j = 0; j < N; ++j) {
        P[j] = exp(S[j] - m);
        l += P[j];
    }
    for (long j = 0; j < N; ++j)
        P[j] /= l;
    /* step 3: O row = P row times V */
    for (long t = 0; t < d; ++t)
        o_row[t] = 0.0;
    for (long j = 0; j < N; ++j) {
        const double *vj = v + j * d;
        const double pj = P[j];
        for (long t = 0; t < d; ++t)
            o_row[t] += pj * vj[t];
    }
    *lse = m + log(l);
}

/*
 * Standard attention for every (b, h): materializes the full N x N score
 * matrix S and probability matrix P of one head at a time, then O = P V.
 * [P1, "Standard Attention: The Memory-Wasteful Way"]
 * [P2, "Attention is not slow because of arithmetic"]
 *
 * q, k, v, o: [B][H][N][d] fp64; lse: [B][H][N] fp64;
 * p_out: NULL, or [B][H][N][N] fp64 to receive P.
 * Rows of a head are computed in parallel (OpenMP); each row's arithmetic is
 * the sequential definition above, so the result does not depend on the
 * thread count.
 */
int oracle_attention_fwd(const double *q, const double *k, const double *v,
                         double *o, double *lse, double *p_out, long B, long H,
                         long N, long d, double scale, int causal)
{
    if (B < 0 || H < 0 || N < 0 || d < 1)
        return ORACLE_ERR_ARG;
    if (B == 0 || H == 0 || N == 0)
        return ORACLE_OK;
    if (!q || !k || !v || !o || !lse || !isfinite(scale))
        return ORACLE_ERR_ARG;
    double *S = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    double *P = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    if (!S || !P) {
        free(S);
        free(P);
        return ORACLE_ERR_NOMEM;
    }
    for (long bh = 0; bh < B * H; ++bh) {
        const size_t off = (size_t)bh * (size_t)N * (size_t)d;
        const double *qh = q + off, *kh = k + off, *vh = v + off;
        double *oh = o + off;
        double *lh = lse + (size_t)bh * (size_t)N;
#pragma omp parallel for schedule(dynamic, 4)
        for (long i = 0; i < N; ++i)
            attention_row(qh, kh, vh, N, d, scale, causal, i,
                          S + (size_t)i * N, P + (size_t)i * N,
                          oh + (size_t)i * d, lh + i);
        if (p_out)
            memcpy(p_out + (size_t)bh * (size_t)N * (size_t)N, P,
                   (size_t)N * (size_t)N * sizeof(double));
    }
    free(S);
    free(P);
    return ORACLE_OK;
}

/*
 * Standard attention for selected query rows only: the same definition as
 * oracle_attention_fwd, materializing S and P one row at a time.
 * rows: [B*H][R] query indices (0 <= row < N) per head;
 * o_rows: [B*H][R][d]; lse_rows: [B*H][R].
 */
int oracle_attention_rows(const double *q, const double *k, const double *v,
                          long B, long H, long N, long d, double scale,
                          int causal, const long *rows, long R, double *o_rows,
                          double *lse_rows)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || R < 0)
        return ORACLE_ERR_ARG;
    if (R == 0)
        return ORACLE_OK;
    if (!q || !k || !v || !rows || !o_rows || !lse_rows || !isfinite(scale))
        return ORACLE_ERR_ARG;
    for (long x = 0; x < B * H * R; ++x)
        if (rows[x] < 0 || rows[x] >= N)
            return ORACLE_ERR_ARG;
    int nt = oracle_num_threads();
    double *scratch = (double *)malloc((size_t)nt * 2 * (size_t)N * sizeof(double));
    if (!scratch)
        return ORACLE_ERR_NOMEM;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long bh = 0; bh < B * H; ++bh)
        for (long r = 0; r < R; ++r) {
            int tid = 0;
#ifdef _OPENMP
            tid = omp_get_thread_num();
#endif
            double *S = scratch + (size_t)tid * 2 * (size_t)N;
            double *P = S + N;
            const size_t off = (size_t)bh * (size_t)N * (size_t)d;
            const long i = rows[bh * R + r];
            attention_row(q + off, k + off, v + off, N, d, scale, causal, i,
                          S, P, o_rows + ((size_t)bh * R + r) * (size_t)d,
                          lse_rows + (size_t)bh * R + r);
        }
    free(scratch);
    return ORACLE_OK;
}

/*
 * Backward pass of standard attention for every (b, h), with S, P, dP and
 * dS materialized for one head at a time.
 * [P2, "Sizing a tile, and why the backward pass recomputes instead of
 *  storing": the backward pass needs P again; gradients are the plain
 *  derivatives of O = softmax(scale * Q K^T + mask) V]
 *
 * With L any scalar loss and dO = dL/dO given:
 *   dV = P^T dO
 *   dP = dO V^T
 *   D_i = sum_j P_ij dP_ij            (the softmax Jacobian's row term)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ = scale * dS K,   dK = scale * dS^T Q
 * Masked entries have P_ij = 0 and so dS_ij = 0.
 *
 * q, k, v, dout, dq, dk, dv: [B][H][N][d] fp64; delta (may be NULL):
 * [B][H][N] fp64, receives D.
 */
int oracle_attention_bwd(const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk,
                         double *dv, double *delta, long B, long H, long N,
                         long d, double scale, int causal)
{
    if (B < 0 || H < 0 || N < 0 || d < 1)
        return ORACLE_ERR_ARG;
    if (B == 0 || H == 0 || N == 0)
        return ORACLE_OK;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !isfinite(scale))
        return ORACLE_ERR_ARG;
    const size_t nn = (size_t)N * (size_t)N;
    double *P = (double *)malloc(nn * sizeof(double));
    double *dS = (double *)malloc(nn * sizeof(double));
    double *D = (double *)malloc((size_t)N * sizeof(double));
    if (!P || !dS || !D) {
        free(P);
        free(dS);
        free(D);
        return ORACLE_ERR_NOMEM;
    }
    for (long bh = 0; bh < B * H; ++bh) {
        const size_t off = (size_t)bh * (size_t)N * (size_t)d;
        const double *qh = q + off, *kh = k + off, *vh = v + off, *doh = dout + off;
        double *dqh = dq + off, *dkh = dk + off, *dvh = dv + off;
        /* P row by row (as in the forward), then dP, D and dS for that row */
#pragma omp parallel for schedule(dynamic, 4)
        for (long i = 0; i < N; ++i) {
            double *Pi = P + (size_t)i * N;
            double *dSi = dS + (size_t)i * N;
            double m = -INFINITY;
            for (long j = 0; j < N; ++j) {
                double dot = 0.0;
                for (long t = 0; t < d; ++t)
                    dot += qh[i * d + t] * kh[j * d + t];
                Pi[j] = (causal && j > i) ? -INFINITY : scale * dot;
                if (Pi[j] > m)
                    m = Pi[j];
            }
            double l = 0.0;
            for (long j = 0; j < N; ++j) {
                Pi[j] = exp(Pi[j] - m);
                l += Pi[j];
            }
            for (long j = 0; j < N; ++j)
                Pi[j] /= l;
            double Di = 0.0;
            for (long j = 0; j < N; ++j) {
                double dp = 0.0;
                for (long t = 0; t < d; ++t)
                    dp += doh[i * d + t] * vh[j * d + t];
                dSi[j] = dp; /* dP_ij for now */
                Di += Pi[j] * dp;
            }
            for (long j = 0; j < N; ++j)
                dSi[j] = Pi[j] * (dSi[j] - Di);
            D[i] = Di;
        }
        /* dQ = scale dS K (rows i). Each dQ_it is the sum over j = 0..N-1 in
         * ascending order; the t loop is innermost so that K is read by rows. */
#pragma omp parallel
        {
            double *acc = (double *)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(static)
            for (long i = 0; i < N; ++i) {
                for (long t = 0; t < d; ++t)
                    acc[t] = 0.0;
                for (long j = 0; j < N; ++j) {
                    const double w = dS[(size_t)i * N + j];
                    for (long t = 0; t < d; ++t)
                        acc[t] += w * kh[j * d + t];
                }
                for (long t = 0; t < d; ++t)
                    dqh[i * d + t] = scale * acc[t];
            }
            free(acc);
        }
        /* dK = scale dS^T Q and dV = P^T dO (rows j), for a run of kKeyRun key
         * rows at a time. Each dK_jt and dV_jt is the sum over i = 0..N-1 in
         * ascending order, as in the plain column-by-column loop; the i loop
         * is outermost so that dS and P are read by rows. */
        enum { kKeyRun = 32 };
#pragma omp parallel
        {
            double *ak = (double *)malloc((size_t)kKeyRun * (size_t)d * sizeof(double));
            double *av = (double *)malloc((size_t)kKeyRun * (size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 1)
            for (long j0 = 0; j0 < N; j0 += kKeyRun) {
                const long nj = j0 + kKeyRun < N ? kKeyRun : N - j0;
                for (long x = 0; x < nj * d; ++x)
                    ak[x] = av[x] = 0.0;
                for (long i = 0; i < N; ++i) {
                    const double *dSi = dS + (size_t)i * N + j0, *Pi = P + (size_t)i * N + j0;
                    for (long jj = 0; jj < nj; ++jj) {
                        const double ws = dSi[jj], wp = Pi[jj];
                        for (long t = 0; t < d; ++t) {
                            ak[jj * d + t] += ws * qh[i * d + t];
                            av[jj * d + t] += wp * doh[i * d + t];
                        }
                    }
                }
                for (long jj = 0; jj < nj; ++jj)
                    for (long t = 0; t < d; ++t) {
                        dkh[(j0 + jj) * d + t] = scale * ak[jj * d + t];
                        dvh[(j0 + jj) * d + t] = av[jj * d + t];
                    }
            }
            free(ak);
            free(av);
        }
        if (delta)
            memcpy(delta + (size_t)bh * (size_t)N, D, (size_t)N * sizeof(double));
    }
    free(P);
    free(dS);
    free(D);
    return ORACLE_OK;
}

/*
 * Backward pass for selected heads, query rows and key rows, for shapes whose
 * N x N matrices are too large to materialize. The definitions are those of
 * oracle_attention_bwd; only the order of evaluation differs:
 *   1. every row i of the head: lse_i and O_i (attention_row), then
 *      D_i = dO_i . O_i, which equals sum_j P_ij dP_ij because O_i is
 *      sum_j P_ij V_j;
 *   2. each sampled query row i: dQ_i = scale * sum_j dS_ij K_j;
 *   3. each sampled key row j: dV_j = sum_i P_ij dO_i and
 *      dK_j = scale * sum_i dS_ij Q_i;
 * with P_ij = exp(scale * Q_i . K_j - lse_i) (0 where masked),
 * dP_ij = dO_i . V_j and dS_ij = P_ij (dP_ij - D_i).
 * heads: [Hs] head indices b * H + h; qrows: [Hs][R]; krows: [Hs][C];
 * dq_rows: [Hs][R][d]; dk_rows, dv_rows: [Hs][C][d].
 */
static double dot_d(const double *a, const double *b, long d)
{
    double s = 0.0;
    for (long t = 0; t < d; ++t)
        s += a[t] * b[t];
    return s;
}

int oracle_attention_bwd_sampled(const double *q, const double *k,
                                 const double *v, const double *dout, long B,
                                 long H, long N, long d, double scale,
                                 int causal, const long *heads, long Hs,
                                 const long *qrows, long R, const long *krows,
                                 long C, double *dq_rows, double *dk_rows,
                                 double *dv_rows)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || Hs < 0 || R < 0 || C < 0)
        return ORACLE_ERR_ARG;
    if (Hs == 0)
        return ORACLE_OK;
    if (!q || !k || !v || !dout || !heads || !isfinite(scale))
        return ORACLE_ERR_ARG;
    if ((R > 0 && (!qrows || !dq_rows)) || (C > 0 && (!krows || !dk_rows || !dv_rows)))
        return ORACLE_ERR_ARG;
    for (long x = 0; x < Hs; ++x)
        if (heads[x] < 0 || heads[x] >= B * H)
            return ORACLE_ERR_ARG;
    for (long x = 0; x < Hs * R; ++x)
        if (qrows[x] < 0 || qrows[x] >= N)
            return ORACLE_ERR_ARG;
    for (long x = 0; x < Hs * C; ++x)
        if (krows[x] < 0 || krows[x] >= N)
            return ORACLE_ERR_ARG;
    int nt = oracle_num_threads();
    double *lse = (double *)malloc((size_t)N * sizeof(double));
    double *D = (double *)malloc((size_t)N * sizeof(double));
    double *scratch = (double *)malloc((size_t)nt * (2 * (size_t)N + (size_t)d) *
                                       sizeof(double));
    if (!lse || !D || !scratch) {
        free(lse);
        free(D);
        free(scratch);
        return ORACLE_ERR_NOMEM;
    }
    for (long x = 0; x < Hs; ++x) {
        const size_t off = (size_t)heads[x] * (size_t)N * (size_t)d;
        const double *qh = q + off, *kh = k + off, *vh = v + off, *doh = dout + off;
        /* step 1: lse_i and D_i for every row */
#pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i) {
            int tid = 0;
#ifdef _OPENMP
            tid = omp_get_thread_num();
#endif
            double *S = scratch + (size_t)tid * (2 * (size_t)N + (size_t)d);
            double *P = S + N;
            double *o_row = P + N;
            attention_row(qh, kh, vh, N, d, scale, causal, i, S, P, o_row, lse + i);
            D[i] = dot_d(doh + i * d, o_row, d);
        }
        /* step 2: sampled rows of dQ */
#pragma omp parallel for schedule(dynamic, 1)
        for (long r = 0; r < R; ++r) {
            const long i = qrows[x * R + r];
            double *dqi = dq_rows + ((size_t)x * R + r) * (size_t)d;
            for (long t = 0; t < d; ++t)
                dqi[t] = 0.0;
            for (long j = 0; j < N; ++j) {
                if (causal && j > i)
                    continue;
                const double p = exp(scale * dot_d(qh + i * d, kh + j * d, d) - lse[i]);
                const double dp = dot_d(doh + i * d, vh + j * d, d);
                const double ds = p * (dp - D[i]);
                for (long t = 0; t < d; ++t)
                    dqi[t] += ds * kh[j * d + t];
            }
            for (long t = 0; t < d; ++t)
                dqi[t] *= scale;
        }
        /* step 3: sampled rows of dK and dV */
#pragma omp parallel for schedule(dynamic, 1)
        for (long c = 0; c < C; ++c) {
            const long j = krows[x * C + c];
            double *dkj = dk_rows + ((size_t)x * C + c) * (size_t)d;
            double *dvj = dv_rows + ((size_t)x * C + c) * (size_t)d;
            for (long t = 0; t < d; ++t) {
                dkj[t] = 0.0;
                dvj[t] = 0.0;
            }
            for (long i = 0; i < N; ++i) {
                if (causal && j > i)
                    continue;
                const double p = exp(scale * dot_d(qh + i * d, kh + j * d, d) - lse[i]);
                const double dp = dot_d(doh + i * d, vh + j * d, d);
                const double ds = p * (dp - D[i]);
                for (long t = 0; t < d; ++t) {
                    dvj[t] += p * doh[i * d + t];
                    dkj[t] += ds * qh[i * d + t];
                }
            }
            for (long t = 0; t < d; ++t)
                dkj[t] *= scale;
        }
    }
    free(lse);
    free(D);
    free(scratch);
    return ORACLE_OK;
}

/*
 * FP8 E4M3 (the OCP 8-bit floating-point format with 4 exponent bits, bias
 * 7, 3 mantissa bits, no infinities; S.1111.111 is NaN) decoded to fp64:
 * exponent field 0 is subnormal, value (m / 8) * 2^-6; otherwise
 * (1 + m / 8) * 2^(e - 7). Used to hand the exact values of 8-bit inputs,
 * times their per-tensor scale, to the attention definitions above.
 * x: n bytes; out: n doubles (each times `scale`). Returns ORACLE_ERR_ARG on
 * a NaN code.
 */
int oracle_decode_e4m3(const unsigned char *x, long n, double scale, double *out)
{
    if (n < 0 || (n > 0 && (!x || !out)))
        return ORACLE_ERR_ARG;
    for (long t = 0; t < n; ++t) {
        const int s = x[t] >> 7, e = (x[t] >> 3) & 15, m = x[t] & 7;
        if (e == 15 && m == 7)
            return ORACLE_ERR_ARG;
        const double mag = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
        out[t] = (s ? -mag : mag) * scale;
    }
    return ORACLE_OK;
}

/*
 * Decode-step attention over a paged KV cache: one new query token per
 * sequence attends to all L_b cached tokens of its sequence, whose keys and
 * values live in fixed-size pages located through a per-sequence page table
 * (the KV-cache layout the pages point to as the next step, "PagedAttention:
 * pages, page tables" in [P1, "What's Next?"]). The result is the definition
 * of attention for that one row: token t of sequence b is page
 * page_table[b][t / page_size], row t % page_size; then
 *   s_t = scale * q . k_t,  P = softmax(s),  o = sum_t P_t v_t,
 *   lse = ln sum_t exp(s_t),
 * computed with attention_row on the gathered rows (no mask: the new token
 * sees every cached token, itself included).
 * q, o: [B][H][d]; k_cache, v_cache: [num_pages][H_kv][page_size][d];
 * page_table: [B][max_pages]; seq_lens: [B]; lse: [B][H]. Query head h
 * reads KV head h / (H / H_kv). Every L_b must be in [1, max_pages *
 * page_size] and every page index used in [0, num_pages).
 */
int oracle_decode_paged(const double *q, const double *k_cache, const double *v_cache,
                        const int *page_table, const int *seq_lens, long B, long H,
                        long H_kv, long d, long num_pages, long page_size, long max_pages,
                        double scale, double *o, double *lse)
{
    if (B < 0 || H < 1 || H_kv < 1 || H % H_kv || d < 1 || num_pages < 1 || page_size < 1 ||
        max_pages < 1)
        return ORACLE_ERR_ARG;
    if (B == 0)
        return ORACLE_OK;
    if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !o || !lse ||
        !isfinite(scale))
        return ORACLE_ERR_ARG;
    long maxlen = 0;
    for (long b = 0; b < B; ++b) {
        const long L = seq_lens[b];
        if (L < 1 || L > max_pages * page_size)
            return ORACLE_ERR_ARG;
        for (long t = 0; t < (L + page_size - 1) / page_size; ++t) {
            const int pg = page_table[b * max_pages + t];
            if (pg < 0 || pg >= num_pages)
                return ORACLE_ERR_ARG;
        }
        if (L > maxlen)
            maxlen = L;
    }
    int nt = oracle_num_threads();
    const size_t per = (size_t)maxlen * (size_t)d * 2 + 2 * (size_t)maxlen;
    double *scratch = (double *)malloc((size_t)nt * per * sizeof(double));
    if (!scratch)
        return ORACLE_ERR_NOMEM;
    const long group = H / H_kv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long b = 0; b < B; ++b)
        for (long h = 0; h < H; ++h) {
            int tid = 0;
#ifdef _OPENMP
            tid = omp_get_thread_num();
#endif
            double *K = scratch + (size_t)tid * per;
            double *V = K + (size_t)maxlen * d;
            double *S = V + (size_t)maxlen * d;
            double *P = S + maxlen;
            const long L = seq_lens[b], hk = h / group;
            /* gather the sequence's rows of this KV head through the page table */
            for (long t = 0; t < L; ++t) {
                const long pg = page_table[b * max_pages + t / page_size];
                const size_t src = (((size_t)pg * H_kv + hk) * page_size + t % page_size) * d;
                memcpy(K + (size_t)t * d, k_cache + src, (size_t)d * sizeof(double));
                memcpy(V + (size_t)t * d, v_cache + src, (size_t)d * sizeof(double));
            }
            const double *qh = q + ((size_t)b * H + h) * d;
            /* one row of standard attention: query row 0 against L keys */
            attention_row(qh, K, V, L, d, scale, 0, 0, S, P, o + ((size_t)b * H + h) * d,
                          lse + (size_t)b * H + h);
        }
    free(scratch);
    return ORACLE_OK;
}
