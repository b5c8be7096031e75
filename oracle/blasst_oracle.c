/*
 * FP64 CPU oracle for skip-softmax ("BLASST") block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code, header or constant
 * with the HIP library; both read the same bf16 input bytes and nothing else.
 *
 * What it computes (BLASST blog, "BLASST: Dynamic BLocked Attention Sparsity
 * via Softmax Thresholding", MLSys 2026 notes):
 *
 *  - section on FlashAttention's online softmax (Eqs. 1-4): for the rows of a
 *    query block, visit the KV blocks j = 0, 1, ... in ascending order keeping a
 *    running max m (starts at -inf), a row sum l (starts at 0) and an output
 *    accumulator O (starts at 0).  For block j: S = Q K_j^T (scaled by
 *    1/sqrt(d)), block row max mt = rowmax(S), updated max m_new = max(m, mt)
 *    [Eq. 1]; then P = exp(S - m_new), l = exp(m - m_new) l + rowsum(P),
 *    O = exp(m - m_new) O + P V_j [Eqs. 2-4].  Finally O / l.
 *  - section on the decision rule (Eq. 5): right after the running-max update,
 *    a row votes to skip block j when mt - m_new < ln(lambda), compared against
 *    the *updated* max, in log space, before any exponential.
 *  - section on what is skipped: a skipped block does no exp, no row sum, no
 *    P V product (and, in decode, no V load); S = Q K^T itself is always formed.
 *  - sections on the lambda = a/L rule and on the decision's cost: in prefill
 *    the block is skipped only if every row of the query block agrees (logical
 *    AND over the block's rows); in decode the single query row decides alone.
 *  - SANTA notes (split-KV / FlashDecoding tiles merged by their true
 *    normaliser): decode splits the KV blocks into contiguous ranges, each with
 *    its own fresh running state, and merges them with a log-sum-exp.
 *
 * Readings where the pages are silent (each also recorded in the design notes):
 *  - scores are scaled by 1/sqrt(d) before the max and the test;
 *  - lambda = 0 means "never skip" (ln 0 = -inf); lambda must lie in [0, 1);
 *  - the test is strict: a difference exactly equal to ln(lambda) keeps;
 *  - query head h reads kv head h / G (G = Hq / Hkv, consecutive heads share);
 *  - a skipped block leaves (m, l, O) untouched.  This is what Eq. 1 followed
 *    by a skip gives: a skipping row has mt < m_new + ln(lambda) < m_new, hence
 *    m_new = m, so the running max does not move;
 *  - a decision imposed through the force argument (used to adopt the other
 *    valid decision of a block whose margin lies within float rounding of the
 *    threshold) replaces only the keep/skip choice; the running max follows
 *    Eq. 1 either way, and a row or split left with no kept key has o = 0,
 *    lse = -inf;
 *  - a query row that sees no key of a visited block (possible only when the
 *    query block is taller than a KV block) votes to skip and adds nothing;
 *  - split s of S covers KV blocks [floor(s*nk/S), floor((s+1)*nk/S));
 *  - a trailing KV block or query block shorter than Bc (Br) is handled by
 *    simply having fewer columns (rows).
 *
 * Numbers: every input is the exact bf16 value widened to double; all
 * arithmetic is double, with no rounding of P or O.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ln(lambda); lambda = 0 gives -inf so that no difference ever falls below it. */
static double log_threshold(double lambda)
{
    return lambda > 0.0 ? log(lambda) : -INFINITY;
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

/* Widen n bf16 values to double. */
static void widen(const uint16_t* src, double* dst, size_t n)
{
    for (size_t i = 0; i < n; ++i) dst[i] = bf16_value(src[i]);
}

/*
 * Eq. 1 for a row whose block is skipped: the running max still becomes
 * m_new = max(m, mt), and (l, O) are rescaled to it.  Under the rule's own
 * decision a skipping row has mt < m + ln(lambda) < m, so m_new = m and nothing
 * changes; only a decision imposed from outside (the force argument) can skip
 * a block that raises the max, and then the max still moves, so that every
 * later decision is taken against the prefix max of the block maxima whatever
 * was kept before it.
 */
static void advance_running_max(double* m, double* l, double* o, int d, double m_new)
{
    if (!(m_new > *m)) return;
    double alpha = (*m == -INFINITY) ? 0.0 : exp(*m - m_new);
    *l *= alpha;
    for (int e = 0; e < d; ++e) o[e] *= alpha;
    *m = m_new;
}

/*
 * One row's state update for a kept block (Eqs. 2-4).
 * s[0..nc) are the row's scores for the block (-inf where the key is hidden),
 * vb the block's value rows (nc x d, double), m_new the updated running max.
 */
static void accumulate_kept_block(double* m, double* l, double* o, const double* s,
                                  const double* vb, int nc, int d, double m_new)
{
    double alpha = (*m == -INFINITY) ? 0.0 : exp(*m - m_new);
    *l *= alpha;
    for (int e = 0; e < d; ++e) o[e] *= alpha;
    for (int c = 0; c < nc; ++c) {
        if (s[c] == -INFINITY) continue;
        double p = exp(s[c] - m_new);
        *l += p;
        for (int e = 0; e < d; ++e) o[e] += p * vb[(size_t)c * d + e];
    }
    *m = m_new;
}

/* ------------------------------------------------------------------------ */
/* Prefill                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * One query block of one query head: unit = (b*Hq + hq) * nq + i, nq = ceil(T/Br).
 * Outputs for the unit:
 *   o      [Br, d]   normalised output rows (rows past T left untouched)
 *   lse    [Br]      m + ln(l) per row
 *   mask   [nk]      0 = kept, 1 = skipped, 2 = not visited (above the diagonal)
 *   margin [nk]      D - ln(lambda) where D = max over rows of (mt - m_new);
 *                    the block is skipped iff margin < 0.  NaN if not visited.
 * force (nullable) [nk]: -1 = own decision, 0 = keep, 1 = skip.
 */
static void prefill_unit(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         int B, int Hq, int Hkv, int T, int d, int Bc, int Br,
                         double thr, int causal, int64_t unit, const int8_t* force,
                         double* o, double* lse, uint8_t* mask, double* margin)
{
    (void)B;
    const int G = Hq / Hkv;
    const int nq = ceil_div(T, Br), nk = ceil_div(T, Bc);
    const int i = (int)(unit % nq);
    const int hq = (int)((unit / nq) % Hq);
    const int b = (int)(unit / nq / Hq);
    const int hkv = hq / G;
    const int r0 = i * Br, nr = (T - r0 < Br) ? T - r0 : Br;
    const double scale = 1.0 / sqrt((double)d);

    const uint16_t* Q = q + (((size_t)b * Hq + hq) * T + r0) * d;
    const uint16_t* K = k + ((size_t)b * Hkv + hkv) * (size_t)T * d;
    const uint16_t* V = v + ((size_t)b * Hkv + hkv) * (size_t)T * d;

    double* qd = malloc(sizeof(double) * (size_t)nr * d);
    double* kb = malloc(sizeof(double) * (size_t)Bc * d);
    double* vb = malloc(sizeof(double) * (size_t)Bc * d);
    double* S = malloc(sizeof(double) * (size_t)nr * Bc);
    double* mt = malloc(sizeof(double) * nr);
    double* m = malloc(sizeof(double) * nr);
    double* l = calloc(nr, sizeof(double));
    double* acc = calloc((size_t)nr * d, sizeof(double));

    widen(Q, qd, (size_t)nr * d);
    for (int r = 0; r < nr; ++r) m[r] = -INFINITY;
    for (int j = 0; j < nk; ++j) { mask[j] = 2; margin[j] = NAN; }

    const int last_row = r0 + nr - 1;
    const int j_end = causal ? last_row / Bc + 1 : nk;
    for (int j = 0; j < j_end; ++j) {
        const int c0 = j * Bc, nc = (T - c0 < Bc) ? T - c0 : Bc;
        widen(K + (size_t)c0 * d, kb, (size_t)nc * d);

        /* S = Q_i K_j^T / sqrt(d); hidden (future) keys get -inf. */
        for (int r = 0; r < nr; ++r) {
            for (int c = 0; c < nc; ++c) {
                double* s = &S[(size_t)r * Bc + c];
                if (causal && c0 + c > r0 + r) { *s = -INFINITY; continue; }
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += qd[(size_t)r * d + e] * kb[(size_t)c * d + e];
                *s = dot * scale;
            }
        }

        /* Eq. 1 and Eq. 5: block row max, updated max, per-row vote, AND over rows. */
        int all_rows_skip = 1;
        double D = -INFINITY;
        for (int r = 0; r < nr; ++r) {
            double row_max = -INFINITY;
            for (int c = 0; c < nc; ++c)
                if (S[(size_t)r * Bc + c] > row_max) row_max = S[(size_t)r * Bc + c];
            mt[r] = row_max;
            if (row_max == -INFINITY) continue; /* sees no key here: votes skip */
            double m_new = (m[r] > row_max) ? m[r] : row_max;
            double diff = row_max - m_new;
            if (!(diff < thr)) all_rows_skip = 0;
            if (diff > D) D = diff;
        }
        int skip = all_rows_skip;
        if (force && force[j] >= 0) skip = force[j];
        mask[j] = (uint8_t)skip;
        margin[j] = (thr == -INFINITY) ? INFINITY : D - thr;
        if (skip) {
            for (int r = 0; r < nr; ++r)
                if (mt[r] > m[r]) advance_running_max(&m[r], &l[r], &acc[(size_t)r * d], d, mt[r]);
            continue;
        }

        /* Eqs. 2-4 for the kept block, every row of the query block. */
        widen(V + (size_t)c0 * d, vb, (size_t)nc * d);
        for (int r = 0; r < nr; ++r) {
            if (mt[r] == -INFINITY) continue;
            double m_new = (m[r] > mt[r]) ? m[r] : mt[r];
            accumulate_kept_block(&m[r], &l[r], &acc[(size_t)r * d], &S[(size_t)r * Bc], vb, nc, d,
                                  m_new);
        }
    }

    /* A row whose kept set is empty (only a forced decision can make one)
     * has no output: o = 0 and lse = -inf. */
    for (int r = 0; r < nr; ++r) {
        for (int e = 0; e < d; ++e) o[(size_t)r * d + e] = (l[r] > 0.0) ? acc[(size_t)r * d + e] / l[r] : 0.0;
        lse[r] = (l[r] > 0.0) ? m[r] + log(l[r]) : -INFINITY;
    }
    free(qd); free(kb); free(vb); free(S); free(mt); free(m); free(l); free(acc);
}

/*
 * Causal (or full) prefill over a list of units.  Per-unit outputs are packed:
 * o [n_units, Br, d], lse [n_units, Br], mask and margin [n_units, nk],
 * force (nullable) [n_units, nk].  Returns 0, or -1 on a bad argument.
 */
int oracle_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   int B, int Hq, int Hkv, int T, int d, int Bc, int Br,
                   double lambda, int causal, const int64_t* units, int n_units,
                   const int8_t* force, double* o, double* lse, uint8_t* mask,
                   double* margin, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || T <= 0 || d <= 0 || Bc <= 0 || Br <= 0) return -1;
    if (!(lambda >= 0.0 && lambda < 1.0)) return -1;
    const double thr = log_threshold(lambda);
    const int nk = ceil_div(T, Bc);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int u = 0; u < n_units; ++u) {
        prefill_unit(q, k, v, B, Hq, Hkv, T, d, Bc, Br, thr, causal, units[u],
                     force ? force + (size_t)u * nk : NULL, o + (size_t)u * Br * d,
                     lse + (size_t)u * Br, mask + (size_t)u * nk, margin + (size_t)u * nk);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Split-KV decode                                                           */
/* ------------------------------------------------------------------------ */

/*
 * One split of one query head: the G query heads of kv head (b, hkv) form
 * unit = b*Hkv + hkv; this computes head g of the unit over split sp, whose
 * blocks are [floor(sp*nk/S), floor((sp+1)*nk/S)).  One query row; every key of
 * the context is visible.  Outputs for (g, sp):
 *   o_part  [d]   the split's normalised output
 *   lse_part[1]   the split's m + ln(l)
 *   skip    the head's row [nk]: entries of the split's blocks, 1 = skipped
 *   margin  the head's row [nk]: (mt - m_new) - ln(lambda), skipped iff < 0
 * force (nullable): the head's row [nk], -1 = own decision, 0 = keep, 1 = skip.
 */
static void decode_head_split(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              int Hq, int Hkv, int N, int d, int Bc, double thr, int S,
                              int64_t unit, int g, int sp, const int8_t* force, double* o_part,
                              double* lse_part, uint8_t* skip, double* margin)
{
    const int G = Hq / Hkv;
    const int nk = ceil_div(N, Bc);
    const int hkv = (int)(unit % Hkv), b = (int)(unit / Hkv);
    const int hq = hkv * G + g;
    const double scale = 1.0 / sqrt((double)d);
    const uint16_t* K = k + ((size_t)b * Hkv + hkv) * (size_t)N * d;
    const uint16_t* V = v + ((size_t)b * Hkv + hkv) * (size_t)N * d;
    const int j0 = (int)((int64_t)sp * nk / S), j1 = (int)((int64_t)(sp + 1) * nk / S);

    double* qd = malloc(sizeof(double) * d);
    double* kb = malloc(sizeof(double) * (size_t)Bc * d);
    double* vb = malloc(sizeof(double) * (size_t)Bc * d);
    double* s = malloc(sizeof(double) * Bc);
    double* acc = calloc(d, sizeof(double));
    widen(q + ((size_t)b * Hq + hq) * d, qd, d);

    double m = -INFINITY, l = 0.0;
    for (int j = j0; j < j1; ++j) {
        const int c0 = j * Bc, nc = (N - c0 < Bc) ? N - c0 : Bc;
        widen(K + (size_t)c0 * d, kb, (size_t)nc * d);
        /* S = q K_j^T / sqrt(d) — always formed. */
        double row_max = -INFINITY;
        for (int c = 0; c < nc; ++c) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e) dot += qd[e] * kb[(size_t)c * d + e];
            s[c] = dot * scale;
            if (s[c] > row_max) row_max = s[c];
        }
        /* Eq. 1 then Eq. 5 for the single row. */
        double m_new = (m > row_max) ? m : row_max;
        double diff = row_max - m_new;
        int sk = diff < thr;
        if (force && force[j] >= 0) sk = force[j];
        skip[j] = (uint8_t)sk;
        margin[j] = (thr == -INFINITY) ? INFINITY : diff - thr;
        if (sk) {
            advance_running_max(&m, &l, acc, d, m_new);
            continue;
        }
        widen(V + (size_t)c0 * d, vb, (size_t)nc * d);
        accumulate_kept_block(&m, &l, acc, s, vb, nc, d, m_new);
    }
    /* A split with no kept key (S > nk, an empty context, or every block
     * skipped by a forced decision) contributes nothing to the merge:
     * o = 0 and lse = -inf. */
    for (int e = 0; e < d; ++e) o_part[e] = (l > 0.0) ? acc[e] / l : 0.0;
    *lse_part = (l > 0.0) ? m + log(l) : -INFINITY;
    free(qd); free(kb); free(vb); free(s); free(acc);
}

/*
 * Split-KV decode over a list of (b, hkv) units; q [B,Hq,1,d], k and v [B,Hkv,N,d].
 * Per-unit outputs:
 *   o_part  [G, S, d]  each split's normalised output
 *   lse_part[G, S]     each split's m + ln(l)
 *   skip    [G, nk]    1 = the head's row skipped the block
 *   vskip   [nk]       1 = no head of the group kept the block (its V is not needed)
 *   margin  [G, nk]    (mt - m_new) - ln(lambda); skipped iff < 0
 *   vmargin [nk]       max over heads of (mt - m_new) - ln(lambda)
 * force (nullable) [U, G, nk]: -1 = own decision, 0 = keep, 1 = skip.
 * Every (unit, head, split) is independent and runs as its own task; the group
 * outputs (vskip, vmargin) are formed from the heads' rows afterwards.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  int B, int Hq, int Hkv, int N, int d, int Bc, double lambda, int num_splits,
                  const int64_t* units, int n_units, const int8_t* force,
                  double* o_part, double* lse_part, uint8_t* skip, uint8_t* vskip,
                  double* margin, double* vmargin, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N < 0 || d <= 0 || Bc <= 0) return -1;
    if (!(lambda >= 0.0 && lambda < 1.0)) return -1;
    const int nk = ceil_div(N, Bc), G = Hq / Hkv, S = num_splits;
    if (S < 1) return -1;
    const double thr = log_threshold(lambda);
    const int64_t tasks = (int64_t)n_units * G * S;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t t = 0; t < tasks; ++t) {
        const int sp = (int)(t % S), g = (int)((t / S) % G);
        const int64_t u = t / ((int64_t)S * G);
        const size_t row = (size_t)u * G + g;  /* the head's row among the units' heads */
        decode_head_split(q, k, v, Hq, Hkv, N, d, Bc, thr, S, units[u], g, sp,
                          force ? force + row * nk : NULL, o_part + (row * S + sp) * d,
                          lse_part + row * S + sp, skip + row * nk, margin + row * nk);
    }
    /* V is needed for a block iff some head of the group keeps it; the group's
     * margin is the largest of its heads' margins. */
    for (int u = 0; u < n_units; ++u) {
        for (int j = 0; j < nk; ++j) {
            uint8_t all_skip = 1;
            double best = -INFINITY;
            for (int g = 0; g < G; ++g) {
                const size_t row = (size_t)u * G + g;
                all_skip &= skip[row * nk + j];
                if (margin[row * nk + j] > best) best = margin[row * nk + j];
            }
            vskip[(size_t)u * nk + j] = all_skip;
            vmargin[(size_t)u * nk + j] = best;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* MLA decode (latent KV, absorbed form)                                     */
/* ------------------------------------------------------------------------ */

/*
 * One query head of multi-head latent attention at decode: every head of
 * sequence b reads the same cache row per token, kv [N, dqk] (the latent part
 * followed by the rotary part), and token t's value is the latent part
 * kv_t[0 .. dv).  Scores s_t = (q . kv_t) * scale.  Blocks, splits, decisions
 * and the kept-block update are those of split-KV decode; the head decides
 * alone.  unit = b*Hq + h.  Per-unit outputs:
 *   o_part [S, dv], lse_part [S], skip [nk], margin [nk] (D - ln(lambda)).
 * force (nullable) [nk]: -1 = own decision, 0 = keep, 1 = skip.
 */
static void mla_unit(const uint16_t* q, const uint16_t* kv, int Hq, int N, int dqk, int dv, int Bc,
                     double scale, double thr, int S, int64_t unit, const int8_t* force,
                     double* o_part, double* lse_part, uint8_t* skip, double* margin)
{
    const int nk = ceil_div(N, Bc);
    const int64_t b = unit / Hq;
    const uint16_t* K = kv + (size_t)b * N * dqk;

    double* qd = malloc(sizeof(double) * dqk);
    double* kb = malloc(sizeof(double) * (size_t)Bc * dqk);
    double* vb = malloc(sizeof(double) * (size_t)Bc * dv);
    double* s = malloc(sizeof(double) * Bc);
    double* acc = malloc(sizeof(double) * dv);
    widen(q + (size_t)unit * dqk, qd, dqk);
    for (int sp = 0; sp < S; ++sp) {
        const int j0 = (int)((int64_t)sp * nk / S), j1 = (int)((int64_t)(sp + 1) * nk / S);
        double m = -INFINITY, l = 0.0;
        for (int e = 0; e < dv; ++e) acc[e] = 0.0;
        for (int j = j0; j < j1; ++j) {
            const int c0 = j * Bc, nc = (N - c0 < Bc) ? N - c0 : Bc;
            widen(K + (size_t)c0 * dqk, kb, (size_t)nc * dqk);
            double row_max = -INFINITY;
            for (int c = 0; c < nc; ++c) {
                double dot = 0.0;
                for (int e = 0; e < dqk; ++e) dot += qd[e] * kb[(size_t)c * dqk + e];
                s[c] = dot * scale;
                if (s[c] > row_max) row_max = s[c];
            }
            double m_new = (m > row_max) ? m : row_max;
            double diff = row_max - m_new;
            int sk = diff < thr;
            if (force && force[j] >= 0) sk = force[j];
            skip[j] = (uint8_t)sk;
            margin[j] = (thr == -INFINITY) ? INFINITY : diff - thr;
            if (sk) {
                advance_running_max(&m, &l, acc, dv, m_new);
                continue;
            }
            /* the value of a token is the latent part of its cache row */
            for (int c = 0; c < nc; ++c)
                for (int e = 0; e < dv; ++e) vb[(size_t)c * dv + e] = kb[(size_t)c * dqk + e];
            accumulate_kept_block(&m, &l, acc, s, vb, nc, dv, m_new);
        }
        for (int e = 0; e < dv; ++e) o_part[(size_t)sp * dv + e] = (l > 0.0) ? acc[e] / l : 0.0;
        lse_part[sp] = (l > 0.0) ? m + log(l) : -INFINITY;
    }
    free(qd); free(kb); free(vb); free(s); free(acc);
}

/*
 * MLA decode over a list of (b, h) units; q [B,Hq,dqk], kv [B,N,dqk], value =
 * kv[..., :dv].  Returns 0, or -1 on a bad argument.
 */
int oracle_decode_mla(const uint16_t* q, const uint16_t* kv, int B, int Hq, int N, int dqk, int dv, int Bc,
                      double scale, double lambda, int num_splits, const int64_t* units, int n_units,
                      const int8_t* force, double* o_part, double* lse_part, uint8_t* skip, double* margin,
                      int nthreads)
{
    if (B < 0 || Hq <= 0 || N < 0 || dqk <= 0 || dv <= 0 || dv > dqk || Bc <= 0 || num_splits < 1) return -1;
    if (!(lambda >= 0.0 && lambda < 1.0) || !(scale > 0.0)) return -1;
    const int nk = ceil_div(N, Bc), S = num_splits;
    const double thr = log_threshold(lambda);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int u = 0; u < n_units; ++u)
        mla_unit(q, kv, Hq, N, dqk, dv, Bc, scale, thr, S, units[u], force ? force + (size_t)u * nk : NULL,
                 o_part + (size_t)u * S * dv, lse_part + (size_t)u * S, skip + (size_t)u * nk,
                 margin + (size_t)u * nk);
    return 0;
}

/*
 * Merge of split results by their true normalisers: with L = ln(sum_s exp(lse_s)),
 * O = sum_s exp(lse_s - L) O_s.  o_part [rows, S, d], lse_part [rows, S];
 * o [rows, d], lse [rows].
 */
int oracle_combine(const double* o_part, const double* lse_part, int rows, int S, int d,
                   double* o, double* lse)
{
    if (rows < 0 || S < 1 || d <= 0) return -1;
    for (int r = 0; r < rows; ++r) {
        const double* ls = lse_part + (size_t)r * S;
        double top = -INFINITY;
        for (int s = 0; s < S; ++s) if (ls[s] > top) top = ls[s];
        if (top == -INFINITY) {  /* every split empty: no key at all */
            for (int e = 0; e < d; ++e) o[(size_t)r * d + e] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (int s = 0; s < S; ++s) z += exp(ls[s] - top);
        const double L = top + log(z);
        for (int e = 0; e < d; ++e) {
            double x = 0.0;
            for (int s = 0; s < S; ++s) x += exp(ls[s] - L) * o_part[((size_t)r * S + s) * d + e];
            o[(size_t)r * d + e] = x;
        }
        lse[r] = L;
    }
    return 0;
}
