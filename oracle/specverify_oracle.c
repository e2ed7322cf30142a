/*
 * specverify_oracle.c -- CPU oracle for the batched verify-and-sample step of
 * speculative decoding and the MTP token shift/insert.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never links,
 * includes or calls it, and it shares no source with the GPU library: this file
 * includes only the C standard library and pthreads.
 *
 * Source of the rules: "Accelerating Sonar through speculation" (Perplexity
 * Research, N. Licker and E. McKnight, 2025-06-10), and the paper that page lists
 * first among its references, "Fast Inference from Transformers via Speculative
 * Decoding", for the acceptance test u < p/q and the residual max(0, p - q).
 *
 *   - Speculative decoding section, second paragraph: every candidate prefix is
 *     scored by probability, the longest acceptable prefix is kept, and the target
 *     supplies one extra token, so n drafts give at most n + 1 tokens per step.
 *   - Speculative decoding section, the acceptance and target-generation stages
 *     of its four inference stages: at the mismatch, or after the last draft, the target
 *     logits of that position yield one more token, which ends the sequence.
 *   - Target-draft section, prefill paragraph: batches without speculation use
 *     standard sampling (here: draft length 0).
 *   - Target-draft section, decode paragraph: acceptance compares the full draft
 *     and target distributions.
 *   - MTP section, first paragraph (figure lost): token t_{i+1} is sampled from
 *     logits L_i derived from hidden state H_i, so the input token buffer is
 *     shifted left one step relative to the target's hidden states.
 *   - Single-token MTP scheduling section, third paragraph: after the target's
 *     input tokens are shifted, a kernel writes the next target token into its
 *     slot, so no CPU sync is needed after acceptance.
 *
 * Everything is computed scalar, with sums taken in ascending index order, in
 * double precision except the final draw: its weights (p_L, or max(0, p_k - q_k)
 * after a rejection) and their running sum are formed in 80-bit extended
 * precision (long double).  When the draft is almost the target, p_k - q_k is
 * a difference of nearly equal numbers; at a residual mass near 1e-10 binary64
 * keeps only about five of its digits, too few to place the draw to 1e-5 of the
 * mass.  As T -> 0 with both rows on one top token no precision suffices for
 * the difference itself (p_0 = 1 / (1 + tail) rounds to 1), so the residual is
 * written as an exact rearrangement in which tokens that the rows share cancel
 * before anything is rounded, and its terms are carried as signed logarithms
 * (resid_t).  Nothing is blocked, fused or reordered.
 *
 * Readings of points the pages leave open:
 *   - acceptance of draft x_j:  u[b][j] < p_j(x_j) / q_j(x_j); q(x) = 0 gives
 *     ratio +inf when p(x) > 0 and 0 when p(x) = 0;
 *   - p and q are softmax(z / T_b) at the same per-sequence temperature T_b;
 *   - after the first rejection at k: draw from max(0, p_k - q_k) normalised; if
 *     its total is not positive (impossible in exact arithmetic) draw from p_k and
 *     flag ZERO_RESIDUAL; after all drafts are accepted: draw from p_L;
 *   - the final draw always uses u[b][n]; inverse CDF with unnormalised weights
 *     in ascending index: y = min{i : C_i > u * Z}, else the last i with w_i > 0;
 *   - T_b = 0 selects the greedy rule (argmax prefix match, lowest index on ties,
 *     raw logits); T_b < 0 or NaN is treated as 0 and flagged;
 *   - draft lengths outside [0, n] are clamped and flagged; a draft token outside
 *     [0, V) is rejected at its position and flagged;
 *   - a uniform outside [0, 1) or NaN is replaced (NaN or < 0 -> 0, >= 1 -> the
 *     largest float below 1) and flagged;
 *   - emitted slots after the correction/bonus token hold -1;
 *   - MTP shift: out[i] = in[i+1] for i < n, out[n] = in[n], then
 *     out[a_b] = emitted[b][a_b]; hidden states are carried unshifted.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2 /* logits already in double (e.g. from sv_oracle_lmhead_logits) */

#define OR_FLAG_LEN_CLAMPED 1u
#define OR_FLAG_TOKEN_OOR 2u
#define OR_FLAG_BAD_TEMP 4u
#define OR_FLAG_BAD_UNIFORM 8u
#define OR_FLAG_ZERO_RESIDUAL 16u
#define OR_FLAG_BAD_PARENT 64u
#define OR_FLAG_TREE_TRUNCATED 128u

#define OR_MODE_SAMPLE 0
#define OR_MODE_GREEDY 1

/* ---------------------------------------------------------------- helpers */

/* Widen one logit to double.  bf16 is the top half of an IEEE binary32, so the
 * widening is exact: place the 16 bits in the high half of a 32-bit word. */
static double logit_at(const void *rows, int dt, size_t idx)
{
    if (dt == OR_F64) return ((const double *)rows)[idx];
    if (dt == OR_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)rows)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)rows)[idx];
}

/* Greedy choice of one row: the maximum raw logit, lowest index on ties
 * (strict '>' scan in ascending index). */
static int row_argmax(const void *rows, int dt, size_t base, int V)
{
    int best = 0;
    double bv = logit_at(rows, dt, base);
    for (int i = 1; i < V; ++i) {
        double v = logit_at(rows, dt, base + (size_t)i);
        if (v > bv) {
            bv = v;
            best = i;
        }
    }
    return best;
}

/* Softmax of z / T over one row, by its definition:
 *   m = max_i z_i,  S = sum_i exp((z_i - m) / T),  lse = m / T + ln S,
 *   p_i = exp((z_i - m) / T - ln S).
 * Returns lse; writes m and ln S for later probability evaluation. */
static double row_softmax_stats(const void *rows, int dt, size_t base, int V, double T,
                                double *m_out, double *logS_out)
{
    double m = logit_at(rows, dt, base);
    for (int i = 1; i < V; ++i) {
        double v = logit_at(rows, dt, base + (size_t)i);
        if (v > m) m = v;
    }
    double S = 0.0;
    for (int i = 0; i < V; ++i)
        S += exp((logit_at(rows, dt, base + (size_t)i) - m) / T);
    double logS = log(S);
    *m_out = m;
    *logS_out = logS;
    return m / T + logS;
}

static double prob_at(const void *rows, int dt, size_t base, int i, double T, double m, double logS)
{
    return exp((logit_at(rows, dt, base + (size_t)i) - m) / T - logS);
}

/* The acceptance ratio p(x) / q(x) of a target and a draft probability at the
 * same temperature (Speculative decoding section: x is kept iff u < p(x) /
 * q(x)), formed from their logarithms log p = (z_t - m_t) / T - log S_t and
 * log q = (z_d - m_d) / T - log S_d, so that it keeps its value when both
 * probabilities lie below the binary64 range (T -> 0).  A -inf logit is a
 * probability of exactly 0: q(x) = 0 < p(x) gives +inf, p(x) = 0 gives 0. */
static double accept_ratio(double zt, double mt, double lst, double zd, double md, double lsd, double T)
{
    if (zt == -INFINITY) return 0.0;
    if (zd == -INFINITY) return INFINITY;
    return exp(((zt - mt) / T - lst) - ((zd - md) / T - lsd));
}

/* The whole distribution softmax(z / T) of one row in extended precision:
 * p_i = exp((z_i - m) / T) / S with S = sum_i exp((z_i - m) / T), m the row max. */
static void row_probs_ld(const void *rows, int dt, size_t base, int V, double T, long double *p)
{
    double m = logit_at(rows, dt, base);
    for (int i = 1; i < V; ++i) {
        double v = logit_at(rows, dt, base + (size_t)i);
        if (v > m) m = v;
    }
    long double S = 0.0L;
    for (int i = 0; i < V; ++i) {
        p[i] = expl(((long double)logit_at(rows, dt, base + (size_t)i) - (long double)m) / (long double)T);
        S += p[i];
    }
    for (int i = 0; i < V; ++i) p[i] /= S;
}

/* Row maximum (-inf for an empty or fully masked row). */
static double row_max(const void *rows, int dt, size_t base, int V)
{
    double m = -INFINITY;
    for (int i = 0; i < V; ++i) {
        double v = logit_at(rows, dt, base + (size_t)i);
        if (v > m) m = v;
    }
    return m;
}

/* A signed quantity s e^l (s = +1, -1, or 0 with l = -inf), so that residual
 * terms far below the range of long double keep their value and sign. */
typedef struct {
    int s;
    long double l;
} slog_t;

static slog_t slog_zero(void)
{
    slog_t z = {0, -INFINITY};
    return z;
}

/* x + y: the larger magnitude keeps its sign; a difference is formed as
 * e^hi (1 - e^{lo - hi}) with -expm1l, so that no digit is lost to 1 - e^d. */
static slog_t slog_add(slog_t x, slog_t y)
{
    if (x.s == 0) return y;
    if (y.s == 0) return x;
    const slog_t hi = x.l >= y.l ? x : y, lo = x.l >= y.l ? y : x;
    const long double d = lo.l - hi.l;
    slog_t r = {hi.s, hi.l};
    if (hi.s == lo.s) {
        r.l = hi.l + log1pl(expl(d));
    } else {
        if (d == 0.0L) return slog_zero();
        r.l = hi.l + logl(-expm1l(d));
    }
    return r;
}

/* The residual of a target row and a draft row at lam (Speculative decoding
 * section, the first reference: after a rejection the token is drawn from
 * max(0, p - q) normalised; SpecInfer: after k rejections at a node, from
 * max(0, p - lam_k q), lam_1 = 1, lam_{k+1} = lam_k + M_k, M_k the mass of
 * max(0, p - lam_k q)).  With a_i = (z_t,i - m_t) / T and b_i = (z_d,i - m_d) / T
 * (each row relative to its own maximum), S_t = sum e^a and S_d = sum e^b:
 *   p_i - lam q_i = R_i / S_d,  R_i = kappa e^{a_i} + lam (e^{a_i} - e^{b_i}),
 *   kappa = S_d / S_t - lam,
 * an exact rearrangement in which a token whose relative logits agree
 * (a_i = b_i, "shared") contributes kappa e^{a_i} alone.  As T -> 0 with both
 * rows on one top token, p_i - q_i is a difference of two numbers that agree
 * beyond any precision (1 + tail rounds to 1), and so is kappa = S_d / S_t - lam
 * formed from its parts; here kappa is formed from the differing tokens only:
 *   kappa_1 = Delta / S_t,  Delta = sum over differing tokens of (e^b - e^a),
 *   kappa_{k+1} = kappa_k - M_k = (kappa_k Y - W) / S_d   if kappa_k > 0,
 *               = kappa_k - W / S_d                          otherwise,
 * with Y = sum e^b over the differing tokens (= S_d - the shared tokens' sum)
 * and W = sum max(0, R_i) over the differing tokens (M_k = (W + max(0, kappa_k)
 * times the shared tokens' sum) / S_d).  kappa and every R_i are carried as
 * signed logarithms (slog_t), so none leaves the range however small it is.  A
 * -inf logit is a probability of 0 (its e^a is 0); a row with no finite logit
 * takes every a_i = -inf. */
typedef struct {
    const void *trows, *drows;
    int dt, V;
    size_t tb, db;      /* first element of the target row and of the draft row */
    long double T, mt, md;
    long double St, Sd; /* sum e^{a_i}, sum e^{b_i} */
    long double lY;     /* log of sum e^{b_i} over the tokens with a_i != b_i */
    slog_t kap;         /* kappa at the current lam */
    long double lam;    /* the current lam (1 after the first rejection) */
} resid_t;

static long double rel_logit(const void *rows, int dt, size_t at, long double m, long double T)
{
    if (m == -INFINITY) return -INFINITY;
    return ((long double)logit_at(rows, dt, at) - m) / T;
}

/* e^a - e^b (a != b) as a signed logarithm */
static slog_t exp_diff(long double a, long double b)
{
    slog_t r;
    if (a > b) {
        r.s = 1;
        r.l = a + logl(-expm1l(b - a));
    } else {
        r.s = -1;
        r.l = b + logl(-expm1l(a - b));
    }
    return r;
}

/* The residual of the pair at lam = 1: S_t, S_d, Y and kappa_1 = Delta / S_t. */
static void resid_setup(resid_t *r, const void *trows, const void *drows, int dt, size_t tb, size_t db, int V,
                        double T)
{
    r->trows = trows;
    r->drows = drows;
    r->dt = dt;
    r->V = V;
    r->tb = tb;
    r->db = db;
    r->T = T;
    r->mt = row_max(trows, dt, tb, V);
    r->md = row_max(drows, dt, db, V);
    r->St = r->Sd = 0.0L;
    r->lY = -INFINITY;
    slog_t dlt = slog_zero();
    for (int i = 0; i < V; ++i) {
        const long double a = rel_logit(trows, dt, tb + (size_t)i, r->mt, r->T);
        const long double b = rel_logit(drows, dt, db + (size_t)i, r->md, r->T);
        r->St += expl(a);
        r->Sd += expl(b);
        if (a != b) {
            slog_t d = exp_diff(a, b);
            d.s = -d.s; /* e^b - e^a */
            dlt = slog_add(dlt, d);
            if (b > -INFINITY) {
                const slog_t eb = {1, b};
                const slog_t y = {r->lY > -INFINITY ? 1 : 0, r->lY};
                r->lY = slog_add(y, eb).l;
            }
        }
    }
    r->kap = dlt;
    if (dlt.s != 0) r->kap.l -= logl(r->St);
    r->lam = 1.0L;
}

/* R_i = kappa e^{a_i} + lam (e^{a_i} - e^{b_i}) at the current lam (resid_t),
 * as a signed logarithm; *shared receives whether a_i = b_i. */
static slog_t resid_at(const resid_t *r, int i, int *shared)
{
    const long double a = rel_logit(r->trows, r->dt, r->tb + (size_t)i, r->mt, r->T);
    const long double b = rel_logit(r->drows, r->dt, r->db + (size_t)i, r->md, r->T);
    slog_t R = slog_zero();
    if (r->kap.s != 0 && a > -INFINITY) {
        R.s = r->kap.s;
        R.l = r->kap.l + a;
    }
    *shared = (a == b);
    if (a != b) {
        slog_t d = exp_diff(a, b);
        d.l += logl(r->lam);
        R = slog_add(R, d);
    }
    return R;
}

/* The log-weights lw_i = log max(0, R_i) (-inf where R_i <= 0) into lw[V];
 * returns log of their sum (-inf: no residual mass), and the log of the
 * differing tokens' part of it in *lw_diff. */
static long double resid_log_weights(const resid_t *r, long double *lw, long double *lw_diff)
{
    slog_t tot = slog_zero(), dif = slog_zero();
    for (int i = 0; i < r->V; ++i) {
        int shared = 0;
        const slog_t R = resid_at(r, i, &shared);
        lw[i] = R.s > 0 ? R.l : -INFINITY;
        if (R.s > 0) {
            tot = slog_add(tot, R);
            if (!shared) dif = slog_add(dif, R);
        }
    }
    if (lw_diff) *lw_diff = dif.l;
    return tot.l;
}

/* lam_{k+1} = lam_k + M_k and kappa_{k+1} (resid_t) from the log of the
 * residual's total lw_tot and of its differing tokens' part lw_diff. */
static void resid_advance(resid_t *r, long double lw_tot, long double lw_diff)
{
    const long double lSd = logl(r->Sd);
    const slog_t W = {lw_diff > -INFINITY ? 1 : 0, lw_diff};
    slog_t next;
    if (r->kap.s > 0) {
        slog_t kY = slog_zero();
        if (r->lY > -INFINITY) {
            kY.s = 1;
            kY.l = r->kap.l + r->lY;
        }
        slog_t mW = W;
        mW.s = -mW.s;
        next = slog_add(kY, mW);
        next.l -= lSd;
    } else {
        slog_t mWS = W;
        mWS.s = -mWS.s;
        mWS.l -= lSd;
        next = slog_add(r->kap, mWS);
    }
    if (next.s == 0) next.l = -INFINITY;
    r->kap = next;
    if (lw_tot > -INFINITY) r->lam += expl(lw_tot - lSd);
}

/* Weights proportional to max(0, p_i - lam q_i) from the log-weights: w_i =
 * e^{lw_i - max lw}; returns 1 if any is positive, 0 if none is. */
static int resid_weights_from_log(const long double *lw, int V, long double *w)
{
    long double mx = -INFINITY;
    for (int i = 0; i < V; ++i)
        if (lw[i] > mx) mx = lw[i];
    for (int i = 0; i < V; ++i) w[i] = (mx > -INFINITY && lw[i] > -INFINITY) ? expl(lw[i] - mx) : 0.0L;
    return mx > -INFINITY;
}

/* Inverse CDF over unnormalised weights in ascending index order.
 *   Z = sum w_i,  t = u * Z,  C_i = w_0 + ... + w_i,  y = min{i : C_i > t};
 *   if no index qualifies (t >= C_{V-1} through rounding), y = the last i with
 *   w_i > 0 (or 0 if all weights are zero).
 * *margin receives min(t - C_{y-1}, C_y - t) / Z with C_{-1} = 0: the distance of
 * the threshold to the nearest CDF boundary of the chosen bucket. */
static int draw_inverse_cdf(const long double *w, int V, double u, double *margin)
{
    long double Z = 0.0L;
    for (int i = 0; i < V; ++i) Z += w[i];
    long double t = (long double)u * Z;
    long double C = 0.0L;
    for (int i = 0; i < V; ++i) {
        long double prev = C;
        C += w[i];
        if (C > t) {
            if (margin) {
                long double a = t - prev, b = C - t;
                *margin = (Z > 0.0L) ? (double)((a < b ? a : b) / Z) : 0.0;
            }
            return i;
        }
    }
    int last = 0;
    for (int i = 0; i < V; ++i)
        if (w[i] > 0.0L) last = i;
    if (margin) *margin = 0.0;
    return last;
}

static double sanitize_uniform(float uf, uint32_t *flags)
{
    double u = (double)uf;
    if (!(u >= 0.0)) { /* NaN or negative */
        *flags |= OR_FLAG_BAD_UNIFORM;
        return 0.0;
    }
    if (u >= 1.0) {
        *flags |= OR_FLAG_BAD_UNIFORM;
        return 1.0 - ldexp(1.0, -24); /* largest float below 1 */
    }
    return u;
}

/* ------------------------------------------------------- one sequence step */

typedef struct {
    const void *target;  /* [B][n+1][V] */
    const void *draft;   /* [B][n][V], may be NULL if every T_b = 0 */
    int dt;
    const int32_t *draft_tokens; /* [B][n] */
    const int32_t *draft_lens;   /* [B] */
    const float *temperature;    /* [B], NULL in greedy mode */
    const float *uniforms;       /* [B][n+1], NULL in greedy mode */
    int B, n, V, mode;
    int32_t *accepted_len;  /* [B] */
    int32_t *emitted;       /* [B][n+1] */
    double *row_lse;        /* [B][2n+1] nullable */
    double *accept_margin;  /* [B][n] nullable */
    double *draw_margin;    /* [B] nullable */
    uint32_t *seq_flags;    /* [B] nullable */
} job_t;

static void verify_one(const job_t *J, int b, long double *w /* scratch [2V] */)
{
    const int n = J->n, V = J->V;
    uint32_t flags = 0;
    int L = J->draft_lens[b];
    if (L < 0) { L = 0; flags |= OR_FLAG_LEN_CLAMPED; }
    if (L > n) { L = n; flags |= OR_FLAG_LEN_CLAMPED; }

    double T = 0.0;
    if (J->mode == OR_MODE_SAMPLE) {
        T = (double)J->temperature[b];
        if (!(T >= 0.0)) { T = 0.0; flags |= OR_FLAG_BAD_TEMP; }
    }
    const int32_t *x = J->draft_tokens + (size_t)b * n;
    const size_t trow0 = (size_t)b * (size_t)(n + 1) * (size_t)V; /* target row 0 of b */
    const size_t drow0 = (size_t)b * (size_t)n * (size_t)V;       /* draft row 0 of b  */

    if (J->row_lse)
        for (int r = 0; r < 2 * n + 1; ++r) J->row_lse[(size_t)b * (2 * n + 1) + r] = NAN;
    if (J->accept_margin)
        for (int j = 0; j < n; ++j) J->accept_margin[(size_t)b * n + j] = INFINITY;
    if (J->draw_margin) J->draw_margin[b] = INFINITY;

    int k = L, y = -1;
    if (J->mode == OR_MODE_GREEDY || T == 0.0) {
        /* greedy rule: accept x_j iff it is the target argmax of row j */
        k = L;
        for (int j = 0; j < L; ++j) {
            int g = row_argmax(J->target, J->dt, trow0 + (size_t)j * V, V);
            if (x[j] < 0 || x[j] >= V) flags |= OR_FLAG_TOKEN_OOR;
            if (x[j] != g) { k = j; y = g; break; }
        }
        if (k == L) y = row_argmax(J->target, J->dt, trow0 + (size_t)L * V, V);
    } else {
        /* softmax statistics of every row the step may read */
        double mt[129], lst[129], md[129], lsd[129]; /* n <= 128 */
        for (int r = 0; r <= L; ++r) {
            double lse = row_softmax_stats(J->target, J->dt, trow0 + (size_t)r * V, V, T, &mt[r], &lst[r]);
            if (J->row_lse) J->row_lse[(size_t)b * (2 * n + 1) + r] = lse;
        }
        for (int r = 0; r < L; ++r) {
            double lse = row_softmax_stats(J->draft, J->dt, drow0 + (size_t)r * V, V, T, &md[r], &lsd[r]);
            if (J->row_lse) J->row_lse[(size_t)b * (2 * n + 1) + (n + 1) + r] = lse;
        }
        /* acceptance tests in order; the first rejection ends the scan */
        int rejected = 0;
        for (int j = 0; j < L; ++j) {
            if (x[j] < 0 || x[j] >= V) {
                flags |= OR_FLAG_TOKEN_OOR;
                k = j;
                rejected = 1;
                break;
            }
            double u = sanitize_uniform(J->uniforms[(size_t)b * (n + 1) + j], &flags);
            const double zt = logit_at(J->target, J->dt, trow0 + (size_t)j * V + (size_t)x[j]);
            const double zd = logit_at(J->draft, J->dt, drow0 + (size_t)j * V + (size_t)x[j]);
            double ratio = accept_ratio(zt, mt[j], lst[j], zd, md[j], lsd[j], T);
            if (J->accept_margin) J->accept_margin[(size_t)b * n + j] = fabs(u - ratio);
#if SV_ORACLE_PLANT == 3
            /* planted mistake for negative-control tests: the ratio inverted */
            ratio = accept_ratio(zd, md[j], lsd[j], zt, mt[j], lst[j], T);
#endif
            if (!(u < ratio)) {
                k = j;
                rejected = 1;
                break;
            }
        }
        double ufinal = sanitize_uniform(J->uniforms[(size_t)b * (n + 1) + n], &flags);
#if SV_ORACLE_PLANT == 2
        /* planted mistake: the rejected position's own uniform drives the draw */
        if (rejected) ufinal = sanitize_uniform(J->uniforms[(size_t)b * (n + 1) + k], &flags);
#endif
        if (rejected) {
            /* residual distribution max(0, p_k - q_k), formed exactly (resid_t) */
            resid_t rs;
            resid_setup(&rs, J->target, J->draft, J->dt, trow0 + (size_t)k * V, drow0 + (size_t)k * V, V, T);
            long double *lw = w + V;
            (void)resid_log_weights(&rs, lw, NULL);
            long double Z = resid_weights_from_log(lw, V, w) ? 1.0L : 0.0L;
#if SV_ORACLE_PLANT == 1
            /* planted mistake: plain target sampling at the rejection */
            row_probs_ld(J->target, J->dt, trow0 + (size_t)k * V, V, T, w);
            Z = 1.0L;
#endif
            if (!(Z > 0.0L)) {
                flags |= OR_FLAG_ZERO_RESIDUAL;
                row_probs_ld(J->target, J->dt, trow0 + (size_t)k * V, V, T, w);
            }
        } else {
            /* every draft accepted: the bonus token comes from p_L */
            row_probs_ld(J->target, J->dt, trow0 + (size_t)L * V, V, T, w);
        }
        double margin = 0.0;
        y = draw_inverse_cdf(w, V, ufinal, &margin);
        if (J->draw_margin) J->draw_margin[b] = margin;
    }

    /* emit: accepted prefix, then the correction or bonus token, then -1 */
    J->accepted_len[b] = k;
    int32_t *e = J->emitted + (size_t)b * (n + 1);
    for (int j = 0; j < k; ++j) e[j] = x[j];
    e[k] = y;
    for (int j = k + 1; j <= n; ++j) e[j] = -1;
    if (J->seq_flags) J->seq_flags[b] = flags;
}

typedef struct {
    const job_t *job;
    int b0, b1;
    int status;
} slice_t;

static void *run_slice(void *arg)
{
    slice_t *s = (slice_t *)arg;
    long double *w = (long double *)malloc(sizeof(long double) * 2 * (size_t)s->job->V);
    if (!w) { s->status = -2; return NULL; }
    for (int b = s->b0; b < s->b1; ++b) verify_one(s->job, b, w);
    free(w);
    s->status = 0;
    return NULL;
}

static int run_job(const job_t *J, int threads)
{
    if (J->B <= 0) return 0;
    if (threads < 1) threads = 1;
    if (threads > J->B) threads = J->B;
    slice_t *sl = (slice_t *)calloc((size_t)threads, sizeof(slice_t));
    pthread_t *th = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!sl || !th) { free(sl); free(th); return -2; }
    for (int t = 0; t < threads; ++t) {
        sl[t].job = J;
        sl[t].b0 = (int)((long long)J->B * t / threads);
        sl[t].b1 = (int)((long long)J->B * (t + 1) / threads);
    }
    int rc = 0;
    if (threads == 1) {
        run_slice(&sl[0]);
        rc = sl[0].status;
    } else {
        for (int t = 0; t < threads; ++t) pthread_create(&th[t], NULL, run_slice, &sl[t]);
        for (int t = 0; t < threads; ++t) {
            pthread_join(th[t], NULL);
            if (sl[t].status) rc = sl[t].status;
        }
    }
    free(sl);
    free(th);
    return rc;
}

static int check_dims(int B, int n, int V)
{
    if (B < 0 || n < 0 || n > 128 || V < 1) return -1;
    return 0;
}

/* ---------------------------------------------------------------- exports */

/* Verify-and-sample for every sequence.  Returns 0 on success, -1 on bad sizes,
 * -2 if scratch memory cannot be had.  seq_flags receives per-sequence OR_FLAG_*
 * bits (the GPU library reports their OR). */
int sv_oracle_verify_sample(const void *target_logits, const void *draft_logits, int dt,
                            const int32_t *draft_tokens, const int32_t *draft_lens,
                            const float *temperature, const float *uniforms, int B, int n, int V,
                            int32_t *accepted_len, int32_t *emitted, double *row_lse,
                            double *accept_margin, double *draw_margin, uint32_t *seq_flags,
                            int threads)
{
    if (check_dims(B, n, V)) return -1;
    job_t J = {target_logits, draft_logits, dt, draft_tokens, draft_lens, temperature, uniforms,
               B, n, V, OR_MODE_SAMPLE, accepted_len, emitted, row_lse, accept_margin,
               draw_margin, seq_flags};
    return run_job(&J, threads);
}

/* Greedy verify: accept the longest prefix whose drafts equal the target argmax;
 * the emitted token after it is the argmax of the first mismatching (or bonus)
 * row. */
int sv_oracle_verify_greedy(const void *target_logits, int dt, const int32_t *draft_tokens,
                            const int32_t *draft_lens, int B, int n, int V, int32_t *accepted_len,
                            int32_t *emitted, uint32_t *seq_flags, int threads)
{
    if (check_dims(B, n, V)) return -1;
    job_t J = {target_logits, NULL, dt, draft_tokens, draft_lens, NULL, NULL, B, n, V,
               OR_MODE_GREEDY, accepted_len, emitted, NULL, NULL, NULL, seq_flags};
    return run_job(&J, threads);
}

/* MTP bookkeeping.  The draft's input slot i pairs the target hidden state H_i
 * with the token that follows position i, so the token buffer moves left by one
 * relative to the hidden states, and the token the target just produced (emitted
 * at slot a_b) goes into slot a_b.  Slot n keeps its old value unless a_b = n.
 * Hidden states are copied unchanged (elem_bytes per element, B*(n+1)*H
 * elements); hidden_src == hidden_dst, or both NULL, copies nothing.  accepted
 * lengths outside [0, n] are clamped. */
int sv_oracle_mtp_shift_insert(int32_t *tokens, const void *hidden_src, void *hidden_dst, int H,
                               int elem_bytes, const int32_t *accepted_len,
                               const int32_t *emitted, int B, int n)
{
    if (B < 0 || n < 0 || H < 0 || elem_bytes < 0) return -1;
    int32_t *old = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n + 1));
    if (!old) return -2;
    for (int b = 0; b < B; ++b) {
        int32_t *t = tokens + (size_t)b * (n + 1);
        for (int i = 0; i <= n; ++i) old[i] = t[i];
        for (int i = 0; i < n; ++i) t[i] = old[i + 1];
        t[n] = old[n];
        int a = accepted_len[b];
        if (a < 0) a = 0;
        if (a > n) a = n;
        t[a] = emitted[(size_t)b * (n + 1) + a];
    }
    free(old);
    if (hidden_src && hidden_dst && hidden_src != hidden_dst)
        memcpy(hidden_dst, hidden_src, (size_t)B * (size_t)(n + 1) * (size_t)H * (size_t)elem_bytes);
    return 0;
}

/* Standard sampling of one token per sequence from a row chosen per sequence:
 * sequence b draws from logits[b][r_b][:] with r_b = row_index[b] clamped to
 * [0, R) (row 0 when row_index is NULL), by the same rule as a verify step with
 * no drafts (draft length 0): inverse CDF of softmax(z / T_b) with uniforms[b],
 * or the argmax when T_b = 0.  This is how the first draft token of the next
 * step comes from the carried draft logits at the accepted slot (Target-draft
 * section, decode paragraph; Single-token MTP scheduling section, second
 * paragraph).  seq_flags bit 32 marks a clamped row index. */
int sv_oracle_sample_rows(const void *logits, int dt, int R, const int32_t *row_index,
                          const float *temperature, const float *uniforms, int B, int V,
                          int32_t *tokens, uint32_t *seq_flags, int threads)
{
    if (B < 0 || R < 1 || V < 1) return -1;
    if (B == 0) return 0;
    const size_t es = (dt == OR_BF16) ? 2 : (dt == OR_F64) ? 8 : 4;
    unsigned char *rows = (unsigned char *)malloc((size_t)B * (size_t)V * es);
    int32_t *zeros = (int32_t *)calloc((size_t)B, sizeof(int32_t));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)B);
    if (!rows || !zeros || !acc) { free(rows); free(zeros); free(acc); return -2; }
    for (int b = 0; b < B; ++b) {
        int r = row_index ? row_index[b] : 0;
        uint32_t f = 0;
        if (r < 0) { r = 0; f = 32u; }
        if (r >= R) { r = R - 1; f = 32u; }
        if (seq_flags) seq_flags[b] = f;
        memcpy(rows + (size_t)b * V * es, (const unsigned char *)logits + ((size_t)b * R + r) * V * es,
               (size_t)V * es);
    }
    uint32_t *fl = (uint32_t *)calloc((size_t)B, sizeof(uint32_t));
    job_t J = {rows, NULL, dt, NULL, zeros, temperature, uniforms, B, 0, V, OR_MODE_SAMPLE,
               acc, tokens, NULL, NULL, NULL, fl};
    int rc = fl ? run_job(&J, threads) : -2;
    if (seq_flags && fl)
        for (int b = 0; b < B; ++b) seq_flags[b] |= fl[b];
    free(fl);
    free(rows);
    free(zeros);
    free(acc);
    return rc;
}

/* ------------------------------------------------- tree verification (greedy)
 *
 * EAGLE section of "Accelerating Sonar through speculation": the draft explores
 * a tree of candidate tokens, the target scores the candidate sequences, the
 * longest suitable one is kept and one more token from the target is appended.
 * Greedy reading, written out:
 *   - node 0 is the root (the last committed token); node j + 1 (j < L_b) holds
 *     draft token x_j and hangs below node parents[b][j], which must lie in
 *     [0, j] (nodes in topological order); a node with another parent is left
 *     out of the tree (flag OR_FLAG_BAD_PARENT);
 *   - target row r holds the logits after node r; g_r = its argmax (lowest index
 *     on ties);
 *   - node i is accepted iff its parent p is accepted (the root is) and
 *     x_{i-1} == g_p;
 *   - the kept path runs from the root to the deepest accepted node (the lowest
 *     index among equally deep ones); its draft tokens are emitted in order, then
 *     g of its last node, then -1;
 *   - path[b][0..]: the kept path's node indices (root excluded), then -1.
 * With parents[b][j] = j (a chain) this is the linear greedy rule. */
static void tree_one(const void *target, int dt, const int32_t *tokens, const int32_t *parents,
                     int L, int n, int V, size_t trow0, int32_t *acc, int32_t *emitted, int32_t *path,
                     uint32_t *flags_out)
{
    uint32_t flags = 0;
    if (L < 0) { L = 0; flags |= OR_FLAG_LEN_CLAMPED; }
    if (L > n) { L = n; flags |= OR_FLAG_LEN_CLAMPED; }
    int parent[129], depth[129], accepted[129];
    accepted[0] = 1;
    depth[0] = 0;
    int best = 0;
    for (int i = 1; i <= L; ++i) {
        const int p = parents[i - 1];
        const int x = tokens[i - 1];
        if (x < 0 || x >= V) flags |= OR_FLAG_TOKEN_OOR;
        parent[i] = p;
        accepted[i] = 0;
        depth[i] = 0;
        if (p < 0 || p >= i) {
            flags |= OR_FLAG_BAD_PARENT;
            continue;
        }
#if SV_ORACLE_PLANT == 6 /* negative control: the node's own row instead of its parent's */
        const int gp = row_argmax(target, dt, trow0 + (size_t)i * V, V);
#else
        const int gp = row_argmax(target, dt, trow0 + (size_t)p * V, V);
#endif
#if SV_ORACLE_PLANT == 7 /* negative control: the parent's acceptance is not required */
        if (x == gp) {
#else
        if (accepted[p] && x == gp) {
#endif
            accepted[i] = 1;
            depth[i] = depth[p] + 1;
            if (depth[i] > depth[best]) best = i;
        }
    }
    const int k = depth[best];
    /* the kept path, root excluded, from the root down */
    int node = best;
    for (int d = k - 1; d >= 0; --d) {
        path[d] = node;
        emitted[d] = tokens[node - 1];
        node = parent[node];
    }
    emitted[k] = row_argmax(target, dt, trow0 + (size_t)best * V, V);
    for (int d = k + 1; d <= n; ++d) emitted[d] = -1;
    for (int d = k; d < n; ++d) path[d] = -1;
    *acc = k;
    *flags_out = flags;
}

/* Greedy tree verification for every sequence; target logits [B][n+1][V],
 * draft_tokens and draft_parents [B][n], draft_lens [B]; outputs accepted_len
 * [B], emitted [B][n+1], path [B][n] (nullable), seq_flags [B] (nullable).
 * Returns 0, or -1 on bad sizes. */
int sv_oracle_verify_tree_greedy(const void *target_logits, int dt, const int32_t *draft_tokens,
                                 const int32_t *draft_parents, const int32_t *draft_lens, int B, int n,
                                 int V, int32_t *accepted_len, int32_t *emitted, int32_t *path,
                                 uint32_t *seq_flags)
{
    if (check_dims(B, n, V)) return -1;
    int32_t scratch_path[128];
    for (int b = 0; b < B; ++b) {
        uint32_t f = 0;
        tree_one(target_logits, dt, draft_tokens + (size_t)b * n, draft_parents + (size_t)b * n,
                 draft_lens[b], n, V, (size_t)b * (size_t)(n + 1) * (size_t)V, &accepted_len[b],
                 emitted + (size_t)b * (n + 1), path ? path + (size_t)b * n : scratch_path, &f);
        if (seq_flags) seq_flags[b] = f;
    }
    return 0;
}

/* ----------------------------------------------- tree verification (sampling)
 *
 * EAGLE section of "Accelerating Sonar through speculation": the draft proposes
 * a tree of candidate tokens (several candidates per node), the target scores
 * every candidate sequence, the longest suitable one is kept and one more token
 * from the target is appended.  The page gives no acceptance rule for sampling;
 * the rule taken is SpecInfer's multi-step speculative sampling (Miao et al.,
 * "SpecInfer: Accelerating Large Language Model Serving with Tree-based
 * Speculative Inference and Verification"), which keeps the target's
 * distribution when every node's children are independent draws from the
 * draft's distribution at that node:
 *   - node 0 is the root; node j + 1 (j < L) holds x_j below parents[j] in
 *     [0, j] (other parents leave the node out, flagged);
 *   - target row r is p_r = softmax(z_t[r] / T), the target after node r; draft
 *     row r is q_r = softmax(z_d[r] / T), the draft at node r, from which node
 *     r's children were drawn;
 *   - at node u with children c_1 < c_2 < ... (index order): the current target
 *     residual starts as p' = p_u; child c_i is accepted iff
 *     u[c_i - 1] < p'(x) / q_u(x) (q_u(x) = 0: ratio +inf if p'(x) > 0, else 0);
 *     accepting it moves the walk to c_i; rejecting it replaces p' by
 *     max(0, p' - q_u) normalised.  After k rejections p' is
 *     max(0, p_u - lam_k q_u) / M_k with lam_0 = 0, M_0 = 1 and
 *     lam_{k+1} = lam_k + M_k, M_{k+1} = sum_i max(0, p_u,i - lam_{k+1} q_u,i)
 *     (the same residual, written without nesting);
 *   - when no child of the current node is accepted the token is drawn with
 *     u[n] from p' (p_u itself when the node has no children: the bonus
 *     token); a residual with no mass left falls back to p_u (flagged);
 *   - outputs as in the greedy tree rule: the kept path's tokens, the drawn
 *     token, then -1; path[] the kept path's nodes.
 * With parents[j] = j (a chain) this is the linear sampling rule.  T_b = 0 takes
 * the greedy tree rule.  A limit on the number of M_k a walk may form
 * (max_rounds >= 0; negative: none) is the same rule on a smaller tree: when a
 * rejection leaves a later sibling to test and the walk has formed its
 * max_rounds sums already, the untested siblings are dropped, the token is
 * drawn from max(0, p_u - lam_{k+1} q_u) (that residual needs no new sum
 * before the draw), and the sequence is flagged.  The residual sums, the later
 * siblings' ratios and the draw are formed from resid_t in extended precision,
 * the first acceptance test at a node as the linear rule forms it. */
typedef struct {
    const void *target, *draft;
    int dt;
    const int32_t *tokens, *parents, *lens;
    const float *temperature, *uniforms;
    int B, n, V, max_rounds;
    int32_t *acc, *emitted, *path;
    double *accept_margin, *draw_margin;
    uint32_t *seq_flags;
} tree_job_t;

static void tree_sample_one(const tree_job_t *J, int b, long double *w /* scratch [3V] */)
{
    const int n = J->n, V = J->V;
    uint32_t flags = 0;
    int L = J->lens[b];
    if (L < 0) { L = 0; flags |= OR_FLAG_LEN_CLAMPED; }
    if (L > n) { L = n; flags |= OR_FLAG_LEN_CLAMPED; }
    double T = (double)J->temperature[b];
    if (!(T >= 0.0)) { T = 0.0; flags |= OR_FLAG_BAD_TEMP; }
    const int32_t *x = J->tokens + (size_t)b * n;
    const int32_t *par = J->parents + (size_t)b * n;
    const float *uni = J->uniforms + (size_t)b * (n + 1);
    int32_t *e = J->emitted + (size_t)b * (n + 1);
    int32_t scratch_path[128];
    int32_t *path = J->path ? J->path + (size_t)b * n : scratch_path;
    for (int j = 0; j < n; ++j) J->accept_margin[(size_t)b * n + j] = INFINITY;
    J->draw_margin[b] = INFINITY;
    if (T == 0.0) {
        uint32_t f = 0;
        tree_one(J->target, J->dt, x, par, J->lens[b], n, V, (size_t)b * (size_t)(n + 1) * (size_t)V, &J->acc[b],
                 e, path, &f);
        J->seq_flags[b] = flags | f;
        return;
    }
    for (int j = 0; j < L; ++j) {
        if (par[j] < 0 || par[j] > j) flags |= OR_FLAG_BAD_PARENT;
        if (x[j] < 0 || x[j] >= V) flags |= OR_FLAG_TOKEN_OOR;
    }
    const size_t trow0 = (size_t)b * (size_t)(n + 1) * (size_t)V;
    const size_t drow0 = (size_t)b * (size_t)n * (size_t)V;
    long double *p = w, *q = w + V, *lw = w + 2 * (size_t)V;
    int u = 0, depth = 0, y = -1, sums = 0;
    for (;;) {
        /* the target at node u, and (if u has children) the draft at node u */
        int first = -1;
        for (int j = 0; j < L; ++j)
            if (par[j] == u && par[j] <= j) { first = j; break; }
        row_probs_ld(J->target, J->dt, trow0 + (size_t)u * V, V, T, p);
        if (first < 0) {
            /* no children: the bonus token from p_u */
            double margin = 0.0;
            y = draw_inverse_cdf(p, V, sanitize_uniform(uni[n], &flags), &margin);
            J->draw_margin[b] = margin;
            break;
        }
        double mt, lst, md, lsd;
        (void)row_softmax_stats(J->target, J->dt, trow0 + (size_t)u * V, V, T, &mt, &lst);
        (void)row_softmax_stats(J->draft, J->dt, drow0 + (size_t)u * V, V, T, &md, &lsd);
        /* after k >= 1 rejections at u: the residual max(0, p_u - lam_k q_u) of
         * resid_t (lam_k, kappa_k), its log-weights in lw, log M_k in lM */
        resid_t rs;
        int rejections = 0, accepted = -1, have_rs = 0;
        long double lW = -INFINITY, lWd = -INFINITY, lM = -INFINITY;
        slog_t kap1 = slog_zero(); /* kappa_1, for the planted mistakes below */
        (void)kap1;
        for (int j = first; j < L; ++j) {
            if (par[j] != u || par[j] > j) continue;
            const int xc = x[j];
            double ratio = 0.0;
            if (xc >= 0 && xc < V) {
                if (rejections == 0) {
                    /* p_u(x) / q_u(x), as the linear rule forms it */
                    ratio = accept_ratio(logit_at(J->target, J->dt, trow0 + (size_t)u * V + (size_t)xc), mt, lst,
                                         logit_at(J->draft, J->dt, drow0 + (size_t)u * V + (size_t)xc), md, lsd, T);
                } else {
                    /* the residual's ratio (p_u(x) - lam q_u(x)) / (M_k q_u(x)) =
                     * R_x / (M_k e^{b_x}) (resid_t); q_u(x) = 0 < p_u(x) - lam q_u(x)
                     * gives +inf */
                    int shared = 0;
                    const slog_t R = resid_at(&rs, xc, &shared);
                    const long double bx = rel_logit(J->draft, J->dt, drow0 + (size_t)u * V + (size_t)xc, rs.md, rs.T);
                    if (R.s > 0 && lM > -INFINITY) ratio = (double)expl(R.l - lM - bx);
                }
            }
            const double uu = sanitize_uniform(uni[j], &flags);
            J->accept_margin[(size_t)b * n + j] = fabs(uu - ratio);
            if (uu < ratio) { accepted = j; break; }
            if (!have_rs) {
                resid_setup(&rs, J->target, J->draft, J->dt, trow0 + (size_t)u * V, drow0 + (size_t)u * V, V, T);
                kap1 = rs.kap;
                have_rs = 1;
            }
#if SV_ORACLE_PLANT == 8
            /* planted mistake: every sibling tested against p_u itself (no
             * residual update between siblings); the draw still takes
             * max(0, p_u - q_u) */
            continue;
#endif
            /* rejected: p' <- max(0, p' - q_u) normalised, i.e. lam_{k+1} = lam_k + M_k
             * (the first rejection leaves lam_1 = 1 as resid_setup() formed it) */
            if (rejections > 0) resid_advance(&rs, lW, lWd);
            ++rejections;
            int later = 0;
            for (int t = j + 1; t < L && !later; ++t) later = (par[t] == u);
            if (!later) break; /* the draw forms its own sum */
            if (J->max_rounds >= 0 && sums >= J->max_rounds) {
                flags |= OR_FLAG_TREE_TRUNCATED; /* the later siblings stay untested */
                break;
            }
            ++sums;
            lW = resid_log_weights(&rs, lw, &lWd);
            lM = lW > -INFINITY ? lW - logl(rs.Sd) : -INFINITY;
        }
        if (accepted >= 0) {
            path[depth] = accepted + 1;
            e[depth] = x[accepted];
            ++depth;
            u = accepted + 1;
            continue;
        }
        /* every child rejected: draw from max(0, p_u - lam q_u) */
#if SV_ORACLE_PLANT == 8 || SV_ORACLE_PLANT == 9
        /* planted mistakes: the draw ignores the later siblings' updates */
        rs.kap = kap1;
        rs.lam = 1.0L;
#endif
        (void)resid_log_weights(&rs, lw, NULL);
        double margin = 0.0;
        if (resid_weights_from_log(lw, V, q)) {
            y = draw_inverse_cdf(q, V, sanitize_uniform(uni[n], &flags), &margin);
        } else {
            flags |= OR_FLAG_ZERO_RESIDUAL;
            y = draw_inverse_cdf(p, V, sanitize_uniform(uni[n], &flags), &margin);
        }
        J->draw_margin[b] = margin;
        break;
    }
    J->acc[b] = depth;
    e[depth] = y;
    for (int d = depth + 1; d <= n; ++d) e[d] = -1;
    for (int d = depth; d < n; ++d) path[d] = -1;
    J->seq_flags[b] = flags;
}

/* Sampling tree verification for every sequence.  target [B][n+1][V], draft
 * [B][n][V] (row r = the draft at node r), draft_tokens / draft_parents [B][n],
 * draft_lens [B], temperature [B], uniforms [B][n+1] (u[j]: the test of node
 * j + 1, u[n]: the final draw), max_rounds (the limit on the residual sums a
 * walk forms before a later sibling's test; negative: none).  Outputs accepted_len [B], emitted [B][n+1],
 * path [B][n] (nullable), accept_margin [B][n] (+inf for nodes not tested),
 * draw_margin [B], seq_flags [B].  Returns 0, -1 on bad sizes, -2 without memory. */
int sv_oracle_verify_tree_sample(const void *target_logits, const void *draft_logits, int dt,
                                 const int32_t *draft_tokens, const int32_t *draft_parents,
                                 const int32_t *draft_lens, const float *temperature, const float *uniforms,
                                 int B, int n, int V, int max_rounds, int32_t *accepted_len, int32_t *emitted,
                                 int32_t *path, double *accept_margin, double *draw_margin, uint32_t *seq_flags)
{
    if (check_dims(B, n, V)) return -1;
    long double *w = (long double *)malloc(sizeof(long double) * 3 * (size_t)V);
    if (!w) return -2;
    tree_job_t J = {target_logits, draft_logits, dt, draft_tokens, draft_parents, draft_lens, temperature,
                    uniforms, B, n, V, max_rounds, accepted_len, emitted, path, accept_margin, draw_margin, seq_flags};
    for (int b = 0; b < B; ++b) tree_sample_one(&J, b, w);
    free(w);
    return 0;
}

/* ------------------------------------------------------- logit projection */

/* The target's logit projection (its lm_head): a [V][H] matrix that maps a
 * final hidden state to one logit per vocabulary entry.  The MTP section of
 * "Accelerating Sonar through speculation" (the paragraph on the MTP head's
 * normalisation layers) notes that the MTP head reuses this projection, which is
 * about 2 GB for a 70B Llama; the model runs it to produce the logits the step
 * samples from (Inference with speculative decoding section, first paragraph).
 *
 *   logits[i][v] = sum_k hidden[r_i][k] * weight[v][k]
 *
 * for the hidden rows r_i = rows[i] (rows NULL: r_i = i, nrows = M).  bf16
 * inputs are widened exactly; each product is exact in double (two 8-bit
 * significands) and the sum runs in double in ascending k. */
typedef struct {
    const uint16_t *hidden, *weight;
    int M, H, V;
    const int32_t *rows;
    int nrows;
    double *out;
    long long i0, i1; /* flat output range [i0, i1) of this thread */
    int status;
} lm_job_t;

static double bf16_at(const uint16_t *p, size_t idx)
{
    uint32_t bits = ((uint32_t)p[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static void *lm_slice(void *arg)
{
    lm_job_t *J = (lm_job_t *)arg;
    const int H = J->H, V = J->V;
    for (long long o = J->i0; o < J->i1; ++o) {
        const int i = (int)(o / V), v = (int)(o % V);
        const int r = J->rows ? J->rows[i] : i;
        if (r < 0 || r >= J->M) {
            J->status = -1;
            return NULL;
        }
        double acc = 0.0;
#if SV_ORACLE_PLANT == 4 /* negative control: the last product is dropped */
        for (int k = 0; k < H - 1; ++k)
#else
        for (int k = 0; k < H; ++k)
#endif
#if SV_ORACLE_PLANT == 5 /* negative control: the weight is indexed transposed */
            acc += bf16_at(J->hidden, (size_t)r * H + k) * bf16_at(J->weight, (size_t)k * V + v);
#else
            acc += bf16_at(J->hidden, (size_t)r * H + k) * bf16_at(J->weight, (size_t)v * H + k);
#endif
        J->out[o] = acc;
    }
    return NULL;
}

int sv_oracle_lmhead_logits(const uint16_t *hidden, const uint16_t *weight, int M, int H, int V,
                            const int32_t *rows, int nrows, double *out, int threads)
{
    if (M < 0 || H < 1 || V < 1 || nrows < 0 || (!rows && nrows != M)) return -1;
    if (threads < 1) threads = 1;
    const long long total = (long long)nrows * V;
    if (total == 0) return 0;
    if (threads > total) threads = (int)total;
    lm_job_t *sl = (lm_job_t *)calloc((size_t)threads, sizeof(lm_job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!sl || !th) { free(sl); free(th); return -2; }
    int rc = 0;
    for (int t = 0; t < threads; ++t) {
        lm_job_t J = {hidden, weight, M, H, V, rows, nrows, out,
                      total * t / threads, total * (t + 1) / threads, 0};
        sl[t] = J;
    }
    if (threads == 1) {
        lm_slice(&sl[0]);
        rc = sl[0].status;
    } else {
        /* a slice whose thread cannot be started runs on the calling thread */
        unsigned char *started = (unsigned char *)calloc((size_t)threads, 1);
        if (!started) { free(sl); free(th); return -2; }
        for (int t = 0; t < threads; ++t) {
            started[t] = pthread_create(&th[t], NULL, lm_slice, &sl[t]) == 0;
            if (!started[t]) lm_slice(&sl[t]);
        }
        for (int t = 0; t < threads; ++t) {
            if (started[t]) pthread_join(th[t], NULL);
            if (sl[t].status) rc = sl[t].status;
        }
        free(started);
    }
    free(sl);
    free(th);
    return rc;
}

/* Softmax of one row at temperature T (> 0): returns lse = log sum exp(z / T) and,
 * if p_out is not NULL, writes p_i = exp(z_i / T - lse). */
double sv_oracle_softmax_row(const void *z, int dt, int V, double T, double *p_out)
{
    double m, logS;
    double lse = row_softmax_stats(z, dt, 0, V, T, &m, &logS);
    if (p_out)
        for (int i = 0; i < V; ++i) p_out[i] = prob_at(z, dt, 0, i, T, m, logS);
    return lse;
}

/* Greedy choice of one row (lowest index of the maximum). */
int sv_oracle_argmax_row(const void *z, int dt, int V)
{
    return row_argmax(z, dt, 0, V);
}

/* The inverse-CDF step on explicit weights (exposed for pinning; the weights
 * are widened to extended precision as the step's own draw forms them).
 * Returns -2 if scratch memory cannot be had. */
int sv_oracle_draw_weights(const double *w, int V, double u, double *margin)
{
    long double *wl = (long double *)malloc(sizeof(long double) * (size_t)(V > 0 ? V : 1));
    if (!wl) return -2;
    for (int i = 0; i < V; ++i) wl[i] = w[i];
    int y = draw_inverse_cdf(wl, V, u, margin);
    free(wl);
    return y;
}

/* Which planted mistake this compiled oracle carries (0 = none).  Test-only builds set
 * SV_ORACLE_PLANT to show that the statistical tests reject a wrong rule. */
int sv_oracle_plant(void)
{
#ifdef SV_ORACLE_PLANT
    return SV_ORACLE_PLANT;
#else
    return 0;
#endif
}
