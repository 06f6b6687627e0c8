/*
 * smcsd_oracle.c -- plain, slow CPU reference of one SMC-SD round, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY. It exists to check the GPU library, not to run in its place:
 * only the test suite, the smoke check and the CPU-baseline leg of the benchmark load it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What one round computes is taken from "Faster LLM Inference via Sequential Monte Carlo"
 * (SMC-SD), section 2 "Methodology":
 *   - a request keeps N particles, each a partially generated string;
 *   - the draft model extends every particle by K tokens;
 *   - the target model scores all extended particles in one batched pass;
 *   - no token is rejected; each particle instead receives an importance weight;
 *   - low-weight particles are evicted and high-weight ones duplicated, giving N again,
 *     as in sequential Monte Carlo;
 *   - every round also yields one bonus token from the target, so K+1 tokens per round;
 *   - a duplicated particle shares KV pages with its source by copying page metadata and
 *     exchanging pointers, never by copying KV tensors.
 * The per-position total-variation distance is the block-divergence signal of the METASD
 * page (section 2, "alignment feedback as reward"). Bonus noise is precomputed Gumbel noise
 * as in the STAND page (method item 2, Gumbel-Top-K with cached noise), used here with k=1.
 *
 * The pages print no formulas. Where they are silent this file takes the plainest reading:
 *   R1 weight: log w_i = sum_k [log p(x_k) - log q(x_k)] over the K drafted tokens; the bonus
 *      token is drawn from p itself, so its ratio is 1 and it adds nothing.
 *   R2 temperature: one T per request divides both target and draft logits.
 *   R3 carried weights: l_i = logW_prev_i + log w_i; logZ = LSE_i l_i; after resampling every
 *      log-weight becomes -log N, otherwise l_i - logZ is carried (normalised).
 *   R4 resampling scheme: systematic, U_j = (j+u)/N, ancestor = min{i : U_j < C_i} with C the
 *      inclusive prefix sum of the normalised weights, clamped to N-1.
 *   R5 ESS = 1 / sum W_i^2; mode ESS resamples iff ESS < ess_frac * N (strict).
 *   R6 bonus: drawn per original particle from its row K and inherited through the ancestor.
 *   R7 the bonus key is the real number z_v/T + G_v, evaluated here in double; an exact tie
 *      goes to the lowest index. The gap between the best and the second-best key is returned
 *      with every decision, so that a check can tell a clear winner from a near tie.
 *   R8 page table: [N][P] int32 per request, negative = unused; a refcount counts table
 *      entries that reference a page.
 *   R9 potential (optional): the SMC-SD page's section 5 names constrained generation and
 *      reward-weighted decoding as targets the same machinery can sample. Reading: the
 *      target becomes p times a potential phi, so particle i's incremental log weight gains
 *      log phi_i (given per particle and round; -inf removes the particle).
 * Summation order: over v ascending within a row, over k ascending, over i ascending.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_ALWAYS = 0, ORC_ESS = 1, ORC_NEVER = 2 };

/* A bf16 value is the upper 16 bits of an IEEE-754 binary32, so widening is exact. */
static float elem_f32(const void *row, int dtype, int64_t v)
{
    if (dtype == ORC_F32)
        return ((const float *)row)[v];
    uint32_t bits = (uint32_t)((const uint16_t *)row)[v] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

static double elem(const void *row, int dtype, int64_t v)
{
    return (double)elem_f32(row, dtype, v);
}

static size_t esize(int dtype) { return dtype == ORC_F32 ? 4u : 2u; }

/*
 * Temperature-scaled log-softmax normaliser of one logits row:
 *   LSE(z/T) = m + log sum_v exp(z_v/T - m),  m = max_v z_v/T.
 * log p(v) = z_v/T - LSE. (SMC-SD page, section 2: the weights need normalised target and
 * draft probabilities at the drafted tokens; reading R2 for T.)
 */
double orc_row_logsumexp(const void *row, int dtype, int64_t V, double T)
{
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double a = elem(row, dtype, v) / T;
        if (a > m)
            m = a;
    }
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v)
        s += exp(elem(row, dtype, v) / T - m);
    return m + log(s);
}

/*
 * Total-variation distance between the target and draft distributions of one position:
 *   TV = 1/2 sum_v |exp(zp_v/T - A) - exp(zq_v/T - B)|
 * with A, B the normalisers above (METASD page, section 2: block divergence is built on the
 * total-variation distance between drafter and target distributions).
 */
static double tv_given_norms(const void *zp, const void *zq, int dtype, int64_t V, double T,
                             double A, double B)
{
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v)
        s += fabs(exp(elem(zp, dtype, v) / T - A) - exp(elem(zq, dtype, v) / T - B));
    return 0.5 * s;
}

double orc_row_tv(const void *zp, const void *zq, int dtype, int64_t V, double T)
{
    double A = orc_row_logsumexp(zp, dtype, V, T);
    double B = orc_row_logsumexp(zq, dtype, V, T);
    return tv_given_norms(zp, zq, dtype, V, T, A, B);
}

/*
 * Bonus token by Gumbel-max: argmax_v (z_v/T + G_v) with G precomputed standard Gumbel
 * noise. Adding the row's normaliser to every key changes nothing, so this is argmax of
 * log p(v) + G_v, i.e. one draw from p (STAND page, method item 2: Gumbel noise added to
 * log-probabilities, top-k of the sum, noise precomputed and cached; here k = 1).
 * Keys in double (reading R7), lowest index on an exact tie. *gap receives
 * key(best) - key(second best), 0 on a tie, +inf when V == 1.
 */
int32_t orc_row_gumbel_argmax(const void *row, int dtype, const float *g, int64_t V, float T,
                              double *gap)
{
    const double t = (double)T;
    double k1 = -INFINITY, k2 = -INFINITY;
    int32_t best = 0;
    for (int64_t v = 0; v < V; ++v) {
        double key = elem(row, dtype, v) / t + (double)g[v];
        if (key > k1) {
            k2 = k1;
            k1 = key;
            best = (int32_t)v;
        } else if (key > k2) {
            k2 = key;
        }
    }
    if (gap)
        *gap = V > 1 ? k1 - k2 : INFINITY;
    return best;
}

/*
 * Normalise, ESS, resample decision and systematic resampling for one request
 * (SMC-SD page, section 2: evict low-weight particles, duplicate high-weight ones, keep N;
 * readings R3, R4, R5).
 *   l_i = logw_prev_i + lw_i
 *   e_i = exp(l_i - max l),  W_i = e_i / sum e,  logZ = max l + log sum e,  ESS = 1/sum W_i^2
 * Resampled: anc_j = min{i : (j+u)/N < C_i} (clamped to N-1), logw_new_i = -log N.
 * Otherwise: anc_j = j, logw_new_i = l_i - logZ.
 * gap[j] = min_i |U_j - C_i| (infinity when not resampled): how close ancestor j is to a tie.
 * Returns 1 if the request was resampled.
 */
int32_t orc_resample_request(int32_t N, const double *lw, const double *logw_prev, double u,
                             int32_t mode, double ess_frac, double *logZ, double *ess,
                             int32_t *anc, double *logw_new, double *gap)
{
    double *l = malloc(sizeof(double) * (size_t)N * 3);
    double *W = l + N, *C = l + 2 * (size_t)N;
    double m = -INFINITY;
    for (int32_t i = 0; i < N; ++i) {
        l[i] = logw_prev[i] + lw[i];
        if (l[i] > m)
            m = l[i];
    }
    double se = 0.0;
    for (int32_t i = 0; i < N; ++i) {
        W[i] = exp(l[i] - m);
        se += W[i];
    }
    double s2 = 0.0;
    for (int32_t i = 0; i < N; ++i) {
        W[i] = W[i] / se;
        s2 += W[i] * W[i];
    }
    *logZ = m + log(se);
    *ess = 1.0 / s2;
    int32_t rs = mode == ORC_ALWAYS || (mode == ORC_ESS && *ess < ess_frac * (double)N);
    if (rs) {
        double c = 0.0;
        for (int32_t i = 0; i < N; ++i) {
            c += W[i];
            C[i] = c;
        }
        for (int32_t j = 0; j < N; ++j) {
            double U = ((double)j + u) / (double)N;
            int32_t i = 0;
            while (i < N - 1 && !(U < C[i]))
                ++i;
            anc[j] = i;
            double g = INFINITY;
            for (int32_t t = 0; t < N; ++t)
                g = fmin(g, fabs(U - C[t]));
            gap[j] = g;
        }
        for (int32_t i = 0; i < N; ++i)
            logw_new[i] = -log((double)N);
    } else {
        for (int32_t j = 0; j < N; ++j) {
            anc[j] = j;
            gap[j] = INFINITY;
        }
        for (int32_t i = 0; i < N; ++i)
            logw_new[i] = l[i] - *logZ;
    }
    free(l);
    return rs;
}

/*
 * Page-table remap by pointer exchange for one request (SMC-SD page, section 2: a
 * duplicated particle gets a copy of its source's page metadata and shares the KV pages
 * through pointers; KV tensors are never copied; reading R8).
 *   pt_out[j][c] = pt_in[anc_j][c]
 *   o_i = #{j : anc_j = i};  for each valid pt_in[i][c]: refcount[page] += o_i - 1
 * Returns 0, or -1 if an ancestor or page id is out of range or a refcount ends negative.
 */
int32_t orc_remap_request(int32_t N, int32_t P, const int32_t *anc, const int32_t *pt_in,
                          int32_t *pt_out, int32_t *refcount, int32_t num_pages)
{
    int32_t err = 0;
    int32_t *o = calloc((size_t)N, sizeof(int32_t));
    for (int32_t j = 0; j < N; ++j) {
        if (anc[j] < 0 || anc[j] >= N) {
            free(o);
            return -1;
        }
        o[anc[j]] += 1;
    }
    for (int32_t j = 0; j < N; ++j)
        for (int32_t c = 0; c < P; ++c)
            pt_out[(size_t)j * P + c] = pt_in[(size_t)anc[j] * P + c];
    for (int32_t i = 0; i < N; ++i)
        for (int32_t c = 0; c < P; ++c) {
            int32_t page = pt_in[(size_t)i * P + c];
            if (page < 0)
                continue;
            if (page >= num_pages) {
                err = -1;
                continue;
            }
            refcount[page] += o[i] - 1;
        }
    for (int32_t i = 0; i < N; ++i)
        for (int32_t c = 0; c < P; ++c) {
            int32_t page = pt_in[(size_t)i * P + c];
            if (page >= 0 && page < num_pages && refcount[page] < 0)
                err = -1;
        }
    free(o);
    return err;
}

/*
 * One whole round over R requests (SMC-SD page, section 2, in the order propose -> weight
 * -> resample -> remap; reading R6 for the bonus).
 *
 * Layouts (row stride ld elements, ld >= V; element type per dtype):
 *   target [R][N][K+1][ld]  rows 0..K-1 score the drafted tokens, row K is the bonus position
 *   draft  [R][N][K][ld]    row k is the distribution x_k was drawn from
 *   tokens [R][N][K] int32, temperature [R], gumbel [R][N][ld] fp32, uniform [R] in [0,1),
 *   logw_in [R][N] fp32 (normalised), page tables [R][N][P] int32, refcount [num_pages].
 * Outputs in double where the value is real: lw [R][N], logw_out [R][N], log_norm [R],
 * ess [R], tv [R][N][K] (NULL skips TV), anc_gap [R][N], bonus_gap [R][N]; int32 elsewhere.
 * out_tokens [R][N][K+1] may be NULL; pt_in == NULL skips the remap. log_potential [R][N]
 * (R9) may be NULL.
 * Returns 0, or a negative code on an out-of-range token (-1) or remap error (-2).
 */
int32_t orc_round(int32_t R, int32_t N, int32_t K, int64_t V, int64_t ld, int32_t dtype,
                  const void *target, const void *draft, const int32_t *tokens,
                  const float *temperature, const float *gumbel, const float *uniform,
                  int32_t mode, float ess_frac, const float *logw_in,
                  double *lw, double *logw_out, double *log_norm, double *ess,
                  int32_t *resampled, int32_t *anc, int32_t *bonus, int32_t *out_tokens,
                  double *tv, int32_t P, int32_t num_pages, const int32_t *pt_in,
                  int32_t *pt_out, int32_t *refcount, double *anc_gap, double *bonus_gap,
                  const float *log_potential)
{
    const size_t es = esize(dtype);
    const int64_t rows = (int64_t)R * N * K;
    double *d = malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
    int32_t bad_token = 0;

    /* Per drafted position: log p(x_k) - log q(x_k), and the TV of that position. */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad_token)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t r = row / ((int64_t)N * K);
        int64_t ik = row % ((int64_t)N * K);
        int64_t i = ik / K, k = ik % K;
        const char *zp = (const char *)target + (size_t)(((r * N + i) * (K + 1) + k) * ld) * es;
        const char *zq = (const char *)draft + (size_t)(((r * N + i) * K + k) * ld) * es;
        double T = (double)temperature[r];
        double A = orc_row_logsumexp(zp, dtype, V, T);
        double B = orc_row_logsumexp(zq, dtype, V, T);
        int32_t x = tokens[row];
        if (x < 0 || x >= V) {
            bad_token = 1;
            d[row] = 0.0;
        } else {
            d[row] = (elem(zp, dtype, x) / T - A) - (elem(zq, dtype, x) / T - B);
        }
        if (tv)
            tv[row] = tv_given_norms(zp, zq, dtype, V, T, A, B);
    }

    /* Bonus token of every original particle. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < (int64_t)R * N; ++ri) {
        int64_t r = ri / N;
        const char *zb = (const char *)target + (size_t)((ri * (K + 1) + K) * ld) * es;
        bonus[ri] = orc_row_gumbel_argmax(zb, dtype, gumbel + (size_t)ri * ld, V, temperature[r],
                                          bonus_gap ? &bonus_gap[ri] : NULL);
    }

    int32_t err = bad_token ? -1 : 0;
    double *prev = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *gap_tmp = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    for (int32_t r = 0; r < R; ++r) {
        for (int32_t i = 0; i < N; ++i) {
            double s = 0.0;
            for (int32_t k = 0; k < K; ++k)
                s += d[((size_t)r * N + i) * K + k];
            if (log_potential)
                s += (double)log_potential[(size_t)r * N + i];
            lw[(size_t)r * N + i] = s;
            prev[i] = (double)logw_in[(size_t)r * N + i];
        }
        resampled[r] = orc_resample_request(N, lw + (size_t)r * N, prev, (double)uniform[r], mode,
                                            (double)ess_frac, &log_norm[r], &ess[r],
                                            anc + (size_t)r * N, logw_out + (size_t)r * N,
                                            anc_gap ? anc_gap + (size_t)r * N : gap_tmp);
        if (out_tokens) {
            for (int32_t j = 0; j < N; ++j) {
                int32_t a = anc[(size_t)r * N + j];
                int32_t *dst = out_tokens + ((size_t)r * N + j) * (K + 1);
                for (int32_t k = 0; k < K; ++k)
                    dst[k] = tokens[((size_t)r * N + a) * K + k];
                dst[K] = bonus[(size_t)r * N + a];
            }
        }
        if (pt_in) {
            if (orc_remap_request(N, P, anc + (size_t)r * N, pt_in + (size_t)r * N * P,
                                  pt_out + (size_t)r * N * P, refcount, num_pages) != 0)
                err = err ? err : -2;
        }
    }
    free(gap_tmp);
    free(prev);
    free(d);
    return err;
}

/*
 * Standard speculative-decoding verification of one particle's K drafted tokens, the
 * baseline the SMC-SD page compares against (section 1: the target verifies the draft, the
 * first rejection discards every later draft token). The pages give no formulas; this is
 * standard speculative sampling written from its definition (readings S1-S3):
 *   S1 positions k = 0..K-1 in order; x_k is accepted iff acc_u[k] < min(1, p_k(x_k)/q_k(x_k)),
 *      and the first rejection ends the block;
 *   S2 at the first rejection k*, the next token is drawn from the residual
 *      r(v) = max(p_k*(v) - q_k*(v), 0) / sum_w max(p_k*(w) - q_k*(w), 0) by inverse CDF over
 *      increasing v with one uniform b: the first v whose inclusive prefix sum of the
 *      unnormalised residual exceeds b * sum r (clamped to the last v with r > 0);
 *   S3 if all K tokens are accepted, the next token is the bonus draw from p_K (the Gumbel-max
 *      of the round, reading R7); *bonus_gap then receives its top-2 key gap (+inf otherwise).
 * p and q are temperature-scaled softmaxes as in the round (R2). Outputs: *n_acc in 0..K and
 * *next the token that follows the accepted ones. *acc_gap = min over the examined positions
 * of |acc_u[k] - min(1, p/q)|. For a residual draw with target t = b sum r landing in
 * (C_lo, C_hi] of the chosen token: res[0] = (t - C_lo) / sum r and res[1] = (C_hi - t) / sum r
 * (distances to the two boundaries), nb[0] / nb[1] the nearest tokens with positive residual
 * below / above the chosen one (-1 if none). Without a residual draw res = {1, 1}, nb = {-1, -1}.
 */
static void sd_verify_particle(int32_t K, int64_t V, int64_t ld, int32_t dtype,
                               const char *tgt, const char *dft, const int32_t *tok, float Tf,
                               const float *gumbel, const float *acc_u, float res_u,
                               int32_t *n_acc, int32_t *next, double *acc_gap, double *res,
                               int32_t *nb, double *bonus_gap)
{
    const size_t es = esize(dtype);
    const double T = (double)Tf;
    double agap = INFINITY;
    res[0] = res[1] = 1.0;
    nb[0] = nb[1] = -1;
    *bonus_gap = INFINITY;
    for (int32_t k = 0; k < K; ++k) {
        const char *zp = tgt + (size_t)k * (size_t)ld * es;
        const char *zq = dft + (size_t)k * (size_t)ld * es;
        double A = orc_row_logsumexp(zp, dtype, V, T);
        double B = orc_row_logsumexp(zq, dtype, V, T);
        int32_t x = tok[k];
        double ratio = exp((elem(zp, dtype, x) / T - A) - (elem(zq, dtype, x) / T - B));
        double m = ratio < 1.0 ? ratio : 1.0;
        double d = fabs((double)acc_u[k] - m);
        if (d < agap)
            agap = d;
        if ((double)acc_u[k] < m)
            continue;
        /* first rejection: residual draw */
        double R = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double r = exp(elem(zp, dtype, v) / T - A) - exp(elem(zq, dtype, v) / T - B);
            if (r > 0.0)
                R += r;
        }
        double target = (double)res_u * R;
        double C = 0.0, lo = 0.0, hi = 0.0;
        int32_t pick = -1, last = -1, before = -1, after = -1;
        for (int64_t v = 0; v < V; ++v) {
            double r = exp(elem(zp, dtype, v) / T - A) - exp(elem(zq, dtype, v) / T - B);
            if (r <= 0.0)
                continue;
            if (pick >= 0) {
                after = (int32_t)v;
                break;
            }
            double prev_c = C;
            C += r;
            if (target < C) {
                pick = (int32_t)v;
                before = last;
                lo = prev_c;
                hi = C;
            }
            last = (int32_t)v;
        }
        if (pick < 0) {            /* rounding past the end: the last token with r > 0 */
            pick = last;
            lo = hi = C;
        }
        *n_acc = k;
        *next = pick >= 0 ? pick : 0;
        *acc_gap = agap;
        if (R > 0.0) {
            res[0] = (target - lo) / R;
            res[1] = (hi - target) / R;
        } else {
            res[0] = res[1] = 0.0;
        }
        nb[0] = before;
        nb[1] = after;
        return;
    }
    *n_acc = K;
    *next = orc_row_gumbel_argmax(tgt + (size_t)K * (size_t)ld * es, dtype, gumbel, V, Tf,
                                  bonus_gap);
    *acc_gap = agap;
}

/*
 * sd_verify_particle over a batch: R requests x N particles, each an independent sequence.
 * Layouts as in orc_round; acc_u [R][N][K], res_u [R][N]; outputs [R][N], res and nb [R][N][2],
 * bonus_gap [R][N].
 */
void orc_sd_verify(int32_t R, int32_t N, int32_t K, int64_t V, int64_t ld, int32_t dtype,
                   const void *target, const void *draft, const int32_t *tokens,
                   const float *temperature, const float *gumbel, const float *acc_u,
                   const float *res_u, int32_t *n_acc, int32_t *next, double *acc_gap,
                   double *res, int32_t *nb, double *bonus_gap)
{
    const size_t es = esize(dtype);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < (int64_t)R * N; ++ri) {
        int64_t r = ri / N;
        sd_verify_particle(K, V, ld, dtype,
                           (const char *)target + (size_t)(ri * (K + 1)) * (size_t)ld * es,
                           (const char *)draft + (size_t)(ri * K) * (size_t)ld * es,
                           tokens + (size_t)ri * K, temperature[r], gumbel + (size_t)ri * ld,
                           acc_u + (size_t)ri * K, res_u[ri], &n_acc[ri], &next[ri],
                           &acc_gap[ri], res + 2 * (size_t)ri, nb + 2 * (size_t)ri,
                           &bonus_gap[ri]);
    }
}

/*
 * Gumbel-Top-K: k distinct tokens drawn without replacement from softmax(z/T) in one step,
 * as the STAND page describes for drafting (method item 2: add Gumbel noise to the
 * log-probabilities and keep the indices of the k largest sums; the noise is precomputed and
 * cached). Keys as for the bonus token (reading R7), key_v = z_v/T + G_v in double; the k
 * tokens come out in decreasing key order, equal keys in increasing index. out_keys and
 * out_gaps ([rows][k], may be NULL) receive the keys and, for rank j, key_j - key_(j+1), the
 * gap to the next rank (+inf after the last token when k == V). k <= V.
 */
typedef struct {
    double key;
    int32_t idx;
} orc_kv;

static int kv_order(const void *a, const void *b)
{
    const orc_kv *x = (const orc_kv *)a, *y = (const orc_kv *)b;
    if (x->key > y->key)
        return -1;
    if (x->key < y->key)
        return 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);
}

void orc_gumbel_topk(int64_t rows, int64_t V, int64_t ld, int32_t dtype, const void *logits,
                     const float *temperature, const float *gumbel, int32_t k,
                     int32_t *out_tokens, double *out_keys, double *out_gaps)
{
    const size_t es = esize(dtype);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const char *z = (const char *)logits + (size_t)r * (size_t)ld * es;
        const float *g = gumbel + (size_t)r * (size_t)ld;
        const double t = (double)temperature[r];
        orc_kv *kv = malloc(sizeof(orc_kv) * (size_t)V);
        for (int64_t v = 0; v < V; ++v) {
            kv[v].key = elem(z, dtype, v) / t + (double)g[v];
            kv[v].idx = (int32_t)v;
        }
        qsort(kv, (size_t)V, sizeof(orc_kv), kv_order);
        for (int32_t j = 0; j < k; ++j) {
            out_tokens[(size_t)r * k + j] = kv[j].idx;
            if (out_keys)
                out_keys[(size_t)r * k + j] = kv[j].key;
            if (out_gaps)
                out_gaps[(size_t)r * k + j] = j + 1 < V ? kv[j].key - kv[j + 1].key : INFINITY;
        }
        free(kv);
    }
}

/*
 * Bonus token drawn after resampling, the alternative to drawing it per original particle
 * inside the pass (the SMC-SD page, section 2, emits K + 1 tokens a round without saying when
 * the last one is drawn). Reading: new slot j of request r draws from the target's bonus row
 * of its ancestor, row K of particle ancestors[r][j], with its own noise row gumbel[r][j],
 * by the same Gumbel-max key as the in-pass bonus (STAND page, method item 2, k = 1).
 * bonus [R][N] out; gap [R][N] optional (key(best) - key(second)). Returns -1 if an
 * ancestor is outside [0, N) (that slot's bonus is -1), else 0.
 */
int32_t orc_bonus_resampled(int32_t R, int32_t N, int32_t K, int64_t V, int64_t ld, int32_t dtype,
                            const void *target, const float *temperature,
                            const int32_t *ancestors, const float *gumbel, int32_t *bonus,
                            double *gap)
{
    const size_t es = esize(dtype);
    int32_t err = 0;
    for (int64_t rj = 0; rj < (int64_t)R * N; ++rj) {
        int64_t r = rj / N;
        int32_t a = ancestors[rj];
        if (a < 0 || a >= N) {
            bonus[rj] = -1;
            err = -1;
            continue;
        }
        const char *zb = (const char *)target + (size_t)(((r * N + a) * (K + 1) + K) * ld) * es;
        bonus[rj] = orc_row_gumbel_argmax(zb, dtype, gumbel + (size_t)rj * ld, V, temperature[r],
                                          gap ? &gap[rj] : NULL);
    }
    return err;
}

/*
 * Page lifecycle between rounds (the steps around the SMC-SD round: the page says duplicated
 * particles share KV pages by copying page metadata and exchanging pointers, section 2; a
 * shared page that will be written must then be copied first, and pages nobody references
 * return to the pool). The pages fix none of this; readings P1-P4:
 *   P1 a page's refcount is -1 while it is free (on the free list) and otherwise counts the
 *      table entries naming it; the free list is a stack of page ids, popped from the top;
 *   P2 release: every page with refcount 0 becomes free (refcount -1), pushed in increasing
 *      page id;
 *   P3 copy-on-write of the tail: if a request's length is not a multiple of page_size, its
 *      last (partly filled) column will be written next; there, the first particle (lowest j)
 *      naming a page keeps it, and every later particle naming the same page gets a fresh
 *      page (popped), a copy of the page's KV bytes, and refcount 1, the shared page losing
 *      one reference each time;
 *   P4 append: the columns the request's new length needs beyond the old one get fresh
 *      pages, particle by particle (j ascending), column by column.
 * Pops happen request by request, within a request first every copy (j ascending), then every
 * append (j, then column ascending). If the free list runs dry, the remaining entries stay -1
 * and -3 is returned.
 * Layouts: pt [R][N][P] int32, refcount / free_ids [num_pages], kv [kv_count][num_pages]
 * [page_bytes]: a page id names the same page in every one of the kv_count KV tensors (one
 * per layer and per K / V), and a copy copies it in all of them. With token_rows (a token
 * pool's layout: a page is page_size rows of page_bytes / page_size bytes, in token order)
 * a copy moves only the rows the tail holds, len_before mod page_size of them; the rest of
 * the destination page keeps its bytes (the next round writes them).
 */
int32_t orc_pages_advance(int32_t R, int32_t N, int32_t P, int32_t page_size,
                          const int32_t *len_before, const int32_t *len_after, int32_t *pt,
                          int32_t num_pages, int32_t *refcount, int32_t *free_ids,
                          int32_t *n_free, uint8_t *kv, int64_t page_bytes, int32_t kv_count,
                          int32_t token_rows)
{
    const size_t tensor_bytes = (size_t)num_pages * (size_t)page_bytes;
    int32_t err = 0;
    /* P2 */
    for (int32_t p = 0; p < num_pages; ++p) {
        if (refcount[p] == 0) {
            refcount[p] = -1;
            free_ids[(*n_free)++] = p;
        }
    }
    for (int32_t r = 0; r < R; ++r) {
        int32_t *row0 = pt + (size_t)r * N * P;
        /* P3 */
        int32_t lb = len_before[r];
        if (lb > 0 && lb % page_size != 0) {
            int32_t c = (lb - 1) / page_size;
            size_t copy_bytes = token_rows ? (size_t)(lb % page_size) * (size_t)(page_bytes / page_size)
                                           : (size_t)page_bytes;
            for (int32_t j = 0; j < N; ++j) {
                int32_t p = row0[(size_t)j * P + c];
                if (p < 0)
                    continue;
                int shared = 0;
                for (int32_t jj = 0; jj < j; ++jj)
                    if (row0[(size_t)jj * P + c] == p)
                        shared = 1;
                if (!shared)
                    continue;
                if (*n_free == 0) {
                    err = -3;
                    row0[(size_t)j * P + c] = -1;
                    refcount[p] -= 1;
                    continue;
                }
                int32_t q = free_ids[--(*n_free)];
                for (int32_t t = 0; t < kv_count; ++t)
                    memcpy(kv + t * tensor_bytes + (size_t)q * (size_t)page_bytes,
                           kv + t * tensor_bytes + (size_t)p * (size_t)page_bytes, copy_bytes);
                row0[(size_t)j * P + c] = q;
                refcount[p] -= 1;
                refcount[q] = 1;
            }
        }
        /* P4 */
        int32_t c0 = (lb + page_size - 1) / page_size;
        int32_t c1 = (len_after[r] + page_size - 1) / page_size;
        for (int32_t j = 0; j < N; ++j) {
            for (int32_t c = c0; c < c1 && c < P; ++c) {
                if (*n_free == 0) {
                    err = -3;
                    row0[(size_t)j * P + c] = -1;
                    continue;
                }
                int32_t q = free_ids[--(*n_free)];
                row0[(size_t)j * P + c] = q;
                refcount[q] = 1;
            }
        }
    }
    return err;
}

/* Threads OpenMP would use for the parallel loops above (1 when built without OpenMP). */
int32_t orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
