/*
 * Plain serial fp64 oracle for the finite-automaton-constrained sampler.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * calls it.  It shares no code, header or table with the GPU library.
 *
 * Sources (two summaries of one paper, "Constrained Decoding for Diffusion
 * Language Models via Efficient Inference over Finite Automata"):
 *   [P1] the paperfeed.app English summary, sections "The insight: the
 *        constraint is a hidden Markov model" and "The scan trick: log-depth
 *        exact sampling";
 *   [P2] the papernotes.org summary, 关键设计 1 (mean-field emission
 *        reweighting), 关键设计 2 (log-depth tree sampling) and 关键设计 3
 *        (constrained-marginal remasking).
 *
 * Model.  An automaton (S, V, delta, s0, F) with edges e = (src, dst, label)
 * is a chain model whose transitions are fixed and whose emissions are
 * reweighted by the per-position token probabilities p[i][v] [P1 HMM,
 * P2 关键设计 1].  Summing the edge paths over states gives per-position
 * weights M_i[a][b] = sum over edges a->b of sum_{v in label} p[i][v]; an
 * NFA string is weighted by its number of accepting paths [P1 "Arbitrary
 * schedules and NFAs"].  Everything below is computed in fp64, serially, in
 * plain loops; no blocking, no reordering beyond the stated definitions.
 *
 * Conventions (readings of the pages where they are silent):
 *  - tokens are 0-based, position i sits between boundary states z_i and
 *    z_{i+1}; z_0 = s0; L is padded to Lpad = 2^ceil(log2 L) with identity
 *    transitions so every span of the tree is 2^k long;
 *  - the sampler draws z_Lpad over F, then midpoints level by level, then
 *    the tokens, each by inverse CDF over ascending candidate ids: the
 *    chosen index is the smallest j with w_j > 0 and C_j > u*T, where C is
 *    the inclusive prefix sum and T its last element;
 *  - u = (r0 >> 8) * 2^-24 with r0 the first word of Philox4x32-10 keyed by
 *    the 64-bit seed and counter (b, level, node, 0); level 0 is the root
 *    draw, levels 1..K the midpoint levels (node = heap index - 2^(level-1)),
 *    level K+1 the token stage (node = position).
 *  - range labels: sums over [lo, hi) are taken as differences of an fp64
 *    running prefix sum of the row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_INFEASIBLE 1
#define OR_UNDERFLOW 2
#define OR_BADARG 3

typedef struct {
    int32_t S, V, start, n_accept;
    const int32_t *accept;
    int64_t E;
    const int32_t *src, *dst;
    const int64_t *label_off;
    const int32_t *label_tok; /* token ids, or flat (lo, hi) pairs */
    int32_t ranges;
} or_aut;

/* ------------------------------------------------------------------ Philox
 * Philox4x32 with 10 rounds, written from its published definition (Salmon,
 * Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11):
 * each round multiplies counter words 0 and 2 by two fixed 32-bit constants,
 * keeps both 32-bit halves of the products, and mixes the high halves with the
 * other two counter words and the round key; the key is advanced by the two
 * Weyl constants between rounds. */
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

double or_uniform(uint64_t seed, uint32_t b, uint32_t level, uint32_t node)
{
    uint32_t ctr[4] = {b, level, node, 0u};
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t r[4];
    or_philox4x32_10(ctr, key, r);
    return (double)(r[0] >> 8) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------- emission weights
 * [P2 关键设计 1]: reweighting each emission by p and summing over the tokens
 * of an edge gives the edge's weight at position i; M_i[a][b] is the sum of
 * the weights of the edges a->b.  W[i*E + e] = sum_{v in label(e)} p[i][v]. */
int or_edge_weights(const or_aut *A, const float *p, int32_t L, double *W)
{
    double *pre = NULL;
    if (A->ranges) {
        pre = (double *)malloc(sizeof(double) * ((size_t)A->V + 1));
        if (!pre) return OR_BADARG;
    }
    for (int32_t i = 0; i < L; ++i) {
        const float *row = p + (size_t)i * A->V;
        if (A->ranges) {
            pre[0] = 0.0;
            for (int32_t v = 0; v < A->V; ++v) pre[v + 1] = pre[v] + (double)row[v];
        }
        for (int64_t e = 0; e < A->E; ++e) {
            double s = 0.0;
            if (A->ranges) {
                for (int64_t k = A->label_off[e]; k + 1 < A->label_off[e + 1]; k += 2)
                    s += pre[A->label_tok[k + 1]] - pre[A->label_tok[k]];
            } else {
                for (int64_t k = A->label_off[e]; k < A->label_off[e + 1]; ++k)
                    s += (double)row[A->label_tok[k]];
            }
            W[(size_t)i * A->E + e] = s;
        }
    }
    free(pre);
    return OR_OK;
}

/* Dense M_i from the edge weights (small automata only). */
void or_dense_M(const or_aut *A, const double *W, int32_t i, double *M)
{
    memset(M, 0, sizeof(double) * (size_t)A->S * A->S);
    for (int64_t e = 0; e < A->E; ++e)
        M[(size_t)A->src[e] * A->S + A->dst[e]] += W[(size_t)i * A->E + e];
}

/* one forward step v_out = v_in * M_i (M_i = identity beyond L) */
static void step_forward(const or_aut *A, const double *W, int32_t L, int32_t i,
                         const double *vin, double *vout)
{
    if (i >= L) { memcpy(vout, vin, sizeof(double) * A->S); return; }
    memset(vout, 0, sizeof(double) * A->S);
    for (int64_t e = 0; e < A->E; ++e)
        vout[A->dst[e]] += vin[A->src[e]] * W[(size_t)i * A->E + e];
}

/* one backward step v_out = M_i * v_in */
static void step_backward(const or_aut *A, const double *W, int32_t L, int32_t i,
                          const double *vin, double *vout)
{
    if (i >= L) { memcpy(vout, vin, sizeof(double) * A->S); return; }
    memset(vout, 0, sizeof(double) * A->S);
    for (int64_t e = 0; e < A->E; ++e)
        vout[A->src[e]] += W[(size_t)i * A->E + e] * vin[A->dst[e]];
}

/* rescale by the maximum; returns ln(max) or -inf if the vector is zero */
static double rescale(double *v, int32_t n)
{
    double mx = 0.0;
    for (int32_t k = 0; k < n; ++k) if (v[k] > mx) mx = v[k];
    if (mx == 0.0) return -INFINITY;
    for (int32_t k = 0; k < n; ++k) v[k] /= mx;
    return log(mx);
}

/* ------------------------------------------------------ forward-backward
 * [P1 HMM]: exact normalization, marginals and sampling of the reweighted
 * chain follow from forward-backward message passing.  Scaled messages:
 * alpha_0 = e_{s0}, alpha_{i+1} = alpha_i M_i / kappa; beta_L = 1_F,
 * beta_i = M_i beta_{i+1} / kappa'.  alog/blog hold the accumulated ln kappa.
 * log Z = alog_L + ln sum_{f in F} alpha_L[f]. */
int or_forward_backward(const or_aut *A, const double *W, int32_t L,
                        double *alpha, double *alog, double *beta, double *blog,
                        double *logZ)
{
    const int32_t S = A->S;
    int status = OR_OK;
    memset(alpha, 0, sizeof(double) * S);
    alpha[A->start] = 1.0;
    alog[0] = 0.0;
    for (int32_t i = 0; i < L; ++i) {
        step_forward(A, W, L, i, alpha + (size_t)i * S, alpha + (size_t)(i + 1) * S);
        double lk = rescale(alpha + (size_t)(i + 1) * S, S);
        if (lk == -INFINITY) status = OR_INFEASIBLE;
        alog[i + 1] = alog[i] + lk;
    }
    double zf = 0.0;
    for (int32_t k = 0; k < A->n_accept; ++k) zf += alpha[(size_t)L * S + A->accept[k]];
    if (zf == 0.0) status = OR_INFEASIBLE;
    *logZ = (status == OR_OK) ? alog[L] + log(zf) : -INFINITY;

    double *bl = beta + (size_t)L * S;
    memset(bl, 0, sizeof(double) * S);
    for (int32_t k = 0; k < A->n_accept; ++k) bl[A->accept[k]] = 1.0;
    blog[L] = 0.0;
    for (int32_t i = L - 1; i >= 0; --i) {
        step_backward(A, W, L, i, beta + (size_t)(i + 1) * S, beta + (size_t)i * S);
        double lk = rescale(beta + (size_t)i * S, S);
        blog[i] = blog[i + 1] + lk;
    }
    return status;
}

/* ------------------------------------------------------ constrained marginals
 * [P2 关键设计 3], [P1 "Two immediate bonuses"]: the constrained per-token
 * marginal is q[i][v] = p[i][v] * sum over edges e containing v of
 * alpha_i[src e] beta_{i+1}[dst e], normalized over v.  Computed for the
 * positions listed in pos[0..npos); q is [npos][V].  lognorm[k] receives
 * ln(normalizer) + alog_i + blog_{i+1}, which equals log Z in exact
 * arithmetic.  conf (optional): mode 0 = q at tokens[i] (the sampled
 * token's constrained probability), mode 1 = sum_v q ln q (0 ln 0 = 0),
 * mode 2 = p at tokens[i] (the unconstrained probability of the sampled
 * token, the comparison score of [P2 消融实验]). */
int or_marginals(const or_aut *A, const float *p, int32_t L, const double *alpha,
                 const double *alog, const double *beta, const double *blog,
                 const int32_t *pos, int32_t npos, double *q, double *lognorm,
                 const int32_t *tokens, int32_t conf_mode, double *conf)
{
    const int32_t S = A->S, V = A->V;
    double *r = (double *)malloc(sizeof(double) * V);
    if (!r) return OR_BADARG;
    for (int32_t k = 0; k < npos; ++k) {
        int32_t i = pos[k];
        if (i < 0 || i >= L) { free(r); return OR_BADARG; }
        const double *al = alpha + (size_t)i * S;
        const double *be = beta + (size_t)(i + 1) * S;
        memset(r, 0, sizeof(double) * V);
        for (int64_t e = 0; e < A->E; ++e) {
            double g = al[A->src[e]] * be[A->dst[e]];
            if (g == 0.0) continue;
            if (A->ranges) {
                for (int64_t t = A->label_off[e]; t + 1 < A->label_off[e + 1]; t += 2)
                    for (int32_t v = A->label_tok[t]; v < A->label_tok[t + 1]; ++v) r[v] += g;
            } else {
                for (int64_t t = A->label_off[e]; t < A->label_off[e + 1]; ++t)
                    r[A->label_tok[t]] += g;
            }
        }
        const float *row = p + (size_t)i * V;
        double nrm = 0.0;
        for (int32_t v = 0; v < V; ++v) nrm += (double)row[v] * r[v];
        double *qk = q + (size_t)k * V;
        for (int32_t v = 0; v < V; ++v) qk[v] = nrm > 0.0 ? (double)row[v] * r[v] / nrm : 0.0;
        lognorm[k] = nrm > 0.0 ? log(nrm) + alog[i] + blog[i + 1] : -INFINITY;
        if (conf) {
            if (conf_mode == 0) {
                conf[k] = (tokens && nrm > 0.0) ? qk[tokens[i]] : -INFINITY;
            } else if (conf_mode == 2) {
                conf[k] = (tokens && nrm > 0.0 && tokens[i] >= 0) ? (double)row[tokens[i]]
                                                                  : -INFINITY;
            } else {
                double h = 0.0;
                for (int32_t v = 0; v < V; ++v) if (qk[v] > 0.0) h += qk[v] * log(qk[v]);
                conf[k] = nrm > 0.0 ? h : -INFINITY;
            }
        }
    }
    free(r);
    return OR_OK;
}

/* ------------------------------------------------------------- draws */

/* inverse CDF: smallest j with w_j > 0 and C_j > u*T (C inclusive prefix,
 * T = C_last); -1 if T == 0 */
static int32_t icdf(const double *w, int32_t n, double u)
{
    double T = 0.0;
    for (int32_t j = 0; j < n; ++j) T += w[j];
    if (!(T > 0.0)) return -1;
    double target = u * T, c = 0.0;
    int32_t last = -1;
    for (int32_t j = 0; j < n; ++j) {
        c += w[j];
        if (w[j] > 0.0) {
            last = j;
            if (c > target) return j;
        }
    }
    return last;
}

static int32_t ilog2_pad(int32_t L, int32_t *Lpad)
{
    int32_t K = 0, P = 1;
    while (P < L) { P <<= 1; ++K; }
    *Lpad = P;
    return K;
}

/* count c(a, v, b) of edges a->b whose label contains v */
static int32_t edge_count(const or_aut *A, int32_t a, int32_t v, int32_t b)
{
    int32_t c = 0;
    for (int64_t e = 0; e < A->E; ++e) {
        if (A->src[e] != a || A->dst[e] != b) continue;
        if (A->ranges) {
            for (int64_t t = A->label_off[e]; t + 1 < A->label_off[e + 1]; t += 2)
                if (v >= A->label_tok[t] && v < A->label_tok[t + 1]) { ++c; break; }
        } else {
            for (int64_t t = A->label_off[e]; t < A->label_off[e + 1]; ++t)
                if (A->label_tok[t] == v) { ++c; break; }
        }
    }
    return c;
}

/* token weights w[v] = p[i][v] * c(a, v, b) over all v */
static void token_weights(const or_aut *A, const float *row, int32_t a, int32_t b, double *w)
{
    memset(w, 0, sizeof(double) * A->V);
    for (int64_t e = 0; e < A->E; ++e) {
        if (A->src[e] != a || A->dst[e] != b) continue;
        if (A->ranges) {
            for (int64_t t = A->label_off[e]; t + 1 < A->label_off[e + 1]; t += 2)
                for (int32_t v = A->label_tok[t]; v < A->label_tok[t + 1]; ++v) w[v] += 1.0;
        } else {
            for (int64_t t = A->label_off[e]; t < A->label_off[e + 1]; ++t)
                w[A->label_tok[t]] += 1.0;
        }
    }
    for (int32_t v = 0; v < A->V; ++v) if (w[v] != 0.0) w[v] *= (double)row[v];
}

/* row chain e_{a} M_l ... M_{m-1} and column chain M_m ... M_{r-1} e_{b},
 * each rescaled after every step (a positive factor per vector does not
 * change the normalized midpoint weights). */
static void span_row(const or_aut *A, const double *W, int32_t L, int32_t a, int32_t l,
                     int32_t m, double *v, double *tmp)
{
    memset(v, 0, sizeof(double) * A->S);
    v[a] = 1.0;
    for (int32_t i = l; i < m; ++i) {
        step_forward(A, W, L, i, v, tmp);
        memcpy(v, tmp, sizeof(double) * A->S);
        rescale(v, A->S);
    }
}

static void span_col(const or_aut *A, const double *W, int32_t L, int32_t b, int32_t m,
                     int32_t r, double *v, double *tmp)
{
    memset(v, 0, sizeof(double) * A->S);
    v[b] = 1.0;
    for (int32_t i = r - 1; i >= m; --i) {
        step_backward(A, W, L, i, v, tmp);
        memcpy(v, tmp, sizeof(double) * A->S);
        rescale(v, A->S);
    }
}

/* Replay record of one draw, filled in by the shared walker below. */
typedef struct {
    int64_t n_draws, n_hard, n_near, n_margin, first_hard;
} or_replay_report;

/* Boundary distance between two choices j1 < j2 of a draw: the largest
 * |C_k/T - u| over the CDF boundaries k in [j1, j2).  Another implementation
 * whose fp32 prefix sums moved every one of those boundaries across u picks
 * j2 where this one picks j1 (or the reverse); that is a rounding effect
 * only when all of them lie close to u.  A candidate of real weight between
 * the two choices puts a boundary far from u, and the draw is then wrong. */
static double boundary_gap(const double *w, int32_t n, double u, int32_t j1, int32_t j2)
{
    double T = 0.0;
    for (int32_t j = 0; j < n; ++j) T += w[j];
    double c = 0.0, worst = 0.0;
    for (int32_t j = 0; j < j2 && j < n; ++j) {
        c += w[j];
        if (j >= j1) {
            double d = fabs(c / T - u);
            if (d > worst) worst = d;
        }
    }
    return worst;
}

/* Judge one draw.  chosen = the candidate index the other implementation
 * picked (or -1 to accept the oracle's own choice).  Returns the index to
 * condition on. */
static int32_t judge(const double *w, int32_t n, double u, int32_t chosen, int64_t draw_id,
                     or_replay_report *rep)
{
    int32_t mine = icdf(w, n, u);
    if (rep) rep->n_draws++;
    if (chosen < 0 || !rep) return mine;
    if (chosen == mine) return chosen;
    if (chosen >= n || mine < 0 || !(w[chosen] > 0.0)) {
        rep->n_hard++;
        if (rep->first_hard < 0) rep->first_hard = draw_id;
        return chosen;
    }
    int32_t j1 = chosen < mine ? chosen : mine, j2 = chosen < mine ? mine : chosen;
    double gap = boundary_gap(w, n, u, j1, j2);
    if (gap <= 1e-6) rep->n_near++;
    else {
        rep->n_hard++;
        if (gap <= 1e-4) rep->n_margin++;
        if (rep->first_hard < 0) rep->first_hard = draw_id;
    }
    return chosen;
}

/* One draw judged on its own, for tests: weights w[0..n), uniform u, and the
 * index another implementation chose.  out[0] = the oracle's own choice
 * (-1 when the weights vanish), out[1] = 0 same choice, 1 NEAR, 2 HARD,
 * out[2] = 1 when a HARD draw lies within 1e-4 of the boundaries (the
 * fp32-margin count). */
void or_judge_draw(const double *w, int32_t n, double u, int32_t chosen, int32_t out[3])
{
    or_replay_report rep = {0, 0, 0, 0, -1};
    out[0] = icdf(w, n, u);
    judge(w, n, u, chosen, 0, &rep);
    out[1] = rep.n_hard ? 2 : (rep.n_near ? 1 : 0);
    out[2] = rep.n_margin ? 1 : 0;
}

/* ------------------------------------------------- tree-order sampler
 * [P1 "The scan trick"], [P2 关键设计 2]: draw the final boundary state from
 * its marginal (the start state is pinned), then for every segment [l, r)
 * with both boundary states known draw the midpoint state m = (l+r)/2 with
 * weight P_{l->m}[z_l, z_m] * P_{m->r}[z_m, z_r], level by level, and finally
 * every token given its two boundary states.  The span rows and columns are
 * evaluated as fp64 vector chains.
 *
 * Walker shared by the sampler (z_in = NULL) and the replay verifier
 * (z_in/x_in = another implementation's states and tokens, original ids,
 * states of length L+1).  Outputs z_out [L+1], x_out [L]. */
static int tree_walk(const or_aut *A, const float *p, const double *W, int32_t L, uint64_t seed,
                     uint32_t b, const int32_t *z_in, const int32_t *x_in, int32_t *z_out,
                     int32_t *x_out, or_replay_report *rep)
{
    const int32_t S = A->S;
    int32_t Lpad;
    int32_t K = ilog2_pad(L, &Lpad);
    int32_t *z = (int32_t *)malloc(sizeof(int32_t) * ((size_t)Lpad + 1));
    double *row = (double *)malloc(sizeof(double) * S);
    double *col = (double *)malloc(sizeof(double) * S);
    double *tmp = (double *)malloc(sizeof(double) * S);
    double *w = (double *)malloc(sizeof(double) * (S > A->V ? S : A->V));
    int status = OR_OK;
    if (!z || !row || !col || !tmp || !w) { status = OR_BADARG; goto done; }
    for (int32_t k = 0; k <= Lpad; ++k) z[k] = -1;
    z[0] = A->start;

    /* root: weights over accepting states, ascending id */
    span_row(A, W, L, A->start, 0, Lpad, row, tmp);
    {
        int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (A->n_accept > 0 ? A->n_accept : 1));
        memcpy(acc, A->accept, sizeof(int32_t) * A->n_accept);
        for (int32_t a1 = 1; a1 < A->n_accept; ++a1)  /* insertion sort */
            for (int32_t a2 = a1; a2 > 0 && acc[a2 - 1] > acc[a2]; --a2) {
                int32_t t = acc[a2]; acc[a2] = acc[a2 - 1]; acc[a2 - 1] = t;
            }
        for (int32_t k = 0; k < A->n_accept; ++k) w[k] = row[acc[k]];
        int32_t chosen = -1;
        if (z_in) {
            chosen = -2;
            for (int32_t k = 0; k < A->n_accept; ++k) if (acc[k] == z_in[L]) chosen = k;
            if (chosen == -2) chosen = A->n_accept; /* not accepting: judged hard */
        }
        int32_t j = judge(w, A->n_accept, or_uniform(seed, b, 0, 0), chosen, 0, rep);
        if (j < 0) { status = OR_INFEASIBLE; free(acc); goto done; }
        z[Lpad] = (j < A->n_accept) ? acc[j] : (z_in ? z_in[L] : -1);
        free(acc);
    }
    /* midpoint levels */
    for (int32_t lev = 1; lev <= K; ++lev) {
        int32_t span = Lpad >> (lev - 1);
        int32_t nn = 1 << (lev - 1);
        for (int32_t node = 0; node < nn; ++node) {
            int32_t l = node * span, r = l + span, m = l + span / 2;
            if (z[l] < 0 || z[r] < 0) { status = OR_UNDERFLOW; goto done; }
            span_row(A, W, L, z[l], l, m, row, tmp);
            span_col(A, W, L, z[r], m, r, col, tmp);
            for (int32_t j = 0; j < S; ++j) w[j] = row[j] * col[j];
            int32_t chosen = -1;
            if (z_in) chosen = (m <= L) ? z_in[m] : z_in[L];
            int32_t j = judge(w, S, or_uniform(seed, b, (uint32_t)lev, (uint32_t)node), chosen,
                              ((int64_t)lev << 32) | node, rep);
            if (j < 0) { status = OR_UNDERFLOW; goto done; }
            z[m] = j;
        }
    }
    /* tokens */
    for (int32_t i = 0; i < L; ++i) {
        token_weights(A, p + (size_t)i * A->V, z[i], z[i + 1], w);
        int32_t chosen = x_in ? x_in[i] : -1;
        int32_t j = judge(w, A->V, or_uniform(seed, b, (uint32_t)(K + 1), (uint32_t)i), chosen,
                          ((int64_t)(K + 1) << 32) | i, rep);
        if (j < 0) { status = OR_UNDERFLOW; goto done; }
        if (x_out) x_out[i] = j;
    }
    if (z_out) for (int32_t k = 0; k <= L; ++k) z_out[k] = z[k];
done:
    free(z); free(row); free(col); free(tmp); free(w);
    return status;
}

int or_sample_tree(const or_aut *A, const float *p, const double *W, int32_t L, uint64_t seed,
                   uint32_t b, int32_t *states, int32_t *tokens)
{
    return tree_walk(A, p, W, L, seed, b, NULL, NULL, states, tokens, NULL);
}

/* [P1 "The scan trick"]: replay another implementation's draws under the same
 * uniforms; a differing choice is NEAR when every CDF boundary between the
 * two choices lies within 1e-6 of u, else HARD (also HARD: a zero-weight
 * choice). */
int or_replay_verify(const or_aut *A, const float *p, const double *W, int32_t L, uint64_t seed,
                     uint32_t b, const int32_t *states, const int32_t *tokens, int64_t report[5])
{
    or_replay_report rep = {0, 0, 0, 0, -1};
    int st = tree_walk(A, p, W, L, seed, b, states, tokens, NULL, NULL, &rep);
    report[0] = rep.n_draws; report[1] = rep.n_hard; report[2] = rep.n_near;
    report[3] = rep.n_margin; report[4] = rep.first_hard;
    return st;
}

/* ------------------------------------------------------------------ FFBS
 * Textbook forward-filtering backward-sampling of the same chain, used only
 * as an independent distributional cross-check of the tree-order sampler.
 * u holds L+1 + L uniforms supplied by the caller (states then tokens). */
int or_ffbs(const or_aut *A, const float *p, const double *W, int32_t L, const double *alpha,
            const double *u, int32_t *states, int32_t *tokens)
{
    const int32_t S = A->S;
    double *w = (double *)malloc(sizeof(double) * (S > A->V ? S : A->V));
    if (!w) return OR_BADARG;
    memset(w, 0, sizeof(double) * S);
    for (int32_t k = 0; k < A->n_accept; ++k) w[A->accept[k]] = alpha[(size_t)L * S + A->accept[k]];
    int32_t j = icdf(w, S, u[0]);
    if (j < 0) { free(w); return OR_INFEASIBLE; }
    states[L] = j;
    for (int32_t i = L - 1; i >= 0; --i) {
        memset(w, 0, sizeof(double) * S);
        for (int64_t e = 0; e < A->E; ++e)
            if (A->dst[e] == states[i + 1])
                w[A->src[e]] += alpha[(size_t)i * S + A->src[e]] * W[(size_t)i * A->E + e];
        j = icdf(w, S, u[L - i]);
        if (j < 0) { free(w); return OR_UNDERFLOW; }
        states[i] = j;
    }
    for (int32_t i = 0; i < L; ++i) {
        token_weights(A, p + (size_t)i * A->V, states[i], states[i + 1], w);
        j = icdf(w, A->V, u[L + 1 + i]);
        if (j < 0) { free(w); return OR_UNDERFLOW; }
        tokens[i] = j;
    }
    free(w);
    return OR_OK;
}

/* c(a, v, b) for tests */
int32_t or_edge_count(const or_aut *A, int32_t a, int32_t v, int32_t b)
{
    return edge_count(A, a, v, b);
}

/* ======================================================= MAP decoding
 * Greedy (temperature 0) constrained decoding: the most probable accepted
 * string, argmax_x prod_i p[i][x_i] over x in C (paperfeed summary, "The
 * evidence": greedy decoding next to sampling; "Why constrained decoding
 * breaks for diffusion LMs": MAP inference over DFAs by dynamic
 * programming).  Readings: an NFA string counts once however many accepting
 * paths it has (every path of a string has the same product, so the maximum
 * over (string, path) pairs is the maximum over accepted strings); all
 * values are natural logs in fp64, log 0 = -inf.
 *
 * Max-times weights: Wm[i*E + e] = max_{v in label(e)} p[i][v] (0 for an
 * empty label). */
int or_map_weights(const or_aut *A, const float *p, int32_t L, double *Wm)
{
    for (int32_t i = 0; i < L; ++i) {
        const float *row = p + (size_t)i * A->V;
        for (int64_t e = 0; e < A->E; ++e) {
            double m = 0.0;
            if (A->ranges) {
                for (int64_t k = A->label_off[e]; k + 1 < A->label_off[e + 1]; k += 2)
                    for (int32_t v = A->label_tok[k]; v < A->label_tok[k + 1]; ++v)
                        if ((double)row[v] > m) m = (double)row[v];
            } else {
                for (int64_t k = A->label_off[e]; k < A->label_off[e + 1]; ++k)
                    if ((double)row[A->label_tok[k]] > m) m = (double)row[A->label_tok[k]];
            }
            Wm[(size_t)i * A->E + e] = m;
        }
    }
    return OR_OK;
}

static double lg(double x) { return x > 0.0 ? log(x) : -INFINITY; }

/* one max-plus step forward: vout[b] = max over edges a->b of vin[a] + ln Wm */
static void map_forward(const or_aut *A, const double *Wm, int32_t L, int32_t i,
                        const double *vin, double *vout)
{
    if (i >= L) { memcpy(vout, vin, sizeof(double) * A->S); return; }
    for (int32_t k = 0; k < A->S; ++k) vout[k] = -INFINITY;
    for (int64_t e = 0; e < A->E; ++e) {
        double t = vin[A->src[e]] + lg(Wm[(size_t)i * A->E + e]);
        if (t > vout[A->dst[e]]) vout[A->dst[e]] = t;
    }
}

/* one max-plus step backward: vout[a] = max over edges a->b of ln Wm + vin[b] */
static void map_backward(const or_aut *A, const double *Wm, int32_t L, int32_t i,
                         const double *vin, double *vout)
{
    if (i >= L) { memcpy(vout, vin, sizeof(double) * A->S); return; }
    for (int32_t k = 0; k < A->S; ++k) vout[k] = -INFINITY;
    for (int64_t e = 0; e < A->E; ++e) {
        double t = lg(Wm[(size_t)i * A->E + e]) + vin[A->dst[e]];
        if (t > vout[A->src[e]]) vout[A->src[e]] = t;
    }
}

/* Serial Viterbi: delta_0 = ln e_{s0}, delta_{i+1} = delta_i (max,+) ln M_i,
 * log-max = max_{f in F} delta_L[f] (-inf: no accepted string has positive
 * weight). */
int or_viterbi(const or_aut *A, const double *Wm, int32_t L, double *logmax)
{
    double *a = (double *)malloc(sizeof(double) * A->S), *b = (double *)malloc(sizeof(double) * A->S);
    if (!a || !b) { free(a); free(b); return OR_BADARG; }
    for (int32_t k = 0; k < A->S; ++k) a[k] = -INFINITY;
    a[A->start] = 0.0;
    for (int32_t i = 0; i < L; ++i) {
        map_forward(A, Wm, L, i, a, b);
        memcpy(a, b, sizeof(double) * A->S);
    }
    double m = -INFINITY;
    for (int32_t k = 0; k < A->n_accept; ++k) if (a[A->accept[k]] > m) m = a[A->accept[k]];
    *logmax = m;
    free(a); free(b);
    return m == -INFINITY ? OR_INFEASIBLE : OR_OK;
}

/* max-plus span row e_{a} M_l ... M_{m-1} and column M_m ... M_{r-1} e_{b} */
static void map_span_row(const or_aut *A, const double *Wm, int32_t L, int32_t a, int32_t l,
                         int32_t m, double *v, double *tmp)
{
    for (int32_t k = 0; k < A->S; ++k) v[k] = -INFINITY;
    v[a] = 0.0;
    for (int32_t i = l; i < m; ++i) {
        map_forward(A, Wm, L, i, v, tmp);
        memcpy(v, tmp, sizeof(double) * A->S);
    }
}

static void map_span_col(const or_aut *A, const double *Wm, int32_t L, int32_t b, int32_t m,
                         int32_t r, double *v, double *tmp)
{
    for (int32_t k = 0; k < A->S; ++k) v[k] = -INFINITY;
    v[b] = 0.0;
    for (int32_t i = r - 1; i >= m; --i) {
        map_backward(A, Wm, L, i, v, tmp);
        memcpy(v, tmp, sizeof(double) * A->S);
    }
}

/* argmax with the smallest index among equal maxima; -1 when all are -inf */
static int32_t argmax_first(const double *w, int32_t n)
{
    int32_t best = -1;
    for (int32_t j = 0; j < n; ++j)
        if (w[j] > -INFINITY && (best < 0 || w[j] > w[best])) best = j;
    return best;
}

/* the MAP token of position i between states a and b: argmax_v p[i][v] over
 * v with c(a, v, b) > 0, smallest v among equal values; -1 if none has p > 0 */
static int32_t map_token(const or_aut *A, const float *row, int32_t a, int32_t b, double *w)
{
    token_weights(A, row, a, b, w);   /* p[i][v] c(a, v, b) */
    int32_t best = -1;
    for (int32_t v = 0; v < A->V; ++v)
        if (w[v] > 0.0 && (best < 0 || (double)row[v] > (double)row[best])) best = v;
    return best;
}

/* Judge of one MAP decision: the other implementation chose `chosen`;
 * NEAR when its value equals the best up to fp64 rounding of the sums
 * (|best - value| <= 1e-9 max(1, |best|)), else HARD. */
static int32_t map_judge(const double *w, int32_t n, int32_t chosen, int64_t id,
                         or_replay_report *rep)
{
    int32_t mine = argmax_first(w, n);
    if (rep) rep->n_draws++;
    if (chosen < 0 || !rep) return mine;
    if (chosen == mine) return chosen;
    if (chosen >= n || mine < 0 || !(w[chosen] > -INFINITY) ||
        !(fabs(w[mine] - w[chosen]) <= 1e-9 * fmax(1.0, fabs(w[mine])))) {
        rep->n_hard++;
        if (rep->first_hard < 0) rep->first_hard = id;
    } else {
        rep->n_near++;
    }
    return chosen;
}

/* Tree-order MAP decoding [P1 "The scan trick", with max in place of sum]:
 * the final boundary state over F, then for every segment [l, r) with known
 * boundary states the midpoint m = (l+r)/2 maximizing
 * P_{l->m}[z_l][z_m] + P_{m->r}[z_m][z_r] (max-plus span products as vector
 * chains), level by level, then every token as the most probable token of
 * its edge; smallest id among equal values at every decision.  With z_in /
 * x_in (another implementation's states, original ids, and tokens) it
 * replays their decisions and judges each one instead. */
static int map_walk(const or_aut *A, const float *p, const double *Wm, int32_t L,
                    const int32_t *z_in, const int32_t *x_in, int32_t *z_out, int32_t *x_out,
                    double *logmax, or_replay_report *rep)
{
    const int32_t S = A->S;
    int32_t Lpad;
    int32_t K = ilog2_pad(L, &Lpad);
    int32_t *z = (int32_t *)malloc(sizeof(int32_t) * ((size_t)Lpad + 1));
    double *row = (double *)malloc(sizeof(double) * S);
    double *col = (double *)malloc(sizeof(double) * S);
    double *tmp = (double *)malloc(sizeof(double) * S);
    double *w = (double *)malloc(sizeof(double) * (S > A->V ? S : A->V));
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (A->n_accept > 0 ? A->n_accept : 1));
    int status = OR_OK;
    if (!z || !row || !col || !tmp || !w || !acc) { status = OR_BADARG; goto done; }
    for (int32_t k = 0; k <= Lpad; ++k) z[k] = -1;
    z[0] = A->start;
    memcpy(acc, A->accept, sizeof(int32_t) * A->n_accept);
    for (int32_t a1 = 1; a1 < A->n_accept; ++a1)
        for (int32_t a2 = a1; a2 > 0 && acc[a2 - 1] > acc[a2]; --a2) {
            int32_t t = acc[a2]; acc[a2] = acc[a2 - 1]; acc[a2 - 1] = t;
        }
    map_span_row(A, Wm, L, A->start, 0, Lpad, row, tmp);
    for (int32_t k = 0; k < A->n_accept; ++k) w[k] = row[acc[k]];
    {
        int32_t j0 = argmax_first(w, A->n_accept);
        if (logmax) *logmax = j0 >= 0 ? w[j0] : -INFINITY;
        int32_t chosen = -1;
        if (z_in) {
            chosen = A->n_accept;  /* not accepting: judged hard */
            for (int32_t k = 0; k < A->n_accept; ++k) if (acc[k] == z_in[L]) chosen = k;
        }
        int32_t j = map_judge(w, A->n_accept, chosen, 0, rep);
        if (j0 < 0) { status = OR_INFEASIBLE; goto done; }
        z[Lpad] = j < A->n_accept ? acc[j] : z_in[L];
    }
    for (int32_t lev = 1; lev <= K; ++lev) {
        int32_t span = Lpad >> (lev - 1), nn = 1 << (lev - 1);
        for (int32_t node = 0; node < nn; ++node) {
            int32_t l = node * span, r = l + span, m = l + span / 2;
            if (z[l] < 0 || z[r] < 0) { status = OR_UNDERFLOW; goto done; }
            map_span_row(A, Wm, L, z[l], l, m, row, tmp);
            map_span_col(A, Wm, L, z[r], m, r, col, tmp);
            for (int32_t j = 0; j < S; ++j) w[j] = row[j] + col[j];
            int32_t chosen = z_in ? ((m <= L) ? z_in[m] : z_in[L]) : -1;
            int32_t j = map_judge(w, S, chosen, ((int64_t)lev << 32) | node, rep);
            if (j < 0) { status = OR_UNDERFLOW; goto done; }
            z[m] = j;
        }
    }
    for (int32_t i = 0; i < L; ++i) {
        const float *prow = p + (size_t)i * A->V;
        int32_t t = map_token(A, prow, z[i], z[i + 1], w);
        if (t < 0) { status = OR_UNDERFLOW; goto done; }
        if (x_in && rep) {
            rep->n_draws++;
            /* tokens compare fp32 values exactly: only equal values may differ */
            int32_t o = x_in[i];
            int ok = o == t || (o >= 0 && o < A->V && edge_count(A, z[i], o, z[i + 1]) > 0 &&
                                prow[o] == prow[t]);
            if (!ok) {
                rep->n_hard++;
                if (rep->first_hard < 0) rep->first_hard = ((int64_t)(K + 1) << 32) | i;
            } else if (o != t) {
                rep->n_near++;
            }
        }
        if (x_out) x_out[i] = t;
    }
    if (z_out) for (int32_t k = 0; k <= L; ++k) z_out[k] = z[k];
done:
    free(z); free(row); free(col); free(tmp); free(w); free(acc);
    return status;
}

int or_map_tree(const or_aut *A, const float *p, const double *Wm, int32_t L, int32_t *states,
                int32_t *tokens, double *logmax)
{
    return map_walk(A, p, Wm, L, NULL, NULL, states, tokens, logmax, NULL);
}

/* Replay another implementation's MAP decisions (states original ids
 * [L+1], tokens [L]); report as or_replay_verify: draws = decisions,
 * hard, near (equal up to fp64 rounding, or equal p for a token), 0, first
 * hard decision. */
int or_map_verify(const or_aut *A, const float *p, const double *Wm, int32_t L,
                  const int32_t *states, const int32_t *tokens, int64_t report[5])
{
    or_replay_report rep = {0, 0, 0, 0, -1};
    int st = map_walk(A, p, Wm, L, states, tokens, NULL, NULL, NULL, &rep);
    report[0] = rep.n_draws; report[1] = rep.n_hard; report[2] = rep.n_near;
    report[3] = rep.n_margin; report[4] = rep.first_hard;
    return st;
}

/* ===================================================== chain (FFBS) replay
 * The serial chain baseline of [P1 "The scan trick"] (forward filtering over
 * the positions, then backward sampling): z_L ~ alpha_L[f] over f in F,
 * then z_i ~ alpha_i[a] M_i[a][z_{i+1}] for i = L-1 .. 0, then every token
 * as in the tree sampler.  Uniforms keyed like the tree sampler's with
 * level K+2 and node i for the draw of z_i, and level K+1, node i for token
 * i (K = log2 Lpad).  Replays another implementation's states (original
 * ids, [L+1]) and tokens [L], each draw conditioned on that implementation's
 * later state and judged as in or_replay_verify; alpha from
 * or_forward_backward.  report as or_replay_verify. */
int or_ffbs_verify(const or_aut *A, const float *p, const double *W, int32_t L,
                   const double *alpha, uint64_t seed, uint32_t b, const int32_t *states,
                   const int32_t *tokens, int64_t report[5])
{
    const int32_t S = A->S;
    int32_t Lpad;
    int32_t K = ilog2_pad(L, &Lpad);
    or_replay_report rep = {0, 0, 0, 0, -1};
    double *w = (double *)malloc(sizeof(double) * (S > A->V ? S : A->V));
    if (!w) return OR_BADARG;
    int status = OR_OK;
    memset(w, 0, sizeof(double) * S);
    for (int32_t k = 0; k < A->n_accept; ++k) w[A->accept[k]] = alpha[(size_t)L * S + A->accept[k]];
    int32_t z = judge(w, S, or_uniform(seed, b, (uint32_t)(K + 2), (uint32_t)L),
                      states[L] >= 0 && states[L] < S ? states[L] : S, ((int64_t)(K + 2) << 32) | L,
                      &rep);
    for (int32_t i = L - 1; i >= 0 && status == OR_OK; --i) {
        if (z < 0 || z >= S) { status = OR_UNDERFLOW; break; }
        memset(w, 0, sizeof(double) * S);
        for (int64_t e = 0; e < A->E; ++e)
            if (A->dst[e] == z) w[A->src[e]] += alpha[(size_t)i * S + A->src[e]] * W[(size_t)i * A->E + e];
        z = judge(w, S, or_uniform(seed, b, (uint32_t)(K + 2), (uint32_t)i),
                  states[i] >= 0 && states[i] < S ? states[i] : S, ((int64_t)(K + 2) << 32) | i, &rep);
    }
    for (int32_t i = 0; i < L && status == OR_OK; ++i) {
        if (states[i] < 0 || states[i] >= S || states[i + 1] < 0 || states[i + 1] >= S) {
            status = OR_UNDERFLOW;
            break;
        }
        token_weights(A, p + (size_t)i * A->V, states[i], states[i + 1], w);
        judge(w, A->V, or_uniform(seed, b, (uint32_t)(K + 1), (uint32_t)i), tokens[i],
              ((int64_t)(K + 1) << 32) | i, &rep);
    }
    report[0] = rep.n_draws; report[1] = rep.n_hard; report[2] = rep.n_near;
    report[3] = rep.n_margin; report[4] = rep.first_hard;
    free(w);
    return status;
}
