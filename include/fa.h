/*
 * fa.h - C ABI of the finite-automaton-constrained sampler for one
 * denoising step of a diffusion language model, for AMD MI355X (gfx950).
 *
 * The operation, from "Constrained Decoding for Diffusion Language Models via
 * Efficient Inference over Finite Automata" (paperfeed.app summary, sections
 * "The insight: the constraint is a hidden Markov model" and "The scan trick:
 * log-depth exact sampling"; papernotes.org summary, 关键设计 1-3):
 *   given per-position token probabilities p[b][i][v] (the denoiser's
 *   mean-field prediction) and an automaton M = (S, V, delta, s0, F), draw
 *   x ~ prod_i p[i][x_i] * paths(x) / Z, where paths(x) is the number of
 *   accepting paths of x (1 or 0 for a DFA), and return log Z, the sampled
 *   boundary states z_0..z_L and tokens, the constrained per-token marginals
 *   q[b][i][v] and the confidence score used for remasking.
 *
 * One step is four calls on one stream: fa_build_transitions (emission
 * reduce into per-position transition matrices), fa_span_tree (bottom-up
 * 2^k-span products and log Z), fa_sample (top-down midpoint draws, then
 * parallel token draws), fa_marginals (constrained marginals and confidence).
 *
 * Ownership: the caller owns every device buffer and the stream.  The
 * library owns only the host-side fa_table; it never allocates device memory
 * and never synchronizes the stream.  Calls are asynchronous on `stream`
 * (a hipStream_t; NULL is the default stream).  Distinct buffers may be used
 * concurrently from different streams; one table may be shared.
 *
 * Errors: every call returns FA_OK or a synchronous error code; on a
 * synchronous error nothing is launched.  Data-dependent conditions are
 * OR-ed asynchronously into row_status[b] (FA_ROW_*); the caller clears
 * row_status before a step.  Rows with a status bit set get states/tokens
 * -1, q = 0 and conf = -inf; logZ = -inf for the rows fa_build_transitions
 * or fa_span_tree flag (a row that only fa_sample flags keeps the log Z of
 * its tree).  No C++ exception crosses this interface.
 *
 * Layout (all device arrays row-major, C order):
 *   p      float  [B][L][V]
 *   tree   float  [B][2*Lpad][Sp][Sp]   heap order: node 1 = root over
 *                 [0, Lpad), node n has children 2n (left) and 2n+1 (right),
 *                 leaves Lpad + i hold the transition matrix of position i
 *                 (identity for i >= L).  Nodes with an odd index >= 3 are
 *                 stored transposed, all others as is.
 *   meta   int32  [B][2*Lpad][3][Sp]    per stored row/column power-of-two
 *                 exponents of every node (row scale, column scale, row
 *                 fold normalizer); the true matrix is
 *                 diag(2^ro) P diag(2^co) in stored orientation.
 *   states int32  [B][L+1]  original state ids z_0 = s0 .. z_L
 *   tokens int32  [B][L]
 *   q      float  [B][L][V]
 *   conf   float  [B][L]
 *   logZ   double [B]
 * Lpad = smallest power of two >= L; Sp = trimmed state count rounded up to
 * a multiple of 64 (padding rows and columns are zero).  Sizes come from
 * fa_sizes().
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *fa_stream_t; /* a hipStream_t */
typedef struct fa_table fa_table;

enum {
    FA_OK = 0,
    FA_EINVAL = 1,  /* bad size, id, range, pointer or workspace */
    FA_ENOTDET = 2, /* FA_DFA given but some (state, token) has two edges */
    FA_ETOOBIG = 3, /* a size exceeds what the kernels index */
    FA_EHIP = 4,    /* a HIP call or launch failed */
    FA_ESTATE = 5   /* table not uploaded */
};

enum { FA_ROW_INFEASIBLE = 1, FA_ROW_UNDERFLOW = 2, FA_ROW_BADPROB = 4 };

enum {
    FA_DFA = 1,          /* check determinism */
    FA_NFA = 2,          /* strings weighted by their number of accepting paths */
    FA_LABEL_RANGES = 4, /* label_tok holds flat half-open [lo, hi) pairs */
    FA_NO_TRIM = 8,      /* keep states unreachable from s0 or unable to reach F */
    FA_FIRST_LEVEL_SPARSE = 16, /* first span level from the pair values (row combination) */
    FA_FIRST_LEVEL_DENSE = 32,  /* first span level as dense matrix products */
    FA_SECOND_LEVEL_SPARSE = 64, /* also the second level from the two-step pattern (needs the
                                    first level sparse) */
    FA_LIVE_STATES = 128, /* span products over the states live at their midpoint (see fa_span_tree) */
    FA_FIRST_LEVEL_PAIRS = 256 /* first span level as dense matrix products whose operands are
                                  staged from the pair values (no dense leaves) */
};

enum { FA_CONF_PROB = 0, FA_CONF_NEGENT = 1, FA_CONF_UNCONSTRAINED = 2 };

/*
 * fa_compile_table - validate and compile an automaton (host only).
 * Cite: the automaton as a chain model, paperfeed summary "The insight: the
 * constraint is a hidden Markov model"; NFAs, "Arbitrary schedules and
 * NFAs"; papernotes 整体框架 (M = (S, V, delta, s0, F)).
 *   S, V            state and vocabulary sizes (>= 1)
 *   start           s0 in [0, S)
 *   accept          n_accept accepting state ids in [0, S) (host pointer)
 *   E, src, dst     edge list, ids in [0, S) (host pointers)
 *   label_off       E+1 non-decreasing offsets into label_tok, label_off[0]=0
 *   label_tok       token ids in [0, V) (a label is a set: repeats count
 *                   once), or with FA_LABEL_RANGES flat [lo, hi) pairs with
 *                   0 <= lo <= hi <= V, disjoint within one edge
 *   flags           FA_DFA | FA_NFA | FA_LABEL_RANGES | FA_NO_TRIM, and at
 *                   most one of FA_FIRST_LEVEL_SPARSE / FA_FIRST_LEVEL_DENSE /
 *                   FA_FIRST_LEVEL_PAIRS (how fa_span_tree forms the first
 *                   level; default: the sparse form when its work is at
 *                   most 1/256 of S^3, else the pair-staged dense form when
 *                   the table allows it (Sp a multiple of 256, Sp <= 2048,
 *                   no FA_LIVE_STATES, the pairs fit the message pass's
 *                   pair-value leaf level: FA_ETOOBIG when forced without
 *                   that, FA_EINVAL with FA_LIVE_STATES), else dense
 *                   products over dense leaves), and
 *                   FA_SECOND_LEVEL_SPARSE (the second level likewise, over
 *                   the pairs (a, c) joined through some k; default: when
 *                   the first is sparse and its own work is at most 1/256 of
 *                   S^3), and FA_LIVE_STATES (fa_span_tree restricts the
 *                   256x256-tile products to the states live at their
 *                   midpoint under the step's p)
 *   out             receives the handle (free with fa_table_destroy)
 *   device_bytes    receives the size of the device image
 * Dead states (unreachable from s0 or unable to reach F) are removed unless
 * FA_NO_TRIM; state order is preserved, so ascending compact ids are
 * ascending original ids.  Errors: FA_EINVAL, FA_ENOTDET, FA_ETOOBIG.
 */
int fa_compile_table(int32_t S, int32_t V, int32_t start, const int32_t *accept,
                     int32_t n_accept, int64_t E, const int32_t *src, const int32_t *dst,
                     const int64_t *label_off, const int32_t *label_tok, uint32_t flags,
                     fa_table **out, size_t *device_bytes);

/*
 * fa_table_upload - copy the compiled image into dev_buf (device memory of at
 * least device_bytes, 256-byte aligned, owned by the caller, which must
 * outlive every later call with this table) with one asynchronous
 * host-to-device copy on `stream`.  The handle keeps the host image alive.
 * Errors: FA_EINVAL, FA_EHIP.
 */
int fa_table_upload(fa_table *t, void *dev_buf, size_t bytes, fa_stream_t stream);

/* fa_table_destroy - free the host handle (not the caller's device buffer). */
void fa_table_destroy(fa_table *t);

/*
 * fa_table_info - host-side facts about a compiled table.  Writes up to n of:
 * [0] S' (kept states), [1] Sp, [2] start (compact), [3] accepting states
 * kept, [4] pairs, [5] LIST pairs, [6] DENSE pairs, [7] RANGE pairs,
 * [8] LIST entries, [9] range segments, [10] cut points, [11] sel tokens,
 * [12] 1 if LIST entries index the selected-token gather, [13] V,
 * [14] S (original), [15] 1 if fa_span_tree forms the first level from the
 * pair values, [16] that form's multiply-adds per first-level product (the
 * number of pairs (a, k), (k, c) sharing k), [17] 1 if the second level is
 * formed likewise, [18] its multiply-adds per product, [19] the pairs of the
 * two-step pattern it uses, [20] 1 if the step keeps no dense leaves (the
 * first level is sparse or pair-staged, and the message pass's leaf level and
 * the leaf-level midpoint draws read the pair values), [21] 1 if the message
 * pass's leaf level (L > 1) reads the pair values instead of the dense
 * leaves, [22] 1 if the table was compiled with FA_LIVE_STATES, [23] 1 if
 * the first level is a dense product with operands staged from the pair
 * values, [24] 1 if fa_map_decode forms its first max-plus level from the
 * pairs (FA_FIRST_LEVEL_SPARSE forces it and FA_FIRST_LEVEL_DENSE keeps it
 * dense; else when 256 [16] <= S^3).  Returns FA_OK or FA_EINVAL.
 */
int fa_table_info(const fa_table *t, int64_t *info, int32_t n);

/*
 * fa_table_state_map - orig_of[k] = original id of compact state k, for k in
 * [0, S').  Host pointer of S' entries.
 */
int fa_table_state_map(const fa_table *t, int32_t *orig_of);

/*
 * fa_sizes - bytes of the tree, meta and workspace buffers a step with batch
 * B and length L needs.  Any output pointer may be NULL.  The four calls of
 * one step take the same workspace, in order on one stream, and it must not
 * be written in between: fa_marginals reads pair-value sources that
 * fa_build_transitions leaves in it.  Any B is taken: the step calls run a
 * batch in chunks of at most 32767 / Lpad rows, one after the other on the
 * stream, each chunk with its own slot of the workspace (the draws keyed by
 * the row's index in the whole batch, so chunking changes no result).
 * Errors: FA_EINVAL, FA_ETOOBIG (L >= 2^24, or 2 Lpad > 65535).
 */
int fa_sizes(const fa_table *t, int32_t B, int32_t L, size_t *tree_bytes, size_t *meta_bytes,
             size_t *ws_bytes);

/*
 * fa_build_transitions - emission reduce: for every row b and position i,
 * M_i[s][s'] = sum_v c(s, v, s') p[b][i][v] with c the number of edges s->s'
 * whose label holds v; leaves i >= L are the identity.
 * Cite: papernotes 关键设计 1 (each position's state transition matrix sums
 * the reweighted emissions over the vocabulary); paperfeed "The insight"
 * (a factorized model times a chain model is a chain model; the |E||V| term).
 *   p        device [B][L][V] fp32, read only (values must be >= 0; NaN or
 *            negative entries that are read set FA_ROW_BADPROB)
 *   tree     device, fa_sizes bytes; leaves written, except on a table
 *            whose every leaf reader takes the pair values (fa_table_info
 *            [20]; the first span level then sparse or pair-staged) when
 *            L > 1
 *   meta     device, fa_sizes bytes; leaf exponents written
 *   ws       device workspace of ws_bytes >= fa_sizes; keeps, for the step's
 *            fa_marginals, the compact copy of p at token-list tokens and the
 *            values of the pairs that are not a single token's probability
 *   row_status device int32 [B], OR-ed
 * Errors: FA_EINVAL, FA_ESTATE, FA_EHIP.
 */
int fa_build_transitions(const fa_table *t, const float *p, int32_t B, int32_t L, float *tree,
                         int32_t *meta, void *ws, size_t ws_bytes, int32_t *row_status,
                         fa_stream_t stream);

/*
 * fa_span_tree - bottom-up span products: level by level every internal node
 * n gets P_n = P_2n P_2n+1 (log2 Lpad levels of batched fp32 matrix
 * products), with power-of-two row and column exponents so long chains
 * neither underflow nor overflow; then
 * logZ[b] = ln sum_{f in F} P_1[s0][f].
 * Cite: paperfeed "The scan trick: log-depth exact sampling" (2^k-step
 * transitions from 2^(k-1)-step ones in log L rounds of batched matrix
 * multiplication); papernotes 关键设计 2.
 *   tree, meta  written by fa_build_transitions; internal nodes written
 *   ws          device workspace of ws_bytes >= fa_sizes (partial products
 *               of the upper levels, whose few large products are split
 *               along K).  When the table computes the first level from
 *               the pair values (FA_FIRST_LEVEL_SPARSE, or chosen at compile
 *               time when the products' sparse work is at most 1/256 of
 *               the dense S^3), ws must hold what this step's
 *               fa_build_transitions wrote; the level is then a sum over
 *               pairs (a, k), (k, c) of the two leaves instead of a dense
 *               product, the same fp32 folded operands in another order.
 *               With FA_SECOND_LEVEL_SPARSE (or chosen likewise) the second
 *               level is formed the same way over the pairs (a, c) joined
 *               through some k, for its products whose four leaves lie
 *               inside the sequence.  With FA_FIRST_LEVEL_PAIRS (or
 *               chosen likewise) the first level is the dense product,
 *               each K step of its operands built in LDS from the leaves'
 *               folded pair values in ws (zeros elsewhere): the same
 *               operands as from dense leaves, and the same products bit
 *               for bit.  With FA_LIVE_STATES the call first
 *               finds, per row and boundary, the states reachable from s0
 *               and able to reach F through transitions of positive value
 *               (a forward and a backward pass over the positions), and
 *               the products on 256x256 tiles sum only over the states
 *               live at their midpoint: exact, since every path of the
 *               posterior visits live states only, and cheaper where
 *               committed positions (one-hot p) leave few of them.
 *   logZ        device double [B]; -inf for infeasible rows
 *   row_status  device int32 [B]; FA_ROW_INFEASIBLE when Z = 0
 * Errors: FA_EINVAL, FA_ESTATE, FA_EHIP.
 */
int fa_span_tree(const fa_table *t, int32_t B, int32_t L, float *tree, int32_t *meta,
                 void *ws, size_t ws_bytes, double *logZ, int32_t *row_status,
                 fa_stream_t stream);

/*
 * fa_sample - top-down exact sampling: z_Lpad ~ P_1[s0][f] over f in F (the
 * start state is pinned), then for every segment [l, r) with known boundary
 * states the midpoint m = (l+r)/2 by z_m ~ P_[l,m)[z_l][z_m] P_[m,r)[z_m][z_r],
 * level by level, then every token x_i ~ p[b][i][v] c(z_i, v, z_{i+1}) in
 * parallel.  Each draw is an inverse CDF over ascending candidate ids (the
 * smallest j with w_j > 0 and C_j > u T, C the inclusive prefix sum, T its
 * total) with u = (r0 >> 8) 2^-24, r0 the first word of Philox4x32-10 keyed by
 * seed and counter (b, level, node, 0): level 0 the root draw, levels 1..K
 * the midpoints (node = heap index - 2^(level-1)), level K+1 the tokens
 * (node = i).
 * Cite: paperfeed "The scan trick" (midpoint conditional independence,
 * top-down pass, parallel token emission); papernotes 关键设计 2.
 *   states  device int32 [B][L+1] original ids; tokens device int32 [B][L]
 *   ws      workspace (>= fa_sizes)
 *   row_status FA_ROW_UNDERFLOW if a draw's weights vanish while Z > 0
 * Errors: FA_EINVAL, FA_ESTATE, FA_EHIP.
 */
int fa_sample(const fa_table *t, const float *p, int32_t B, int32_t L, const float *tree,
              const int32_t *meta, uint64_t seed, int32_t *states, int32_t *tokens, void *ws,
              size_t ws_bytes, int32_t *row_status, fa_stream_t stream);

/*
 * fa_marginals - constrained per-token marginals and the remasking
 * confidence: forward/backward boundary messages alpha_i, beta_i from the
 * span tree (top-down), then
 *   q[b][i][v] = p[b][i][v] sum_{(a, a') pairs holding v} c alpha_i[a]
 *                beta_{i+1}[a'] / Z,
 *   conf[b][i] = q[b][i][tokens[b][i]]   (FA_CONF_PROB), or
 *              = sum_v q ln q            (FA_CONF_NEGENT, 0 ln 0 = 0), or
 *              = p[b][i][tokens[b][i]]   (FA_CONF_UNCONSTRAINED: the
 *                denoiser's own probability of the sampled token, the
 *                score the constrained marginal is compared with;
 *                papernotes 消融实验).
 * Cite: papernotes 关键设计 3 (constrained marginals as the confidence that
 * decides which positions are committed); paperfeed "Two immediate bonuses"
 * (LLaDA: highest probability, Dream: lowest entropy).
 *   logZ    device double [B] from fa_span_tree
 *   tokens  device int32 [B][L] (needed for FA_CONF_PROB and
 *           FA_CONF_UNCONSTRAINED; may be NULL for FA_CONF_NEGENT)
 *   q       device fp32 [B][L][V] or NULL (not written)
 *   conf    device fp32 [B][L]
 *   ws      the workspace this step's fa_build_transitions wrote (the leaf
 *           level of the messages reads pair values from it)
 * Errors: FA_EINVAL, FA_ESTATE, FA_EHIP.
 */
int fa_marginals(const fa_table *t, const float *p, int32_t B, int32_t L, const float *tree,
                 const int32_t *meta, const double *logZ, const int32_t *tokens,
                 int32_t conf_mode, float *q, float *conf, void *ws, size_t ws_bytes,
                 int32_t *row_status, fa_stream_t stream);

/*
 * fa_sample_marginals - fa_sample followed by fa_marginals on the sampled
 * tokens, in one call whose outputs are bit-identical to that pair of calls
 * (states, tokens, q, conf and row_status).  When the table has dense-label
 * pairs, V % 4 == 0, p and q are 16-byte aligned and the q writer streams
 * rows (q non-NULL or FA_CONF_NEGENT), the token draws of positions whose
 * sampled pair is a dense pair take their chunk sums from the q writer's pass
 * over p instead of reading the row again (the same sums in the same order);
 * otherwise the call runs the two calls' launches in order.  On the first
 * path the midpoint draws, which depend only on the tree, run as extra
 * workgroups of the message pass's last launches; everything stays on
 * `stream`.
 * Cite: as fa_sample and fa_marginals.
 *   arguments  as in fa_sample and fa_marginals; tokens is an output here
 *              and required in both confidence modes
 *   ws         workspace (>= fa_sizes) this step's fa_build_transitions wrote
 * Errors: FA_EINVAL, FA_ESTATE, FA_EHIP.
 */
int fa_sample_marginals(const fa_table *t, const float *p, int32_t B, int32_t L,
                        const float *tree, const int32_t *meta, const double *logZ,
                        uint64_t seed, int32_t conf_mode, int32_t *states, int32_t *tokens,
                        float *q, float *conf, void *ws, size_t ws_bytes, int32_t *row_status,
                        fa_stream_t stream);

/*
 * fa_chain_sample - the serial chain sampler, the baseline the span tree
 * replaces: forward filtering over the positions (L dependent steps, one
 * launch each: a_{i+1} = (a_i 2^-e_i) M_i with e_i the exponent of max a_i,
 * a_0 = e_{s0}), log Z = ln 2 sum e_i + ln sum_{f in F} a_L[f], then backward
 * sampling z_L ~ a_L[f] over f in F and z_i ~ a_i[a] M_i[a][z_{i+1}] for
 * i = L-1 .. 0, then the tokens as fa_sample draws them.  Uniforms: the state
 * draw of z_i keyed (b, K+2, i), token i (b, K+1, i), K = log2 Lpad.  The
 * same posterior as fa_sample, other draws.
 * Cite: paperfeed summary "The scan trick: log-depth exact sampling" (the
 * serial forward-backward pass with L dependent steps); papernotes 消融实验
 * (the chain's latency against the tree's).
 *   tree     the leaves fa_build_transitions wrote (read only; a table that
 *            keeps no dense leaves, fa_table_info [20], is refused when L > 1)
 *   logZ     device double [B]; states [B][L+1] original ids; tokens [B][L]
 *   ws       the step's workspace (>= fa_sizes)
 * Errors: FA_EINVAL, FA_ETOOBIG, FA_ESTATE, FA_EHIP.
 */
int fa_chain_sample(const fa_table *t, const float *p, int32_t B, int32_t L, const float *tree,
                    uint64_t seed, double *logZ, int32_t *states, int32_t *tokens, void *ws,
                    size_t ws_bytes, int32_t *row_status, fa_stream_t stream);

/*
 * fa_chain_sample_marginals - the chain's full serial forward-backward
 * pass: fa_chain_sample, then backward messages over the positions
 * (L dependent steps, one launch each: b_L = 1_F, b_i = M_i (b_{i+1}
 * 2^-e'_{i+1}) with e'_j the exponent of max b_j), and the marginals and
 * confidence of fa_marginals from alpha_i = a_i 2^(e_0 + .. + e_{i-1}) and
 * beta_i = b_i 2^(e'_{i+1} + .. + e'_L) instead of the span tree's messages.
 * The same q and conf as the tree path up to rounding (the messages are
 * products of up to L fp32 steps here, of log2 L levels there); the states
 * and tokens of fa_chain_sample.
 * Cite: paperfeed summary "The scan trick: log-depth exact sampling" (the
 * serial forward-backward pass the tree replaces); papernotes 关键设计 3 (the
 * constrained marginals as the remasking confidence).
 *   arguments  as in fa_chain_sample, plus conf_mode, q (or NULL) and conf
 *              as in fa_marginals; ws (>= fa_sizes) the workspace of this
 *              step's fa_build_transitions
 * Errors: FA_EINVAL (also for a table that keeps no dense leaves, L > 1),
 * FA_ETOOBIG, FA_ESTATE, FA_EHIP.
 */
int fa_chain_sample_marginals(const fa_table *t, const float *p, int32_t B, int32_t L,
                              const float *tree, uint64_t seed, int32_t conf_mode, double *logZ,
                              int32_t *states, int32_t *tokens, float *q, float *conf, void *ws,
                              size_t ws_bytes, int32_t *row_status, fa_stream_t stream);

/*
 * fa_map_sizes - bytes of the fp64 tree and of the workspace fa_map_decode
 * needs for batch B and length L.  Errors: FA_EINVAL, FA_ETOOBIG (also for a
 * table with range labels whose per-position range-maximum structure, 4 bytes
 * per elementary interval between cut points plus a sparse table over blocks
 * of 64 of them, exceeds 160 KB: about 34,000 distinct cut points).
 */
int fa_map_sizes(const fa_table *t, int32_t B, int32_t L, size_t *tree_bytes, size_t *ws_bytes);

/*
 * fa_map_decode - greedy (temperature 0) constrained decoding: for every row
 * the most probable accepted string, argmax_x prod_i p[b][i][x_i] over the
 * strings the automaton accepts (an NFA string counts once, whatever its
 * number of accepting paths: every path of one string has the same
 * product), and ln of its probability.
 * Cite: paperfeed summary "The evidence" (greedy decoding beside sampling)
 * and "Why constrained decoding breaks for diffusion LMs" (MAP inference
 * over an automaton by dynamic programming); the tree of "The scan trick:
 * log-depth exact sampling" with max in place of sum.
 * Method: per position the max-times transition matrix
 * Mmax_i[a][b] = max over v with c(a, v, b) > 0 of p[b][i][v] (range labels:
 * per position the maxima of p over the elementary intervals between cut
 * points, a sparse table over blocks of them, and each segment's maximum
 * from at most two partial blocks and two table entries); 2^k-span
 * max-times products level by level in fp64 logs; the final boundary state
 * maximizing root[s0][f] over f in F; top-down, every midpoint z_m
 * maximizing P[l,m)[z_l][z_m] + P[m,r)[z_m][z_r]; every token the most
 * probable one of its edge (z_i, z_{i+1}).  Each decision takes the smallest
 * id (state, token) among equal values.
 *   p        device [B][L][V] fp32 (>= 0; NaN or negative p at a labelled
 *            token sets FA_ROW_BADPROB)
 *   tree     device fp64, fa_map_sizes bytes ([B][2*Lpad][Sp][Sp] heap
 *            order, right children transposed, natural logs)
 *   ws       device workspace of ws_bytes >= fa_map_sizes
 *   logmax   device double [B]: ln of the best string's probability, -inf
 *            (and FA_ROW_INFEASIBLE) when no accepted string has p > 0
 *   states   device int32 [B][L+1] original ids; tokens device int32 [B][L]
 *            (-1 on flagged rows)
 *   row_status device int32 [B], OR-ed
 * Errors: FA_EINVAL, FA_ETOOBIG (also range labels beyond fa_map_sizes'
 * bound), FA_ESTATE, FA_EHIP.
 */
int fa_map_decode(const fa_table *t, const float *p, int32_t B, int32_t L, double *tree,
                  void *ws, size_t ws_bytes, double *logmax, int32_t *states, int32_t *tokens,
                  int32_t *row_status, fa_stream_t stream);

/*
 * fa_commit - the remasking step between denoising steps: per row b, of the
 * n positions still masked (committed[b][i] == 0 and tokens[b][i] >= 0), the
 * k = ceil(n / steps_left) with the largest conf[b][i] (NaN counts as -inf;
 * ties go to the lower position; steps_left == 1 commits all of them) are
 * committed to their sampled tokens: committed[b][i] = 1, fresh[b][i] = 1,
 * and p[b][i][.] becomes one-hot at tokens[b][i], which is how the next step
 * sees a committed position.  Every other fresh entry is 0, and a row with
 * row_status[b] != 0 commits nothing.
 * Cite: papernotes 关键设计 3 (the constrained marginal as the confidence
 * that decides which positions are committed); paperfeed "Two immediate
 * bonuses" (LLaDA: highest probability; Dream: lowest entropy, i.e. pass the
 * FA_CONF_NEGENT confidence).
 *   conf        device fp32 [B][L] (fa_marginals)
 *   tokens      device int32 [B][L] (fa_sample)
 *   committed   device int32 [B][L], read and updated
 *   fresh       device int32 [B][L], written
 *   p           device fp32 [B][L][V], committed rows rewritten
 *   row_status  device int32 [B] or NULL
 * Errors: FA_EINVAL (negative sizes, V < 1, steps_left < 1, NULL buffers),
 * FA_ETOOBIG (L > 8192), FA_EHIP.
 */
int fa_commit(int32_t B, int32_t L, int32_t V, const float *conf, const int32_t *tokens,
              int32_t steps_left, int32_t *committed, int32_t *fresh, float *p,
              const int32_t *row_status, fa_stream_t stream);

/*
 * fa_span_tree_noalloc - fa_span_tree for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc.  The same kernels and outputs as fa_span_tree; the
 * split-K partial tiles of the upper levels (the only scratch memory the
 * span tree uses) live in a library-owned device array of
 * FA_SPAN_TREE_NOALLOC_MAX_BYTES (8 MiB), one copy per GPU, held until the
 * process ends.  A level is split along K only while rows x nodes x splits
 * x (Sp/64)^2 <= 256, so its partial tiles never exceed 2^20 floats: every
 * table and size fa_span_tree takes fits.  No workspace argument; the call
 * allocates nothing.
 *   arguments  as in fa_span_tree (tree, meta, logZ, row_status are the
 *              caller's)
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, or different threads) race and must not be
 * issued.  The array is fully written before it is read by each call.
 * Errors: FA_EINVAL (also for a table whose first span level is formed from
 * the pair values, fa_table_info [15] = 1 or [23] = 1: that level reads the
 * workspace fa_build_transitions wrote, so such tables take fa_span_tree),
 * FA_ETOOBIG (the step's partial tiles exceed FA_SPAN_TREE_NOALLOC_MAX_BYTES,
 * or the grid limits of fa_span_tree), FA_ESTATE, FA_EHIP.
 */
#define FA_SPAN_TREE_NOALLOC_MAX_BYTES ((size_t)8 << 20)
int fa_span_tree_noalloc(const fa_table *t, int32_t B, int32_t L, float *tree, int32_t *meta,
                         double *logZ, int32_t *row_status, fa_stream_t stream);

/* fa_strerror - static description of an error code. */
const char *fa_strerror(int code);

/* Measurement hook; not part of the method.
 * fa_profile_kernel - bracket every launch of one kernel with two HIP events
 *   owned by the caller (hipEvent_t handles passed as void *):
 *   hipEventRecord(start) just before and hipEventRecord(stop) just after the
 *   launch, on the stream the launch uses, until cleared with FA_PROF_NONE.
 *   which:
 *     FA_PROF_EMISSION_DENSE  dense-mask contraction in fa_build_transitions
 *     FA_PROF_TREE_LEVEL1     matrix products of the first span-tree level
 *     FA_PROF_MARG_Q          per-token marginal writer in fa_marginals
 *   The setting belongs to the calling thread (thread-local): it brackets
 *   the launches of the step calls that thread issues.
 * Errors: FA_EINVAL (unknown id, or an event missing for a kernel id).
 */
enum { FA_PROF_NONE = 0, FA_PROF_EMISSION_DENSE = 1, FA_PROF_TREE_LEVEL1 = 2, FA_PROF_MARG_Q = 3 };
int fa_profile_kernel(int32_t which, void *start_event, void *stop_event);

/* Measurement hook; not part of the method.
 * fa_probe_bandwidth - one plain streaming kernel on `stream`, whose rate is
 *   an achievable HBM ceiling for the step's kernels: `blocks` workgroups,
 *   each over its own contiguous chunk, with non-temporal float4 loads: 256
 *   threads and eight loads in flight per thread for the read, 1024 threads
 *   and four for the copy (with non-temporal stores).
 *     FA_PROBE_READ  every byte of src read once; dst receives one float per
 *                    workgroup (at least blocks * 4 bytes)
 *     FA_PROBE_COPY  dst = src (bytes each), streaming stores
 *   src, dst device pointers, 16-byte aligned; bytes a multiple of 16.
 * Errors: FA_EINVAL (mode, alignment, size, blocks outside 1..2^20), FA_EHIP.
 */
enum { FA_PROBE_READ = 0, FA_PROBE_COPY = 1 };
int fa_probe_bandwidth(int32_t mode, const void *src, void *dst, size_t bytes, int32_t blocks,
                       fa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
