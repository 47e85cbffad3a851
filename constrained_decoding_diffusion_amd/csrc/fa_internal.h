// Internal declarations shared by the host table compiler, the C-ABI entry
// points and the gfx950 kernels.  Not part of the public interface.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/fa.h"

namespace fa {

constexpr int kSpAlign = 64;       // trimmed state count padded to this
constexpr int kNeg = -(1 << 29);   // exponent of an all-zero row/column
constexpr int kDenseMax = 32;      // dense-label pairs share one mask word per token
// the first span level is formed from the pair values when its multiply-adds
// are at most 1/kSparseFirstRatio of the dense product's S^3
constexpr int kSparseFirstRatio = 256;
// LDS of one workgroup of the sparse first level (gfx950: 160 KB per CU);
// it holds the product's column exponents and the row pointers, which
// bounds the states the sparse form takes
constexpr size_t kSparseLdsMax = 160 * 1024;
// LDS bound of the sparse levels: the row pointers and column exponents
// (Sp + S words) next to eight waves' 1024-column row buffers and tasks
constexpr int kSparseMaxSpS = 22000;
constexpr int kSpWin = 1024;       // columns of a window when Sp > kSpWin
constexpr int32_t kSparseSecondMaxPairs = 1 << 24;
constexpr int32_t kSparseMaxPairs = 1 << 26;   // a sparse task packs its first item in 26 bits
constexpr int32_t kLeafMsgMaxPairs = 512 * 40; // pairs of the pair-value leaf level of the message pass
constexpr int kLeafTile = 4096;    // floats of the LDS tile of the one-pass leaf writer
constexpr int kDenseStepsMax = 64;  // dense-mask contraction: 256-token steps per V chunk, at most
constexpr int kDenseSlots = 512;    // workgroups of that contraction resident at once (256 CUs x 2)
constexpr int kDenseSelLds = 64;    // token-list tokens per V chunk that its LDS buffer holds
constexpr int kDenseTile = 32;     // positions per workgroup of the dense-mask contraction
constexpr int kSelMax = 8192;      // LIST tokens gathered through a compact copy of p
constexpr int kMapMaxSp = 2048;   // dense (row, column) -> pair maps up to this Sp
// greedy decoding forms its first max-plus level from the pairs when their
// terms, each costing about as much as this many dense terms (a chain of
// dependent gathers against a streamed tile), fall below S^3
constexpr int kMapSparseCost = 256;
constexpr uint32_t kSelBit = 1u << 31;  // tokmask flag of LIST tokens (tables with < 32 dense pairs)
constexpr int kRowChunk4 = 1024;   // float4 groups per chunk of a dense-pair token draw (4096 tokens)
constexpr int kQParts = 4;         // workgroups per position of the streaming q writer
constexpr int kTokChunksMax = 256;  // chunks per candidate list of one token draw
// MAP decoding over range labels: per position, the maxima of p over the
// ncut - 1 elementary intervals between cut points and a sparse table over
// blocks of kMapRangeBlk of them, both in one workgroup's LDS; a table whose
// structure exceeds kMapRangeLdsMax is refused
constexpr int kMapRangeBlk = 64;
constexpr size_t kMapRangeLdsMax = 160 * 1024;
constexpr int map_range_blocks(int nint) { return (nint + kMapRangeBlk - 1) / kMapRangeBlk; }
constexpr int map_range_levels(int nblk)   // floor(log2 nblk) + 1 levels
{
    int lg = 1;
    while ((2LL << (lg - 1)) <= nblk) ++lg;
    return lg;
}
constexpr size_t map_range_lds(int ncut)
{
    const int nint = ncut > 1 ? ncut - 1 : 0;
    const int nblk = map_range_blocks(nint);
    return ((size_t)nint + (size_t)nblk * map_range_levels(nblk)) * sizeof(uint32_t);
}

enum PairClass : int32_t { kList = 0, kDense = 1, kRange = 2 };

// The message pass's leaf level runs from the pair values (marg_leaf) when
// the leaf entries exist (Sp <= kLeafTile), the pairs fit its threads'
// registers and the pairs plus two S-vectors fit in LDS.  The table compiler
// (which drops the dense leaves of such tables) and the launcher (which then
// must not read them) both decide with this one predicate.
inline bool leaf_level_from_pairs(int64_t npairs, int64_t S, int64_t Sp)
{
    return Sp <= kLeafTile && npairs <= kLeafMsgMaxPairs &&
           ((size_t)npairs + 2 * (size_t)S) * 4 <= kSparseLdsMax;
}

// Device view of a compiled automaton.  All pointers address the caller's
// device buffer; passed to kernels by value.
struct DevTable {
    int32_t S;       // kept states
    int32_t Sp;      // padded
    int32_t V;
    int32_t start;   // compact
    int32_t n_acc;
    int32_t npairs;
    int32_t nsel;
    int32_t use_sel;
    int32_t ndense;
    int32_t nseg;
    int32_t ncut;
    int32_t has_cnt;
    int32_t selbit;  // 1: bit 31 of tokmask marks tokens that LIST pairs hold
    const int32_t *acc;        // [n_acc] ascending compact ids
    const int32_t *orig;       // [S] compact -> original id
    const int32_t *pair_a;     // [npairs] sorted by (a, b)
    const int32_t *pair_b;
    const int32_t *row_ptr;    // [S+1] pairs of source a
    const int32_t *col_ptr;    // [S+1] into col_pairs
    const int32_t *col_pairs;  // [npairs] pair ids sorted by (b, a)
    const int32_t *pair_cls;   // [npairs] PairClass
    const int32_t *pair_aux;   // dense index of a dense pair, else -1
    const int32_t *list_off;   // [npairs+1]
    const int32_t *list_tok;   // raw token ids
    const int32_t *list_sel;   // index into sel_tok
    const float *list_cnt;     // counts (nullptr when every count is 1)
    const int32_t *sel_tok;    // [nsel] sorted unique LIST tokens
    const int32_t *tm_off;     // [nsel+1] token-major LIST entries
    const int32_t *tm_pair;
    const float *tm_cnt;       // nullptr when every count is 1
    const int32_t *dense_pair; // [ndense]
    const uint32_t *tokmask;   // [V] bit j set: v in the label of dense pair j
    const int32_t *seg_off;    // [npairs+1] disjoint segments of a RANGE pair
    const int32_t *seg_lo;     // [nseg]
    const int32_t *seg_hi;
    const float *seg_cnt;
    const int32_t *seg_lo_cut; // index of seg_lo in cuts
    const int32_t *seg_hi_cut;
    const int32_t *cuts;       // [ncut] sorted unique segment endpoints
    const int32_t *cut_off;    // [ncut+1] segment events at each cut
    const int32_t *cut_ev;     // 2*seg (start) or 2*seg+1 (end)
    const int32_t *tok2sel;    // [V] index into sel_tok or -1 (nsel > 0)
    const int32_t *tok2cut;    // [V] largest c with cuts[c] <= v, or -1 (nseg > 0)
    const int32_t *seg_pair;   // [nseg] pair of each segment
    const int32_t *map_n;      // [Sp][Sp] pair at (a, b) or -1 (Sp <= kMapMaxSp)
    const int32_t *map_t;      // [Sp][Sp] pair at (b, a) (transposed storage)
    const int32_t *tm_a;       // [list entries] source state of each token-major entry
    const int32_t *tm_b;       // [list entries] target state
    // leaf entries, in pair order (row-major leaves) and in column order
    // (transposed leaves): stored (row << 16 | column), and the value's
    // source: >= 0 a direct index (psel column, or token of p without a
    // compact copy) of a one-token count-1 list pair, else -1 - j for the
    // j-th indirect pair (ind_pair[j])
    const int32_t *ent_n_rc;
    const int32_t *ent_n_src;
    const int32_t *ent_t_rc;
    const int32_t *ent_t_src;
    const int32_t *ind_pair;   // [n_ind] pairs whose value is computed (not one direct read)
    int32_t n_ind;
    int32_t first_sparse;        // 1: the first span level is formed from the pair values
    int32_t first_pairs;         // 1: it is a dense product whose operands are staged from them
    int32_t map_first_sparse;    // 1: greedy decoding forms its first max-plus level from the pairs
    int32_t leafless;            // 1: no dense leaves; every leaf reader takes the pair values
    int32_t second_sparse;       // 1: so is the second, from the two-step pattern
    int32_t live_states;         // 1: dense products contract over the live states (live.hip)
    int32_t np2;                 // pairs of the two-step pattern
    int32_t nwin;                // win_cols-column windows of a row (0: one window)
    int32_t win_cols;            // kSpWin for Sp > kSpWin, kSpWin / 2 for Sp > kSpWin / 2
    const int32_t *p2_a, *p2_b, *p2_row_ptr, *p2_col_ptr, *p2_col_pairs, *p2_colpos;
    const int32_t *w1_n, *w1_t, *w2_n, *w2_t;
    const int32_t *col_a, *p2_col_a;   // a of each column-order entry (column walk targets)
    const uint32_t *dense_bits;  // [ndense][dense_words] bit v%32 of word v/32: v in the label
    int32_t dense_words;
    const int32_t *ev_a;       // [2 nseg] per cut event (cut_ev order): the states of its pair
    const int32_t *ev_b;
    const float *ev_w;         // [2 nseg] its count, negative at a segment end
    const uint32_t *cutbits;   // [(V+31)/32] bit v%32 of word v/32: a cut point at token v < V
    const int32_t *sel_lb;     // [V/256 + 2] first sel_tok index at or after token 256 t
    const int32_t *pair_colpos;  // [npairs] position of each pair in col_pairs
    int32_t n_tm;              // token-major LIST entries
};

// Host representation of a compiled automaton and its device image.
struct HostTable {
    int32_t S_orig = 0, V = 0, S = 0, Sp = 0, start = 0;
    std::vector<int32_t> acc, orig;
    std::vector<int32_t> pair_a, pair_b, row_ptr, col_ptr, col_pairs, pair_cls, pair_aux;
    std::vector<int32_t> list_off, list_tok, list_sel;
    std::vector<float> list_cnt;
    std::vector<int32_t> sel_tok, tm_off, tm_pair;
    std::vector<float> tm_cnt;
    std::vector<int32_t> dense_pair;
    std::vector<uint32_t> tokmask;
    std::vector<int32_t> seg_off, seg_lo, seg_hi, seg_lo_cut, seg_hi_cut, cuts, cut_off, cut_ev;
    std::vector<float> seg_cnt;
    std::vector<int32_t> tok2sel, tok2cut, seg_pair;
    std::vector<int32_t> map_n, map_t;
    std::vector<int32_t> tm_a, tm_b;
    std::vector<int32_t> ent_n_rc, ent_n_src, ent_t_rc, ent_t_src, ind_pair;
    std::vector<uint32_t> dense_bits;
    std::vector<int32_t> ev_a, ev_b;
    std::vector<float> ev_w;
    std::vector<uint32_t> cutbits;
    std::vector<int32_t> sel_lb;
    std::vector<int32_t> pair_colpos;
    bool has_cnt = false;
    bool use_sel = false;
    bool selbit = false;
    bool first_sparse = false;  // first span level by row combination over the pairs
    bool first_pairs = false;   // first span level on the matrix cores, operands from the pairs
    bool map_first_sparse = false;  // greedy decoding's first max-plus level over the pairs
    bool leafless = false;      // dense leaves not written (every leaf reader takes pair values)
    int64_t first_work = 0;     // its multiply-adds per product: pairs (a, k) times pairs (k, c)
    // two-step pattern: pairs (a, c) joined by pairs (a, k), (k, c), sorted
    // (a, c), with the same row/column orders as the pairs (second level)
    std::vector<int32_t> p2_a, p2_b, p2_row_ptr, p2_col_ptr, p2_col_pairs, p2_colpos;
    std::vector<int32_t> col_a, p2_col_a;   // column walks' targets: a of each column-order entry
    bool second_sparse = false;
    int64_t second_work = 0;    // multiply-adds per second-level product
    bool live_states = false;   // FA_LIVE_STATES: products over the live states of their midpoint
    // entry offsets of each state's row walk (_n) and column walk (_t) at
    // every window boundary, [S][nwin + 1]; only when Sp > kSpWin / 2
    std::vector<int32_t> w1_n, w1_t, w2_n, w2_t;
    int32_t nwin = 0, win_cols = 0;   // windows of win_cols columns (0: one window)
    // device image
    std::vector<uint8_t> image;
    std::vector<size_t> offs;  // section offsets, in the order of DevTable pointers
    void *dev = nullptr;
    size_t dev_bytes = 0;

    int32_t npairs() const { return (int32_t)pair_a.size(); }
    int32_t ndense() const { return (int32_t)dense_pair.size(); }
    int32_t nseg() const { return (int32_t)seg_lo.size(); }
    int32_t ncut() const { return (int32_t)cuts.size(); }
    int32_t nsel() const { return (int32_t)sel_tok.size(); }
    bool needs_stream() const { return ndense() > 0 || nseg() > 0; }
    DevTable device_view() const;
};

// Step geometry shared by all calls.
struct Geometry {
    int32_t B, L, Lpad, K, Sp;
    int32_t b0;          // batch row of the chunk's row 0 (the draws' keys use b0 + b)
    size_t mat;          // floats per matrix = Sp*Sp
    size_t tree_floats;  // B * 2*Lpad * mat
    size_t meta_ints;    // B * 2*Lpad * 3 * Sp
};

// Lpad, K and buffer sizes of a step; FA_EINVAL for negative sizes,
// FA_ETOOBIG for L >= 2^24
int make_geometry(const HostTable &t, int32_t B, int32_t L, Geometry *g);

// Rows per launch: the step kernels put (row, node) pairs in a grid
// dimension of at most 65535, so a batch runs in chunks of at most
// 32767 / Lpad rows, one after the other on the caller's stream, each chunk
// with its own workspace slot.  The chunking depends on B and L only, so
// every call of a step finds its chunk's workspace where the previous call
// left it.
struct StepChunks {
    int32_t rows = 0;   // rows per full chunk
    int32_t count = 0;  // chunks
    size_t slot = 0;    // workspace bytes per chunk: the larger of a full and the last chunk
};
// map: slots sized for MAP decoding instead of the sampling step.
// FA_ETOOBIG when even one row does not fit (2 Lpad > 65535).
int plan_chunks(const HostTable &t, int32_t B, int32_t L, bool map, StepChunks *c);

// Workspace layout (bytes from the start of ws), sized for the largest user.
struct WsLayout {
    size_t dpart = 0, dval = 0, psel = 0, cutp = 0, val = 0;  // emission reduce
    size_t pvf = 0;                            // folded leaf pair values (first level from the pairs)
    size_t pv2 = 0;                            // first-level nodes on the two-step pattern (second level)
    size_t pv2alt = 0;                         // the same values in each node's other walk order
    int32_t n_vchunks = 0;                     // dense-mask contraction: V split
    int32_t vchunk = 0;                        // tokens per V chunk (multiple of 256)
    int32_t sel_mode = 0;                      // token-list copy: 1 LDS-buffered, 2 gathered
    size_t zc = 0;                             // sampler: compact boundary states
    size_t tpair = 0, tdbit = 0;               // sampler: per position the drawn pair, its dense bit
    size_t kpart = 0;                          // span tree: split-K partial tiles
    size_t lbits = 0, live = 0, nlive = 0;     // span tree: live-state bitsets, lists, counts
    size_t va = 0, ea = 0, vb = 0, eb = 0;     // marginals: messages
    size_t rcut = 0;                           // marginals: range weights per cut
    size_t ndval = 0;                          // emission: values of the indirect pairs (persist)
    size_t pw = 0;                             // marginals: per-position pair weights
    size_t hpart = 0;                          // marginals: q ln q partial sums per row part
    size_t tcs = 0, tcs_ok = 0;                // joint call: dense-pair chunk sums of the token draws
    int32_t tcs_nch = 0;                       // chunks per row of those sums
    int32_t pw_nl = 0, pw_ld = 0;              // token-list weights per row, row length
    size_t total = 0;
};
WsLayout ws_layout(const HostTable &t, const Geometry &g);


// Kernel launchers (kernels.hip).  Return 0 or a hipError_t value.
int launch_build_transitions(const DevTable &d, const Geometry &g, const float *p, float *tree,
                             int32_t *meta, uint8_t *ws, const WsLayout &w, int32_t *status,
                             void *stream);
int launch_span_tree(const DevTable &d, const Geometry &g, float *tree, int32_t *meta,
                     uint8_t *ws, const WsLayout &w, double *logZ, int32_t *status, void *stream);
// the live states of every boundary (live.hip): lists at w.live, counts at w.nlive
int launch_live_states(const DevTable &d, const Geometry &g, const float *tree, uint8_t *ws,
                       const WsLayout &w, void *stream);

// Measurement hook: records the caller's start (begin) or stop event on
// `stream` when `which` is the kernel selected by fa_profile_kernel.
// Returns 0 or a hipError_t value.
int prof_mark(int which, bool begin, void *stream);

// Split of one tree level's products along K (upper levels with few
// products): 1 = no split.
int tree_ksplit(const Geometry &g, int level);
// the serial chain sampler (chain.hip): forward filtering over the positions,
// backward sampling, the token draws of the tree sampler
int launch_chain_sample(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                        uint64_t seed, double *logZ, int32_t *states, int32_t *tokens,
                        uint8_t *ws, const WsLayout &w, int32_t *status, void *stream);
// the chain sampler, then backward messages and the marginals from the two
// message chains (conf_mode FA_CONF_PROB or FA_CONF_NEGENT)
int launch_chain_sample_marginals(const DevTable &d, const Geometry &g, const float *p,
                                  const float *tree, uint64_t seed, int32_t conf_mode,
                                  double *logZ, int32_t *states, int32_t *tokens, float *q,
                                  float *conf, uint8_t *ws, const WsLayout &w, int32_t *status,
                                  void *stream);

// MAP decoding (map.hip): workspace regions and the launcher
struct MapWs {
    size_t pmax = 0;   // [B*L][npairs] fp32 pair maxima
    size_t zc = 0;     // [B][Lpad+1] int32 compact boundary states
    size_t kpart = 0;  // fp64 split-K partial tiles
    size_t total = 0;
};
MapWs map_ws_layout(const HostTable &t, const Geometry &g);
int launch_map_decode(const DevTable &d, const Geometry &g, const float *p, double *tree,
                      uint8_t *ws, const MapWs &w, double *logmax, int32_t *states,
                      int32_t *tokens, int32_t *status, void *stream);

// conf = p at the sampled token (FA_CONF_UNCONSTRAINED), after the PROB path
int launch_conf_unconstrained(const DevTable &d, const Geometry &g, const float *p,
                              const int32_t *tokens, const int32_t *status, float *conf,
                              void *stream);
int launch_sample(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                  const int32_t *meta, uint64_t seed, int32_t *states, int32_t *tokens,
                  uint8_t *ws, const WsLayout &w, int32_t *status, void *stream);
int launch_marginals(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                     const int32_t *meta, const double *logZ, const int32_t *tokens,
                     int32_t conf_mode, float *q, float *conf, uint8_t *ws, const WsLayout &w,
                     int32_t *status, void *stream);
// The parts of the two calls above, for the joint call fa_sample_marginals.
// States: the root and every midpoint (compact ids in ws at w.zc), and per
// position the pair of its two boundary states (w.tpair: index or -1;
// w.tdbit: its dense-mask bit or 0).  Tokens:
// the token draws and (finish) the state output; `pre` takes the dense-pair
// chunk sums from ws at w.tcs where w.tcs_ok marks a position.
int launch_sample_states(const DevTable &d, const Geometry &g, const float *tree,
                         const int32_t *meta, uint64_t seed, uint8_t *ws, const WsLayout &w,
                         int32_t *status, void *stream);
int launch_sample_tokens(const DevTable &d, const Geometry &g, const float *p, uint64_t seed,
                         int32_t *states, int32_t *tokens, uint8_t *ws, const WsLayout &w,
                         bool pre, int32_t *status, void *stream, bool finish = true);
// Message pass (alpha/beta at every boundary, range weights per cut).  ride
// (K >= 1): the launches of launch_sample_states (with `seed`, flagging
// `status`) ride on its last launches as extra workgroups.
int launch_marg_pass(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                     const int32_t *meta, uint8_t *ws, const WsLayout &w, void *stream,
                     bool ride, uint64_t seed, int32_t *status);
// The q writer and the confidence.  mode 0: the plain writer; 1: the
// streaming writer that also sums the token draws' dense-pair chunks (the
// boundary states in ws at w.zc; tokens unused); 2: after mode 1 and the
// token draws (launched without their finish): the PROB confidence of the
// sampled tokens, zeros and -inf for rows the draws flagged, and the states
// output (and -1 tokens of flagged rows) the draws' finish would write.
// marg_joint_ok tells whether modes 1 and 2 apply.
bool marg_joint_ok(const DevTable &d, const Geometry &g, const float *p, const float *q,
                   int32_t conf_mode, const WsLayout &w);
int launch_marg_out(const DevTable &d, const Geometry &g, const float *p, const double *logZ,
                    const int32_t *tokens, int32_t conf_mode, float *q, float *conf, uint8_t *ws,
                    const WsLayout &w, int mode, int32_t *status, void *stream, int32_t *states);
// The range weights per cut and the plain q writer (mode 0) from alpha/beta
// already in ws at w.va/w.ea and w.vb/w.eb (each vector with its own
// power-of-two exponent), as the chain's messages leave them.
int launch_marg_from_messages(const DevTable &d, const Geometry &g, const float *p,
                              const double *logZ, const int32_t *tokens, int32_t conf_mode,
                              float *q, float *conf, uint8_t *ws, const WsLayout &w,
                              int32_t *status, void *stream);

// The remasking step (commit.hip).
constexpr int kCommitMaxL = 8192;  // positions per row the selection holds in LDS
int launch_commit(int B, int L, int V, const float *conf, const int32_t *tokens, int steps_left,
                  int32_t *committed, int32_t *fresh, float *p, const int32_t *status,
                  void *stream);

}  // namespace fa

struct fa_table {
    fa::HostTable h;
};
