// Host-side automaton compiler: validation, dead-state trimming, the
// state-pair form of the edge chain model, the three label encodings
// (token lists, dense token masks, token ranges), the token-major inverse
// used by the marginals, and the device image.
//
// The state-pair form: a path over edges visits states, and the weight of
// an edge path summed over the edges between two consecutive states is
// c(a, v, b) = #{edges a->b whose label holds v}; this counts accepting edge
// paths exactly, so strings keep the weight the chain over edges gives them
// (paperfeed summary, "The insight: the constraint is a hidden Markov model";
// NFA path counting, "Arbitrary schedules and NFAs").
#include <algorithm>
#include <cstring>
#include <limits>
#include <new>
#include <numeric>
#include <stdexcept>

#include "fa_internal.h"

namespace fa {
namespace {

struct Err {
    int code;
};

template <class T>
void append_section(std::vector<uint8_t> &img, std::vector<size_t> &offs, const std::vector<T> &v)
{
    size_t off = (img.size() + 255) & ~size_t(255);
    img.resize(off + v.size() * sizeof(T));
    if (!v.empty()) std::memcpy(img.data() + off, v.data(), v.size() * sizeof(T));
    offs.push_back(off);
}

void build_image(HostTable &t)
{
    t.image.clear();
    t.offs.clear();
    append_section(t.image, t.offs, t.acc);
    append_section(t.image, t.offs, t.orig);
    append_section(t.image, t.offs, t.pair_a);
    append_section(t.image, t.offs, t.pair_b);
    append_section(t.image, t.offs, t.row_ptr);
    append_section(t.image, t.offs, t.col_ptr);
    append_section(t.image, t.offs, t.col_pairs);
    append_section(t.image, t.offs, t.pair_cls);
    append_section(t.image, t.offs, t.pair_aux);
    append_section(t.image, t.offs, t.list_off);
    append_section(t.image, t.offs, t.list_tok);
    append_section(t.image, t.offs, t.list_sel);
    append_section(t.image, t.offs, t.list_cnt);
    append_section(t.image, t.offs, t.sel_tok);
    append_section(t.image, t.offs, t.tm_off);
    append_section(t.image, t.offs, t.tm_pair);
    append_section(t.image, t.offs, t.tm_cnt);
    append_section(t.image, t.offs, t.dense_pair);
    append_section(t.image, t.offs, t.tokmask);
    append_section(t.image, t.offs, t.seg_off);
    append_section(t.image, t.offs, t.seg_lo);
    append_section(t.image, t.offs, t.seg_hi);
    append_section(t.image, t.offs, t.seg_cnt);
    append_section(t.image, t.offs, t.seg_lo_cut);
    append_section(t.image, t.offs, t.seg_hi_cut);
    append_section(t.image, t.offs, t.cuts);
    append_section(t.image, t.offs, t.cut_off);
    append_section(t.image, t.offs, t.cut_ev);
    append_section(t.image, t.offs, t.tok2sel);
    append_section(t.image, t.offs, t.tok2cut);
    append_section(t.image, t.offs, t.seg_pair);
    append_section(t.image, t.offs, t.map_n);
    append_section(t.image, t.offs, t.map_t);
    append_section(t.image, t.offs, t.tm_a);
    append_section(t.image, t.offs, t.tm_b);
    append_section(t.image, t.offs, t.ent_n_rc);
    append_section(t.image, t.offs, t.ent_n_src);
    append_section(t.image, t.offs, t.ent_t_rc);
    append_section(t.image, t.offs, t.ent_t_src);
    append_section(t.image, t.offs, t.sel_lb);
    append_section(t.image, t.offs, t.ind_pair);
    append_section(t.image, t.offs, t.dense_bits);
    append_section(t.image, t.offs, t.ev_a);
    append_section(t.image, t.offs, t.ev_b);
    append_section(t.image, t.offs, t.ev_w);
    append_section(t.image, t.offs, t.cutbits);
    append_section(t.image, t.offs, t.pair_colpos);
    append_section(t.image, t.offs, t.p2_a);
    append_section(t.image, t.offs, t.p2_b);
    append_section(t.image, t.offs, t.p2_row_ptr);
    append_section(t.image, t.offs, t.p2_col_ptr);
    append_section(t.image, t.offs, t.p2_col_pairs);
    append_section(t.image, t.offs, t.p2_colpos);
    append_section(t.image, t.offs, t.w1_n);
    append_section(t.image, t.offs, t.w1_t);
    append_section(t.image, t.offs, t.w2_n);
    append_section(t.image, t.offs, t.w2_t);
    append_section(t.image, t.offs, t.col_a);
    append_section(t.image, t.offs, t.p2_col_a);
    t.image.resize((t.image.size() + 255) & ~size_t(255));
}

}  // namespace

DevTable HostTable::device_view() const
{
    DevTable d{};
    d.S = S;
    d.Sp = Sp;
    d.V = V;
    d.start = start;
    d.n_acc = (int32_t)acc.size();
    d.npairs = npairs();
    d.nsel = nsel();
    d.use_sel = use_sel ? 1 : 0;
    d.ndense = ndense();
    d.nseg = nseg();
    d.ncut = ncut();
    d.has_cnt = has_cnt ? 1 : 0;
    d.selbit = selbit ? 1 : 0;
    d.first_sparse = first_sparse ? 1 : 0;
    d.first_pairs = first_pairs ? 1 : 0;
    d.map_first_sparse = map_first_sparse ? 1 : 0;
    d.leafless = leafless ? 1 : 0;
    const uint8_t *b = static_cast<const uint8_t *>(dev);
    size_t k = 0;
    auto nxt = [&](auto *&ptr) {
        ptr = reinterpret_cast<std::remove_reference_t<decltype(ptr)>>(b + offs[k++]);
    };
    nxt(d.acc); nxt(d.orig); nxt(d.pair_a); nxt(d.pair_b); nxt(d.row_ptr); nxt(d.col_ptr);
    nxt(d.col_pairs); nxt(d.pair_cls); nxt(d.pair_aux); nxt(d.list_off); nxt(d.list_tok);
    nxt(d.list_sel); nxt(d.list_cnt); nxt(d.sel_tok); nxt(d.tm_off); nxt(d.tm_pair);
    nxt(d.tm_cnt); nxt(d.dense_pair); nxt(d.tokmask); nxt(d.seg_off); nxt(d.seg_lo);
    nxt(d.seg_hi); nxt(d.seg_cnt); nxt(d.seg_lo_cut); nxt(d.seg_hi_cut); nxt(d.cuts);
    nxt(d.cut_off); nxt(d.cut_ev); nxt(d.tok2sel); nxt(d.tok2cut); nxt(d.seg_pair);
    nxt(d.map_n); nxt(d.map_t); nxt(d.tm_a); nxt(d.tm_b);
    nxt(d.ent_n_rc); nxt(d.ent_n_src); nxt(d.ent_t_rc); nxt(d.ent_t_src); nxt(d.sel_lb);
    nxt(d.ind_pair);
    d.n_ind = (int32_t)ind_pair.size();
    nxt(d.dense_bits);
    d.dense_words = (V + 31) / 32;
    nxt(d.ev_a);
    nxt(d.ev_b);
    nxt(d.ev_w);
    nxt(d.cutbits);
    nxt(d.pair_colpos);
    nxt(d.p2_a); nxt(d.p2_b); nxt(d.p2_row_ptr); nxt(d.p2_col_ptr); nxt(d.p2_col_pairs);
    nxt(d.p2_colpos); nxt(d.w1_n); nxt(d.w1_t); nxt(d.w2_n); nxt(d.w2_t);
    nxt(d.col_a); nxt(d.p2_col_a);
    d.second_sparse = second_sparse ? 1 : 0;
    d.live_states = live_states ? 1 : 0;
    d.np2 = (int32_t)p2_a.size();
    d.nwin = nwin;
    d.win_cols = win_cols;
    d.n_tm = (int32_t)tm_pair.size();
    if (map_n.empty()) {
        d.map_n = nullptr;
        d.map_t = nullptr;
    }
    if (!has_cnt) {
        d.list_cnt = nullptr;
        d.tm_cnt = nullptr;
    }
    return d;
}

int make_geometry(const HostTable &t, int32_t B, int32_t L, Geometry *g)
{
    if (B < 0 || L < 0) return FA_EINVAL;
    // positions index 24-bit fields of the kernels; this also keeps Lpad
    // (below 2^24) far from int32 overflow
    if (L >= (1 << 24)) return FA_ETOOBIG;
    int32_t Lpad = 1, K = 0;
    while (Lpad < L) {
        Lpad <<= 1;
        ++K;
    }
    g->B = B;
    g->b0 = 0;
    g->L = L;
    g->Lpad = Lpad;
    g->K = K;
    g->Sp = t.Sp;
    g->mat = (size_t)t.Sp * t.Sp;
    g->tree_floats = L > 0 ? (size_t)B * 2 * Lpad * g->mat : 0;
    g->meta_ints = L > 0 ? (size_t)B * 2 * Lpad * 3 * t.Sp : 0;
    return FA_OK;
}

int plan_chunks(const HostTable &t, int32_t B, int32_t L, bool map, StepChunks *c)
{
    Geometry g;
    if (int rc = make_geometry(t, B, L, &g)) return rc;
    if ((int64_t)g.Lpad * 2 > 65535) return FA_ETOOBIG;
    c->rows = std::max<int32_t>(1, std::min<int32_t>(std::max<int32_t>(B, 1), 32767 / g.Lpad));
    c->count = B == 0 ? 0 : (B + c->rows - 1) / c->rows;
    const int32_t last = B - (c->count - 1) * c->rows;
    size_t slot = 0;
    for (int32_t nb : {c->rows, last}) {
        if (nb <= 0) continue;
        Geometry gc;
        make_geometry(t, nb, L, &gc);
        slot = std::max(slot, map ? map_ws_layout(t, gc).total : ws_layout(t, gc).total);
    }
    c->slot = (slot + 255) & ~size_t(255);
    return FA_OK;
}

int tree_ksplit(const Geometry &g, int level)
{
    // large levels run on the 128x128 kernel; smaller ones on 64x64 tiles,
    // split along K only while the tiles with their splits still fit the
    // 256 compute units once and every split keeps a K range of at least
    // 256: the reduce is a launch of its own (about as long as 8 K blocks of
    // 32), so shorter splits cost more than they save
    const long long nn = g.Lpad >> level;
    const long long big = (long long)g.B * nn * (g.Sp / 128) * (g.Sp / 128);
    if (g.Sp % 128 == 0 && big >= 256) return 1;
    const long long small = (long long)g.B * nn * (g.Sp / 64) * (g.Sp / 64);
    int s = 1;
    // the split must divide the K blocks of 64 exactly
    while ((g.Sp / 64) % (s * 2) == 0 && small * s * 2 <= 256 && g.Sp / (s * 2) >= 256) s *= 2;
    return s;
}

WsLayout ws_layout(const HostTable &t, const Geometry &g)
{
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    WsLayout w;
    size_t BL = (size_t)g.B * g.L;
    size_t o = 0;  // emission reduce region
    size_t BLpad = (BL + kDenseTile - 1) / kDenseTile * kDenseTile;
    if (t.ndense() && BL > 0) {
        // V split of the dense-mask contraction: chunks of whole 256-token
        // steps; the count minimises (rounds of kDenseSlots workgroups) x
        // (steps per chunk + a fixed cost of two steps per workgroup)
        const long long tiles = (long long)(BLpad / kDenseTile);
        const long long steps = (t.V + 255) / 256;
        double best = 1e300;
        const long long nc_lo = (steps + kDenseStepsMax - 1) / kDenseStepsMax;
        const long long nc_hi = std::max(nc_lo, std::min(steps, 64LL));
        for (long long nc = nc_lo; nc <= nc_hi; ++nc) {
            const long long st = (steps + nc - 1) / nc;
            const long long n = (steps + st - 1) / st;
            const long long rounds = (tiles * n + kDenseSlots - 1) / kDenseSlots;
            const double cost = (double)rounds * (double)(st + 2);
            if (cost < best) {
                best = cost;
                w.n_vchunks = (int32_t)n;
                w.vchunk = (int32_t)(st * 256);
            }
        }
        // token-list copy: LDS-buffered when every chunk holds few such tokens
        int32_t most = 0;
        for (int32_t c = 0; c < w.n_vchunks; ++c) {
            const int32_t lo = c * w.vchunk, hi = std::min(t.V, lo + w.vchunk);
            const int32_t n = (int32_t)(std::lower_bound(t.sel_tok.begin(), t.sel_tok.end(), hi) -
                                        std::lower_bound(t.sel_tok.begin(), t.sel_tok.end(), lo));
            most = std::max(most, n);
        }
        w.sel_mode = most <= kDenseSelLds ? 1 : 2;
    }
    // the compact token copy and the stored indirect pair values persist
    // through the step (the leaf level of the marginal message pass reads
    // pair values from them); every other region is a union over one call
    const bool fused = g.Sp <= kLeafTile;  // leaves straight from pair values
    w.psel = o; o = al(o + (t.use_sel ? BL * t.nsel() * sizeof(float) : 0));
    // one spare float: a clamped read of slot 0 stays inside even with no indirect pairs
    w.ndval = o; o = al(o + (fused ? (BL * t.ind_pair.size() + 1) * sizeof(float) : 0));
    // the folded leaf pair values: read by the sparse first level, and on a
    // leafless table by the leaf-level draws too (so kept through the step)
    w.pvf = o; o = al(o + (t.first_sparse || t.first_pairs ? BL * t.npairs() * sizeof(float) : 0));
    const size_t a0 = o;
    w.dpart = o; o = al(o + (size_t)w.n_vchunks * BLpad * kDenseMax * sizeof(float));
    w.dval = o; o = al(o + (t.ndense() && !fused ? BL * kDenseMax * sizeof(float) : 0));
    w.cutp = o; o = al(o + BL * t.ncut() * sizeof(double));
    w.val = o; o = al(o + (fused ? 0 : BL * t.npairs() * sizeof(float)));
    size_t a1 = o;
    o = a0;  // span tree region
    size_t kp = 0;
    for (int level = 1; level <= g.K; ++level) {
        const int s = tree_ksplit(g, level);
        if (s > 1) kp = std::max(kp, (size_t)g.B * (g.Lpad >> level) * s * g.mat);
    }
    w.kpart = o; o = al(o + kp * sizeof(float));
    const size_t nbd = t.live_states ? (size_t)g.B * (g.Lpad + 1) : 0;  // boundaries
    w.lbits = o; o = al(o + nbd * 2 * ((g.Sp + 31) / 32) * sizeof(uint32_t));
    w.live = o; o = al(o + nbd * g.Sp * sizeof(int32_t));
    w.nlive = o; o = al(o + nbd * sizeof(int32_t));
    size_t a2 = o;
    o = a0;  // marginals region
    size_t nv = (size_t)g.B * (g.Lpad + 1);
    w.va = o; o = al(o + nv * g.Sp * sizeof(float));
    w.vb = o; o = al(o + nv * g.Sp * sizeof(float));
    w.ea = o; o = al(o + nv * sizeof(int32_t));
    w.eb = o; o = al(o + nv * sizeof(int32_t));
    w.rcut = o; o = al(o + BL * t.ncut() * sizeof(float));
    w.pw_nl = t.nsel() <= kSelMax ? t.nsel() : 0;
    w.pw_ld = (kDenseMax + w.pw_nl + 3) & ~3;
    w.pw = o; o = al(o + BL * (size_t)w.pw_ld * sizeof(float));
    w.hpart = o; o = al(o + BL * kQParts * sizeof(double));  // the q writer's row parts
    size_t a4 = o;
    // sampler region, apart from the others: the joint call keeps the drawn
    // boundary states through the message pass, and the dense-pair chunk
    // sums of the token draws from the q writer to the draws
    o = al(std::max(std::max(a1, a2), a4));
    w.zc = o; o = al(o + (size_t)g.B * (g.Lpad + 1) * sizeof(int32_t));
    w.tpair = o; o = al(o + BL * sizeof(int32_t));
    w.tdbit = o; o = al(o + BL * sizeof(uint32_t));
    w.tcs_nch = (t.V / 4 + kRowChunk4 - 1) / kRowChunk4;
    const bool joint = t.ndense() > 0 && t.V % 4 == 0;
    w.tcs = o; o = al(o + (joint ? BL * (size_t)w.tcs_nch * 4 * sizeof(double) : 0));
    w.tcs_ok = o; o = al(o + (joint ? BL * sizeof(int32_t) : 0));
    // first-level nodes on the two-step pattern: written by the first level,
    // read by the second, apart from every per-call region
    const size_t n2 = t.second_sparse ? (size_t)g.B * (g.Lpad / 2) * t.p2_a.size() : 0;
    w.pv2 = o; o = al(o + n2 * sizeof(float));
    w.pv2alt = o; o = al(o + n2 * sizeof(float));
    w.total = o;
    if (w.total == 0) w.total = 256;
    return w;
}

// the two-step pattern of the pairs: (a, c) for every pairs (a, k), (k, c),
// sorted by (a, c), with row pointers, the (c, a) order and its inverse
static void build_two_step(HostTable &t)
{
    const int32_t S = t.S;
    std::vector<int32_t> mark(S, -1), cs;
    t.p2_row_ptr.assign(S + 1, 0);
    for (int32_t a = 0; a < S; ++a) {
        cs.clear();
        for (int32_t e = t.row_ptr[a]; e < t.row_ptr[a + 1]; ++e) {
            const int32_t k = t.pair_b[e];
            for (int32_t e2 = t.row_ptr[k]; e2 < t.row_ptr[k + 1]; ++e2) {
                const int32_t c = t.pair_b[e2];
                if (mark[c] != a) {
                    mark[c] = a;
                    cs.push_back(c);
                }
            }
        }
        std::sort(cs.begin(), cs.end());
        for (int32_t c : cs) {
            t.p2_a.push_back(a);
            t.p2_b.push_back(c);
        }
        t.p2_row_ptr[a + 1] = (int32_t)t.p2_a.size();
    }
    const int32_t n2 = (int32_t)t.p2_a.size();
    t.p2_col_ptr.assign(S + 1, 0);
    for (int32_t q = 0; q < n2; ++q) t.p2_col_ptr[t.p2_b[q] + 1]++;
    for (int32_t s = 0; s < S; ++s) t.p2_col_ptr[s + 1] += t.p2_col_ptr[s];
    t.p2_col_pairs.resize(n2);
    std::iota(t.p2_col_pairs.begin(), t.p2_col_pairs.end(), 0);
    std::stable_sort(t.p2_col_pairs.begin(), t.p2_col_pairs.end(), [&](int32_t x, int32_t y) {
        return t.p2_b[x] != t.p2_b[y] ? t.p2_b[x] < t.p2_b[y] : t.p2_a[x] < t.p2_a[y];
    });
    t.p2_colpos.resize(n2);
    for (int32_t k = 0; k < n2; ++k) t.p2_colpos[t.p2_col_pairs[k]] = k;
}

// for every state s and window w: the first entry of s's row walk (targets
// ascending) and of its column walk (sources ascending) at or past column
// w * win_cols; [S][nwin + 1], the last the walk's end
static void window_offsets(const HostTable &t, const std::vector<int32_t> &rp,
                           const std::vector<int32_t> &cp, const std::vector<int32_t> &pa,
                           const std::vector<int32_t> &pb, const std::vector<int32_t> &cpairs,
                           std::vector<int32_t> &wn, std::vector<int32_t> &wt)
{
    const int32_t S = t.S, nw = t.nwin;
    wn.assign((size_t)S * (nw + 1), 0);
    wt.assign((size_t)S * (nw + 1), 0);
    for (int32_t s = 0; s < S; ++s) {
        int32_t e = rp[s], f = cp[s];
        for (int32_t w = 0; w <= nw; ++w) {
            const int64_t lim = (int64_t)w * t.win_cols;
            while (e < rp[s + 1] && pb[e] < lim) ++e;
            while (f < cp[s + 1] && pa[cpairs[f]] < lim) ++f;
            wn[(size_t)s * (nw + 1) + w] = w == nw ? rp[s + 1] : e;
            wt[(size_t)s * (nw + 1) + w] = w == nw ? cp[s + 1] : f;
        }
    }
}

static int compile(int32_t S, int32_t V, int32_t start, const int32_t *accept, int32_t n_accept,
                   int64_t E, const int32_t *src, const int32_t *dst, const int64_t *label_off,
                   const int32_t *label_tok, uint32_t flags, HostTable &t)
{
    const bool ranges = flags & FA_LABEL_RANGES;
    if (S < 1 || V < 1 || start < 0 || start >= S || n_accept < 0 || E < 0) return FA_EINVAL;
    if ((n_accept > 0 && !accept) || (E > 0 && (!src || !dst || !label_off))) return FA_EINVAL;
    if ((flags & FA_DFA) && (flags & FA_NFA)) return FA_EINVAL;
    if (flags & ~uint32_t(FA_DFA | FA_NFA | FA_LABEL_RANGES | FA_NO_TRIM | FA_FIRST_LEVEL_SPARSE |
                          FA_FIRST_LEVEL_DENSE | FA_SECOND_LEVEL_SPARSE | FA_LIVE_STATES |
                          FA_FIRST_LEVEL_PAIRS))
        return FA_EINVAL;
    {
        const uint32_t first = flags & (FA_FIRST_LEVEL_SPARSE | FA_FIRST_LEVEL_DENSE | FA_FIRST_LEVEL_PAIRS);
        if (first & (first - 1)) return FA_EINVAL;  // at most one first-level form
    }
    if (E > std::numeric_limits<int32_t>::max()) return FA_ETOOBIG;
    if (E > 0 && label_off[0] != 0) return FA_EINVAL;
    for (int32_t k = 0; k < n_accept; ++k)
        if (accept[k] < 0 || accept[k] >= S) return FA_EINVAL;
    if (E > 0 && label_off[E] > 0 && !label_tok) return FA_EINVAL;

    // per-edge labels: sorted unique tokens, or sorted disjoint ranges
    std::vector<std::vector<int32_t>> lab((size_t)E);
    for (int64_t e = 0; e < E; ++e) {
        if (src[e] < 0 || src[e] >= S || dst[e] < 0 || dst[e] >= S) return FA_EINVAL;
        int64_t b0 = label_off[e], b1 = label_off[e + 1];
        if (b1 < b0) return FA_EINVAL;
        std::vector<int32_t> &L = lab[(size_t)e];
        if (ranges) {
            if ((b1 - b0) % 2) return FA_EINVAL;
            std::vector<std::pair<int32_t, int32_t>> rr;
            for (int64_t k = b0; k < b1; k += 2) {
                int32_t lo = label_tok[k], hi = label_tok[k + 1];
                if (lo < 0 || hi > V || lo > hi) return FA_EINVAL;
                if (lo < hi) rr.emplace_back(lo, hi);
            }
            std::sort(rr.begin(), rr.end());
            for (size_t k = 1; k < rr.size(); ++k)
                if (rr[k].first < rr[k - 1].second) return FA_EINVAL;
            for (auto &r : rr) {
                L.push_back(r.first);
                L.push_back(r.second);
            }
        } else {
            L.assign(label_tok + b0, label_tok + b1);
            for (int32_t v : L)
                if (v < 0 || v >= V) return FA_EINVAL;
            std::sort(L.begin(), L.end());
            L.erase(std::unique(L.begin(), L.end()), L.end());
        }
    }
    // determinism check on the whole input automaton
    if (flags & FA_DFA) {
        if (ranges) {
            std::vector<std::vector<std::pair<int32_t, int32_t>>> per(S);
            for (int64_t e = 0; e < E; ++e)
                for (size_t k = 0; k < lab[e].size(); k += 2) per[src[e]].emplace_back(lab[e][k], lab[e][k + 1]);
            for (auto &v : per) {
                std::sort(v.begin(), v.end());
                for (size_t k = 1; k < v.size(); ++k)
                    if (v[k].first < v[k - 1].second) return FA_ENOTDET;
            }
        } else {
            std::vector<uint64_t> keys;
            for (int64_t e = 0; e < E; ++e)
                for (int32_t v : lab[e]) keys.push_back(((uint64_t)(uint32_t)src[e] << 32) | (uint32_t)v);
            std::sort(keys.begin(), keys.end());
            for (size_t k = 1; k < keys.size(); ++k)
                if (keys[k] == keys[k - 1]) return FA_ENOTDET;
        }
    }
    // trimming: reachable from start and co-reachable to F over non-empty edges
    std::vector<char> fwd(S, 0), bwd(S, 0), keep(S, 1);
    if (!(flags & FA_NO_TRIM)) {
        std::vector<std::vector<int32_t>> out(S), in(S);
        for (int64_t e = 0; e < E; ++e)
            if (!lab[e].empty()) {
                out[src[e]].push_back(dst[e]);
                in[dst[e]].push_back(src[e]);
            }
        std::vector<int32_t> st{start};
        fwd[start] = 1;
        while (!st.empty()) {
            int32_t a = st.back();
            st.pop_back();
            for (int32_t b : out[a]) if (!fwd[b]) { fwd[b] = 1; st.push_back(b); }
        }
        for (int32_t k = 0; k < n_accept; ++k)
            if (!bwd[accept[k]]) { bwd[accept[k]] = 1; st.push_back(accept[k]); }
        while (!st.empty()) {
            int32_t b = st.back();
            st.pop_back();
            for (int32_t a : in[b]) if (!bwd[a]) { bwd[a] = 1; st.push_back(a); }
        }
        for (int32_t s = 0; s < S; ++s) keep[s] = fwd[s] && bwd[s];
        keep[start] = 1;
    }
    std::vector<int32_t> cid(S, -1);
    t.orig.clear();
    for (int32_t s = 0; s < S; ++s)
        if (keep[s]) {
            cid[s] = (int32_t)t.orig.size();
            t.orig.push_back(s);
        }
    t.S_orig = S;
    t.V = V;
    t.S = (int32_t)t.orig.size();
    // padded to 64; for large automata to 256 (or 128) when that adds at
    // most 10% to the S^3 products, so the span tree runs on the large-tile
    // kernels (Sp a multiple of 256 or 128)
    t.Sp = (t.S + kSpAlign - 1) / kSpAlign * kSpAlign;
    for (int32_t a : {256, 128}) {
        const double sp = (double)((t.S + a - 1) / a * a);
        if (t.S >= 1024 && sp * sp * sp <= 1.10 * (double)t.Sp * t.Sp * t.Sp) {
            t.Sp = (int32_t)sp;
            break;
        }
    }
    t.start = cid[start];
    t.acc.clear();
    for (int32_t k = 0; k < n_accept; ++k)
        if (cid[accept[k]] >= 0) t.acc.push_back(cid[accept[k]]);
    std::sort(t.acc.begin(), t.acc.end());
    t.acc.erase(std::unique(t.acc.begin(), t.acc.end()), t.acc.end());

    // edges between kept states, grouped by (a, b)
    std::vector<int64_t> eids;
    for (int64_t e = 0; e < E; ++e)
        if (!lab[e].empty() && cid[src[e]] >= 0 && cid[dst[e]] >= 0) eids.push_back(e);
    std::sort(eids.begin(), eids.end(), [&](int64_t x, int64_t y) {
        int32_t ax = cid[src[x]], ay = cid[src[y]], bx = cid[dst[x]], by = cid[dst[y]];
        return ax != ay ? ax < ay : (bx != by ? bx < by : x < y);
    });
    t.pair_a.clear(); t.pair_b.clear(); t.pair_cls.clear(); t.pair_aux.clear();
    t.list_off.assign(1, 0); t.list_tok.clear(); t.list_cnt.clear();
    t.seg_off.assign(1, 0); t.seg_lo.clear(); t.seg_hi.clear(); t.seg_cnt.clear();
    t.has_cnt = false;
    std::vector<int64_t> pair_size;
    std::vector<int32_t> maxcnt;
    for (size_t k0 = 0; k0 < eids.size();) {
        size_t k1 = k0;
        int32_t a = cid[src[eids[k0]]], b = cid[dst[eids[k0]]];
        while (k1 < eids.size() && cid[src[eids[k1]]] == a && cid[dst[eids[k1]]] == b) ++k1;
        t.pair_a.push_back(a);
        t.pair_b.push_back(b);
        if (ranges) {
            // sweep the edges' ranges into disjoint segments with counts
            std::vector<std::pair<int32_t, int32_t>> ev;  // (position, +1/-1)
            for (size_t k = k0; k < k1; ++k) {
                const auto &L = lab[eids[k]];
                for (size_t r = 0; r < L.size(); r += 2) {
                    ev.emplace_back(L[r], +1);
                    ev.emplace_back(L[r + 1], -1);
                }
            }
            std::sort(ev.begin(), ev.end());
            int32_t depth = 0, mc = 0;
            int64_t sz = 0;
            for (size_t k = 0; k < ev.size();) {
                int32_t x = ev[k].first;
                int32_t before = depth;
                while (k < ev.size() && ev[k].first == x) depth += ev[k++].second;
                (void)before;
                if (k < ev.size() && depth > 0) {
                    int32_t y = ev[k].first;
                    // merge with the previous segment if contiguous with equal count
                    if (!t.seg_hi.empty() && (int64_t)t.seg_lo.size() > t.seg_off.back() &&
                        t.seg_hi.back() == x && t.seg_cnt.back() == (float)depth)
                        t.seg_hi.back() = y;
                    else {
                        t.seg_lo.push_back(x);
                        t.seg_hi.push_back(y);
                        t.seg_cnt.push_back((float)depth);
                    }
                    sz += (int64_t)(y - x) * depth;
                    mc = std::max(mc, depth);
                }
            }
            t.seg_off.push_back((int32_t)t.seg_lo.size());
            t.list_off.push_back((int32_t)t.list_tok.size());
            t.pair_cls.push_back(kRange);
            pair_size.push_back(sz);
            maxcnt.push_back(mc);
            if (mc > 1) t.has_cnt = true;
        } else {
            std::vector<int32_t> all;
            for (size_t k = k0; k < k1; ++k) all.insert(all.end(), lab[eids[k]].begin(), lab[eids[k]].end());
            std::sort(all.begin(), all.end());
            int32_t mc = 0;
            for (size_t k = 0; k < all.size();) {
                size_t k2 = k;
                while (k2 < all.size() && all[k2] == all[k]) ++k2;
                t.list_tok.push_back(all[k]);
                t.list_cnt.push_back((float)(k2 - k));
                mc = std::max(mc, (int32_t)(k2 - k));
                k = k2;
            }
            if (t.list_tok.size() > (size_t)std::numeric_limits<int32_t>::max()) throw Err{FA_ETOOBIG};
            t.list_off.push_back((int32_t)t.list_tok.size());
            t.seg_off.push_back((int32_t)t.seg_lo.size());
            t.pair_cls.push_back(kList);
            pair_size.push_back((int64_t)all.size());
            maxcnt.push_back(mc);
            if (mc > 1) t.has_cnt = true;
        }
        t.pair_aux.push_back(-1);
        k0 = k1;
    }
    const int32_t np = t.npairs();
    // dense-mask class: the largest count-1 token lists
    t.dense_pair.clear();
    if (!ranges) {
        int64_t dense_min = std::max<int64_t>(2048, V / 16);
        std::vector<int32_t> cand;
        for (int32_t q = 0; q < np; ++q)
            if (maxcnt[q] == 1 && pair_size[q] >= dense_min) cand.push_back(q);
        std::stable_sort(cand.begin(), cand.end(),
                         [&](int32_t x, int32_t y) { return pair_size[x] > pair_size[y]; });
        if ((int32_t)cand.size() > kDenseMax) cand.resize(kDenseMax);
        std::sort(cand.begin(), cand.end());
        for (int32_t q : cand) {
            t.pair_cls[q] = kDense;
            t.pair_aux[q] = (int32_t)t.dense_pair.size();
            t.dense_pair.push_back(q);
        }
        // move dense pairs' tokens into the mask and out of the lists
        t.tokmask.assign(t.ndense() ? (size_t)V : 0, 0u);
        std::vector<int32_t> off2(1, 0), tok2;
        std::vector<float> cnt2;
        for (int32_t q = 0; q < np; ++q) {
            if (t.pair_cls[q] == kDense) {
                uint32_t bit = 1u << t.pair_aux[q];
                for (int32_t k = t.list_off[q]; k < t.list_off[q + 1]; ++k) t.tokmask[t.list_tok[k]] |= bit;
            } else {
                tok2.insert(tok2.end(), t.list_tok.begin() + t.list_off[q], t.list_tok.begin() + t.list_off[q + 1]);
                cnt2.insert(cnt2.end(), t.list_cnt.begin() + t.list_off[q], t.list_cnt.begin() + t.list_off[q + 1]);
            }
            off2.push_back((int32_t)tok2.size());
        }
        t.list_off.swap(off2);
        t.list_tok.swap(tok2);
        t.list_cnt.swap(cnt2);
    } else {
        t.tokmask.clear();
    }
    if (!t.has_cnt) t.list_cnt.clear();
    // row and column orders of the pairs
    t.row_ptr.assign(t.S + 1, 0);
    t.col_ptr.assign(t.S + 1, 0);
    for (int32_t q = 0; q < np; ++q) {
        t.row_ptr[t.pair_a[q] + 1]++;
        t.col_ptr[t.pair_b[q] + 1]++;
    }
    for (int32_t s = 0; s < t.S; ++s) {
        t.row_ptr[s + 1] += t.row_ptr[s];
        t.col_ptr[s + 1] += t.col_ptr[s];
    }
    t.col_pairs.resize(np);
    std::iota(t.col_pairs.begin(), t.col_pairs.end(), 0);
    std::stable_sort(t.col_pairs.begin(), t.col_pairs.end(), [&](int32_t x, int32_t y) {
        return t.pair_b[x] != t.pair_b[y] ? t.pair_b[x] < t.pair_b[y] : t.pair_a[x] < t.pair_a[y];
    });
    t.pair_colpos.resize(np);
    for (int32_t k = 0; k < np; ++k) t.pair_colpos[t.col_pairs[k]] = k;
    // token-major inverse of the LIST pairs
    t.sel_tok = t.list_tok;
    std::sort(t.sel_tok.begin(), t.sel_tok.end());
    t.sel_tok.erase(std::unique(t.sel_tok.begin(), t.sel_tok.end()), t.sel_tok.end());
    const int32_t ns = t.nsel();
    t.list_sel.resize(t.list_tok.size());
    for (size_t k = 0; k < t.list_tok.size(); ++k)
        t.list_sel[k] = (int32_t)(std::lower_bound(t.sel_tok.begin(), t.sel_tok.end(), t.list_tok[k]) - t.sel_tok.begin());
    t.tm_off.assign(ns + 1, 0);
    for (int32_t s : t.list_sel) t.tm_off[s + 1]++;
    for (int32_t s = 0; s < ns; ++s) t.tm_off[s + 1] += t.tm_off[s];
    t.tm_pair.resize(t.list_tok.size());
    t.tm_cnt.assign(t.has_cnt ? t.list_tok.size() : 0, 1.f);
    {
        std::vector<int32_t> fill(t.tm_off.begin(), t.tm_off.end() - 1);
        for (int32_t q = 0; q < np; ++q)
            for (int32_t k = t.list_off[q]; k < t.list_off[q + 1]; ++k) {
                int32_t pos = fill[t.list_sel[k]]++;
                t.tm_pair[pos] = q;
                if (t.has_cnt) t.tm_cnt[pos] = t.list_cnt[k];
            }
    }
    t.tm_a.resize(t.tm_pair.size());
    t.tm_b.resize(t.tm_pair.size());
    for (size_t k = 0; k < t.tm_pair.size(); ++k) {
        t.tm_a[k] = t.pair_a[t.tm_pair[k]];
        t.tm_b[k] = t.pair_b[t.tm_pair[k]];
    }
    // range cut points and events
    t.cuts.clear();
    for (size_t s = 0; s < t.seg_lo.size(); ++s) {
        t.cuts.push_back(t.seg_lo[s]);
        t.cuts.push_back(t.seg_hi[s]);
    }
    std::sort(t.cuts.begin(), t.cuts.end());
    t.cuts.erase(std::unique(t.cuts.begin(), t.cuts.end()), t.cuts.end());
    t.seg_lo_cut.resize(t.seg_lo.size());
    t.seg_hi_cut.resize(t.seg_lo.size());
    for (size_t s = 0; s < t.seg_lo.size(); ++s) {
        t.seg_lo_cut[s] = (int32_t)(std::lower_bound(t.cuts.begin(), t.cuts.end(), t.seg_lo[s]) - t.cuts.begin());
        t.seg_hi_cut[s] = (int32_t)(std::lower_bound(t.cuts.begin(), t.cuts.end(), t.seg_hi[s]) - t.cuts.begin());
    }
    t.cut_off.assign(t.ncut() + 1, 0);
    for (size_t s = 0; s < t.seg_lo.size(); ++s) {
        t.cut_off[t.seg_lo_cut[s] + 1]++;
        t.cut_off[t.seg_hi_cut[s] + 1]++;
    }
    for (int32_t c = 0; c < t.ncut(); ++c) t.cut_off[c + 1] += t.cut_off[c];
    t.cut_ev.resize(2 * t.seg_lo.size());
    {
        std::vector<int32_t> fill(t.cut_off.begin(), t.cut_off.end() - 1);
        for (size_t s = 0; s < t.seg_lo.size(); ++s) {
            t.cut_ev[fill[t.seg_lo_cut[s]]++] = (int32_t)(2 * s);
            t.cut_ev[fill[t.seg_hi_cut[s]]++] = (int32_t)(2 * s + 1);
        }
    }
    if (!t.has_cnt) t.seg_cnt.assign(t.seg_lo.size(), 1.f);
    t.seg_pair.resize(t.seg_lo.size());
    for (int32_t q = 0; q < np; ++q)
        for (int32_t s = t.seg_off[q]; s < t.seg_off[q + 1]; ++s) t.seg_pair[s] = q;
    // per cut event: the states (a, b) of its pair and its count, negative at a segment end
    t.ev_a.resize(t.cut_ev.size());
    t.ev_b.resize(t.cut_ev.size());
    t.ev_w.resize(t.cut_ev.size());
    for (size_t k = 0; k < t.cut_ev.size(); ++k) {
        const int32_t ev = t.cut_ev[k], sg = ev >> 1, q = t.seg_pair[sg];
        t.ev_a[k] = t.pair_a[q];
        t.ev_b[k] = t.pair_b[q];
        t.ev_w[k] = (ev & 1) ? -t.seg_cnt[sg] : t.seg_cnt[sg];
    }
    t.tok2sel.assign(ns > 0 ? (size_t)V : 0, -1);
    for (int32_t s = 0; s < ns; ++s) t.tok2sel[t.sel_tok[s]] = s;
    // bit v % 32 of word v / 32: a cut point sits at token v (cuts below V)
    t.cutbits.assign(t.ncut() > 0 ? (size_t)(V + 31) / 32 : 0, 0u);
    for (int32_t c = 0; c < t.ncut(); ++c)
        if (t.cuts[c] < V) t.cutbits[t.cuts[c] / 32] |= 1u << (t.cuts[c] % 32);
    t.tok2cut.assign(t.ncut() > 0 ? (size_t)V : 0, -1);
    for (int32_t c = 0, v = 0; v < (t.ncut() > 0 ? V : 0); ++v) {
        while (c < t.ncut() && t.cuts[c] <= v) ++c;
        t.tok2cut[v] = c - 1;
    }
    t.map_n.clear();
    t.map_t.clear();
    if (t.Sp <= kMapMaxSp) {
        t.map_n.assign((size_t)t.Sp * t.Sp, -1);
        t.map_t.assign((size_t)t.Sp * t.Sp, -1);
        for (int32_t q = 0; q < np; ++q) {
            t.map_n[(size_t)t.pair_a[q] * t.Sp + t.pair_b[q]] = q;
            t.map_t[(size_t)t.pair_b[q] * t.Sp + t.pair_a[q]] = q;
        }
    }
    // only tables with dense-mask pairs stream p through a kernel that can copy
    // the token-list tokens (range tables hold no token lists)
    t.use_sel = t.ndense() > 0 && ns > 0 && ns <= kSelMax;
    // one bit array per dense pair (bit v%32 of word v/32: v in its label)
    const int32_t nw = (V + 31) / 32;
    t.dense_bits.assign((size_t)t.ndense() * nw, 0u);
    for (int32_t j = 0; j < t.ndense(); ++j)
        for (int32_t v = 0; v < V; ++v)
            if ((t.tokmask[v] >> j) & 1u) t.dense_bits[(size_t)j * nw + v / 32] |= 1u << (v % 32);
    t.selbit = t.ndense() > 0 && t.ndense() < 32 && ns > 0;
    if (t.selbit)
        for (int32_t v : t.sel_tok) t.tokmask[v] |= kSelBit;
    // first token-list token at or after every multiple of 256 tokens
    t.sel_lb.resize((size_t)V / 256 + 2);
    for (size_t k = 0; k < t.sel_lb.size(); ++k)
        t.sel_lb[k] = (int32_t)(std::lower_bound(t.sel_tok.begin(), t.sel_tok.end(), (int64_t)k * 256) -
                                t.sel_tok.begin());
    // leaf entries (stored row, column and value source) in both orders
    t.ent_n_rc.clear(); t.ent_n_src.clear(); t.ent_t_rc.clear(); t.ent_t_src.clear();
    t.ind_pair.clear();
    if (t.Sp < 65536) {
        std::vector<int32_t> ind_of(np, -1);
        for (int32_t q = 0; q < np; ++q) {
            bool direct = false;
            if (t.pair_cls[q] == kList && t.list_off[q + 1] - t.list_off[q] == 1) {
                const int32_t k = t.list_off[q];
                direct = t.list_cnt.empty() || t.list_cnt[k] == 1.f;
            }
            if (!direct) {
                ind_of[q] = (int32_t)t.ind_pair.size();
                t.ind_pair.push_back(q);
            }
        }
        auto src_code = [&](int32_t q) -> int32_t {
            if (ind_of[q] >= 0) return -1 - ind_of[q];
            const int32_t k = t.list_off[q];
            return t.use_sel ? t.list_sel[k] : t.list_tok[k];
        };
        t.ent_n_rc.resize(np); t.ent_n_src.resize(np); t.ent_t_rc.resize(np); t.ent_t_src.resize(np);
        for (int32_t q = 0; q < np; ++q) {
            t.ent_n_rc[q] = (t.pair_a[q] << 16) | t.pair_b[q];
            t.ent_n_src[q] = src_code(q);
        }
        for (int32_t k = 0; k < np; ++k) {
            const int32_t q = t.col_pairs[k];
            t.ent_t_rc[k] = (t.pair_b[q] << 16) | t.pair_a[q];
            t.ent_t_src[k] = src_code(q);
        }
    }
    // first span level: the sparse form costs one multiply-add per pair
    // (a, k) and pair (k, c) of the two leaves, the dense one S^3
    int64_t w1 = 0;
    for (int32_t q = 0; q < np; ++q) w1 += t.row_ptr[t.pair_b[q] + 1] - t.row_ptr[t.pair_b[q]];
    t.first_work = w1;
    t.live_states = (flags & FA_LIVE_STATES) != 0;
    // the dense first level from the pair values: 256x256 tiles, and every
    // other leaf reader takes the pair values too (so no dense leaf is
    // written); the live-state products read dense leaves
    const bool pairs_ok = t.Sp % 256 == 0 && np > 0 && !t.live_states && !t.map_n.empty() &&
                          leaf_level_from_pairs(np, t.S, t.Sp);
    t.first_pairs = false;
    if (flags & FA_FIRST_LEVEL_SPARSE) {
        if (t.Sp + t.S > kSparseMaxSpS || np >= kSparseMaxPairs) return FA_ETOOBIG;
        t.first_sparse = true;
    } else if (flags & FA_FIRST_LEVEL_DENSE) {
        t.first_sparse = false;
    } else if (flags & FA_FIRST_LEVEL_PAIRS) {
        if (!pairs_ok) return t.live_states ? FA_EINVAL : FA_ETOOBIG;
        t.first_sparse = false;
        t.first_pairs = true;
    } else {
        t.first_sparse = t.Sp + t.S <= kSparseMaxSpS && np < kSparseMaxPairs &&
                         (double)kSparseFirstRatio * (double)w1 <= (double)t.Sp * t.Sp * t.Sp;
        t.first_pairs = !t.first_sparse && pairs_ok;
    }
    // greedy decoding's first level: the same forcing flags, else by its
    // own cost rule (a max-plus term over the pairs against a dense one)
    if (flags & FA_FIRST_LEVEL_SPARSE) t.map_first_sparse = true;
    else if (flags & FA_FIRST_LEVEL_DENSE) t.map_first_sparse = false;
    else t.map_first_sparse = (double)kMapSparseCost * (double)w1 <= (double)t.S * t.S * t.S;
    t.p2_a.clear(); t.p2_b.clear(); t.p2_row_ptr.clear(); t.p2_col_ptr.clear();
    t.p2_col_pairs.clear(); t.p2_colpos.clear();
    t.w1_n.clear(); t.w1_t.clear(); t.w2_n.clear(); t.w2_t.clear();
    t.col_a.clear(); t.p2_col_a.clear();
    t.second_sparse = false;
    t.second_work = 0;
    // windows: 1024 columns for wider rows, 512 for rows of 513..1024 (the
    // width at which the sparse kernel can still stage an operand in LDS)
    t.win_cols = t.Sp > kSpWin ? kSpWin : (t.Sp > kSpWin / 2 ? kSpWin / 2 : 0);
    t.nwin = t.win_cols ? (t.Sp + t.win_cols - 1) / t.win_cols : 0;
    if (t.first_sparse) {
        build_two_step(t);
        int64_t w2 = 0;
        for (size_t q = 0; q < t.p2_a.size(); ++q) w2 += t.p2_row_ptr[t.p2_b[q] + 1] - t.p2_row_ptr[t.p2_b[q]];
        t.second_work = w2;
        const bool fits = t.p2_a.size() <= (size_t)kSparseSecondMaxPairs;
        if (flags & FA_SECOND_LEVEL_SPARSE) {
            if (!fits) return FA_ETOOBIG;
            t.second_sparse = true;
        } else {
            t.second_sparse = fits && !(flags & FA_FIRST_LEVEL_DENSE) &&
                              (double)kSparseFirstRatio * (double)w2 <= (double)t.Sp * t.Sp * t.Sp;
        }
        if (t.nwin > 0) {
            window_offsets(t, t.row_ptr, t.col_ptr, t.pair_a, t.pair_b, t.col_pairs, t.w1_n, t.w1_t);
            if (t.second_sparse)
                window_offsets(t, t.p2_row_ptr, t.p2_col_ptr, t.p2_a, t.p2_b, t.p2_col_pairs, t.w2_n,
                               t.w2_t);
        }
        if (!t.second_sparse) {
            t.p2_a.clear(); t.p2_b.clear(); t.p2_row_ptr.clear(); t.p2_col_ptr.clear();
            t.p2_col_pairs.clear(); t.p2_colpos.clear();
        }
        t.col_a.resize(np);
        for (int32_t k = 0; k < np; ++k) t.col_a[k] = t.pair_a[t.col_pairs[k]];
        t.p2_col_a.resize(t.p2_a.size());
        for (size_t k = 0; k < t.p2_a.size(); ++k) t.p2_col_a[k] = t.p2_a[t.p2_col_pairs[k]];
    } else if (flags & FA_SECOND_LEVEL_SPARSE) {
        return FA_EINVAL;
    }
    // no dense leaves when nothing reads them: the first level is sparse or
    // staged from the pairs, the message pass's leaf level takes the pair
    // values (LDS-resident pairs and vectors) and the leaf-level draws look
    // pairs up in map_n (a one-leaf tree, whose root is the leaf, still
    // writes it)
    t.leafless = (t.first_sparse || t.first_pairs) && np > 0 && !t.map_n.empty() &&
                 leaf_level_from_pairs(np, t.S, t.Sp);
    build_image(t);
    return FA_OK;
}

}  // namespace fa

using namespace fa;

extern "C" int fa_compile_table(int32_t S, int32_t V, int32_t start, const int32_t *accept,
                                int32_t n_accept, int64_t E, const int32_t *src, const int32_t *dst,
                                const int64_t *label_off, const int32_t *label_tok, uint32_t flags,
                                fa_table **out, size_t *device_bytes)
{
    if (!out) return FA_EINVAL;
    *out = nullptr;
    fa_table *t = nullptr;
    try {
        t = new fa_table();
        int rc = compile(S, V, start, accept, n_accept, E, src, dst, label_off, label_tok, flags, t->h);
        if (rc != FA_OK) {
            delete t;
            return rc;
        }
    } catch (const Err &e) {
        delete t;
        return e.code;
    } catch (const std::bad_alloc &) {
        delete t;
        return FA_ETOOBIG;
    } catch (...) {
        delete t;
        return FA_EINVAL;
    }
    *out = t;
    if (device_bytes) *device_bytes = t->h.image.size();
    return FA_OK;
}

extern "C" void fa_table_destroy(fa_table *t) { delete t; }

extern "C" int fa_table_info(const fa_table *t, int64_t *info, int32_t n)
{
    if (!t || (!info && n > 0) || n < 0) return FA_EINVAL;
    const HostTable &h = t->h;
    int32_t nl = 0, nd = 0, nr = 0;
    for (int32_t c : h.pair_cls) (c == kList ? nl : c == kDense ? nd : nr)++;
    constexpr int32_t kInfo = 25;
    int64_t v[kInfo] = {h.S, h.Sp, h.start, (int64_t)h.acc.size(), h.npairs(), nl, nd, nr,
                        (int64_t)h.list_tok.size(), h.nseg(), h.ncut(), h.nsel(),
                        h.use_sel ? 1 : 0, h.V, h.S_orig, h.first_sparse ? 1 : 0, h.first_work,
                        h.second_sparse ? 1 : 0, h.second_work, (int64_t)h.p2_a.size(),
                        h.leafless ? 1 : 0,
                        h.npairs() > 0 && leaf_level_from_pairs(h.npairs(), h.S, h.Sp) ? 1 : 0,
                        h.live_states ? 1 : 0, h.first_pairs ? 1 : 0,
                        h.map_first_sparse ? 1 : 0};
    for (int32_t k = 0; k < n && k < kInfo; ++k) info[k] = v[k];
    return FA_OK;
}

extern "C" int fa_table_state_map(const fa_table *t, int32_t *orig_of)
{
    if (!t || !orig_of) return FA_EINVAL;
    std::memcpy(orig_of, t->h.orig.data(), t->h.orig.size() * sizeof(int32_t));
    return FA_OK;
}

extern "C" int fa_sizes(const fa_table *t, int32_t B, int32_t L, size_t *tree_bytes,
                        size_t *meta_bytes, size_t *ws_bytes)
{
    if (!t) return FA_EINVAL;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if ((size_t)g.Lpad * g.Sp > (size_t)1 << 40) return FA_ETOOBIG;
    StepChunks ck;
    if (int rc = plan_chunks(t->h, B, L, false, &ck)) return rc;
    if (tree_bytes) *tree_bytes = g.tree_floats * sizeof(float);
    if (meta_bytes) *meta_bytes = g.meta_ints * sizeof(int32_t);
    if (ws_bytes) *ws_bytes = std::max<size_t>((size_t)ck.count * ck.slot, 256);
    return FA_OK;
}
