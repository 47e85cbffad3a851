// MAP (greedy, temperature 0) constrained decoding through a max-times span
// tree: the most probable accepted string argmax_x prod_i p[i][x_i] over x in
// C (paperfeed summary "The evidence": greedy decoding beside sampling; "Why
// constrained decoding breaks for diffusion LMs": MAP inference over a DFA by
// dynamic programming).  The scan of "The scan trick" with max in place of
// sum: 2^k-span max-times products level by level, then top-down midpoint
// decisions and per-position token decisions.
//
// Numbers: natural logs in fp64 (max-plus), log 0 = -inf.  A max-times
// product is then max_k (x + y): one add and one max per term, no rounding
// beyond the fp64 adds, so the decisions equal those of an fp64 reference
// except where two candidates tie to fp64 rounding.  Every decision takes the
// smallest id among equal values.  Max-times is not a ring, so the products
// run on the vector ALUs, not on MFMA.
//
// Layout: tree fp64 [B][2 Lpad][Sp][Sp] in heap order like the sum tree,
// right children (odd nodes >= 3) stored transposed, so a product is
// D[i][j] = max_k X[i][k] + Y[j][k] over two row-major stored operands and a
// midpoint reads one stored row of each child.
#include "device_common.h"

namespace fa {
namespace {

constexpr int kMapThreads = 256;
constexpr int kMapRows = 8;     // stored rows per workgroup of the leaf writer
constexpr int kMT = 64;         // output tile of the product kernel
constexpr int kMK = 16;         // K step staged in LDS
constexpr int kMapSplitTarget = 2048;  // product workgroups wanted per level
constexpr int kMapSelLds = 4096;       // selected tokens the pair-maximum kernel stages in LDS

__device__ inline double lg(float x) { return x > 0.f ? log((double)x) : -INFINITY; }

__device__ inline double *node_ptr(double *tree, int Sp, int Lpad, int b, int h)
{
    return tree + ((size_t)b * 2 * Lpad + h) * (size_t)Sp * Sp;
}

// ---------------------------------------------------------- pair maxima
// One workgroup per position.  Dense-mask pairs: maxima of p bit patterns
// (non-negative floats order as their bits) per byte value of the mask, then
// per pair over the byte values holding its bit.  Token-list pairs: one
// thread per pair over its sorted tokens.  A NaN or negative p at a
// labelled token flags the row.
// NG: dense pairs rounded up to whole bytes of the mask (0..4); VEC4: V % 4
// == 0 and p 16-byte aligned (float4 loads)
template <int NG, bool VEC4>
__global__ __launch_bounds__(kMapThreads) void map_pairmax(DevTable d, const float *__restrict__ p,
                                                           int L, float *__restrict__ pmax,
                                                           int32_t *__restrict__ status)
{
    const int pos = blockIdx.x;
    const int b = pos / L;
    const float *row = p + (size_t)pos * d.V;
    float *out = pmax + (size_t)pos * d.npairs;
    const int tid = threadIdx.x;
    int bad = 0;
    if constexpr (NG > 0) {
        // tokens grouped by their mask byte: T[g][y] is the largest p bit
        // pattern over the tokens whose byte g of the mask is y (one LDS
        // atomic max per byte and token); dense pair 8g + t is then the
        // largest T[g][y] over the bytes y with bit t set
        constexpr int NB = 8 * NG;
        constexpr uint32_t kBits = (NB == 32) ? 0xFFFFFFFFu : ((1u << NB) - 1u);
        __shared__ uint32_t T[NG][256];
        for (int e = tid; e < NG * 256; e += kMapThreads) T[e >> 8][e & 255] = 0u;
        __syncthreads();
        auto one = [&](float x, uint32_t m) {
            m &= kBits;
            bad |= (m != 0u) & !(x >= 0.f);
            const uint32_t xb = x >= 0.f ? __float_as_uint(x) : 0u;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t y = (m >> (8 * g)) & 255u;
                if (y) atomicMax(&T[g][y], xb);
            }
        };
        if (VEC4) {
            const int n4 = d.V >> 2;
            for (int g = tid; g < n4; g += kMapThreads) {
                const float4 x4 = load_nt(row + 4 * (size_t)g);
                const uint4 m4 = reinterpret_cast<const uint4 *>(d.tokmask)[g];
                one(x4.x, m4.x);
                one(x4.y, m4.y);
                one(x4.z, m4.z);
                one(x4.w, m4.w);
            }
        } else {
            for (int v = tid; v < d.V; v += kMapThreads) one(row[v], d.tokmask[v]);
        }
        __syncthreads();
        for (int j = tid; j < d.ndense; j += kMapThreads) {
            const int g = j >> 3, t = j & 7;
            uint32_t x = 0u;
            for (int y = 1; y < 256; ++y)
                if ((y >> t) & 1) x = max(x, T[g][y]);
            out[d.dense_pair[j]] = __uint_as_float(x);
        }
    }
    // token lists read p at the table's selected tokens: staged in LDS once
    // when they fit, else gathered from the row
    __shared__ float psel[kMapSelLds];
    const bool staged = d.use_sel && d.nsel <= kMapSelLds;
    if (staged) {
        for (int k = tid; k < d.nsel; k += kMapThreads) psel[k] = row[d.sel_tok[k]];
        __syncthreads();
    }
    for (int q = tid; q < d.npairs; q += kMapThreads) {
        if (d.pair_cls[q] != kList) continue;
        float m = 0.f;
        for (int k = d.list_off[q]; k < d.list_off[q + 1]; ++k) {
            const float x = staged ? psel[d.list_sel[k]] : row[d.list_tok[k]];
            bad |= !(x >= 0.f);
            if (x > m) m = x;
        }
        out[q] = m;
    }
    if (bad) atomicOr(&status[b], (int)FA_ROW_BADPROB);
}

// ------------------------------------------------ range-label pair maxima
// A range pair's maximum of p over its segments, from a range-maximum
// structure built per position in LDS.  The sorted cut points split
// [cuts[0], cuts[ncut-1]) into ncut-1 elementary intervals and every segment
// is a run of them.  The workgroup first folds the row into the intervals'
// maxima, as keys: the bit pattern of a p >= 0 (which orders as p does), all
// ones for a NaN or negative p, so that a segment holding one reads as bad.
// Then the maxima of blocks of kMapRangeBlk intervals, and a sparse table over
// the blocks (level k at k * nblk: the maximum of 2^k blocks from each start).
// A segment's maximum is at most two partial blocks of intervals and two
// table entries.  One workgroup per position.
constexpr int kMapRangeThreads = 1024;

__device__ inline uint32_t range_key(float x)
{
    return x >= 0.f ? (__float_as_uint(x) & 0x7FFFFFFFu) : 0xFFFFFFFFu;
}

// maximum key over the intervals [lo, hi)
__device__ inline uint32_t range_query(const uint32_t *rk, const uint32_t *tab, int nblk, int lo,
                                       int hi)
{
    uint32_t m = 0u;
    const int bl = (lo + kMapRangeBlk - 1) / kMapRangeBlk;  // first whole block
    const int br = hi / kMapRangeBlk - 1;                   // last whole block
    if (bl > br) {
        for (int c = lo; c < hi; ++c) m = max(m, rk[c]);
        return m;
    }
    for (int c = lo; c < bl * kMapRangeBlk; ++c) m = max(m, rk[c]);
    for (int c = (br + 1) * kMapRangeBlk; c < hi; ++c) m = max(m, rk[c]);
    const int k = 31 - __clz(br - bl + 1);
    return max(m, max(tab[k * nblk + bl], tab[k * nblk + br - (1 << k) + 1]));
}

// VEC4: V % 4 == 0 and p and tok2cut 16-byte aligned
template <bool VEC4>
__global__ __launch_bounds__(kMapRangeThreads) void map_rangemax(DevTable d,
                                                                 const float *__restrict__ p,
                                                                 int L, float *__restrict__ pmax,
                                                                 int32_t *__restrict__ status)
{
    extern __shared__ uint32_t rk[];  // [nint] interval maxima, then the block table
    const int pos = blockIdx.x;
    const int b = pos / L;
    const float *row = p + (size_t)pos * d.V;
    float *out = pmax + (size_t)pos * d.npairs;
    const int tid = threadIdx.x;
    const int nint = d.ncut - 1;
    const int nblk = map_range_blocks(nint);
    const int lg = map_range_levels(nblk);
    uint32_t *tab = rk + nint;
    for (int c = tid; c < nint; c += kMapRangeThreads) rk[c] = 0u;
    __syncthreads();
    // a thread's tokens ascend, so equal intervals come in runs: one LDS
    // maximum per run
    int rc = -1;
    uint32_t rkey = 0u;
    auto put = [&](int c, float x) {
        const uint32_t k = range_key(x);
        if (c != rc) {
            if (rc >= 0 && rc < nint && rkey) atomicMax(&rk[rc], rkey);
            rc = c;
            rkey = 0u;
        }
        rkey = max(rkey, k);
    };
    if (VEC4) {
        const int n4 = d.V >> 2;
        for (int g = tid; g < n4; g += kMapRangeThreads) {
            const float4 x4 = load_nt(row + 4 * (size_t)g);
            const int4 c4 = reinterpret_cast<const int4 *>(d.tok2cut)[g];
            put(c4.x, x4.x);
            put(c4.y, x4.y);
            put(c4.z, x4.z);
            put(c4.w, x4.w);
        }
    } else {
        for (int v = tid; v < d.V; v += kMapRangeThreads) put(d.tok2cut[v], row[v]);
    }
    put(-1, 0.f);
    __syncthreads();
    for (int j = tid; j < nblk; j += kMapRangeThreads) {
        uint32_t m = 0u;
        for (int c = j * kMapRangeBlk; c < min(nint, (j + 1) * kMapRangeBlk); ++c) m = max(m, rk[c]);
        tab[j] = m;
    }
    __syncthreads();
    for (int k = 1; k < lg; ++k) {
        const int h = 1 << (k - 1);
        for (int j = tid; j + 2 * h <= nblk; j += kMapRangeThreads)
            tab[k * nblk + j] = max(tab[(k - 1) * nblk + j], tab[(k - 1) * nblk + j + h]);
        __syncthreads();
    }
    int bad = 0;
    for (int q = tid; q < d.npairs; q += kMapRangeThreads) {
        if (d.pair_cls[q] != kRange) continue;
        uint32_t m = 0u;
        for (int s = d.seg_off[q]; s < d.seg_off[q + 1]; ++s)
            m = max(m, range_query(rk, tab, nblk, d.seg_lo_cut[s], d.seg_hi_cut[s]));
        bad |= m == 0xFFFFFFFFu;
        out[q] = m == 0xFFFFFFFFu ? 0.f : __uint_as_float(m);
    }
    if (bad) atomicOr(&status[b], (int)FA_ROW_BADPROB);
}

// ---------------------------------------------------------- log leaves
// One workgroup per (leaf, kMapRows stored rows): each stored row is built in
// LDS (-inf, then the log pair maxima of that row, or 0 on the diagonal of an
// identity leaf past the sequence end) and written out whole.
__global__ __launch_bounds__(kMapThreads) void map_leaves(DevTable d, int L, int Lpad,
                                                          const float *__restrict__ pmax,
                                                          double *__restrict__ tree)
{
    extern __shared__ double rowbuf[];  // [Sp]
    const int Sp = d.Sp;
    const int b = blockIdx.y / Lpad, i = blockIdx.y % Lpad;
    const int h = Lpad + i;
    const bool tr = stored_transposed(h);
    double *M = node_ptr(tree, Sp, Lpad, b, h);
    const float *pm = pmax + ((size_t)b * L + i) * d.npairs;
    const int tid = threadIdx.x;
    for (int r = blockIdx.x * kMapRows; r < min(Sp, (int)(blockIdx.x + 1) * kMapRows); ++r) {
        for (int c = tid; c < Sp; c += kMapThreads) rowbuf[c] = -INFINITY;
        __syncthreads();
        if (r < d.S) {
            if (i >= L) {
                if (tid == 0) rowbuf[r] = 0.0;
            } else if (!tr) {
                for (int k = d.row_ptr[r] + tid; k < d.row_ptr[r + 1]; k += kMapThreads)
                    rowbuf[d.pair_b[k]] = lg(pm[k]);
            } else {
                for (int k = d.col_ptr[r] + tid; k < d.col_ptr[r + 1]; k += kMapThreads) {
                    const int q = d.col_pairs[k];
                    rowbuf[d.pair_a[q]] = lg(pm[q]);
                }
            }
        }
        __syncthreads();
        for (int c = tid; c < Sp; c += kMapThreads) M[(size_t)r * Sp + c] = rowbuf[c];
        __syncthreads();
    }
}

// ---------------------------------------- first max-plus level from pairs
// Level-1 products (two leaves each) over the pair structure: D[a][c] is the
// largest sum of the log weights of a pair (a, k) of the left leaf and a
// pair (k, c) of the right one, -inf where there is none; the weights are
// read from the dense log leaves at the pairs' entries.  A node stored as is
// builds its rows a from the left leaf's rows and the right leaf's rows; one
// stored transposed builds its rows c from the right leaf's columns and the
// left leaf's columns.  Each term is the same fp64 add as map_gemm's and the
// maximum does not depend on the order, so the nodes are map_gemm's, bit for
// bit.  A right leaf past the sequence end is the identity (D = the left
// leaf), and so are both when the left one is.  One workgroup per (node,
// `rows` stored rows, held in LDS as order-preserving integer keys); each
// wavefront takes a stored row at a time, each lane one outer pair and its
// inner pair list, four terms in flight, combined by LDS atomic maxima.
constexpr int kMapSpThreads = 1024;

// fp64 -> uint64 key with the same order (no NaN here), and back
__device__ inline unsigned long long dkey(double x)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ inline double dval(unsigned long long k)
{
    return __longlong_as_double((long long)((k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}

__global__ __launch_bounds__(kMapSpThreads) void map_sparse1(DevTable d, int L, int Lpad, int rows,
                                                             double *__restrict__ tree)
{
    extern __shared__ unsigned long long accs[];  // [rows][Sp] keys
    const int Sp = d.Sp;
    const int half = Lpad >> 1;
    const int b = blockIdx.y / half, n = half + blockIdx.y % half;
    const bool tr = stored_transposed(n);
    const int il = 2 * n - Lpad;
    const bool id_l = il >= L, id_r = il + 1 >= L;  // identity leaves past the sequence end
    const double *Xl = node_ptr(tree, Sp, Lpad, b, 2 * n);      // stored as is: Xl[a][k]
    const double *Xr = node_ptr(tree, Sp, Lpad, b, 2 * n + 1);  // transposed: Xr[c][k]
    double *D = node_ptr(tree, Sp, Lpad, b, n);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = blockIdx.x * rows, nr = min(rows, Sp - r0);
    const unsigned long long kinf = dkey(-INFINITY);
    for (int e = tid; e < nr * Sp; e += kMapSpThreads) accs[e] = kinf;
    __syncthreads();
    // the outer pairs of stored row x: the left leaf's row x (as is) or the
    // right leaf's column x (transposed); for each, the inner pairs through k
    const int32_t *optr = tr ? d.col_ptr : d.row_ptr;
    for (int rr = wave; rr < nr; rr += kMapSpThreads / 64) {
        const int x = r0 + rr;
        unsigned long long *acc = accs + (size_t)rr * Sp;
        if (x >= d.S) continue;
        if (id_l) {
            if (lane == 0) acc[x] = dkey(0.0);
            continue;
        }
        for (int o = optr[x] + lane; o < optr[x + 1]; o += 64) {
            if (id_r) {
                // D = the left leaf: its row x, or its column x when transposed
                if (tr) {
                    const int a = d.pair_a[d.col_pairs[o]];
                    acc[a] = dkey(Xl[(size_t)a * Sp + x] + 0.0);
                } else {
                    const int c = d.pair_b[o];
                    acc[c] = dkey(Xl[(size_t)x * Sp + c] + 0.0);
                }
                continue;
            }
            const int k = tr ? d.pair_a[d.col_pairs[o]] : d.pair_b[o];
            const double wo = tr ? Xr[(size_t)x * Sp + k] : Xl[(size_t)x * Sp + k];
            const int q0 = optr[k], q1 = optr[k + 1];
            for (int q = q0; q < q1; q += 4) {
                int t[4];
                double w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int qq = min(q + u, q1 - 1);
                    t[u] = tr ? d.pair_a[d.col_pairs[qq]] : d.pair_b[qq];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    w[u] = tr ? Xl[(size_t)t[u] * Sp + k] : Xr[(size_t)t[u] * Sp + k];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (q + u < q1) atomicMax(&acc[t[u]], dkey(tr ? w[u] + wo : wo + w[u]));
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < nr * Sp; e += kMapSpThreads) D[(size_t)r0 * Sp + e] = dval(accs[e]);
}

// ------------------------------------------------------ max-plus products
// One wavefront per 64 x 64 output tile of D = X (max,+) Y^T over one K
// range (a split); each lane owns an 8 x 8 block of the tile.  Operand tiles
// of 64 rows x kMK are staged in LDS k-major, so a lane reads its eight rows
// of X and eight rows of Y at one k as two contiguous runs.
__global__ __launch_bounds__(64) void map_gemm(int Sp, int Lpad, double *__restrict__ tree, int n0,
                                               int nn, int ksplit, double *__restrict__ part)
{
    __shared__ __align__(16) double Xs[kMK][kMT];
    __shared__ __align__(16) double Ys[kMK][kMT];
    const int tiles = Sp / kMT, T2 = tiles * tiles;
    const int tile = blockIdx.x % T2, split = blockIdx.x / T2;
    const int tm = (tile / tiles) * kMT, tn = (tile % tiles) * kMT;
    const int b = blockIdx.y / nn, n = n0 + blockIdx.y % nn;
    const bool tr = stored_transposed(n);
    const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
    const double *X = node_ptr(tree, Sp, Lpad, b, hF);
    const double *Y = node_ptr(tree, Sp, Lpad, b, hG);
    const int lane = threadIdx.x;
    const int r0 = (lane >> 3) * 8, c0 = (lane & 7) * 8;
    const int kc = Sp / ksplit, k_begin = split * kc, k_end = k_begin + kc;
    double acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = -INFINITY;
    const double *xrow = X + (size_t)(tm + lane) * Sp;
    const double *yrow = Y + (size_t)(tn + lane) * Sp;
    for (int k0 = k_begin; k0 < k_end; k0 += kMK) {
        double2 xv[kMK / 2], yv[kMK / 2];
#pragma unroll
        for (int q = 0; q < kMK / 2; ++q) {
            xv[q] = *reinterpret_cast<const double2 *>(xrow + k0 + 2 * q);
            yv[q] = *reinterpret_cast<const double2 *>(yrow + k0 + 2 * q);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kMK / 2; ++q) {
            Xs[2 * q][lane] = xv[q].x;
            Xs[2 * q + 1][lane] = xv[q].y;
            Ys[2 * q][lane] = yv[q].x;
            Ys[2 * q + 1][lane] = yv[q].y;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMK; ++k) {
            double a[8], c[8];
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                const double2 t = *reinterpret_cast<const double2 *>(&Xs[k][r0 + r]);
                a[r] = t.x;
                a[r + 1] = t.y;
                const double2 u = *reinterpret_cast<const double2 *>(&Ys[k][c0 + r]);
                c[r] = u.x;
                c[r + 1] = u.y;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) acc[r][cc] = fmax(acc[r][cc], a[r] + c[cc]);
        }
    }
    double *D = ksplit > 1 ? part + ((size_t)(blockIdx.y * ksplit + split) * T2 + tile) * (kMT * kMT)
                           : node_ptr(tree, Sp, Lpad, b, n) + (size_t)tm * Sp + tn;
    const int ld = ksplit > 1 ? kMT : Sp;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int cc = 0; cc < 8; cc += 2)
            *reinterpret_cast<double2 *>(D + (size_t)(r0 + r) * ld + c0 + cc) =
                make_double2(acc[r][cc], acc[r][cc + 1]);
}

// the maximum of the K-split partial tiles, into the node
__global__ __launch_bounds__(kMapThreads) void map_reduce(int Sp, int Lpad, double *__restrict__ tree,
                                                          int n0, int nn, int ksplit,
                                                          const double *__restrict__ part)
{
    const int tiles = Sp / kMT, T2 = tiles * tiles;
    constexpr int kChunks = kMT * kMT / kMapThreads;  // workgroups per tile
    const int tile = blockIdx.x / kChunks;
    const int e = (blockIdx.x % kChunks) * kMapThreads + threadIdx.x;
    const int tm = (tile / tiles) * kMT, tn = (tile % tiles) * kMT;
    const int b = blockIdx.y / nn, n = n0 + blockIdx.y % nn;
    double *D = node_ptr(tree, Sp, Lpad, b, n);
    double m = -INFINITY;
    for (int s = 0; s < ksplit; ++s)
        m = fmax(m, part[((size_t)(blockIdx.y * ksplit + s) * T2 + tile) * (kMT * kMT) + e]);
    D[(size_t)(tm + e / kMT) * Sp + tn + e % kMT] = m;
}

// -------------------------------------------------------- top-down decode
// (value, id) of the better of two candidates: the larger value, the smaller
// id among equal values
__device__ inline void better(double &v, int &k, double v2, int k2)
{
    if (v2 > v || (v2 == v && k2 >= 0 && (k < 0 || k2 < k))) {
        v = v2;
        k = k2;
    }
}

__device__ inline void wave_argmax(double &v, int &k)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double v2 = __shfl_xor(v, o);
        const int k2 = __shfl_xor(k, o);
        better(v, k, v2, k2);
    }
}

// Per row: log-max = max over accepting f of root[s0][f]; the final boundary
// state is the best f (smallest among equal values).  One wavefront per row.
__global__ __launch_bounds__(64) void map_root(DevTable d, int Lpad, const double *__restrict__ tree,
                                               double *__restrict__ logmax, int32_t *__restrict__ zc,
                                               int32_t *__restrict__ status)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    const double *R = node_ptr(const_cast<double *>(tree), d.Sp, Lpad, b, 1) + (size_t)d.start * d.Sp;
    double v = -INFINITY;
    int k = -1;
    for (int a = lane; a < d.n_acc; a += 64) better(v, k, R[d.acc[a]], d.acc[a]);
    wave_argmax(v, k);
    const bool ok = status[b] == 0 && v > -INFINITY;
    for (int j = 1 + lane; j < Lpad; j += 64) zc[(size_t)b * (Lpad + 1) + j] = -1;
    if (lane == 0) {
        zc[(size_t)b * (Lpad + 1)] = ok ? d.start : -1;
        zc[(size_t)b * (Lpad + 1) + Lpad] = ok ? k : -1;
        logmax[b] = ok ? v : -INFINITY;
        if (status[b] == 0 && !(v > -INFINITY)) atomicOr(&status[b], (int)FA_ROW_INFEASIBLE);
    }
}

// One level of midpoints: node n of level `lev` (segment [l, r), midpoint m)
// takes the z_m maximizing left[z_l][z_m] + right[z_m][z_r]: stored row z_l of
// the left child and stored row z_r of the (transposed) right child.  One
// wavefront per node.
__global__ __launch_bounds__(64) void map_mid(DevTable d, int Lpad, int lev,
                                              const double *__restrict__ tree,
                                              int32_t *__restrict__ zc, int32_t *__restrict__ status)
{
    const int nn = 1 << (lev - 1);
    const int b = blockIdx.x / nn, j = blockIdx.x % nn;
    const int n = nn + j;
    const int span = Lpad >> (lev - 1);
    const int l = j * span, r = l + span, m = l + span / 2;
    int32_t *z = zc + (size_t)b * (Lpad + 1);
    const int zl = z[l], zr = z[r];
    if (zl < 0 || zr < 0) return;  // a flagged row: its states stay -1
    const double *Lrow = node_ptr(const_cast<double *>(tree), d.Sp, Lpad, b, 2 * n) + (size_t)zl * d.Sp;
    const double *Rrow = node_ptr(const_cast<double *>(tree), d.Sp, Lpad, b, 2 * n + 1) + (size_t)zr * d.Sp;
    double v = -INFINITY;
    int k = -1;
    for (int c = threadIdx.x; c < d.S; c += 64) better(v, k, Lrow[c] + Rrow[c], c);
    wave_argmax(v, k);
    if (threadIdx.x == 0) {
        z[m] = v > -INFINITY ? k : -1;
        if (!(v > -INFINITY)) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
    }
}

// The most probable token of each position's edge (z_i, z_{i+1}): over the
// pair's token list, its segments, or the row with the dense pair's bit array;
// smallest token among equal probabilities.  One workgroup per position.
__global__ __launch_bounds__(kMapThreads) void map_tokens(DevTable d, int L, int Lpad,
                                                          const float *__restrict__ p,
                                                          const int32_t *__restrict__ zc,
                                                          int32_t *__restrict__ tokens,
                                                          int32_t *__restrict__ status)
{
    const int b = blockIdx.y, i = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *z = zc + (size_t)b * (Lpad + 1);
    const int a = z[i], c = z[i + 1];
    const int q = (a >= 0 && c >= 0) ? pair_index(d, a, c) : -1;
    const float *row = p + ((size_t)b * L + i) * d.V;
    double v = -INFINITY;  // value as fp64 of the fp32 p: the order is the same
    int k = -1;
    if (q >= 0) {
        if (d.pair_cls[q] == kDense) {
            const uint32_t *bits = d.dense_bits + (size_t)d.pair_aux[q] * d.dense_words;
            if ((d.V & 3) == 0 && ((uintptr_t)row & 15) == 0) {
                // four tokens per thread and step, two steps in flight; each
                // thread's tokens ascend, so a strict > keeps its first maximum
                const int n4 = d.V >> 2;
                for (int g0 = tid; g0 < n4; g0 += 2 * kMapThreads) {
                    const int g1 = min(g0 + kMapThreads, n4 - 1);
                    const float4 xa = load_nt(row + 4 * (size_t)g0);
                    const float4 xb = load_nt(row + 4 * (size_t)g1);
                    const uint32_t wa = bits[g0 >> 3] >> ((g0 & 7) * 4);
                    const uint32_t wb = bits[g1 >> 3] >> ((g1 & 7) * 4);
                    const float va[4] = {xa.x, xa.y, xa.z, xa.w};
                    const float vb[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (((wa >> u) & 1u) && va[u] > 0.f) better(v, k, (double)va[u], 4 * g0 + u);
                    if (g0 + kMapThreads < n4) {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (((wb >> u) & 1u) && vb[u] > 0.f) better(v, k, (double)vb[u], 4 * g1 + u);
                    }
                }
            } else {
                for (int t = tid; t < d.V; t += kMapThreads)
                    if ((bits[t >> 5] >> (t & 31)) & 1u) {
                        const float x = row[t];
                        if (x > 0.f) better(v, k, (double)x, t);
                    }
            }
        } else if (d.pair_cls[q] == kRange) {
            for (int s = d.seg_off[q]; s < d.seg_off[q + 1]; ++s)
                for (int t = d.seg_lo[s] + tid; t < d.seg_hi[s]; t += kMapThreads) {
                    const float x = row[t];
                    if (x > 0.f) better(v, k, (double)x, t);
                }
        } else {
            for (int e = d.list_off[q] + tid; e < d.list_off[q + 1]; e += kMapThreads) {
                const int t = d.list_tok[e];
                const float x = row[t];
                if (x > 0.f) better(v, k, (double)x, t);
            }
        }
    }
    wave_argmax(v, k);
    __shared__ double sv[kMapThreads / 64];
    __shared__ int sk[kMapThreads / 64];
    if (lane == 0) {
        sv[wave] = v;
        sk[wave] = k;
    }
    __syncthreads();
    if (tid == 0) {
        v = sv[0];
        k = sk[0];
        for (int w = 1; w < kMapThreads / 64; ++w) better(v, k, sv[w], sk[w]);
        tokens[(size_t)b * L + i] = k;
        if (a >= 0 && c >= 0 && k < 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
    }
}

// states in original ids; a flagged row gets -1 states and tokens
__global__ void map_finalize(DevTable d, int L, int Lpad, const int32_t *__restrict__ zc,
                             int32_t *__restrict__ states, int32_t *__restrict__ tokens,
                             const int32_t *__restrict__ status)
{
    const int b = blockIdx.y;
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k > L) return;
    const bool flagged = status[b] != 0;
    const int zz = zc[(size_t)b * (Lpad + 1) + k];
    states[(size_t)b * (L + 1) + k] = (flagged || zz < 0) ? -1 : d.orig[zz];
    if (k < L && flagged) tokens[(size_t)b * L + k] = -1;
}

// L = 0: the empty string, accepted when the start state is accepting
__global__ void map_empty(DevTable d, int B, double *__restrict__ logmax,
                          int32_t *__restrict__ states, int32_t *__restrict__ status)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    bool acc = false;
    for (int a = 0; a < d.n_acc; ++a) acc |= d.acc[a] == d.start;
    const bool ok = acc && status[b] == 0;
    logmax[b] = ok ? 0.0 : -INFINITY;
    states[b] = ok ? d.orig[d.start] : -1;
    if (!acc) atomicOr(&status[b], (int)FA_ROW_INFEASIBLE);
}

// K split of one product level: the largest power of two dividing the K
// blocks that keeps at most kMapSplitTarget workgroups
int map_ksplit(const Geometry &g, int level)
{
    const long long tiles = (long long)g.B * (g.Lpad >> level) * (g.Sp / kMT) * (g.Sp / kMT);
    int s = 1;
    while ((g.Sp / kMK) % (2 * s) == 0 && tiles * s * 2 <= kMapSplitTarget) s *= 2;
    return s;
}

}  // namespace

MapWs map_ws_layout(const HostTable &t, const Geometry &g)
{
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    MapWs w;
    size_t o = 0;
    w.pmax = o; o = al(o + (size_t)g.B * g.L * t.npairs() * sizeof(float));
    w.zc = o; o = al(o + (size_t)g.B * (g.Lpad + 1) * sizeof(int32_t));
    size_t kp = 0;
    if (g.Sp % kMT == 0)
        for (int level = 1; level <= g.K; ++level) {
            const int s = map_ksplit(g, level);
            if (s > 1) kp = std::max(kp, (size_t)g.B * (g.Lpad >> level) * s * g.mat);
        }
    w.kpart = o; o = al(o + kp * sizeof(double));
    w.total = o ? o : 256;
    return w;
}

int launch_map_decode(const DevTable &d, const Geometry &g, const float *p, double *tree,
                      uint8_t *ws, const MapWs &w, double *logmax, int32_t *states,
                      int32_t *tokens, int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (g.L == 0) {
        map_empty<<<(g.B + 255) / 256, 256, 0, st>>>(d, g.B, logmax, states, status);
        return (int)hipGetLastError();
    }
    float *pmax = (float *)(ws + w.pmax);
    int32_t *zc = (int32_t *)(ws + w.zc);
    double *part = (double *)(ws + w.kpart);
    const int npos = g.B * g.L;
    const int ng = (d.ndense + 7) / 8;
    const bool vec4 = (d.V & 3) == 0 && ((uintptr_t)p & 15) == 0;
#define FA_MAP_PM(NG, V4) map_pairmax<NG, V4><<<npos, kMapThreads, 0, st>>>(d, p, g.L, pmax, status)
    if (ng == 0) FA_MAP_PM(0, false);
    else if (vec4) {
        if (ng == 1) FA_MAP_PM(1, true);
        else if (ng == 2) FA_MAP_PM(2, true);
        else if (ng == 3) FA_MAP_PM(3, true);
        else FA_MAP_PM(4, true);
    } else {
        if (ng == 1) FA_MAP_PM(1, false);
        else if (ng == 2) FA_MAP_PM(2, false);
        else if (ng == 3) FA_MAP_PM(3, false);
        else FA_MAP_PM(4, false);
    }
#undef FA_MAP_PM
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    if (d.nseg > 0) {
        // the entry points refuse tables whose structure exceeds kMapRangeLdsMax
        const size_t rlds = map_range_lds(d.ncut);
        const bool rv4 = vec4 && ((uintptr_t)d.tok2cut & 15) == 0;
        const void *fn = rv4 ? reinterpret_cast<const void *>(&map_rangemax<true>)
                             : reinterpret_cast<const void *>(&map_rangemax<false>);
        if (rlds > 48 * 1024) {
            e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)rlds);
            if (e != hipSuccess) return (int)e;
        }
        if (rv4)
            map_rangemax<true><<<npos, kMapRangeThreads, rlds, st>>>(d, p, g.L, pmax, status);
        else
            map_rangemax<false><<<npos, kMapRangeThreads, rlds, st>>>(d, p, g.L, pmax, status);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    const size_t llds = (size_t)g.Sp * sizeof(double);
    if (llds > 48 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&map_leaves),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)llds);
        if (e != hipSuccess) return (int)e;
    }
    map_leaves<<<dim3((g.Sp + kMapRows - 1) / kMapRows, g.B * g.Lpad), kMapThreads, llds, st>>>(
        d, g.L, g.Lpad, pmax, tree);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const int tiles = g.Sp / kMT;
    for (int k = 1; k <= g.K; ++k) {
        const int n0 = g.Lpad >> k, nn = n0;
        if (k == 1 && d.map_first_sparse) {
            // rows per workgroup: one per wavefront, at most 64 KB of LDS
            const int rows = std::max(1, std::min(kMapSpThreads / 64,
                                                  (int)(65536 / ((size_t)g.Sp * sizeof(double)))));
            const size_t slds = (size_t)rows * g.Sp * sizeof(double);
            if (slds > 48 * 1024) {
                e = hipFuncSetAttribute(reinterpret_cast<const void *>(&map_sparse1),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)slds);
                if (e != hipSuccess) return (int)e;
            }
            map_sparse1<<<dim3((g.Sp + rows - 1) / rows, g.B * nn), kMapSpThreads, slds, st>>>(
                d, g.L, g.Lpad, rows, tree);
            e = hipGetLastError();
            if (e != hipSuccess) return (int)e;
            continue;
        }
        const int ks = map_ksplit(g, k);
        map_gemm<<<dim3(tiles * tiles * ks, g.B * nn), 64, 0, st>>>(g.Sp, g.Lpad, tree, n0, nn, ks,
                                                                      part);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
        if (ks > 1) {
            map_reduce<<<dim3(tiles * tiles * (kMT * kMT / kMapThreads), g.B * nn), kMapThreads, 0,
                         st>>>(g.Sp, g.Lpad, tree, n0, nn, ks, part);
            e = hipGetLastError();
            if (e != hipSuccess) return (int)e;
        }
    }
    map_root<<<g.B, 64, 0, st>>>(d, g.Lpad, tree, logmax, zc, status);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    for (int lev = 1; lev <= g.K; ++lev) {
        map_mid<<<g.B << (lev - 1), 64, 0, st>>>(d, g.Lpad, lev, tree, zc, status);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    map_tokens<<<dim3(g.L, g.B), kMapThreads, 0, st>>>(d, g.L, g.Lpad, p, zc, tokens, status);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    map_finalize<<<dim3((g.L + 1 + 255) / 256, g.B), 256, 0, st>>>(d, g.L, g.Lpad, zc, states,
                                                                    tokens, status);
    return (int)hipGetLastError();
}

}  // namespace fa
