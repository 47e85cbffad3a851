// Span tree: bottom-up 2^k-span transition products, level by level, as
// batched matrix products in fp32 precision on the bf16 matrix cores (the
// three-piece operand split below; paperfeed "The scan trick: log-depth
// exact sampling": 2^k-step transitions from two 2^(k-1)-step ones in log L
// rounds of batched matrix multiplication; papernotes 关键设计 2).
//
// Scaling.  A stored matrix P carries power-of-two exponent vectors ro (per
// stored row) and co (per stored column): the true span matrix is
// diag(2^ro) P diag(2^co) in stored orientation.  rf[r] = max_c (e(P[r][c]) +
// co[c]) is the fold normalizer of stored row r: the consumed row
// P[r][c] 2^(co[c] - rf[r]) has its maximum in [0.5, 1).  A product of a left
// child (stored as is) and a right child (stored transposed) consumes both in
// this row form, so both operands are K-contiguous and every scale stays
// outside the contraction:
//   T_n = diag(2^(ro_L + rf_L)) (X Y^T) diag(2^(ro_R + rf_R)),
// with X, Y the consumed stored rows.  Odd (right-child) nodes are produced
// transposed by swapping the operands.  No entry is lost unless it is 2^-126
// below the maximum of its own row.
//
// Products are stored with plain (write-back) stores: a level is read next
// by the level above and, in the joint call, by the message pass right after
// the tree, so the last-level cache keeps much of it for them (measured
// faster than writing it straight to HBM with non-temporal stores).
#include "device_common.h"
#include <algorithm>
#include <atomic>

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;        // output tile (rows and columns)
constexpr int kBK = 32;          // K step staged in LDS (two MFMA K steps of 16)
constexpr int kLdb2 = kBK + 8;   // padded LDS row of one bf16 piece
constexpr int kGemmThreads = 256;

// rf of the internal nodes 1 .. hend-1 of every row: kNeg (the levels whose
// tiles split rows fill it by atomicMax), over the whole grid
__device__ inline void init_rf_nodes(const StepView &sv, int32_t *__restrict__ meta, int hend)
{
    const size_t per_row = (size_t)(hend - 1) * sv.Sp;
    const size_t total = per_row * sv.B;
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < total;
         k += (size_t)gridDim.x * blockDim.x) {
        const int b = (int)(k / per_row);
        const size_t rem = k % per_row;
        const int h = 1 + (int)(rem / sv.Sp);
        const int r = (int)(rem % sv.Sp);
        sv.meta_ptr(meta, b, h, 2)[r] = kNeg;
    }
}

__global__ void tree_init_rf(StepView sv, int32_t *__restrict__ meta)
{
    init_rf_nodes(sv, meta, sv.Lpad);
}

// exact power-of-two rescale of four consumed entries; zero stays zero and
// values more than 2^126 below the row maximum flush to zero
__device__ inline float4 fold4(float4 x, int4 c, int rfrow)
{
    x.x = ldexpf(x.x, c.x - rfrow);
    x.y = ldexpf(x.y, c.y - rfrow);
    x.z = ldexpf(x.z, c.z - rfrow);
    x.w = ldexpf(x.w, c.w - rfrow);
    return x;
}

// The largest exponent e(D[i][j]) + coD[j] of each row of an output tile,
// reduced through LDS instead of lane shuffles: every lane has written its
// maximum over its own columns of row i to E[i * ld + slot] (one slot per
// lane and column group), and after a barrier thread t < rows reads row t's
// `slots` entries (a multiple of 4; ld too) and folds it into rfD, which
// holds kNeg or another tile's maximum of the row.
__device__ inline void rowmax_from_lds(const int *E, int ld, int slots, int rows, int32_t *rfD)
{
    const int t = threadIdx.x;
    if (t < rows) {
        const int4 *r4 = reinterpret_cast<const int4 *>(E + t * ld);
        int e = kNeg;
        for (int k = 0; k < slots / 4; ++k) {
            const int4 x = r4[k];
            e = max(e, max(max(x.x, x.y), max(x.z, x.w)));
        }
        if (e > kNeg) atomicMax(&rfD[t], e);
    }
}

// this lane's exponent of x scaled by 2^c: kNeg unless both are present
__device__ inline int scaled_exp(float x, int c)
{
    int ex;
    frexpf(x, &ex);
    return ((x > 0.f) & (c > kNeg)) ? ex + c : kNeg;
}

// The dense span kernels run the fp32 products on the bf16 matrix cores:
// every folded operand entry x is split, when it is staged, into
// three bf16 pieces x = h + m + l (round to nearest at each step, so each
// residual is exact and the pieces hold all 24 bits of x), and the product
// x y takes the six partial products hh' + hm' + mh' + hl' + mm' + lh'.  The
// three dropped ones are below 2^-23 |x y| together, and all entries are
// non-negative, so every output entry keeps that relative bound on top of
// the fp32 accumulation's rounding: the precision of the fp32 MFMA path at
// 6/16 of its matrix-core time.  Every kernel adds, per K step of 16, the
// six products in the same order (by the second operand's piece, then the
// first's), so a product does not depend on the kernel that forms it.
constexpr int kBK3 = 16;        // K step per LDS stage of the 128- and 256-tile kernels
constexpr int kLdb = kBK3 + 8;  // padded LDS row of one piece (bf16 entries)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// two fp32 values rounded to bf16 (to nearest even), packed low | high
__device__ inline uint32_t bf16_pair(float a, float b)
{
    const f32x2v v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// the three bf16 pieces of four fp32 entries, two per word (h + m + l == x
// exactly while x is a normal fp32 number of at least 2^-110)
__device__ inline void split3(float4 x, uint2 &h, uint2 &m, uint2 &l)
{
    const float v[4] = {x.x, x.y, x.z, x.w};
    uint32_t hw[2], mw[2], lw[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float a = v[2 * u], b = v[2 * u + 1];
        hw[u] = bf16_pair(a, b);
        const float ra = a - __uint_as_float(hw[u] << 16), rb = b - __uint_as_float(hw[u] & 0xffff0000u);
        mw[u] = bf16_pair(ra, rb);
        const float sa = ra - __uint_as_float(mw[u] << 16), sb = rb - __uint_as_float(mw[u] & 0xffff0000u);
        lw[u] = bf16_pair(sa, sb);
    }
    h = make_uint2(hw[0], hw[1]);
    m = make_uint2(mw[0], mw[1]);
    l = make_uint2(lw[0], lw[1]);
}


// One 64x64 output tile of D = X Y^T for node n of row b, over the K range
// of split blockIdx.x / tiles^2.  With one split the tile is final; with
// several it is a partial sum written to `part` and added by span_reduce.
// The levels that take this kernel hold few products, so a tile's K loop,
// not the chip's throughput, sets its time: each thread keeps DEPTH K
// blocks of loads in flight (a ring in registers; DEPTH divides the split's
// K blocks, which come in pairs, so every step of the loop is the same and
// the loads stay in flight across its iterations) and the LDS is
// double-buffered, one barrier per K block.  A deeper ring (4) measured
// slower: its registers cost more than the extra loads in flight gain.
constexpr int DEPTH = 2;

__global__ __launch_bounds__(kGemmThreads) void span_gemm(StepView sv, float *__restrict__ tree,
                                                          int32_t *__restrict__ meta, int n0,
                                                          int nn, int ksplit,
                                                          float *__restrict__ part)
{
    const int Sp = sv.Sp;
    const int tiles = Sp / kTile;
    const int T2 = tiles * tiles;
    const int tile = blockIdx.x % T2, split = blockIdx.x / T2;
    const int tm = (tile / tiles) * kTile, tn = (tile % tiles) * kTile;
    const int kc = Sp / ksplit, k_begin = split * kc;
    const int nb = kc / kBK;  // K blocks of this split
    const int b = blockIdx.y / nn, n = n0 + blockIdx.y % nn;
    const bool tr = stored_transposed(n);
    const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
    const float *F = sv.mat_ptr((const float *)tree, b, hF);
    const float *G = sv.mat_ptr((const float *)tree, b, hG);
    const int32_t *roF = sv.meta_ptr((const int32_t *)meta, b, hF, 0);
    const int32_t *coF = sv.meta_ptr((const int32_t *)meta, b, hF, 1);
    const int32_t *rfF = sv.meta_ptr((const int32_t *)meta, b, hF, 2);
    const int32_t *roG = sv.meta_ptr((const int32_t *)meta, b, hG, 0);
    const int32_t *coG = sv.meta_ptr((const int32_t *)meta, b, hG, 1);
    const int32_t *rfG = sv.meta_ptr((const int32_t *)meta, b, hG, 2);
    float *D = sv.mat_ptr(tree, b, n);
    int32_t *roD = sv.meta_ptr(meta, b, n, 0);
    int32_t *coD = sv.meta_ptr(meta, b, n, 1);
    int32_t *rfD = sv.meta_ptr(meta, b, n, 2);

    // per buffer and operand: the pieces h, m, l of 64 stored rows
    __shared__ __align__(16) __bf16 Fs[2][3][kTile][kLdb2];
    __shared__ __align__(16) __bf16 Gs[2][3][kTile][kLdb2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // loader: thread t stages float4 (t & 7) of rows (t >> 3) and (t >> 3) + 32
    // of both operands (the four entries share their column exponents)
    const int lrow = tid >> 3, lk = (tid & 7) * 4;
    const int rfF0 = rfF[tm + lrow], rfF1 = rfF[tm + lrow + 32];
    const int rfG0 = rfG[tn + lrow], rfG1 = rfG[tn + lrow + 32];
    const float *Frow = F + (size_t)(tm + lrow) * Sp + k_begin + lk;
    const float *Grow = G + (size_t)(tn + lrow) * Sp + k_begin + lk;
    const size_t r32 = (size_t)32 * Sp;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
    const int l32 = lane & 31, half = lane >> 5;

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    struct Blk {
        float4 f0, f1, g0, g1;
        int4 cf, cg;
    };
    // block bi of the split (past the last one it re-reads the last, so that
    // every step issues the same loads)
    auto gl = [&](Blk &x, int bi) {
        const int k0 = min(bi, nb - 1) * kBK;
        x.f0 = *reinterpret_cast<const float4 *>(Frow + k0);
        x.f1 = *reinterpret_cast<const float4 *>(Frow + r32 + k0);
        x.g0 = *reinterpret_cast<const float4 *>(Grow + k0);
        x.g1 = *reinterpret_cast<const float4 *>(Grow + r32 + k0);
        x.cf = *reinterpret_cast<const int4 *>(coF + k_begin + k0 + lk);
        x.cg = *reinterpret_cast<const int4 *>(coG + k_begin + k0 + lk);
    };
    auto put = [&](__bf16 (*X)[kTile][kLdb2], int row, float4 x) {
        uint2 h, m, l;
        split3(x, h, m, l);
        *reinterpret_cast<uint2 *>(&X[0][row][lk]) = h;
        *reinterpret_cast<uint2 *>(&X[1][row][lk]) = m;
        *reinterpret_cast<uint2 *>(&X[2][row][lk]) = l;
    };
    auto ls = [&](const Blk &x, int buf) {
        put(Fs[buf], lrow, fold4(x.f0, x.cf, rfF0));
        put(Fs[buf], lrow + 32, fold4(x.f1, x.cf, rfF1));
        put(Gs[buf], lrow, fold4(x.g0, x.cg, rfG0));
        put(Gs[buf], lrow + 32, fold4(x.g1, x.cg, rfG1));
    };
    // the block's two K steps of 16, each the six partial products
    auto mm = [&](int buf) {
#pragma unroll
        for (int t = 0; t < kBK; t += kBK3) {
            bf16x8 a[3], c[3];
#pragma unroll
            for (int pc = 0; pc < 3; ++pc) {
                a[pc] = *reinterpret_cast<const bf16x8 *>(&Fs[buf][pc][wr + l32][t + half * 8]);
                c[pc] = *reinterpret_cast<const bf16x8 *>(&Gs[buf][pc][wc + l32][t + half * 8]);
            }
#pragma unroll
            for (int pb = 0; pb < 3; ++pb)
#pragma unroll
                for (int pa = 0; pa < 3 - pb; ++pa)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[pa], c[pb], acc, 0, 0, 0);
        }
    };
    // block bi sits in ring[bi % DEPTH] until it is stored to LDS buffer
    // bi & 1; the slot is then refilled with block bi + DEPTH
    Blk ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) gl(ring[d], d);
    ls(ring[0], 0);
    gl(ring[0], DEPTH);
    __syncthreads();
    for (int bi = 0; bi < nb; bi += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            mm(d & 1);
            __builtin_amdgcn_sched_barrier(0);
            ls(ring[(d + 1) % DEPTH], (d + 1) & 1);
            gl(ring[(d + 1) % DEPTH], bi + d + 1 + DEPTH);
            __syncthreads();
        }
    }
    if (ksplit > 1) {  // partial tile, row-major 64x64
        float *pt = part + ((size_t)(blockIdx.y * ksplit + split) * T2 + tile) * (kTile * kTile);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = wr + (r >> 2) * 8 + half * 4 + (r & 3);
            pt[i * kTile + wc + l32] = acc[r];
        }
        return;
    }
    // epilogue: store, row fold normalizer (row maxima through the LDS of
    // the operand buffers, free after the loop's last barrier), outer scales
    const int j = tn + wc + l32;
    const int coDj = add_exp(roG[j], rfG[j]);
    int *E = reinterpret_cast<int *>(&Fs[0][0][0][0]);  // [kTile][2 * 32 + 4]
    constexpr int ldE = 2 * 32 + 4;
    static_assert(kTile * ldE * sizeof(int) <= sizeof(Fs), "row-maximum exchange fits the operand buffers");
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int il = wr + (r >> 2) * 8 + half * 4 + (r & 3);
        const float x = acc[r];
        D[(size_t)(tm + il) * Sp + j] = x;
        E[il * ldE + (wc >> 5) * 32 + l32] = scaled_exp(x, coDj);
    }
    __syncthreads();
    rowmax_from_lds(E, ldE, 64, kTile, rfD + tm);
    if (tn == 0 && tid < kTile) roD[tm + tid] = add_exp(roF[tm + tid], rfF[tm + tid]);
    if (tm == 0 && tid >= kTile && tid < 2 * kTile)
        coD[tn + tid - kTile] = add_exp(roG[tn + tid - kTile], rfG[tn + tid - kTile]);
}

// add the K-split partial tiles in split order and finish the tile as the
// single-split epilogue does
__global__ __launch_bounds__(kGemmThreads) void span_reduce(StepView sv, float *__restrict__ tree,
                                                            int32_t *__restrict__ meta, int n0,
                                                            int nn, int ksplit,
                                                            const float *__restrict__ part)
{
    const int Sp = sv.Sp;
    const int tiles = Sp / kTile;
    const int T2 = tiles * tiles;
    const int tile = blockIdx.x;
    const int tm = (tile / tiles) * kTile, tn = (tile % tiles) * kTile;
    const int b = blockIdx.y / nn, n = n0 + blockIdx.y % nn;
    const bool tr = stored_transposed(n);
    const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
    const int32_t *roF = sv.meta_ptr((const int32_t *)meta, b, hF, 0);
    const int32_t *rfF = sv.meta_ptr((const int32_t *)meta, b, hF, 2);
    const int32_t *roG = sv.meta_ptr((const int32_t *)meta, b, hG, 0);
    const int32_t *rfG = sv.meta_ptr((const int32_t *)meta, b, hG, 2);
    float *D = sv.mat_ptr(tree, b, n);
    int32_t *roD = sv.meta_ptr(meta, b, n, 0);
    int32_t *coD = sv.meta_ptr(meta, b, n, 1);
    int32_t *rfD = sv.meta_ptr(meta, b, n, 2);
    const int tid = threadIdx.x;
    const int i = tid >> 2, c0 = (tid & 3) * 16;  // row i, 16 columns
    float4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < ksplit; ++s) {
        const float *pt = part + ((size_t)(blockIdx.y * ksplit + s) * T2 + tile) * (kTile * kTile) +
                          i * kTile + c0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 y = *reinterpret_cast<const float4 *>(pt + 4 * q);
            acc[q].x += y.x;
            acc[q].y += y.y;
            acc[q].z += y.z;
            acc[q].w += y.w;
        }
    }
    int e = kNeg;
    float *drow = D + (size_t)(tm + i) * Sp + tn + c0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<float4 *>(drow + 4 * q) = acc[q];
        const float v4[4] = {acc[q].x, acc[q].y, acc[q].z, acc[q].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = tn + c0 + 4 * q + u;
            const int coDj = add_exp(roG[j], rfG[j]);
            if (v4[u] > 0.f && coDj > kNeg) e = max(e, fexp(v4[u]) + coDj);
        }
    }
    e = max(e, __shfl_xor(e, 1));
    e = max(e, __shfl_xor(e, 2));
    if ((tid & 3) == 0 && e > kNeg) atomicMax(&rfD[tm + i], e);
    if (tn == 0 && tid < kTile) roD[tm + tid] = add_exp(roF[tm + tid], rfF[tm + tid]);
    if (tm == 0 && tid < kTile) coD[tn + tid] = add_exp(roG[tn + tid], rfG[tn + tid]);
}

constexpr int kBig = 128;       // output tile of the large-level kernel
constexpr int kBigThreads = 512;

// 128x128 output tiles, eight wavefronts of 32x64 (1x2 MFMA 32x32 blocks),
// double-buffered LDS stages of K = 16 (74 KB of LDS); the global data of
// stage s+1 is loaded while stage s runs.  Small per-wave state keeps four
// wavefronts per SIMD resident.  grid.x enumerates (product, tile) so that
// the tiles of one product land on one XCD.
__global__ __launch_bounds__(kBigThreads) void span_gemm128(StepView sv, float *__restrict__ tree,
                                                            int32_t *__restrict__ meta, int n0,
                                                            int nn)
{
    const int Sp = sv.Sp;
    const int tiles = Sp / kBig;
    const int per_prod = tiles * tiles;
    const int nwork = sv.B * nn * per_prod;
    int w = blockIdx.x;
    const int full = nwork & ~7;
    if (w < full) w = (w & 7) * (full >> 3) + (w >> 3);  // XCD-contiguous work order
    const int prod = w / per_prod, tile = w % per_prod;
    const int tm = (tile / tiles) * kBig, tn = (tile % tiles) * kBig;
    const int b = prod / nn, n = n0 + prod % nn;
    const bool tr = stored_transposed(n);
    const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
    const float *F = sv.mat_ptr((const float *)tree, b, hF);
    const float *G = sv.mat_ptr((const float *)tree, b, hG);
    const int32_t *roF = sv.meta_ptr((const int32_t *)meta, b, hF, 0);
    const int32_t *coF = sv.meta_ptr((const int32_t *)meta, b, hF, 1);
    const int32_t *rfF = sv.meta_ptr((const int32_t *)meta, b, hF, 2);
    const int32_t *roG = sv.meta_ptr((const int32_t *)meta, b, hG, 0);
    const int32_t *coG = sv.meta_ptr((const int32_t *)meta, b, hG, 1);
    const int32_t *rfG = sv.meta_ptr((const int32_t *)meta, b, hG, 2);
    float *D = sv.mat_ptr(tree, b, n);
    int32_t *roD = sv.meta_ptr(meta, b, n, 0);
    int32_t *coD = sv.meta_ptr(meta, b, n, 1);
    int32_t *rfD = sv.meta_ptr(meta, b, n, 2);

    // per buffer and operand: the pieces h, m, l of 128 stored rows
    __shared__ __align__(16) __bf16 Fs[2][3][kBig][kLdb];
    __shared__ __align__(16) __bf16 Gs[2][3][kBig][kLdb];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // loader: thread t stages float4 (t & 3) of row t >> 2 of both
    // operands, so four lanes read one 64-byte row segment
    const int lrow = tid >> 2, lk = (tid & 3) * 4;
    const int rfF0 = rfF[tm + lrow], rfG0 = rfG[tn + lrow];
    const float *Frow = F + (size_t)(tm + lrow) * Sp + lk;
    const float *Grow = G + (size_t)(tn + lrow) * Sp + lk;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 64;
    const int l32 = lane & 31, half = lane >> 5;

    f32x16 acc[2];
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[y][r] = 0.f;

    float4 fr, gr;
    int4 cf, cg;
    auto gload = [&](int k0) {
        fr = *reinterpret_cast<const float4 *>(Frow + k0);
        gr = *reinterpret_cast<const float4 *>(Grow + k0);
        cf = *reinterpret_cast<const int4 *>(coF + k0 + lk);
        cg = *reinterpret_cast<const int4 *>(coG + k0 + lk);
    };
    auto put = [&](__bf16 (*X)[kBig][kLdb], float4 x) {
        uint2 h, m, l;
        split3(x, h, m, l);
        *reinterpret_cast<uint2 *>(&X[0][lrow][lk]) = h;
        *reinterpret_cast<uint2 *>(&X[1][lrow][lk]) = m;
        *reinterpret_cast<uint2 *>(&X[2][lrow][lk]) = l;
    };
    auto lstore = [&](int buf) {
        put(Fs[buf], fold4(fr, cf, rfF0));
        put(Gs[buf], fold4(gr, cg, rfG0));
    };
    const int nk = Sp / kBK3;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        // unconditional (the last step re-reads the final K block), and kept
        // ahead of the MFMAs, with the split arithmetic after them
        gload(min(ks + 1, nk - 1) * kBK3);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 a[3], c[3][2];
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
            a[pc] = *reinterpret_cast<const bf16x8 *>(&Fs[buf][pc][wr + l32][half * 8]);
#pragma unroll
            for (int y = 0; y < 2; ++y)
                c[pc][y] = *reinterpret_cast<const bf16x8 *>(&Gs[buf][pc][wc + 32 * y + l32][half * 8]);
        }
        // the six partial products, grouped by the second operand's piece
#pragma unroll
        for (int pb = 0; pb < 3; ++pb)
#pragma unroll
            for (int pa = 0; pa < 3 - pb; ++pa)
#pragma unroll
                for (int y = 0; y < 2; ++y)
                    acc[y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[pa], c[pb][y], acc[y], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        lstore(buf ^ 1);
        __syncthreads();
    }
    // epilogue: D, then the row maxima through the LDS of the operand
    // buffers (free after the loop's last barrier)
    int coDj[2];
#pragma unroll
    for (int y = 0; y < 2; ++y) {
        const int j = tn + wc + 32 * y + l32;
        coDj[y] = add_exp(roG[j], rfG[j]);
    }
    int *E = reinterpret_cast<int *>(&Fs[0][0][0][0]);  // [kBig][2 * 32 + 4]
    constexpr int ldE = 2 * 32 + 4;
    static_assert(kBig * ldE * sizeof(int) <= sizeof(Fs), "row-maximum exchange fits the operand buffers");
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int il = wr + (r >> 2) * 8 + half * 4 + (r & 3);
        int e = kNeg;
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const float v = acc[y][r];
            D[(size_t)(tm + il) * Sp + tn + wc + 32 * y + l32] = v;
            e = max(e, scaled_exp(v, coDj[y]));
        }
        E[il * ldE + (wc >> 6) * 32 + l32] = e;
    }
    __syncthreads();
    rowmax_from_lds(E, ldE, 64, kBig, rfD + tm);
    if (tn == 0 && tid < kBig) roD[tm + tid] = add_exp(roF[tm + tid], rfF[tm + tid]);
    if (tm == 0 && tid >= kBig && tid < 2 * kBig)
        coD[tn + tid - kBig] = add_exp(roG[tn + tid - kBig], rfG[tn + tid - kBig]);
}

// log Z[b] = ln sum_{f in F} T_root[s0][f]
__global__ void tree_logz(DevTable d, StepView sv, const float *__restrict__ tree,
                          const int32_t *__restrict__ meta, double *__restrict__ logZ,
                          int32_t *__restrict__ status)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    const float *R = sv.mat_ptr(tree, b, 1) + (size_t)d.start * sv.Sp;
    const int32_t *co = sv.meta_ptr(meta, b, 1, 1);
    const int32_t ro = sv.meta_ptr(meta, b, 1, 0)[d.start];
    int e = kNeg;
    for (int k = lane; k < d.n_acc; k += 64) {
        const int f = d.acc[k];
        const float x = R[f];
        if (x > 0.f && co[f] > kNeg) e = max(e, fexp(x) + co[f]);
    }
    const int m = wave_max_i(e);
    double z = 0.0;
    if (m > kNeg)
        for (int k = lane; k < d.n_acc; k += 64) {
            const int f = d.acc[k];
            z += (double)scale2(R[f], co[f] - m);
        }
    z = wave_sum_d(z);
    if (lane == 0) {
        const bool bad = (status[b] & FA_ROW_BADPROB) != 0;
        if (z > 0.0 && m > kNeg && ro > kNeg && !bad) {
            logZ[b] = ((double)ro + (double)m) * 0.69314718055994530942 + log(z);
        } else {
            logZ[b] = -INFINITY;
            if (!bad) atomicOr(&status[b], (int)FA_ROW_INFEASIBLE);
        }
    }
}

// L == 0: the empty string is accepted iff s0 is accepting
__global__ void tree_logz_empty(DevTable d, int B, double *__restrict__ logZ,
                                int32_t *__restrict__ status)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    bool ok = false;
    for (int k = 0; k < d.n_acc; ++k) ok |= d.acc[k] == d.start;
    logZ[b] = ok ? 0.0 : -INFINITY;
    if (!ok) atomicOr(&status[b], (int)FA_ROW_INFEASIBLE);
}

constexpr int kHuge = 256;
constexpr int kHugeThreads = 512;

// The tiles of one 256x256-tile launch: products n0 .. n0+nn-1 of every
// batch row, each of (Sp/256)^2 tiles.  With several tiles per product, the
// tiles that run on one XCD (every eighth workgroup) are consecutive ones,
// which share operand rows in L2.
struct HugeWork {
    int Sp, tiles, per_prod, nwork, full, n0, nn;
    __device__ HugeWork(const StepView &sv, int n0_, int nn_)
        : Sp(sv.Sp), tiles(sv.Sp / 256), per_prod((sv.Sp / 256) * (sv.Sp / 256)),
          nwork(sv.B * nn_ * (sv.Sp / 256) * (sv.Sp / 256)), full(0), n0(n0_), nn(nn_)
    {
        full = nwork & ~7;
    }
    __device__ int work(int v) const
    {
        return (per_prod > 1 && v < full) ? (v & 7) * (full >> 3) + (v >> 3) : v;
    }
    // tile v: batch row, node, first output row and column
    __device__ void node_of(int v, int &b, int &n, int &tm, int &tn) const
    {
        const int w = work(v);
        const int prod = w / per_prod, tile = w % per_prod;
        tm = (tile / tiles) * 256;
        tn = (tile % tiles) * 256;
        b = prod / nn;
        n = n0 + prod % nn;
    }
};

// Epilogue of a 256x256 output tile held by 8 waves of 64 x 128 (2 x 4
// tiles of 32x32): D, and per row the largest e(D[i][j]) + coD[j], reduced
// through E0 (the waves of columns 0..127) and E1 (128..255), two LDS
// regions of 256 x kLde ints that are free until the caller's next barrier;
// the first tile row / column also writes coD / roD.  All 512 threads call
// it (it holds a barrier).
constexpr int kLde = 36;

__device__ __forceinline__ void huge_epilogue(const StepView &sv, float *__restrict__ tree,
                                              int32_t *__restrict__ meta, f32x16 (&acc)[2][4],
                                              int *E0, int *E1, int b, int n, int tm, int tn,
                                              const int32_t *rfF, const int32_t *rfG)
{
    const int Sp = sv.Sp;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 128;
    const int l32 = lane & 31, half = lane >> 5;
    const bool tr = stored_transposed(n);
    const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
    const int32_t *roF = sv.meta_ptr((const int32_t *)meta, b, hF, 0);
    const int32_t *roG = sv.meta_ptr((const int32_t *)meta, b, hG, 0);
    float *D = sv.mat_ptr(tree, b, n);
    // this lane's first row and column in the tile; the empty asm keeps
    // the addresses derived from them out of the tile loop (where they
    // would stay live through the MFMAs)
    int row0 = wr + half * 4, col0 = wc + l32;
    asm volatile("" : "+v"(row0), "+v"(col0));
    // every exponent the epilogue needs is loaded first, so that one
    // load latency covers them all and the stores of D go out meanwhile
    int coDj[4];
#pragma unroll
    for (int cy = 0; cy < 4; ++cy) {
        const int j = tn + col0 + 32 * cy;
        coDj[cy] = add_exp(roG[j], rfG[j]);
    }
    int outer = kNeg;  // roD[tm + tid] (tid < 256) or coD[tn + tid - 256]
    if (tid < 256) {
        if (tn == 0) outer = add_exp(roF[tm + tid], rfF[tm + tid]);
    } else if (tm == 0) {
        outer = add_exp(roG[tn + tid - 256], rfG[tn + tid - 256]);
    }
#pragma unroll
    for (int ry = 0; ry < 2; ++ry)
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int cy = 0; cy < 4; ++cy)
                D[(size_t)(tm + row0 + 32 * ry + (r >> 2) * 8 + (r & 3)) * Sp + tn + col0 + 32 * cy] =
                    acc[ry][cy][r];
    // per row the maximum over this lane's four columns: E[il][l32] of the
    // wave's column half, rows padded to kLde entries
    int *E = wc == 0 ? E0 : E1;
#pragma unroll
    for (int ry = 0; ry < 2; ++ry) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int e = kNeg;
#pragma unroll
            for (int cy = 0; cy < 4; ++cy) {
                const float x = acc[ry][cy][r];
                int ex;
                frexpf(x, &ex);
                const bool ok = (x > 0.f) & (coDj[cy] > kNeg);
                e = max(e, ok ? ex + coDj[cy] : kNeg);
            }
            E[(row0 + 32 * ry + (r >> 2) * 8 + (r & 3)) * kLde + l32] = e;
        }
    }
    __syncthreads();
    if (tid < 256) {
        const int4 *e0 = reinterpret_cast<const int4 *>(E0 + tid * kLde);
        const int4 *e1 = reinterpret_cast<const int4 *>(E1 + tid * kLde);
        int e = kNeg;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int4 x = e0[k], y = e1[k];
            e = max(e, max(max(max(x.x, x.y), max(x.z, x.w)), max(max(y.x, y.y), max(y.z, y.w))));
        }
        int32_t *rfD = sv.meta_ptr(meta, b, n, 2);
        if (Sp == 256) rfD[tm + tid] = e;
        else if (e > kNeg) atomicMax(&rfD[tm + tid], e);
        if (tn == 0) sv.meta_ptr(meta, b, n, 0)[tm + tid] = outer;
    } else if (tm == 0) {
        sv.meta_ptr(meta, b, n, 1)[tn + tid - 256] = outer;
    }
}

// Large levels with 256x256 output tiles (one whole product when Sp = 256),
// one persistent workgroup per CU walking tiles v = blockIdx.x + k gridDim.x:
// 8 waves of 64 x 128 (2 x 4 MFMA tiles of 32x32), double-buffered LDS
// (147 KB) with K steps of 16 (the bf16 pieces above).  The loads of block
// ks+1 are in flight while block ks computes (48 MFMAs per wave); during
// the last K step of a tile they fetch block 0 of the workgroup's next tile
// (or re-read block 0 of the current one when there is none), so the next
// tile starts from a filled buffer while the current one is stored.  Row
// exponents are reduced inside the workgroup through the free LDS buffer:
// one store (full rows) or atomicMax (several column tiles) per row.
// the operand side of one 256x256 tile: stored rows tm.. of F, tn.. of G
struct HugeSrc {
    const float *F, *G;
    const int32_t *coF, *coG, *rfF, *rfG;
    const int32_t *kidx;  // LIVE: the states live at the midpoint, padded with -1
    int tm, tn;
    int nk;               // K steps of 16
};

// LIVE (tables compiled with FA_LIVE_STATES): the contraction runs over the
// states live at the product's midpoint (lists and counts from
// launch_live_states), each K step gathering 16 listed columns of both
// operands; list entries of -1 load zero.
template <bool LIVE>
__global__ __launch_bounds__(kHugeThreads) void span_gemm256(StepView sv, float *__restrict__ tree,
                                                             int32_t *__restrict__ meta, int n0,
                                                             int nn, const int32_t *__restrict__ live,
                                                             const int32_t *__restrict__ nlive)
{
    const int Sp = sv.Sp;
    const HugeWork hw(sv, n0, nn);
    const int nwork = hw.nwork;
    auto src_of = [&](int v) {
        int b, n, tm, tn;
        hw.node_of(v, b, n, tm, tn);
        const bool tr = stored_transposed(n);
        const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
        HugeSrc s;
        s.F = sv.mat_ptr((const float *)tree, b, hF);
        s.G = sv.mat_ptr((const float *)tree, b, hG);
        s.coF = sv.meta_ptr((const int32_t *)meta, b, hF, 1);
        s.coG = sv.meta_ptr((const int32_t *)meta, b, hG, 1);
        s.rfF = sv.meta_ptr((const int32_t *)meta, b, hF, 2);
        s.rfG = sv.meta_ptr((const int32_t *)meta, b, hG, 2);
        s.tm = tm;
        s.tn = tn;
        s.kidx = nullptr;
        s.nk = Sp / kBK3;
        if constexpr (LIVE) {
            // node n of level k: the level's nodes start at 2^(K-k) = Lpad / span
            const int first = 1 << (31 - __clz(n));
            const int span = sv.Lpad / first;
            const int m = (n - first) * span + span / 2;  // midpoint boundary
            const size_t bm = (size_t)b * (sv.Lpad + 1) + m;
            s.kidx = live + bm * Sp;
            s.nk = max(4, (nlive[bm] + 63) / 64 * 4);
        }
        return s;
    };

    // per buffer and operand: the pieces h, m, l of 256 stored rows
    __shared__ __align__(16) __bf16 Fs[2][3][kHuge][kLdb];
    __shared__ __align__(16) __bf16 Gs[2][3][kHuge][kLdb];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // loader: thread t stages float4 (t & 3) of rows (t >> 2) + 128 q, q < 2,
    // of both operands: four lanes read one 64-byte row segment
    const int lrow = tid >> 2, lk = (tid & 3) * 4;
    const size_t q_rows = (size_t)128 * Sp;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 128;
    const int l32 = lane & 31, half = lane >> 5;

    struct Stage {
        float4 f[2], g[2];
        int4 cf, cg;
        int rf[2], rg[2];
    };
    // the rows' exponents come with block 0 of a tile and stay for its other blocks
    auto gload = [&](Stage &st, const HugeSrc &s, int ks, bool rows) {
        const int k0 = ks * kBK3;
        if constexpr (LIVE) {
            const int4 kk = *reinterpret_cast<const int4 *>(s.kidx + k0 + lk);
            const int k[4] = {max(kk.x, 0), max(kk.y, 0), max(kk.z, 0), max(kk.w, 0)};
            const bool ok[4] = {kk.x >= 0, kk.y >= 0, kk.z >= 0, kk.w >= 0};
            const float *Fr = s.F + (size_t)(s.tm + lrow) * Sp;
            const float *Gr = s.G + (size_t)(s.tn + lrow) * Sp;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float *fr = Fr + q * q_rows, *gr = Gr + q * q_rows;
                float fv[4], gv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    fv[u] = fr[k[u]];
                    gv[u] = gr[k[u]];
                }
                st.f[q] = make_float4(ok[0] ? fv[0] : 0.f, ok[1] ? fv[1] : 0.f, ok[2] ? fv[2] : 0.f,
                                      ok[3] ? fv[3] : 0.f);
                st.g[q] = make_float4(ok[0] ? gv[0] : 0.f, ok[1] ? gv[1] : 0.f, ok[2] ? gv[2] : 0.f,
                                      ok[3] ? gv[3] : 0.f);
            }
            st.cf = make_int4(s.coF[k[0]], s.coF[k[1]], s.coF[k[2]], s.coF[k[3]]);
            st.cg = make_int4(s.coG[k[0]], s.coG[k[1]], s.coG[k[2]], s.coG[k[3]]);
        } else {
            const float *Fr = s.F + (size_t)(s.tm + lrow) * Sp + lk + k0;
            const float *Gr = s.G + (size_t)(s.tn + lrow) * Sp + lk + k0;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                st.f[q] = *reinterpret_cast<const float4 *>(Fr + q * q_rows);
                st.g[q] = *reinterpret_cast<const float4 *>(Gr + q * q_rows);
            }
            st.cf = *reinterpret_cast<const int4 *>(s.coF + k0 + lk);
            st.cg = *reinterpret_cast<const int4 *>(s.coG + k0 + lk);
        }
        if (rows) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                st.rf[q] = s.rfF[s.tm + lrow + 128 * q];
                st.rg[q] = s.rfG[s.tn + lrow + 128 * q];
            }
        }
    };
    auto put = [&](__bf16 (*X)[kHuge][kLdb], int row, float4 x) {
        uint2 h, m, l;
        split3(x, h, m, l);
        *reinterpret_cast<uint2 *>(&X[0][row][lk]) = h;
        *reinterpret_cast<uint2 *>(&X[1][row][lk]) = m;
        *reinterpret_cast<uint2 *>(&X[2][row][lk]) = l;
    };
    auto lstore = [&](const Stage &st, int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            put(Fs[buf], lrow + 128 * q, fold4(st.f[q], st.cf, st.rf[q]));
            put(Gs[buf], lrow + 128 * q, fold4(st.g[q], st.cg, st.rg[q]));
        }
    };
    f32x16 acc[2][4];
    // the six partial products, grouped by the second operand's piece, each
    // over the 8 output tiles in turn (no MFMA waits for the one before it)
    auto mfmas = [&](int buf) {
        bf16x8 a[3][2], c[4];
#pragma unroll
        for (int pa = 0; pa < 3; ++pa)
#pragma unroll
            for (int ry = 0; ry < 2; ++ry)
                a[pa][ry] = *reinterpret_cast<const bf16x8 *>(&Fs[buf][pa][wr + 32 * ry + l32][half * 8]);
#pragma unroll
        for (int pb = 0; pb < 3; ++pb) {
#pragma unroll
            for (int cy = 0; cy < 4; ++cy)
                c[cy] = *reinterpret_cast<const bf16x8 *>(&Gs[buf][pb][wc + 32 * cy + l32][half * 8]);
#pragma unroll
            for (int pa = 0; pa < 3 - pb; ++pa)
#pragma unroll
                for (int ry = 0; ry < 2; ++ry)
#pragma unroll
                    for (int cy = 0; cy < 4; ++cy)
                        acc[ry][cy] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[pa][ry], c[cy], acc[ry][cy],
                                                                              0, 0, 0);
        }
    };

    int v = blockIdx.x;
    if (v >= nwork) return;
    HugeSrc cur = src_of(v);
    Stage st;
    gload(st, cur, 0, true);
    lstore(st, 0);
    __syncthreads();
    for (;;) {
        const int vn = v + (int)gridDim.x;
        const bool more = vn < nwork;
        const HugeSrc nxt = more ? src_of(vn) : cur;
#pragma unroll
        for (int ry = 0; ry < 2; ++ry)
#pragma unroll
            for (int cy = 0; cy < 4; ++cy)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[ry][cy][r] = 0.f;
        // step ks: issue the loads of K block ks+1 (of the next tile after
        // the last block), compute buffer ks & 1 (48 MFMAs per wave cover
        // the load latency), store that block into the other buffer.
        // A tile's K steps (Sp / 16, or its live list's length / 16) are
        // even.  The scheduling barriers keep the compiler from moving the
        // fold arithmetic of the stores (which waits for the loads) into
        // the MFMAs.
        for (int ks = 0; ks < cur.nk; ks += 2) {
            gload(st, cur, ks + 1, false);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(0);
            __builtin_amdgcn_sched_barrier(0);
            lstore(st, 1);
            __syncthreads();
            const bool last = ks + 2 == cur.nk;
            gload(st, last ? nxt : cur, last ? 0 : ks + 2, last);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(1);
            __builtin_amdgcn_sched_barrier(0);
            lstore(st, 0);
            __syncthreads();
        }
        // epilogue, the row maxima through buffer 1 (free until the next
        // tile's first store into it)
        int b, n, tm, tn;
        hw.node_of(v, b, n, tm, tn);
        static_assert(kHuge * kLde * sizeof(int) <= sizeof(Fs[1]), "row-maximum exchange fits one buffer");
        huge_epilogue(sv, tree, meta, acc, reinterpret_cast<int *>(&Fs[1][0][0][0]),
                      reinterpret_cast<int *>(&Gs[1][0][0][0]), b, n, tm, tn, cur.rfF, cur.rfG);
        if (!more) break;
        __syncthreads();  // buffer 1 is read above and written by the next tile
        v = vn;
        cur = nxt;
    }
}


// The first level as the dense product of 256x256 tiles, its operands
// staged from the leaves' folded pair values (value times 2^-rf of its
// stored row, as fa_build_transitions leaves them in the workspace) instead
// of dense leaves: a K step of 16 stored columns holds the entries of the
// pairs whose stored column lies in it, zeros elsewhere, which are the
// values the dense kernel folds from a dense leaf (an identity leaf past the
// sequence end: 2^-rf on its diagonal).  A row-major leaf is walked in
// column order (col_ptr, ent_t_rc), a transposed one in pair order
// (row_ptr, ent_n_rc), both giving (stored column << 16 | stored row); the
// values are stored in that walk order, so entry e of a step and its value
// are two independent loads.
//
// LDS: a ring of three slots of both operands' three bf16 pieces (rows of
// 16 entries, 32 bytes, the two 16-byte halves swapped on rows with bit 3
// set so that the fragment reads of 16 lanes hit distinct banks).  During K
// step s the MFMAs read slot s % 3 while slot (s+2) % 3 is cleared and the
// entries of step s+1 (loaded before the MFMAs) are written into slot
// (s+1) % 3, cleared during step s-1: one barrier per step.  Each thread
// holds kPvPer entries per operand and step; more are read when written.
// The MFMAs, their order and the epilogue are those of span_gemm256, so the
// products equal the dense-leaf ones bit for bit.
constexpr int kPvSlots = 3;
constexpr int kPvPer = 2;
constexpr int kPvMaxSteps = kMapMaxSp / kBK3;  // Sp <= kMapMaxSp (the pair maps exist)

struct PvOperand {
    const int32_t *rc;   // walk order: stored (column << 16 | row)
    const float *pv;     // walk order: the leaf's folded values; nullptr for an identity leaf
    const int32_t *rf;   // the leaf's row exponents
    const int *wofs;     // LDS: walk offset of each K step's first column, [steps + 1]
    int t0;              // first stored row of the tile
};

// the held entries of one operand and K step
struct PvHeld {
    int rc[kPvPer];
    float v[kPvPer];
};

__device__ inline int pv_swz(int row, int col) { return row * kBK3 + (col ^ (((row >> 3) & 1) << 3)); }

__global__ __launch_bounds__(kHugeThreads) void span_pairs256(DevTable d, StepView sv,
                                                              float *__restrict__ tree,
                                                              int32_t *__restrict__ meta,
                                                              const float *__restrict__ pvf, int n0,
                                                              int nn, int init_upper)
{
    const int Sp = sv.Sp;
    const HugeWork hw(sv, n0, nn);
    const int nk = Sp / kBK3;
    // with one tile per product (rows stored whole), the first level needs no
    // rf initialized and clears that of the levels above it instead of a
    // launch of its own (they run after this launch)
    if (init_upper) init_rf_nodes(sv, meta, sv.Lpad >> 1);
    // [slot][operand][piece][row][16]
    __shared__ __align__(16) __bf16 Ls[kPvSlots][2][3][kHuge * kBK3];
    __shared__ int wofs_t[kPvMaxSteps + 1], wofs_n[kPvMaxSteps + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 128;
    const int l32 = lane & 31, half = lane >> 5;
    for (int j = tid; j <= nk; j += kHugeThreads) {
        const int c = min(j * kBK3, d.S);
        wofs_t[j] = d.col_ptr[c];
        wofs_n[j] = d.row_ptr[c];
    }
    int v = blockIdx.x;
    if (v >= hw.nwork) return;

    auto operand = [&](int b, int h, int t0) {
        PvOperand o;
        const int i = h - sv.Lpad;  // position of the leaf
        const bool tr = stored_transposed(h);
        o.rc = tr ? d.ent_n_rc : d.ent_t_rc;
        o.pv = i < sv.L ? pvf + ((size_t)b * sv.L + i) * d.npairs : nullptr;
        o.rf = sv.meta_ptr((const int32_t *)meta, b, h, 2);
        o.wofs = tr ? wofs_n : wofs_t;
        o.t0 = t0;
        return o;
    };
    auto load = [&](const PvOperand &o, int ks, PvHeld &x) {
        const int e0 = o.wofs[ks], e1 = o.wofs[ks + 1];
#pragma unroll
        for (int u = 0; u < kPvPer; ++u) {
            const int e = e0 + tid + u * kHugeThreads;
            const bool ok = o.pv != nullptr && e < e1;
            const int ec = ok ? e : 0;
            const int rc = o.rc[ec];
            const float v = o.pv ? o.pv[ec] : 0.f;
            x.rc[u] = ok ? rc : -1;
            x.v[u] = v;
        }
    };
    auto put1 = [&](__bf16 *X, int row, int col, float x) {
        const __bf16 h = (__bf16)x;
        const float r = x - (float)h;
        const __bf16 m = (__bf16)r;
        const int a = pv_swz(row, col);
        X[a] = h;
        X[kHuge * kBK3 + a] = m;
        X[2 * kHuge * kBK3 + a] = (__bf16)(r - (float)m);
    };
    // the entries of K step ks into slot sl: the held ones, then any beyond
    // kPvPer per thread, or the identity's diagonal
    auto scatter = [&](const PvOperand &o, int opi, int sl, int ks, const PvHeld &x) {
        __bf16 *X = &Ls[sl][opi][0][0];
        const int k0 = ks * kBK3;
        if (o.pv) {
#pragma unroll
            for (int u = 0; u < kPvPer; ++u) {
                const int rc = x.rc[u];
                const int row = (rc & 0xffff) - o.t0;
                if (rc >= 0 && (unsigned)row < (unsigned)kHuge) put1(X, row, (rc >> 16) - k0, x.v[u]);
            }
            const int e1 = o.wofs[ks + 1];
            for (int e = o.wofs[ks] + tid + kPvPer * kHugeThreads; e < e1; e += kHugeThreads) {
                const int rc = o.rc[e];
                const int row = (rc & 0xffff) - o.t0;
                if ((unsigned)row < (unsigned)kHuge) put1(X, row, (rc >> 16) - k0, o.pv[e]);
            }
        } else if (tid < kBK3) {
            const int k = k0 + tid, row = k - o.t0;
            if (k < d.S && (unsigned)row < (unsigned)kHuge) put1(X, row, tid, ldexpf(1.f, 0 - o.rf[k]));
        }
    };
    auto clear = [&](int sl) {
        uint4 *z = reinterpret_cast<uint4 *>(&Ls[sl][0][0][0]);
        constexpr int n16 = (int)(sizeof(Ls[0]) / sizeof(uint4));
        static_assert(n16 % kHugeThreads == 0, "one slot clears in whole rounds");
#pragma unroll
        for (int k = 0; k < n16 / kHugeThreads; ++k) z[tid + k * kHugeThreads] = make_uint4(0u, 0u, 0u, 0u);
    };
    f32x16 acc[2][4];
    auto mfmas = [&](int sl) {
        const __bf16 *F = &Ls[sl][0][0][0], *G = &Ls[sl][1][0][0];
        bf16x8 a[3][2], c[4];
#pragma unroll
        for (int pa = 0; pa < 3; ++pa)
#pragma unroll
            for (int ry = 0; ry < 2; ++ry) {
                const int row = wr + 32 * ry + l32;
                a[pa][ry] = *reinterpret_cast<const bf16x8 *>(F + pa * kHuge * kBK3 + pv_swz(row, half * 8));
            }
#pragma unroll
        for (int pb = 0; pb < 3; ++pb) {
#pragma unroll
            for (int cy = 0; cy < 4; ++cy) {
                const int row = wc + 32 * cy + l32;
                c[cy] = *reinterpret_cast<const bf16x8 *>(G + pb * kHuge * kBK3 + pv_swz(row, half * 8));
            }
#pragma unroll
            for (int pa = 0; pa < 3 - pb; ++pa)
#pragma unroll
                for (int ry = 0; ry < 2; ++ry)
#pragma unroll
                    for (int cy = 0; cy < 4; ++cy)
                        acc[ry][cy] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[pa][ry], c[cy], acc[ry][cy],
                                                                              0, 0, 0);
        }
    };

    for (;;) {
        int b, n, tm, tn;
        hw.node_of(v, b, n, tm, tn);
        const bool tr = stored_transposed(n);
        const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
        const PvOperand oF = operand(b, hF, tm), oG = operand(b, hG, tn);
#pragma unroll
        for (int ry = 0; ry < 2; ++ry)
#pragma unroll
            for (int cy = 0; cy < 4; ++cy)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[ry][cy][r] = 0.f;
        // prologue: slots 0 and 1 cleared, step 0 written into slot 0
        PvHeld xF, xG;
        clear(0);
        clear(1);
        __syncthreads();  // the window offsets, and the clears
        load(oF, 0, xF);
        load(oG, 0, xG);
        scatter(oF, 0, 0, 0, xF);
        scatter(oG, 1, 0, 0, xG);
        __syncthreads();
        for (int ks = 0; ks < nk; ++ks) {
            const bool nxt = ks + 1 < nk;
            if (nxt) {  // the entries of step ks+1, in flight during the MFMAs
                load(oF, ks + 1, xF);
                load(oG, ks + 1, xG);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfmas(ks % 3);
            __builtin_amdgcn_sched_barrier(0);
            clear((ks + 2) % 3);
            if (nxt) {
                scatter(oF, 0, (ks + 1) % 3, ks + 1, xF);
                scatter(oG, 1, (ks + 1) % 3, ks + 1, xG);
            }
            __syncthreads();
        }
        // epilogue, the row maxima through slots 0 and 1 (every slot is
        // free after the last step's barrier)
        static_assert(kHuge * kLde * sizeof(int) <= sizeof(Ls[0]), "row-maximum exchange fits one slot");
        huge_epilogue(sv, tree, meta, acc, reinterpret_cast<int *>(&Ls[0][0][0][0]),
                      reinterpret_cast<int *>(&Ls[1][0][0][0]), b, n, tm, tn, oF.rf, oG.rf);
        v += (int)gridDim.x;
        if (v >= hw.nwork) break;
        __syncthreads();  // slots 0 and 1 are read above and cleared by the next tile
    }
}

// Sparse levels.  A leaf holds one value per pair (a, b) of the automaton,
// so a first-level product is a row combination: stored row s of node n is
// the sum over the first operand's pairs (s, k) of x1 times the second
// operand's row k, where both operands are the folded entries the dense
// kernels consume (value times 2^(co - rf) of its stored row and column),
// given per node in its stored entry order; identity leaves past the
// sequence end hold their diagonal.  A node stored as is walks rows (pair
// order, row pointers); a transposed node walks columns (column order),
// which are its stored rows.  Both operands use the same walk, so the first
// operand's entry e has target array entry e as its k.  The second level is
// the same over the two-step pattern (pairs (a, c) joined through some k),
// whose values the first level extracts from its output rows.
//
// One wave builds one output row, a window of `win` columns at a time, in
// two LDS row buffers.  The row's work in a window is cut into tasks of at
// most 32 items (one k, a slice of its row inside the window), numbered by
// a ballot or a prefix sum over the entries; lane group g (32 lanes) runs
// tasks g, g + 2, ... into buffer g, one item per lane, both groups in
// lockstep.  Within one task the targets are distinct pairs and one wave's
// LDS accesses stay in program order, so the buffers need no atomics; the
// row is buffer 0 + buffer 1, each summed in task order, so the result does
// not depend on timing.  The task two steps ahead and the next item are
// read before the current item's buffer update, and the next row's
// first-operand values are loaded while the current row is built.  The
// column exponents of the product and the walk's row pointers sit in LDS;
// with STAGED also the second operand's targets and folded values.
constexpr int kSpThreads = 512;
constexpr int kSpWaves = kSpThreads / 64;
constexpr int kSpRows = 256;   // output rows per workgroup
constexpr int kSpEnt = 64;     // first-operand entries per chunk (one per lane)
constexpr int kSpTasks = 128;  // tasks per wave per pass (64 when the operand is not staged)
constexpr int kSpTaskPad = 8;  // empty tasks after a pass's last one

typedef float f32x4 __attribute__((ext_vector_type(4)));

// a pair pattern: row walk (row pointers, targets = b) and column walk
// (column pointers, column order, targets = a), and per-window offsets of
// both walks when rows span several windows
struct SpPat {
    const int32_t *row_ptr, *col_ptr, *pa, *pb, *col_pairs, *colpos, *wn, *wt;
    const int32_t *cola;   // a of each column-order entry
    int32_t np;
};

struct SpLevel {
    SpPat in;              // the operands' pattern
    SpPat out;             // pattern whose values are taken from the output (out.np = 0: none)
    const float *vin;      // folded operand values, [B][vin_nodes][in.np], stored entry order
    const float *valt;     // the same in each node's other walk order, or nullptr
    float *vout;           // raw output values on `out`, [B][vout_nodes][out.np]
    int vin_nodes, vout_nodes;
    int level, n0, nsp;    // products: nodes n0 .. n0 + nsp - 1 of every row
    int win, tcap, nwin;
};

template <bool STAGED, bool ONEWIN>
__global__ __launch_bounds__(kSpThreads) void span_sparse(DevTable d, StepView sv, SpLevel lv,
                                                          float *__restrict__ tree,
                                                          int32_t *__restrict__ meta)
{
    extern __shared__ __align__(16) float sm[];
    const int Sp = sv.Sp, S = d.S, np = lv.in.np;
    if (np <= 0) return;   // the launcher takes patterns with pairs only
    const int win = lv.win, tcap = lv.tcap, nwin = lv.nwin;
    const int rblocks = (Sp + kSpRows - 1) / kSpRows;
    const int prod = blockIdx.x / rblocks, r0 = (blockIdx.x % rblocks) * kSpRows;
    const int r1 = min(r0 + kSpRows, Sp);
    const int b = prod / lv.nsp, n = lv.n0 + prod % lv.nsp;
    const bool tr = stored_transposed(n);
    const int hF = tr ? 2 * n + 1 : 2 * n, hG = tr ? 2 * n : 2 * n + 1;
    const int cbase = sv.Lpad >> (lv.level - 1);   // first node of the children's level
    const int iF = hF - cbase, iG = hG - cbase;
    // first level: leaves past the sequence end are the identity
    const bool realF = lv.level > 1 || iF < sv.L, realG = lv.level > 1 || iG < sv.L;
    const int32_t *roF = sv.meta_ptr((const int32_t *)meta, b, hF, 0);
    const int32_t *rfF = sv.meta_ptr((const int32_t *)meta, b, hF, 2);
    const int32_t *roG = sv.meta_ptr((const int32_t *)meta, b, hG, 0);
    const int32_t *rfG = sv.meta_ptr((const int32_t *)meta, b, hG, 2);
    // both operands' entries are in their stored order: the first operand's
    // is its walk order; the second's is the other one
    const float *vF = lv.vin + ((size_t)b * lv.vin_nodes + (realF ? iF : 0)) * np;
    const float *vG = lv.vin + ((size_t)b * lv.vin_nodes + (realG ? iG : 0)) * np;
    const int32_t *ptr = tr ? lv.in.col_ptr : lv.in.row_ptr;
    const int32_t *far = tr ? lv.in.pa : lv.in.pb;
    const int32_t *wfar = tr ? lv.in.cola : lv.in.pb;   // target of walk entry e
    const int32_t *perm = tr ? lv.in.col_pairs : lv.in.colpos;
    // the second operand's values in its walk order (other than its stored one)
    const float *vGw = lv.valt ? lv.valt + ((size_t)b * lv.vin_nodes + iG) * np : nullptr;
    const int32_t *woff = tr ? lv.in.wt : lv.in.wn;
    const int npc = np - 1;
    // output values on the `out` pattern, in this node's stored entry order
    const bool extract = lv.out.np > 0 && realF && realG;
    const int32_t *optr = tr ? lv.out.col_ptr : lv.out.row_ptr;
    const int32_t *ofar = tr ? lv.out.cola : lv.out.pb;
    const int32_t *owoff = tr ? lv.out.wt : lv.out.wn;
    float *vout = extract ? lv.vout + ((size_t)b * lv.vout_nodes + (n - lv.n0)) * lv.out.np : nullptr;
    float *D = sv.mat_ptr(tree, b, n);
    int32_t *roD = sv.meta_ptr(meta, b, n, 0);
    int32_t *coD = sv.meta_ptr(meta, b, n, 1);
    int32_t *rfD = sv.meta_ptr(meta, b, n, 2);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 5, sub = lane & 31;
    float *bufw = sm + wave * 2 * win;           // this wave's two row buffers
    float *bufg = bufw + grp * win;              // this lane group's buffer
    // a task: (first item | item count << 26, x1 bits)
    int2 *task = reinterpret_cast<int2 *>(sm + kSpWaves * 2 * win) + wave * (tcap + kSpTaskPad);
    int32_t *sco = reinterpret_cast<int32_t *>(sm + kSpWaves * (2 * win + 2 * (tcap + kSpTaskPad)));
    int32_t *sptr = sco + Sp;
    float *sx = reinterpret_cast<float *>(sptr + ((S + 4) & ~3));
    uint16_t *stt = reinterpret_cast<uint16_t *>(sx + np);

    // second operand entry e of the walk: target and folded value
    auto g_entry = [&](int e, int &t, float &x2) {
        if (STAGED) {
            t = stt[e];
            x2 = sx[e];
        } else if (vGw) {
            t = wfar[e];
            x2 = vGw[e];
        } else {
            t = wfar[e];
            x2 = vG[perm[e]];
        }
    };
    // item index: staged reads of an empty task's items stay inside the LDS
    // block (unused); memory reads are clamped into the arrays
    auto item = [&](int e) { return STAGED ? e : min(max(e, 0), npc); };
    int w0 = 0, wn = Sp, wi = 0;
    auto add = [&](int t, float x1, float x2) {
        if (ONEWIN) {
            bufg[t] = fmaf(x1, x2, bufg[t]);
        } else {
            const int c = t - w0;
            if ((unsigned)c < (unsigned)wn) bufg[c] = fmaf(x1, x2, bufg[c]);
        }
    };
    for (int t = tid; t < Sp; t += kSpThreads) {
        const int c = add_exp(roG[t], rfG[t]);
        sco[t] = c;
        if (r0 == 0) coD[t] = c;
    }
    for (int k = tid; k <= S; k += kSpThreads) sptr[k] = ptr[k];
    // row exponents of the product: those of the first operand, folded
    for (int r = r0 + tid; r < r1; r += kSpThreads) roD[r] = add_exp(roF[r], rfF[r]);
    if (STAGED) {
        // eight entries per thread in flight: the pair id q (column order,
        // or the column position for values stored transposed), then target
        // and value
        constexpr int kU = 8;
        for (int e0 = tid; e0 < np; e0 += kSpThreads * kU) {
            int q[kU], t[kU];
            float x[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) q[u] = perm[min(e0 + u * kSpThreads, npc)];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int e = min(e0 + u * kSpThreads, npc);
                t[u] = far[tr ? q[u] : e];
                x[u] = vG[q[u]];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int e = e0 + u * kSpThreads;
                if (e < np) {
                    stt[e] = (uint16_t)t[u];
                    sx[e] = realG ? x[u] : 0.f;
                }
            }
        }
    }
    __syncthreads();

    // first-operand entries of row s: [e0, e1) of the walk (identity: one
    // entry k = s), and lane's entry e0 + lane (clamped) loaded
    struct RowPf {
        int e0, e1, k, rf;
        float x;
    };
    auto row_pf = [&](int s) {
        RowPf r;
        const int sc = min(s, S - 1);
        const bool has = s < S;
        r.e0 = has && realF ? sptr[sc] : 0;
        r.e1 = has ? (realF ? sptr[sc + 1] : 1) : 0;
        const int ei = min(r.e0 + lane, npc);
        r.x = vF[ei];
        r.k = STAGED ? 0 : wfar[ei];
        r.rf = rfF[min(s, Sp - 1)];
        return r;
    };
    int s = r0 + wave;
    RowPf pf = row_pf(s);
    for (; s < r1; s += kSpWaves) {
        const int e0 = pf.e0, e1 = pf.e1;
        const float cx0 = realF ? pf.x : ldexpf(1.f, 0 - pf.rf);
        const int ck0 = realF ? (STAGED ? (int)stt[min(e0 + lane, npc)] : pf.k) : s;
        pf = row_pf(s + kSpWaves);   // next row, in flight while this one is built
        int emax = kNeg;
        for (w0 = 0, wi = 0; w0 < Sp; w0 += win, ++wi) {
            wn = min(win, Sp - w0);
            for (int c = lane * 4; c < 2 * win; c += 256)
                *reinterpret_cast<f32x4 *>(&bufw[c]) = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int eb = e0; eb < e1; eb += kSpEnt) {
                const int cnt = min(kSpEnt, e1 - eb);
                float cx = cx0;
                int ck = ck0;
                if (eb != e0) {   // rows with more than 64 entries
                    const int ei = min(eb + lane, npc);
                    cx = vF[ei];
                    ck = STAGED ? (int)stt[ei] : wfar[ei];
                }
                if (!realG) {
                    // identity second operand: entry k adds x1 2^-rf[k] at column k
                    if (lane < cnt) {
                        const int c = ck - w0;
                        if ((unsigned)c < (unsigned)wn)
                            bufw[c] = fmaf(cx, ldexpf(1.f, 0 - rfG[ck]), bufw[c]);
                    }
                    continue;
                }
                // tasks of this chunk: entry j has ceil(deg / 32) of them
                // (deg: its items in this window), numbered from the
                // exclusive prefix sum pre
                // (windows without offsets walk the whole row; `add` keeps
                // the window's targets)
                int lo, hiw;
                if (ONEWIN || nwin == 0) {
                    lo = sptr[ck];
                    hiw = sptr[ck + 1];
                } else {
                    lo = woff[(size_t)ck * (nwin + 1) + wi];
                    hiw = woff[(size_t)ck * (nwin + 1) + wi + 1];
                }
                const int deg = lane < cnt ? hiw - lo : 0;
                const int nt = (deg + 31) >> 5;
                int pre, T;
                if (!__any(nt > 1)) {   // at most one task per entry: a ballot
                    const unsigned long long m = __ballot(nt > 0);
                    pre = __popcll(m & ((1ull << lane) - 1ull));
                    T = __popcll(m);
                } else {
                    int inc = nt;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const int y = __shfl_up(inc, o);
                        if (lane >= o) inc += y;
                    }
                    pre = inc - nt;
                    T = __shfl(inc, 63);
                }
                for (int P = 0; P < T; P += tcap) {
                    const int Tp = min(T - P, tcap);
                    for (int u = max(pre, P); u < min(pre + nt, P + tcap); ++u) {
                        const int q0 = lo + ((u - pre) << 5);
                        const int c = min(32, lo + deg - q0);
                        task[u - P] = make_int2(q0 | (c << 26), __float_as_int(cx));
                    }
                    // empty tasks (no items) after the last one: the step
                    // loop runs whole pairs of steps and reads two ahead
                    if (lane < kSpTaskPad) task[Tp + lane] = make_int2(0, 0);
                    const int steps = (Tp + 1) >> 1;
                    // step st runs task 2 st + grp; its item is loaded one
                    // step ahead and the task two steps ahead
                    constexpr int kLoMask = (1 << 26) - 1;
                    int2 ta = task[grp];
                    int2 tb = task[2 + grp];
                    int t0;
                    float x0;
                    g_entry(item((ta.x & kLoMask) + sub), t0, x0);
                    float w0x = __int_as_float(ta.y);
                    bool v0 = sub < (int)((unsigned)ta.x >> 26);
                    for (int st = 0; st < steps; st += 2) {
                        int t1;
                        float x1v;
                        g_entry(item((tb.x & kLoMask) + sub), t1, x1v);
                        const float w1x = __int_as_float(tb.y);
                        const bool v1 = sub < (int)((unsigned)tb.x >> 26);
                        ta = task[2 * st + 4 + grp];
                        if (v0) add(t0, w0x, x0);
                        g_entry(item((ta.x & kLoMask) + sub), t0, x0);
                        w0x = __int_as_float(ta.y);
                        v0 = sub < (int)((unsigned)ta.x >> 26);
                        tb = task[2 * st + 6 + grp];
                        if (v1) add(t1, w1x, x1v);
                    }
                }
            }
            float *Drow = D + (size_t)s * Sp + w0;
            for (int c = lane * 4; c < wn; c += 256) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(&bufw[c]) +
                                *reinterpret_cast<const f32x4 *>(&bufw[win + c]);
                *reinterpret_cast<f32x4 *>(&Drow[c]) = v;
                const int4 co = *reinterpret_cast<const int4 *>(&sco[w0 + c]);
                const int cv[4] = {co.x, co.y, co.z, co.w};
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (v[u] > 0.f && cv[u] > kNeg) emax = max(emax, fexp(v[u]) + cv[u]);
            }
            if (extract && s < S) {
                // the row's values at the `out` pattern's targets in this window
                const bool whole = ONEWIN || nwin == 0;
                const int oa = whole ? optr[s] : owoff[(size_t)s * (nwin + 1) + wi];
                const int ob = whole ? optr[s + 1] : owoff[(size_t)s * (nwin + 1) + wi + 1];
                for (int e = oa + lane; e < ob; e += 64) {
                    const int c = ofar[e] - w0;
                    if ((unsigned)c < (unsigned)wn) vout[e] = bufw[c] + bufw[win + c];
                }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) emax = max(emax, __shfl_xor(emax, o));
        if (lane == 0) rfD[s] = emax;
    }
}

// The second level's operands: the first-level nodes' values on the
// two-step pattern, folded in place as the dense kernels fold them (value
// times 2^(co - rf) of its stored column and row), and copied in the node's
// other walk order (the order the second level reads a second operand in).
__global__ void sparse_fold(DevTable d, StepView sv, SpPat pat, float *__restrict__ v,
                            float *__restrict__ valt, const int32_t *__restrict__ meta, int nodes)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= pat.np) return;
    for (int y = blockIdx.y; y < sv.B * nodes; y += gridDim.y) {
        const int b = y / nodes, j = y % nodes;
        const int n = (sv.Lpad >> 1) + j;
        const bool tr = stored_transposed(n);
        const int q = tr ? pat.col_pairs[e] : e;
        const int row = tr ? pat.pb[q] : pat.pa[q], col = tr ? pat.pa[q] : pat.pb[q];
        const int32_t *co = sv.meta_ptr(meta, b, n, 1);
        const int32_t *rf = sv.meta_ptr(meta, b, n, 2);
        const size_t base = ((size_t)b * nodes + j) * pat.np;
        const float x = ldexpf(v[base + e], co[col] - rf[row]);
        v[base + e] = x;
        // the other walk order: column position of pair e, or pair q
        valt[base + (tr ? q : pat.colpos[e])] = x;
    }
}

// LDS bytes of span_sparse: per wave two row buffers and the tasks; the
// product's column exponents and the walk's row pointers; with staging the
// second operand's folded values and 16-bit targets
size_t sparse_lds(const DevTable &d, int Sp, int np, int win, bool staged)
{
    const int tcap = staged ? kSpTasks : kSpTasks / 2;
    size_t b = (size_t)kSpWaves * (2 * win + 2 * (tcap + kSpTaskPad)) * sizeof(float);
    b += ((size_t)Sp + ((d.S + 4) & ~3)) * sizeof(int32_t);
    if (staged)
        b += (size_t)np * sizeof(float) + (((size_t)np * sizeof(uint16_t) + 15) & ~size_t(15));
    return b;
}

SpPat pattern1(const DevTable &d)
{
    return SpPat{d.row_ptr, d.col_ptr, d.pair_a, d.pair_b, d.col_pairs, d.pair_colpos,
                 d.w1_n, d.w1_t, d.col_a, d.npairs};
}

SpPat pattern2(const DevTable &d)
{
    return SpPat{d.p2_row_ptr, d.p2_col_ptr, d.p2_a, d.p2_b, d.p2_col_pairs, d.p2_colpos,
                 d.w2_n, d.w2_t, d.p2_col_a, d.np2};
}

int launch_sparse(const DevTable &d, const Geometry &g, StepView sv, SpLevel lv, float *tree,
                  int32_t *meta, hipStream_t st)
{
    // rows wider than kSpWin / 2 columns take the table's windows (the
    // per-window offsets are built for them); narrower rows one window, or
    // 256 columns (each window walking the whole row) when that lets the
    // second operand be staged
    int win = d.nwin > 0 ? d.win_cols : g.Sp;
    bool staged = g.Sp <= 65536 && sparse_lds(d, g.Sp, lv.in.np, win, true) <= kSparseLdsMax;
    if (!staged && d.nwin == 0 && g.Sp > 256 && sparse_lds(d, g.Sp, lv.in.np, 256, true) <= kSparseLdsMax) {
        win = 256;
        staged = true;
    }
    const size_t lds = sparse_lds(d, g.Sp, lv.in.np, win, staged);
    if (lds > kSparseLdsMax) return (int)hipErrorInvalidConfiguration;
    lv.win = win;
    lv.tcap = staged ? kSpTasks : kSpTasks / 2;
    lv.nwin = d.nwin;
    const long long grid = (long long)g.B * lv.nsp * ((g.Sp + kSpRows - 1) / kSpRows);
    if (grid > 0x7fffffffLL) return (int)hipErrorInvalidConfiguration;
    if (grid == 0) return 0;
    const bool one = win == g.Sp;
    const void *fn = staged ? (one ? reinterpret_cast<const void *>(&span_sparse<true, true>)
                                   : reinterpret_cast<const void *>(&span_sparse<true, false>))
                            : (one ? reinterpret_cast<const void *>(&span_sparse<false, true>)
                                   : reinterpret_cast<const void *>(&span_sparse<false, false>));
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
#define FA_SPARSE(ST, ONE) span_sparse<ST, ONE><<<(unsigned)grid, kSpThreads, lds, st>>>(d, sv, lv, tree, meta)
    if (staged) {
        if (one) FA_SPARSE(true, true);
        else FA_SPARSE(true, false);
    } else {
        if (one) FA_SPARSE(false, true);
        else FA_SPARSE(false, false);
    }
#undef FA_SPARSE
    return (int)hipGetLastError();
}

// compute units of the current device (the persistent grid size), queried
// once per device; any grid size gives the same result
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// one tree level as dense products over nodes n0 .. n0 + nn - 1 of every row
int launch_dense_level(const Geometry &g, StepView sv, int k, int n0, int nn, float *tree,
                       int32_t *meta, uint8_t *ws, const WsLayout &w, hipStream_t st,
                       const int32_t *live, const int32_t *nlive)
{
    if (nn <= 0) return 0;
    const int tiles = g.Sp / kTile;
    const int big_tiles = g.Sp / kBig;
    const long long big_wgs = (long long)g.B * nn * big_tiles * big_tiles;
    const int ks = tree_ksplit(g, k);
    const int huge_tiles = g.Sp / kHuge;
    const long long huge_wgs = (long long)g.B * nn * huge_tiles * huge_tiles;
    if (ks == 1 && g.Sp % kHuge == 0 && huge_wgs >= 256) {
        const unsigned grid = (unsigned)std::min<long long>(huge_wgs, device_cus());
        if (live)
            span_gemm256<true><<<grid, kHugeThreads, 0, st>>>(sv, tree, meta, n0, nn, live, nlive);
        else
            span_gemm256<false><<<grid, kHugeThreads, 0, st>>>(sv, tree, meta, n0, nn, nullptr, nullptr);
    } else if (ks == 1 && g.Sp % kBig == 0 && big_wgs >= 256) {
        span_gemm128<<<(unsigned)big_wgs, kBigThreads, 0, st>>>(sv, tree, meta, n0, nn);
    } else {
        float *part = (float *)(ws + w.kpart);
        dim3 grid(tiles * tiles * ks, g.B * nn);
        span_gemm<<<grid, kGemmThreads, 0, st>>>(sv, tree, meta, n0, nn, ks, part);
        if (ks > 1) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return (int)e;
            dim3 rgrid(tiles * tiles, g.B * nn);
            span_reduce<<<rgrid, kGemmThreads, 0, st>>>(sv, tree, meta, n0, nn, ks, part);
        }
    }
    return (int)hipGetLastError();
}

}  // namespace

int launch_span_tree(const DevTable &d, const Geometry &g, float *tree, int32_t *meta,
                     uint8_t *ws, const WsLayout &w, double *logZ, int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (g.L == 0) {
        tree_logz_empty<<<(g.B + 255) / 256, 256, 0, st>>>(d, g.B, logZ, status);
        return (int)hipGetLastError();
    }
    StepView sv = step_view(g);
    // the pair-staged first level at Sp = 256 clears the upper levels' rf itself
    const bool pairs_init = d.first_pairs && d.npairs > 0 && g.Sp == kHuge && g.K >= 1;
    if (g.Lpad > 1 && !pairs_init) {
        const size_t total = (size_t)g.B * (g.Lpad - 1) * g.Sp;
        const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
        tree_init_rf<<<blocks, 256, 0, st>>>(sv, meta);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    const float *pvf = (const float *)(ws + w.pvf);
    float *pv2 = (float *)(ws + w.pv2);
    float *pv2alt = (float *)(ws + w.pv2alt);
    const bool sparse1 = d.first_sparse && d.npairs > 0;
    // second level from the two-step pattern: its products whose four
    // leaves are all inside the sequence (the rest, if any, dense)
    const int nsp2 = d.second_sparse && d.np2 > 0 && sparse1 && g.K >= 2 ? g.L / 4 : 0;
    // FA_LIVE_STATES: the states live at every boundary, for the products
    // on 256x256 tiles
    const int32_t *live = nullptr, *nlive = nullptr;
    if (d.live_states) {
        const int e = launch_live_states(d, g, tree, ws, w, stream);
        if (e) return e;
        live = (const int32_t *)(ws + w.live);
        nlive = (const int32_t *)(ws + w.nlive);
    }
    for (int k = 1; k <= g.K; ++k) {
        const int n0 = g.Lpad >> k, nn = n0;
        if (k == 1) {
            const int pe = prof_mark(FA_PROF_TREE_LEVEL1, true, stream);
            if (pe) return pe;
        }
        int e = 0;
        if (k == 1 && d.first_pairs && d.npairs > 0) {
            const long long wgs = (long long)g.B * nn * (g.Sp / kHuge) * (g.Sp / kHuge);
            const unsigned grid = (unsigned)std::min<long long>(wgs, device_cus());
            span_pairs256<<<grid, kHugeThreads, 0, st>>>(d, sv, tree, meta, pvf, n0, nn,
                                                         pairs_init ? 1 : 0);
            e = (int)hipGetLastError();
        } else if (k == 1 && sparse1) {
            SpLevel lv{};
            lv.in = pattern1(d);
            if (nsp2 > 0) lv.out = pattern2(d);
            lv.vin = pvf;
            lv.vout = pv2;
            lv.vin_nodes = g.L;
            lv.vout_nodes = g.Lpad / 2;
            lv.level = 1;
            lv.n0 = n0;
            lv.nsp = nn;
            e = launch_sparse(d, g, sv, lv, tree, meta, st);
            if (!e && nsp2 > 0) {
                dim3 fgrid((d.np2 + 255) / 256, std::min(g.B * (g.Lpad / 2), 65535));
                sparse_fold<<<fgrid, 256, 0, st>>>(d, sv, pattern2(d), pv2, pv2alt, meta, g.Lpad / 2);
                e = (int)hipGetLastError();
            }
        } else if (k == 2 && nsp2 > 0) {
            SpLevel lv{};
            lv.in = pattern2(d);
            lv.vin = pv2;
            lv.valt = pv2alt;
            lv.vin_nodes = g.Lpad / 2;
            lv.level = 2;
            lv.n0 = n0;
            lv.nsp = nsp2;
            e = launch_sparse(d, g, sv, lv, tree, meta, st);
            if (!e)
                e = launch_dense_level(g, sv, k, n0 + nsp2, nn - nsp2, tree, meta, ws, w, st, live,
                                       nlive);
        } else {
            e = launch_dense_level(g, sv, k, n0, nn, tree, meta, ws, w, st, live, nlive);
        }
        if (e) return e;
        if (k == 1) {
            const int pe = prof_mark(FA_PROF_TREE_LEVEL1, false, stream);
            if (pe) return pe;
        }
    }
    tree_logz<<<g.B, 64, 0, st>>>(d, sv, tree, meta, logZ, status);
    return (int)hipGetLastError();
}

}  // namespace fa
