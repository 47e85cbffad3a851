// Emission reduce: M_i[a][b] = sum_v c(a, v, b) p[i][v] for every position,
// written as dense leaves of the span tree (papernotes 关键设计 1: each
// position's transition matrix sums the mean-field-reweighted emissions over
// the vocabulary; paperfeed "The insight": the |E||V| term).
//
// Up to three kernels, by label class:
//  * emission_dense: pairs whose labels are large token sets (dense masks).
//    Their sums form a contraction  D[j][pos] = sum_v mask[j][v] p[pos][v]
//    with a 0/1 operand.  It runs on bf16 MFMA (32 pairs x 32 positions per
//    tile, K = tokens) without rounding any term: each p value is cut into
//    three bf16 pieces that add up to it exactly, so every product with a
//    0/1 mask value is exact, and each short MFMA chain is added into an
//    fp32 total.  V is split over workgroups into chunks (sized so the
//    workgroups fill whole rounds of the chip) whose partials are summed in
//    chunk order.  The same pass copies p at the tokens that token-list
//    pairs use (a compact gather source).
//  * emission_ranges: one workgroup per position streams the row and keeps
//    an fp64 running prefix sum at every range cut point.
//  * emission_densify: one wavefront per stored leaf row evaluates the pair
//    values of that row and writes the row (Sp floats) in 64-column chunks,
//    zeros included, with its power-of-two row exponent.  Odd leaves are
//    stored transposed, so their stored rows are the columns of M_i.
#include "device_common.h"
#include "pair_value.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8, v);
}

// the upper halves of two words, a's in the low half: two bf16 values
__device__ inline uint32_t upper_halves(uint32_t a, uint32_t b)
{
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// 0xffffffff when bit k of w is set, else 0
__device__ inline uint32_t bit_fill(uint32_t w, int k)
{
    return (uint32_t)__builtin_amdgcn_sbfe((int)w, k, 1);
}

constexpr int kDenseThreads = 256;
constexpr int kSub = 256;         // tokens staged per step
constexpr int kSubLd = kSub + 4;  // padded LDS row

// One workgroup: 32 positions x one V chunk (a multiple of 256 tokens).
// Tokens are staged 256 at a time through double-buffered LDS (every
// wavefront load reads 1 KB of one row); each of the four waves runs the
// MFMAs of 64 tokens per step into its own 32x32 tile, and the four tiles
// are summed at the end.  A value x is cut as x = hi + mid + lo, each an
// exact bf16: hi is the top half of x's bits, mid the top half of x - hi,
// lo the rest (at most 8 significant bits); the three pieces share the mask
// operand (1.0 or 0).  Every global load of the loop
// is unconditional (out-of-range elements read an in-range address and are
// zeroed when stored to LDS), so the loop has a fixed number of memory
// operations per step and the loads of step s+2 stay in flight while step s
// computes.
//
// SEL selects how the tokens of token-list pairs are copied to psel:
//   0: no copy; 1: from the staged LDS tiles into an LDS buffer, written out
//   after the loop (at most kDenseSelLds such tokens per chunk); 2: gathered from
//   p after the loop.
template <bool VEC, int SEL>
__global__ __launch_bounds__(kDenseThreads) void emission_dense(
    DevTable d, const float *__restrict__ p, int L, int npos, int BLpad, int vchunk,
    float *__restrict__ dpart, float *__restrict__ psel, int32_t *__restrict__ status)
{
    __shared__ __align__(16) float pt[2][kDenseTile][kSubLd];
    __shared__ __align__(16) uint32_t mk[2][kSub];
    __shared__ int sel_at[kDenseStepsMax + 1];  // first token-list index at or after each step
    __shared__ uint16_t sel_off[SEL == 1 ? kDenseSelLds : 1];
    __shared__ float selv[SEL == 1 ? kDenseTile : 1][SEL == 1 ? kDenseSelLds : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk = blockIdx.x;
    const int pos0 = blockIdx.y * kDenseTile;
    const int v_begin = chunk * vchunk;
    const int v_end = min(d.V, v_begin + vchunk);
    const int nsteps = (v_end - v_begin + kSub - 1) / kSub;
    if (SEL != 0 && tid <= nsteps) sel_at[tid] = d.sel_lb[v_begin / kSub + tid];
    if (SEL == 1) {
        __syncthreads();
        const int s0 = sel_at[0], nc = sel_at[nsteps] - s0;  // nc <= kDenseSelLds (host check)
        if (tid < nc) sel_off[tid] = (uint16_t)(d.sel_tok[s0 + tid] - v_begin);
    }
    // staging map: load k of thread t is float4 number 256k + t of the
    // 32 x 256 tile, i.e. row 4k + wave, column 4*lane, so each wavefront
    // reads one contiguous 1 KB row segment; rows past npos read row npos-1
    const int scol = 4 * lane;
    const float *prow[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        prow[k] = p + (size_t)min(pos0 + 4 * k + wave, npos - 1) * d.V;
    int bad = 0;
    f32x16 tot, zero16;
#pragma unroll
    for (int r = 0; r < 16; ++r) tot[r] = zero16[r] = 0.f;
    struct Step {
        float4 x[8];
        uint32_t m;
    };
    Step sa, sb;
    auto load = [&](Step &st, int v0) {
        const int v = v0 + scol;
        if (VEC) {
            // V % 4 == 0: v and v_end are multiples of 4
            const int vc = v < v_end ? v : v_end - 4;
#pragma unroll
            for (int k = 0; k < 8; ++k) st.x[k] = load_nt(prow[k] + vc);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                st.x[k].x = prow[k][min(v, v_end - 1)];
                st.x[k].y = prow[k][min(v + 1, v_end - 1)];
                st.x[k].z = prow[k][min(v + 2, v_end - 1)];
                st.x[k].w = prow[k][min(v + 3, v_end - 1)];
            }
        }
        st.m = d.tokmask[min(v0 + tid, v_end - 1)];
    };
    auto store = [&](const Step &st, int v0, int buf) {
        float4 xs[8];
        if (v0 + kSub <= v_end && pos0 + kDenseTile <= npos) {  // whole tile in range
#pragma unroll
            for (int k = 0; k < 8; ++k) xs[k] = st.x[k];
        } else {
            const int v = v0 + scol;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bool rok = pos0 + 4 * k + wave < npos;
                xs[k].x = (rok && v < v_end) ? st.x[k].x : 0.f;
                xs[k].y = (rok && v + 1 < v_end) ? st.x[k].y : 0.f;
                xs[k].z = (rok && v + 2 < v_end) ? st.x[k].z : 0.f;
                xs[k].w = (rok && v + 3 < v_end) ? st.x[k].w : 0.f;
            }
        }
        // screen: as unsigned bit patterns, every value that is not >= 0
        // (negative, NaN) and also -0 exceeds 0x7F800000; only then take the
        // exact test per staged row
        uint32_t mx = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            mx = max(mx, max(max(__float_as_uint(xs[k].x), __float_as_uint(xs[k].y)),
                             max(__float_as_uint(xs[k].z), __float_as_uint(xs[k].w))));
        if (mx > 0x7F800000u) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bool b = !(xs[k].x >= 0.f) | !(xs[k].y >= 0.f) | !(xs[k].z >= 0.f) |
                               !(xs[k].w >= 0.f);
                bad |= (int)b << k;  // which staged rows saw a negative or NaN value
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) *reinterpret_cast<float4 *>(&pt[buf][4 * k + wave][scol]) = xs[k];
        mk[buf][tid] = v0 + tid < v_end ? st.m : 0u;
    };
    const int half = lane >> 5, l32 = lane & 31;
    // first token of stage s; stages past the chunk re-read its last stage
    // (the values are zeroed when stored, since they lie past v_end)
    auto vstage = [&](int s) { return v_begin + min(s, nsteps - 1) * kSub; };
    // step s: MFMAs over LDS buffer s&1 (and the token-list copy), then
    // stage s+1 from registers into the other buffer and issue the loads of
    // stage s+3 into the freed registers; one barrier per step.  Loads and
    // stores are unconditional so that every step issues the same memory
    // operations (a conditional load makes the compiler wait for all
    // outstanding loads at the next use of the registers).
    auto step = [&](int s, Step &next, int buf) {
        const float *brow = &pt[buf][l32][64 * wave + 32 * half];
        const uint32_t *mrow = &mk[buf][64 * wave + 32 * half];
        // k-slot v of this lane half is token 8q + v of its 32; the mask
        // operand is the same for the three pieces
        f32x16 acc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 x0 = *reinterpret_cast<const float4 *>(brow + 8 * q);
            const float4 x1 = *reinterpret_cast<const float4 *>(brow + 8 * q + 4);
            const uint4 m0 = *reinterpret_cast<const uint4 *>(mrow + 8 * q);
            const uint4 m1 = *reinterpret_cast<const uint4 *>(mrow + 8 * q + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const uint32_t ms[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            uint32_t ub[8], rb[8], lb[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                ub[v] = __float_as_uint(xs[v]);
                const float r = xs[v] - __uint_as_float(ub[v] & 0xFFFF0000u);
                rb[v] = __float_as_uint(r);
                lb[v] = __float_as_uint(r - __uint_as_float(rb[v] & 0xFFFF0000u));
            }
            uint32_t am[4], bh[4], bm[4], bl[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                am[j] = (bit_fill(ms[2 * j], l32) & 0x3F80u) | (bit_fill(ms[2 * j + 1], l32) & 0x3F800000u);
                bh[j] = upper_halves(ub[2 * j], ub[2 * j + 1]);
                bm[j] = upper_halves(rb[2 * j], rb[2 * j + 1]);
                bl[j] = upper_halves(lb[2 * j], lb[2 * j + 1]);
            }
            const bf16x8 A = as_bf16x8(am[0], am[1], am[2], am[3]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, as_bf16x8(bh[0], bh[1], bh[2], bh[3]),
                                                          q == 0 ? zero16 : acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, as_bf16x8(bm[0], bm[1], bm[2], bm[3]),
                                                          acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, as_bf16x8(bl[0], bl[1], bl[2], bl[3]),
                                                          acc, 0, 0, 0);
        }
        // the step's twelve-MFMA chain goes into the total, so no long fp32
        // chain drops terms far below its own ulp
#pragma unroll
        for (int r = 0; r < 16; ++r) tot[r] += acc[r];
        if (SEL == 1 && s < nsteps) {
            const int j0 = sel_at[s] - sel_at[0], n = sel_at[s + 1] - sel_at[s];
            for (int i = tid; i < n * kDenseTile; i += kDenseThreads) {
                const int r = i & (kDenseTile - 1), j = j0 + (i >> 5);
                selv[r][j] = pt[buf][r][sel_off[j] - s * kSub];
            }
        }
        store(next, v_begin + (s + 1) * kSub, buf ^ 1);
        load(next, vstage(s + 3));
        __syncthreads();
    };
    load(sa, vstage(0));
    load(sb, vstage(1));
    store(sa, v_begin, 0);
    load(sa, vstage(2));
    __syncthreads();
    // stage s sits in sa (s even) or sb (s odd); an odd step count gets one
    // all-zero step
    for (int s = 0; s < nsteps; s += 2) {
        step(s, sb, 0);
        step(s + 1, sa, 1);
    }
    // sum the four waves' tiles in wave order (reusing the staging LDS)
    float *red = &pt[0][0][0];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = (r >> 2) * 8 + half * 4 + (r & 3);
        red[wave * (kDenseTile * kDenseTile) + i * kDenseTile + l32] = tot[r];
    }
    __syncthreads();
    float *outp = dpart + ((size_t)chunk * BLpad + pos0) * kDenseMax;
    for (int k = tid; k < kDenseTile * kDenseTile; k += kDenseThreads) {
        const int i = k / kDenseTile, j = k % kDenseTile;  // pair i, position j
        const int W = kDenseTile * kDenseTile;
        const float sum = ((red[k] + red[W + k]) + red[2 * W + k]) + red[3 * W + k];
        outp[(size_t)j * kDenseMax + i] = sum;
    }
    if (SEL != 0) {
        const int s0 = sel_at[0], nc = sel_at[nsteps] - s0;
        for (int i = tid; i < nc * kDenseTile; i += kDenseThreads) {
            const int r = i / nc, j = i - r * nc;
            if (pos0 + r < npos) {
                float x;
                if (SEL == 1) x = selv[r][j];
                else x = p[(size_t)(pos0 + r) * d.V + d.sel_tok[s0 + j]];
                psel[(size_t)(pos0 + r) * d.nsel + s0 + j] = x;
            }
        }
    }
    for (int k = 0; k < 8; ++k) {
        const int row = 4 * k + wave;
        if (((bad >> k) & 1) && pos0 + row < npos)
            atomicOr(&status[(pos0 + row) / L], (int)FA_ROW_BADPROB);
    }
}

constexpr int kStreamThreads = 256;

// fp64 prefix sums of the row at every range cut point: cutp[pos][c] =
// sum_{v < cuts[c]} p[pos][v].  One workgroup per position reads the row in
// tiles of kRangeTile tokens, each thread a run of kRangePer consecutive
// tokens (four float4 loads; the next tile's loads are in flight while one
// is summed).  A thread sums its run in fp64, one block scan gives the runs'
// offsets, and each thread then writes the prefix at every cut point inside
// its run: the run's first cut index (tok2cut) and its 16 cut bits (one word
// of cutbits) are loaded with the run, so the writes need no further loads.
constexpr int kRangePer = 16;
constexpr int kRangeTile = kStreamThreads * kRangePer;

// VEC: float4 loads (V % 4 == 0 and p 16-byte aligned), decided on the host
// so the loads of the pipelined loop sit on no branch.
template <bool VEC>
__global__ __launch_bounds__(kStreamThreads) void emission_ranges(
    DevTable d, const float *__restrict__ p, int L, double *__restrict__ cutp,
    int32_t *__restrict__ status)
{
    const int pos = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *row = p + (size_t)pos * d.V;
    double *out = cutp + (size_t)pos * d.ncut;
    __shared__ double sh_wsum[kStreamThreads / 64];
    __shared__ int sh_bad;
    if (tid == 0) sh_bad = 0;
    struct Run {
        float x[kRangePer];
        int c_lo;       // first cut index at or after the run's first token
        uint32_t cbit;  // the run's cut bits (bit k: a cut at token v0 + k)
    };
    const int nwords = (d.V + 31) / 32;
    auto load = [&](Run &r, int t0) {
        const int v0 = t0 + kRangePer * tid;
        r.c_lo = d.tok2cut[min(max(v0 - 1, 0), d.V - 1)];
        r.cbit = d.cutbits[min(v0 >> 5, nwords - 1)];
        if constexpr (VEC) {
            const float4 *r4 = reinterpret_cast<const float4 *>(row);
            const int g0 = v0 >> 2, gl = (d.V >> 2) - 1;
#pragma unroll
            for (int j = 0; j < kRangePer / 4; ++j) {
                const float4 y = r4[min(g0 + j, gl)];
                r.x[4 * j] = y.x;
                r.x[4 * j + 1] = y.y;
                r.x[4 * j + 2] = y.z;
                r.x[4 * j + 3] = y.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kRangePer; ++j) r.x[j] = row[min(v0 + j, d.V - 1)];
        }
    };
    double carry = 0.0;
    int bad = 0;
    Run A, B;
    load(A, 0);
    auto tile = [&](const Run &r, int t0) {
        const int v0 = t0 + kRangePer * tid;
        // this run's values (zero past the row) and their fp64 sum
        float xs[kRangePer];
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < kRangePer; ++j) {
            xs[j] = v0 + j < d.V ? r.x[j] : 0.f;
            bad |= !(xs[j] >= 0.f);
            s += (double)xs[j];
        }
        // exclusive block scan of the run sums
        const double inc = wave_incl_scan_d(s, lane);
        if (lane == 63) sh_wsum[wave] = inc;
        __syncthreads();
        double off = carry + (inc - s);
        double tot = carry;
        for (int w = 0; w < kStreamThreads / 64; ++w) {
            if (w < wave) off += sh_wsum[w];
            tot += sh_wsum[w];
        }
        __syncthreads();  // sh_wsum is rewritten by the next tile
        // cut points inside [v0, v0 + kRangePer): consecutive indices from c
        // (a cut at token v0 + j holds the sum of the tokens before it: the
        // run's prefix, added in token order; static indices keep xs in
        // registers)
        if (v0 < d.V) {
            int c = v0 > 0 ? r.c_lo + 1 : 0;
            uint32_t m = (r.cbit >> (v0 & 31)) & ((1u << kRangePer) - 1u);
            if (v0 + kRangePer > d.V) m &= (1u << (d.V - v0)) - 1u;
            double run = off;
#pragma unroll
            for (int j = 0; j < kRangePer; ++j) {
                if ((m >> j) & 1u) out[c++] = run;
                run += (double)xs[j];
            }
        }
        carry = tot;
    };
    // both tiles of a pass unconditionally (a tile past the row adds zeros
    // and holds no cut): a tile summed inside a branch made the compiler wait
    // for every outstanding load there, the prefetch included
    for (int t0 = 0; t0 < d.V; t0 += 2 * kRangeTile) {
        load(B, t0 + kRangeTile);
        tile(A, t0);
        load(A, t0 + 2 * kRangeTile);
        tile(B, t0 + kRangeTile);
    }
    // cut points equal to V hold the row total
    const int nin = d.tok2cut[d.V - 1] + 1;  // cuts below V
    for (int idx = nin + tid; idx < d.ncut; idx += kStreamThreads) out[idx] = carry;
    if (bad) atomicOr(&sh_bad, 1);
    __syncthreads();
    if (tid == 0 && sh_bad) atomicOr(&status[pos / L], (int)FA_ROW_BADPROB);
}

// dense-mask pair sums: add the V-chunk partials of one (position, pair) in
// chunk order
__global__ void emission_dense_reduce(int n_vchunks, int BLpad, int npos, int nd,
                                      const float *__restrict__ dpart, float *__restrict__ dval)
{
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    const int pos = k / kDenseMax, j = k % kDenseMax;
    if (pos >= npos || j >= nd) return;
    float acc = 0.f;
    for (int c = 0; c < n_vchunks; ++c) acc += dpart[((size_t)c * BLpad + pos) * kDenseMax + j];
    dval[(size_t)pos * kDenseMax + j] = acc;
}

constexpr int kPairsPerThread = 4;

// every (position, pair) value: grid.x over pair groups, grid.y over positions
__global__ void emission_pairs(DevTable d, int L, EmitSrc src, float *__restrict__ val,
                               int32_t *__restrict__ status)
{
    const int q0 = (blockIdx.x * blockDim.x + threadIdx.x) * kPairsPerThread;
    const size_t pos = blockIdx.y;
    int bad = 0;
#pragma unroll
    for (int u = 0; u < kPairsPerThread; ++u) {
        const int q = q0 + u;
        if (q < d.npairs) val[pos * d.npairs + q] = pair_value(d, q, pos, src, bad);
    }
    if (bad) atomicOr(&status[pos / L], (int)FA_ROW_BADPROB);
}

// values of the pairs that are not one token's probability (ind_pair), for
// the one-pass leaf writer and the leaf level of the marginal message pass:
// one pair per thread (each value is a short chain of dependent loads),
// grid.x over groups of those pairs, grid.y over positions
constexpr int kIndThreads = 128;

__global__ __launch_bounds__(kIndThreads) void emission_indirect(DevTable d, int L, EmitSrc src,
                                                                int32_t *__restrict__ status)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    const size_t pos = blockIdx.y;
    int bad = 0;
    if (j < d.n_ind) src.ndval[pos * d.n_ind + j] = pair_value_direct(d, d.ind_pair[j], pos, src, bad);
    if (bad) atomicOr(&status[pos / L], (int)FA_ROW_BADPROB);
}

// dense leaf rows through the (row, column) -> pair maps: one wavefront per
// stored row, four columns per lane per step, float4 stores
__global__ __launch_bounds__(256) void emission_densify_map(DevTable d, StepView sv,
                                                            const float *__restrict__ val,
                                                            float *__restrict__ tree,
                                                            int32_t *__restrict__ meta)
{
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int b = blockIdx.y / sv.Lpad, i = blockIdx.y % sv.Lpad;
    if (r >= sv.Sp) return;
    const int h = sv.Lpad + i;
    const bool tr = stored_transposed(h);
    const size_t pos = (size_t)b * sv.L + i;
    float *out = sv.mat_ptr(tree, b, h) + (size_t)r * sv.Sp;
    const int32_t *map = (tr ? d.map_t : d.map_n) + (size_t)r * sv.Sp;
    const float *pv = val + pos * d.npairs;
    int emax = kNeg;
    for (int c = 4 * lane; c < sv.Sp; c += 256) {
        float4 x;
        if (i < sv.L) {
            const int4 m = *reinterpret_cast<const int4 *>(map + c);
            x.x = m.x >= 0 ? pv[m.x] : 0.f;
            x.y = m.y >= 0 ? pv[m.y] : 0.f;
            x.z = m.z >= 0 ? pv[m.z] : 0.f;
            x.w = m.w >= 0 ? pv[m.w] : 0.f;
        } else {  // identity leaf
            x.x = (c == r && r < d.S) ? 1.f : 0.f;
            x.y = (c + 1 == r && r < d.S) ? 1.f : 0.f;
            x.z = (c + 2 == r && r < d.S) ? 1.f : 0.f;
            x.w = (c + 3 == r && r < d.S) ? 1.f : 0.f;
        }
        *reinterpret_cast<float4 *>(out + c) = x;
        emax = max(max(emax, fexp(x.x)), max(fexp(x.y), max(fexp(x.z), fexp(x.w))));
    }
    emax = wave_max_i(emax);
    if (lane == 0) {
        sv.meta_ptr(meta, b, h, 2)[r] = emax;
        sv.meta_ptr(meta, b, h, 0)[r] = 0;
        sv.meta_ptr(meta, b, h, 1)[r] = 0;
    }
}

constexpr int kRowsPerWave = 2;
constexpr int kDensifyThreads = 256;

__global__ __launch_bounds__(kDensifyThreads) void emission_densify(
    DevTable d, StepView sv, const float *__restrict__ val, float *__restrict__ tree,
    int32_t *__restrict__ meta)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b = blockIdx.y / sv.Lpad, i = blockIdx.y % sv.Lpad;
    const int h = sv.Lpad + i;
    const bool tr = stored_transposed(h);
    const size_t pos = (size_t)b * sv.L + i;
    float *M = sv.mat_ptr(tree, b, h);
    int32_t *ro = sv.meta_ptr(meta, b, h, 0);
    int32_t *co = sv.meta_ptr(meta, b, h, 1);
    int32_t *rf = sv.meta_ptr(meta, b, h, 2);
    __shared__ float stage[4][64];
    const float *pv = val + pos * d.npairs;
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int r = (blockIdx.x * 4 + wave) * kRowsPerWave + rr;
        if (r >= sv.Sp) break;
        float *out = M + (size_t)r * sv.Sp;
        int emax = kNeg;
        if (i >= sv.L) {  // identity leaf
            for (int c = lane; c < sv.Sp; c += 64) {
                const float x = (c == r && r < d.S) ? 1.f : 0.f;
                out[c] = x;
                emax = max(emax, fexp(x));
            }
        } else {
            int k0 = 0, k1 = 0;
            if (r < d.S) {
                if (tr) { k0 = d.col_ptr[r]; k1 = d.col_ptr[r + 1]; }
                else { k0 = d.row_ptr[r]; k1 = d.row_ptr[r + 1]; }
            }
            int kp = k0;
            for (int cw = 0; cw < sv.Sp; cw += 64) {
                if (kp >= k1) {  // no pair left in this row: zeros
                    out[cw + lane] = 0.f;
                    continue;
                }
                stage[wave][lane] = 0.f;
                const int k = kp + lane;
                int q = -1, col = 0x7fffffff;
                if (k < k1) {
                    q = tr ? d.col_pairs[k] : k;
                    col = tr ? d.pair_a[q] : d.pair_b[q];
                }
                const bool in = col < cw + 64;
                wave_sync();
                if (in) stage[wave][col - cw] = pv[q];
                wave_sync();
                const float x = stage[wave][lane];
                out[cw + lane] = x;
                emax = max(emax, fexp(x));
                kp += __popcll(__ballot(in));
                wave_sync();
            }
        }
        emax = wave_max_i(emax);
        if (lane == 0) {
            rf[r] = emax;
            ro[r] = 0;
            co[r] = 0;
        }
    }
}

// Leaves from pair values in one pass.  One workgroup per group of rg
// stored rows of one leaf (rg * Sp <= kLeafTile): the tile is cleared in
// LDS, every pair of those rows is evaluated in parallel (they are one
// contiguous range of the leaf entries, in pair order or in column order for
// a transposed leaf; a one-token list pair reads its value directly) and
// placed in the tile with its row's largest exponent, then the tile is
// written out with float4 stores.  The value of every pair that is not one
// token's probability comes from emission_indirect (one load, like a direct
// value).  The first entries and their values are loaded before the tile is
// cleared.
constexpr int kLeafThreads = 256;
constexpr int kLeafPre = 4;      // leaf entries per thread loaded ahead

__global__ __launch_bounds__(kLeafThreads) void emission_leaves(DevTable d, StepView sv, int rg,
                                                                EmitSrc src, float *__restrict__ tree,
                                                                int32_t *__restrict__ meta,
                                                                float *__restrict__ pv,
                                                                int32_t *__restrict__ status)
{
    __shared__ __align__(16) float tile[kLeafTile];
    __shared__ int remax[kLeafTile / kSpAlign];
    const int tid = threadIdx.x;
    const int Sp = sv.Sp;
    const int b = blockIdx.y / sv.Lpad, i = blockIdx.y % sv.Lpad;
    const int r0 = blockIdx.x * rg;
    const int nr = min(rg, Sp - r0);
    const int h = sv.Lpad + i;
    const bool tr = stored_transposed(h);
    const size_t pos = (size_t)b * sv.L + i;
    float4 *tile4 = reinterpret_cast<float4 *>(tile);
    const int n4 = nr * Sp / 4;
    const bool real = i < sv.L;
    const int rlo = min(r0, d.S), rhi = min(r0 + nr, d.S);
    const int k0 = real ? (tr ? d.col_ptr[rlo] : d.row_ptr[rlo]) : 0;
    const int ne = real ? (tr ? d.col_ptr[rhi] : d.row_ptr[rhi]) - k0 : 0;
    const int32_t *erc = (tr ? d.ent_t_rc : d.ent_n_rc) + k0;
    const int32_t *esrc = (tr ? d.ent_t_src : d.ent_n_src) + k0;
    const float *direct = d.use_sel ? src.psel + pos * d.nsel : src.p + pos * d.V;
    // the first kLeafPre entries per thread, and their direct values, are
    // loaded (clamped, unconditionally) before the tile is cleared
    const float *indv = src.ndval + pos * d.n_ind;
    int prc[kLeafPre], pcode[kLeafPre];
    float pval[kLeafPre];
    if (ne > 0) {
#pragma unroll
        for (int u = 0; u < kLeafPre; ++u) {
            const int k = min(tid + u * kLeafThreads, ne - 1);
            prc[u] = erc[k];
            pcode[u] = esrc[k];
        }
#pragma unroll
        for (int u = 0; u < kLeafPre; ++u) {
            const float xd = direct[max(pcode[u], 0)];
            const float xi = indv[max(-1 - pcode[u], 0)];
            pval[u] = pcode[u] >= 0 ? xd : xi;
        }
    }
    for (int k = tid; k < n4; k += kLeafThreads) tile4[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = tid; r < nr; r += kLeafThreads) remax[r] = kNeg;
    __syncthreads();
    if (real) {
        int bad = 0;
        auto place = [&](int rc, float v) {
            const int row = (rc >> 16) - r0, col = rc & 0xffff;
            tile[row * Sp + col] = v;
            if (v > 0.f) atomicMax(&remax[row], fexp(v));
        };
#pragma unroll
        for (int u = 0; u < kLeafPre; ++u) {
            if (tid + u * kLeafThreads < ne) {
                const float v = pval[u];
                if (pcode[u] >= 0 && !d.use_sel) bad |= !(v >= 0.f);
                place(prc[u], v);
            }
        }
        for (int k = tid + kLeafPre * kLeafThreads; k < ne; k += kLeafThreads) {
            const int code = esrc[k];
            const float v = code >= 0 ? direct[code] : indv[-1 - code];
            if (code >= 0 && !d.use_sel) bad |= !(v >= 0.f);
            place(erc[k], v);
        }
        if (bad) atomicOr(&status[b], (int)FA_ROW_BADPROB);
    } else {  // identity leaf past the sequence end
        for (int r = tid; r < nr; r += kLeafThreads)
            if (r0 + r < d.S) {
                tile[r * Sp + r0 + r] = 1.f;
                remax[r] = fexp(1.f);
            }
    }
    __syncthreads();
    if (pv && real) {
        // the folded entries (value times 2^-rf of its stored row) in the
        // leaf's stored entry order, for a first span level from the pairs
        float *pvrow = pv + pos * d.npairs + k0;
        for (int k = tid; k < ne; k += kLeafThreads) {
            const int rc = erc[k];
            const int row = (rc >> 16) - r0, col = rc & 0xffff;
            pvrow[k] = ldexpf(tile[row * Sp + col], 0 - remax[row]);
        }
    }
    if (!d.leafless || sv.K == 0) {   // a one-leaf tree's root is the leaf
        float4 *M4 = reinterpret_cast<float4 *>(sv.mat_ptr(tree, b, h) + (size_t)r0 * Sp);
        for (int k = tid; k < n4; k += kLeafThreads) M4[k] = tile4[k];
    }
    int32_t *ro = sv.meta_ptr(meta, b, h, 0), *co = sv.meta_ptr(meta, b, h, 1);
    int32_t *rf = sv.meta_ptr(meta, b, h, 2);
    for (int r = tid; r < nr; r += kLeafThreads) {
        rf[r0 + r] = remax[r];
        ro[r0 + r] = 0;
        co[r0 + r] = 0;
    }
}

// Leaves of a table that keeps no dense leaves (L > 1): only the folded
// pair values and the row exponents, no dense tile.  One workgroup per
// leaf: every pair's value is evaluated in parallel in the leaf's stored
// entry order into LDS, then each row's largest exponent is taken over the
// row's contiguous entries, then the values are written times 2^-rf of
// their row (what the dense leaf's consumers fold them to) with coalesced
// stores, in stored order, or with `walk` (the pair-staged first level) in
// the order that level walks the leaf: column order for a row-major leaf
// (output o is stored entry col_pairs[o]), pair order for a transposed one
// (output q is stored entry pair_colpos[q]).  Identity leaves past the
// sequence end write only their row exponents (those of a diagonal of
// ones).
constexpr int kLpThreads = 1024;
constexpr int kLpUnroll = 4;

__global__ __launch_bounds__(kLpThreads) void emission_leaf_pairs(DevTable d, StepView sv, EmitSrc src,
                                                                  int32_t *__restrict__ meta,
                                                                  float *__restrict__ pv, int walk,
                                                                  int32_t *__restrict__ status)
{
    extern __shared__ float lpv[];  // [npairs] values in stored order | [Sp] row exponents
    const int np = d.npairs;
    int *remax = reinterpret_cast<int *>(lpv + np);
    const int tid = threadIdx.x;
    const int b = blockIdx.x / sv.Lpad, i = blockIdx.x % sv.Lpad;
    const int h = sv.Lpad + i;
    const bool tr = stored_transposed(h);
    const bool real = i < sv.L;
    const size_t pos = (size_t)b * sv.L + i;
    for (int r = tid; r < sv.Sp; r += kLpThreads) remax[r] = (!real && r < d.S) ? fexp(1.f) : kNeg;
    __syncthreads();
    if (real) {
        const int32_t *erc = tr ? d.ent_t_rc : d.ent_n_rc;
        const int32_t *esrc = tr ? d.ent_t_src : d.ent_n_src;
        const float *direct = d.use_sel ? src.psel + pos * d.nsel : src.p + pos * d.V;
        const float *indv = src.ndval + pos * d.n_ind;
        int bad = 0;
        // kLpUnroll entries per thread in flight: codes first (clamped), then values
        for (int e0 = 0; e0 < np; e0 += kLpThreads * kLpUnroll) {
            int code[kLpUnroll], row[kLpUnroll];
#pragma unroll
            for (int u = 0; u < kLpUnroll; ++u) {
                const int e = min(e0 + u * kLpThreads + tid, np - 1);
                code[u] = esrc[e];
                row[u] = erc[e] >> 16;
            }
#pragma unroll
            for (int u = 0; u < kLpUnroll; ++u) {
                const int e = e0 + u * kLpThreads + tid;
                const float xd = direct[max(code[u], 0)];
                const float xi = indv[max(-1 - code[u], 0)];
                const float v = code[u] >= 0 ? xd : xi;
                if (e < np) {
                    lpv[e] = v;
                    if (code[u] >= 0 && !d.use_sel) bad |= !(v >= 0.f);
                }
            }
        }
        if (bad) atomicOr(&status[b], (int)FA_ROW_BADPROB);
        __syncthreads();
        // each row's largest exponent: four threads per row over its
        // contiguous stored entries, combined across the four lanes (LDS
        // atomics on one row's word would serialize its lanes)
        const int32_t *ptr = tr ? d.col_ptr : d.row_ptr;
        for (int r0 = 0; r0 < sv.Sp; r0 += kLpThreads / 4) {
            const int r = r0 + (tid >> 2), part = tid & 3;
            int m = kNeg;
            if (r < d.S) {
                const int e1 = ptr[r + 1];
                for (int e = ptr[r] + part; e < e1; e += 4) {
                    const float v = lpv[e];
                    if (v > 0.f) m = max(m, fexp(v));
                }
            }
            m = max(m, __shfl_xor(m, 1));
            m = max(m, __shfl_xor(m, 2));
            if (part == 0 && r < sv.Sp) remax[r] = m;
        }
    }
    __syncthreads();
    if (real) {
        // output o: stored entry e and its stored row (low half of the walk's codes)
        const int32_t *perm = tr ? d.pair_colpos : d.col_pairs;
        const int32_t *orc = walk ? (tr ? d.ent_n_rc : d.ent_t_rc) : nullptr;
        const int32_t *erc = tr ? d.ent_t_rc : d.ent_n_rc;
        float *out = pv + pos * np;
        for (int o0 = 0; o0 < np; o0 += kLpThreads * kLpUnroll) {
            int e[kLpUnroll], row[kLpUnroll];
#pragma unroll
            for (int u = 0; u < kLpUnroll; ++u) {
                const int o = min(o0 + u * kLpThreads + tid, np - 1);
                e[u] = walk ? perm[o] : o;
                row[u] = walk ? (orc[o] & 0xffff) : (erc[o] >> 16);
            }
#pragma unroll
            for (int u = 0; u < kLpUnroll; ++u) {
                const int o = o0 + u * kLpThreads + tid;
                if (o < np) out[o] = ldexpf(lpv[e[u]], 0 - remax[row[u]]);
            }
        }
    }
    int32_t *ro = sv.meta_ptr(meta, b, h, 0), *co = sv.meta_ptr(meta, b, h, 1);
    int32_t *rf = sv.meta_ptr(meta, b, h, 2);
    for (int r = tid; r < sv.Sp; r += kLpThreads) {
        rf[r] = remax[r];
        ro[r] = 0;
        co[r] = 0;
    }
}

// Folded entries of every leaf for a first span level from the pairs, on the path
// whose leaves are densified from pair-order values: in the leaf's stored
// entry order (pair order, or column order for a transposed leaf), each
// value times 2^-rf of its stored row, as the dense kernels consume it.
__global__ void emission_fold_pairs(DevTable d, StepView sv, const float *__restrict__ val,
                                    const int32_t *__restrict__ meta, float *__restrict__ pvf)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const size_t pos = blockIdx.y;
    if (e >= d.npairs) return;
    const int b = (int)(pos / sv.L), i = (int)(pos % sv.L);
    const int h = sv.Lpad + i;
    const bool tr = stored_transposed(h);
    const int q = tr ? d.col_pairs[e] : e;
    const int row = tr ? d.pair_b[q] : d.pair_a[q];
    const int32_t *rf = sv.meta_ptr(meta, b, h, 2);
    pvf[pos * d.npairs + e] = ldexpf(val[pos * d.npairs + q], 0 - rf[row]);
}

}  // namespace

int launch_build_transitions(const DevTable &d, const Geometry &g, const float *p, float *tree,
                             int32_t *meta, uint8_t *ws, const WsLayout &w, int32_t *status,
                             void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    const int npos = g.B * g.L;
    const int BLpad = (npos + kDenseTile - 1) / kDenseTile * kDenseTile;
    const EmitSrc src = emit_src(d, g, p, ws, w);
    // leaves straight from pair values when an LDS tile holds a row
    const bool fused = g.Sp <= kLeafTile;  // the leaf entries exist for Sp < 65536
    if (d.ndense > 0) {
        dim3 grid(w.n_vchunks, BLpad / kDenseTile);
        const bool vec = (d.V & 3) == 0 && ((uintptr_t)p & 15) == 0;
        int pe = prof_mark(FA_PROF_EMISSION_DENSE, true, stream);
        if (pe) return pe;
        const int sel = d.use_sel ? w.sel_mode : 0;
#define FA_DENSE(VEC, SEL)                                                                      \
    emission_dense<VEC, SEL><<<grid, kDenseThreads, 0, st>>>(d, p, g.L, npos, BLpad, w.vchunk, \
                                                             (float *)src.dpart,                \
                                                             (float *)src.psel, status)
        if (vec) {
            if (sel == 0) FA_DENSE(true, 0);
            else if (sel == 1) FA_DENSE(true, 1);
            else FA_DENSE(true, 2);
        } else {
            if (sel == 0) FA_DENSE(false, 0);
            else if (sel == 1) FA_DENSE(false, 1);
            else FA_DENSE(false, 2);
        }
#undef FA_DENSE
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
        pe = prof_mark(FA_PROF_EMISSION_DENSE, false, stream);
        if (pe) return pe;
        if (!fused) {
            const int n = npos * kDenseMax;
            emission_dense_reduce<<<(n + 255) / 256, 256, 0, st>>>(w.n_vchunks, BLpad, npos, d.ndense,
                                                                   src.dpart, (float *)src.dval);
            e = hipGetLastError();
            if (e != hipSuccess) return (int)e;
        }
    }
    if (d.nseg > 0) {
        if ((d.V & 3) == 0 && ((uintptr_t)p & 15) == 0)
            emission_ranges<true><<<npos, kStreamThreads, 0, st>>>(d, p, g.L, (double *)src.cutp,
                                                                   status);
        else
            emission_ranges<false><<<npos, kStreamThreads, 0, st>>>(d, p, g.L, (double *)src.cutp,
                                                                    status);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    StepView sv = step_view(g);
    if (fused) {
        if (d.n_ind > 0) {
            dim3 igrid((d.n_ind + kIndThreads - 1) / kIndThreads, npos);
            emission_indirect<<<igrid, kIndThreads, 0, st>>>(d, g.L, src, status);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return (int)e;
        }
        if (d.leafless && g.K >= 1) {
            // the table keeps no dense leaves: pair values and row exponents only
            const size_t lds = ((size_t)d.npairs + g.Sp) * 4;
            if (lds > 48 * 1024) {
                const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&emission_leaf_pairs),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                                         (int)lds);
                if (e != hipSuccess) return (int)e;
            }
            emission_leaf_pairs<<<g.B * g.Lpad, kLpThreads, lds, st>>>(d, sv, src, meta, (float *)(ws + w.pvf),
                                                                      d.first_pairs, status);
            return (int)hipGetLastError();
        }
        const int rg = kLeafTile / g.Sp;
        dim3 grid((g.Sp + rg - 1) / rg, g.B * g.Lpad);
        float *pv = d.first_sparse || d.first_pairs ? (float *)(ws + w.pvf) : nullptr;
        emission_leaves<<<grid, kLeafThreads, 0, st>>>(d, sv, rg, src, tree, meta, pv, status);
        return (int)hipGetLastError();
    }
    float *val = (float *)(ws + w.val);
    if (d.npairs > 0) {
        dim3 pgrid((d.npairs + 256 * kPairsPerThread - 1) / (256 * kPairsPerThread), npos);
        emission_pairs<<<pgrid, 256, 0, st>>>(d, g.L, src, val, status);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    if (d.map_n) {
        dim3 grid((g.Sp + 3) / 4, g.B * g.Lpad);
        emission_densify_map<<<grid, 256, 0, st>>>(d, sv, val, tree, meta);
    } else {
        dim3 grid((g.Sp + 4 * kRowsPerWave - 1) / (4 * kRowsPerWave), g.B * g.Lpad);
        emission_densify<<<grid, kDensifyThreads, 0, st>>>(d, sv, val, tree, meta);
    }
    if ((d.first_sparse || d.first_pairs) && d.npairs > 0 && npos > 0) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
        dim3 fgrid((d.npairs + 255) / 256, npos);
        emission_fold_pairs<<<fgrid, 256, 0, st>>>(d, sv, val, meta, (float *)(ws + w.pvf));
    }
    return (int)hipGetLastError();
}

}  // namespace fa
