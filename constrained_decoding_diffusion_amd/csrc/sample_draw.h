// Midpoint draws of the top-down sampler, shared by the sampler's own
// launches and by the joint call's message-pass launches, which carry them as
// extra workgroups (device code is not linked across files).
//
// Every draw is an inverse CDF over ascending candidate ids: the smallest j
// with w_j > 0 and C_j > u T (C the inclusive prefix sum, T its total), u
// from Philox4x32-10 keyed (seed, b, level, node).  A zero-weight candidate
// is never chosen, so every sample is accepted by the automaton.
#pragma once

#include "device_common.h"

namespace fa {
namespace {

// wavefront inverse CDF over n candidates (fp32 weights, fp64 prefix sums);
// weight(k) is evaluated twice in the same order, so the total of the second
// pass equals the first
template <class Wt>
__device__ int wave_icdf(int n, float u, int lane, Wt weight)
{
    double carry = 0.0;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const float x = (c0 + lane < n) ? weight(c0 + lane) : 0.f;
        const double s = wave_incl_scan_d((double)x, lane);
        carry += __shfl(s, 63);
    }
    const double T = carry;
    if (!(T > 0.0)) return -1;
    const double target = (double)u * T;
    carry = 0.0;
    int last = -1;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const bool valid = c0 + lane < n;
        const float x = valid ? weight(c0 + lane) : 0.f;
        const double s = wave_incl_scan_d((double)x, lane);
        const bool pos = valid && x > 0.f;
        const uint64_t hit = __ballot(pos && carry + s > target);
        if (hit) return c0 + __ffsll((unsigned long long)hit) - 1;
        const uint64_t any = __ballot(pos);
        if (any) last = c0 + 63 - __clzll((unsigned long long)any);
        carry += __shfl(s, 63);
    }
    return last;
}

// the same inverse CDF over weights held in registers: candidate
// 64*c + lane is w[c]
template <int C>
__device__ int wave_icdf_regs(const float (&w)[C], int n, float u, int lane)
{
    double carry = 0.0;
    double incl[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const double s = wave_incl_scan_d((double)w[c], lane);
        incl[c] = carry + s;
        carry += __shfl(s, 63);
    }
    const double T = carry;
    if (!(T > 0.0)) return -1;
    const double target = (double)u * T;
    int last = -1;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const bool pos = 64 * c + lane < n && w[c] > 0.f;
        const uint64_t hit = __ballot(pos && incl[c] > target);
        if (hit) return 64 * c + __ffsll((unsigned long long)hit) - 1;
        const uint64_t any = __ballot(pos);
        if (any) last = 64 * c + 63 - __clzll((unsigned long long)any);
    }
    return last;
}

// root: z_Lpad over the accepting states
// the root draw of row b by one wavefront: z[0] = start, z[Lpad] = the
// drawn accepting state (-1, and the row flagged, when every weight vanishes)
__device__ void draw_root(const DevTable &d, const StepView &sv, const float *__restrict__ tree,
                          const int32_t *__restrict__ meta, uint64_t seed, int b, int lane,
                          int32_t *__restrict__ zc, int32_t *__restrict__ status)
{
    int32_t *z = zc + (size_t)b * (sv.Lpad + 1);
    const float *R = sv.mat_ptr(tree, b, 1) + (size_t)d.start * sv.Sp;
    const int32_t *co = sv.meta_ptr(meta, b, 1, 1);
    int e = kNeg;
    for (int k = lane; k < d.n_acc; k += 64) {
        const int f = d.acc[k];
        if (R[f] > 0.f && co[f] > kNeg) e = max(e, fexp(R[f]) + co[f]);
    }
    const int m = wave_max_i(e);
    int j = -1;
    if (status[b] == 0 && m > kNeg) {
        const float u = philox_u01(seed, (uint32_t)(sv.b0 + b), 0u, 0u);
        j = wave_icdf(d.n_acc, u, lane, [&](int k) {
            const int f = d.acc[k];
            const float x = R[f];
            return (x > 0.f && co[f] > kNeg) ? scale2(mant(x), fexp(x) + co[f] - m) : 0.f;
        });
    }
    if (lane == 0) {
        z[0] = d.start;
        z[sv.Lpad] = j >= 0 ? d.acc[j] : -1;
        if (j < 0 && status[b] == 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
    }
}

// pair of the boundary states (a, c) of one position, for the token draw
__device__ inline void put_pair(const DevTable &d, int a, int c, int32_t *tpair, uint32_t *tdbit)
{
    const int q = pair_index(d, a, c);
    *tpair = q;
    *tdbit = (q >= 0 && d.pair_cls[q] == kDense) ? 1u << d.pair_aux[q] : 0u;
}

// The midpoint draw of a first-level node on a table without dense leaves:
// candidate k weighs L[zl][k] R[k][zr], the two leaves' pair values (folded:
// a factor 2^-rf per leaf that is the same for every candidate) looked up in
// map_n, or the identity past the sequence end.  The weights are formed as in
// draw_mid from the same mantissas and exponent differences, so the draw is
// the one the dense leaves give.  The values are in each leaf's stored
// order (pair order left, column order right), or, on a table whose first
// level is staged from the pairs, in its walk order (the other one).
__device__ int draw_mid_pairs(const DevTable &d, const StepView &sv, const int32_t *__restrict__ meta,
                              uint64_t seed, int b, int level, int idx, int n, int zl, int zr,
                              int lane, int32_t *__restrict__ status)
{
    const int iL = 2 * n - sv.Lpad, iR = iL + 1;
    const float *vL = sv.pvf + ((size_t)b * sv.L + min(iL, sv.L - 1)) * d.npairs;
    const float *vR = sv.pvf + ((size_t)b * sv.L + min(iR, sv.L - 1)) * d.npairs;
    const bool realL = iL < sv.L, realR = iR < sv.L;
    const int32_t *coL = sv.meta_ptr(meta, b, 2 * n, 1);
    const int32_t *coR = sv.meta_ptr(meta, b, 2 * n + 1, 1);
    const size_t Sp = sv.Sp;
    const bool walk = d.first_pairs != 0;
    auto pl = [&](int k) -> float {
        if (!realL) return k == zl ? 1.f : 0.f;
        const int q = d.map_n[(size_t)zl * Sp + k];
        return q >= 0 ? vL[walk ? d.pair_colpos[q] : q] : 0.f;
    };
    auto pr = [&](int k) -> float {
        if (!realR) return k == zr ? 1.f : 0.f;
        const int q = d.map_n[(size_t)k * Sp + zr];
        return q >= 0 ? vR[walk ? q : d.pair_colpos[q]] : 0.f;
    };
    auto expo = [&](int k) {
        const float a = pl(k), c = pr(k);
        if (!(a > 0.f) || !(c > 0.f) || coL[k] <= kNeg || coR[k] <= kNeg) return kNeg;
        return fexp(a) + coL[k] + fexp(c) + coR[k];
    };
    const float u = philox_u01(seed, (uint32_t)(sv.b0 + b), (uint32_t)level, (uint32_t)idx);
    int j = -1;
    int e = kNeg;
    for (int k = lane; k < d.S; k += 64) e = max(e, expo(k));
    const int emax = wave_max_i(e);
    if (emax > kNeg) {
        j = wave_icdf(d.S, u, lane, [&](int k) {
            const int ek = expo(k);
            return ek > kNeg ? scale2(mant(pl(k)) * mant(pr(k)), ek - emax) : 0.f;
        });
    }
    if (j < 0 && lane == 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
    return j;
}

// one midpoint level: node n = nn + idx covers [l, r); children 2n (stored as
// is) and 2n+1 (stored transposed): both needed vectors are stored rows
// midpoint draw of node n (level `level`, index idx within the level) by
// one wavefront, given its boundary states; -1 when they are -1 or when every
// candidate's weight vanishes (then the row is flagged)
__device__ int draw_mid(const DevTable &d, const StepView &sv, const float *__restrict__ tree,
                        const int32_t *__restrict__ meta, uint64_t seed, int b, int level, int idx,
                        int n, int zl, int zr, int lane, int32_t *__restrict__ status)
{
    int j = -1;
    if (zl < 0 || zr < 0) return -1;
    if (sv.pvf && n >= (sv.Lpad >> 1))
        return draw_mid_pairs(d, sv, meta, seed, b, level, idx, n, zl, zr, lane, status);
    const float *PL = sv.mat_ptr(tree, b, 2 * n) + (size_t)zl * sv.Sp;
    const float *PR = sv.mat_ptr(tree, b, 2 * n + 1) + (size_t)zr * sv.Sp;
    const int32_t *coL = sv.meta_ptr(meta, b, 2 * n, 1);
    const int32_t *coR = sv.meta_ptr(meta, b, 2 * n + 1, 1);
    auto expo2 = [&](float a, float c, int cl, int cr) {
        if (!(a > 0.f) || !(c > 0.f) || cl <= kNeg || cr <= kNeg) return kNeg;
        return fexp(a) + cl + fexp(c) + cr;
    };
    const float u = philox_u01(seed, (uint32_t)(sv.b0 + b), (uint32_t)level, (uint32_t)idx);
    constexpr int C = 8;
    if (d.S <= 64 * C) {
        // every candidate's data in registers: one round of loads
        float pa[C], pb[C];
        int ek[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int k = 64 * c + lane;
            const bool ok = k < d.S;
            pa[c] = ok ? PL[k] : 0.f;
            pb[c] = ok ? PR[k] : 0.f;
            ek[c] = ok ? coL[k] : kNeg;
            const int cr = ok ? coR[k] : kNeg;
            ek[c] = expo2(pa[c], pb[c], ek[c], cr);
        }
        int e = kNeg;
#pragma unroll
        for (int c = 0; c < C; ++c) e = max(e, ek[c]);
        const int emax = wave_max_i(e);
        if (emax > kNeg) {
            float wv[C];
#pragma unroll
            for (int c = 0; c < C; ++c)
                wv[c] = ek[c] > kNeg ? scale2(mant(pa[c]) * mant(pb[c]), ek[c] - emax) : 0.f;
            j = wave_icdf_regs(wv, d.S, u, lane);
        }
    } else {
        auto expo = [&](int k) { return expo2(PL[k], PR[k], coL[k], coR[k]); };
        int e = kNeg;
        for (int k = lane; k < d.S; k += 64) e = max(e, expo(k));
        const int emax = wave_max_i(e);
        if (emax > kNeg) {
            j = wave_icdf(d.S, u, lane, [&](int k) {
                const int ek = expo(k);
                return ek > kNeg ? scale2(mant(PL[k]) * mant(PR[k]), ek - emax) : 0.f;
            });
        }
    }
    if (j < 0 && lane == 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
    return j;
}

// Midpoints of `depth` (<= kSubDepth) consecutive levels from level0, one
// subtree per workgroup: at sub-level t wavefront w < 2^t draws node w of the
// subtree.  The subtree's boundary states stay in LDS between sub-levels
// (slot q holds position l0 + q * span0 / 2^depth); each draw is also written
// to zc.  The launch that reaches the leaves also records, per position,
// the pair its token draw uses.
constexpr int kSubDepth = 3;
constexpr int kSubThreads = 64 << (kSubDepth - 1);  // the waves one subtree uses

// the subtree of workgroup `blk` of a midpoint launch; the workgroup has at
// least kSubThreads threads (waves past the first 2^(kSubDepth-1) only meet
// the barriers)
__device__ void sample_levels_wg(const DevTable &d, const StepView &sv,
                                 const float *__restrict__ tree, const int32_t *__restrict__ meta,
                                 uint64_t seed, int level0, int depth, int32_t *__restrict__ zc,
                                 int32_t *__restrict__ tpair, uint32_t *__restrict__ tdbit,
                                 int32_t *__restrict__ status, int blk)
{
    // a launch outside the tree's levels draws nothing (uniform per workgroup)
    if (level0 < 1 || depth < 1 || depth > kSubDepth || level0 + depth - 1 > sv.K) return;
    __shared__ int zs[(1 << kSubDepth) + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nn0 = 1 << (level0 - 1);
    const int b = blk / nn0, idx0 = blk % nn0;
    const int span0 = sv.Lpad / nn0;
    const int q = 1 << depth;
    const int unit = span0 / q;
    const int l0 = idx0 * span0;
    int32_t *z = zc + (size_t)b * (sv.Lpad + 1);
    if (level0 == 1) {  // the first launch also draws the root (wavefront 0)
        if (wave == 0) draw_root(d, sv, tree, meta, seed, b, lane, zc, status);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        zs[0] = z[l0];
        zs[q] = z[l0 + span0];
    }
    __syncthreads();
    for (int t = 0; t < depth; ++t) {
        if (wave < (1 << t)) {
            const int width = q >> t;
            const int ql = wave * width, qm = ql + width / 2;
            const int nn = nn0 << t;
            const int idx = (idx0 << t) + wave;
            const int j = draw_mid(d, sv, tree, meta, seed, b, level0 + t, idx, nn + idx, zs[ql],
                                   zs[ql + width], lane, status);
            if (lane == 0) {
                zs[qm] = j;
                z[l0 + qm * unit] = j;
            }
        }
        __syncthreads();
    }
    if (level0 + depth - 1 == sv.K) {  // unit = 1: slots are positions
        const int t = threadIdx.x, i = l0 + t;
        if (t < q && i < sv.L) {
            const size_t pos = (size_t)b * sv.L + i;
            put_pair(d, zs[t], zs[t + 1], tpair + pos, tdbit + pos);
        }
    }
}

// one launch of midpoint draws riding on another launch: nwg workgroups
// (none when nwg = 0)
struct MidDraws {
    const float *tree;
    const int32_t *meta;
    uint64_t seed;
    int level0, depth, nwg;
    int32_t *zc, *tpair;
    uint32_t *tdbit;
    int32_t *status;
};

__device__ inline void mid_draws_wg(const DevTable &d, const StepView &sv, const MidDraws &m, int blk)
{
    sample_levels_wg(d, sv, m.tree, m.meta, m.seed, m.level0, m.depth, m.zc, m.tpair, m.tdbit,
                     m.status, blk);
}

}  // namespace
}  // namespace fa
