// Value of one automaton pair (a, b) at one position, sum_v c(a, v, b) p[i][v],
// from what the emission reduce keeps in the workspace: the V-chunk partials
// of the dense-mask pairs, the compact copy of p at the token-list tokens,
// fp64 prefix sums of p at the range cut points, or p itself.  Shared by the
// leaf writer and the leaf level of the marginal message pass, so both see
// bit-identical values.
#pragma once

#include "device_common.h"

#include <type_traits>

namespace fa {

struct EmitSrc {
    float *ndval;       // [npos][n_ind] values of the indirect pairs (leaf writer output)
    const float *p;
    const float *dpart;
    const float *dval;  // [npos][kDenseMax] chunk sums of the dense-mask pairs
    const float *psel;
    const double *cutp;
    int n_vchunks;
    int BLpad;
};

// value of pair q at position pos (a dense-mask pair from its summed chunks)
__device__ inline float pair_value(const DevTable &d, int q, size_t pos, const EmitSrc &s,
                                   int &bad)
{
    const int cls = d.pair_cls[q];
    if (cls == kDense) return s.dval[pos * kDenseMax + d.pair_aux[q]];
    if (cls == kRange) {
        double acc = 0.0;
        const double *cp = s.cutp + pos * d.ncut;
        for (int k = d.seg_off[q]; k < d.seg_off[q + 1]; ++k)
            acc += (cp[d.seg_hi_cut[k]] - cp[d.seg_lo_cut[k]]) * (double)d.seg_cnt[k];
        return (float)acc;
    }
    // blocked sum: kListBlock terms at a time, then the block sums in order.
    // A single running fp32 sum over a long label drops terms that fall
    // below half an ulp of the total (a systematic loss when p decays along
    // the label); blocks keep each addition between similar magnitudes.
    // Inside a block the terms are fetched in batches of up to eight (their
    // indices, then their values: two rounds of independent loads instead of
    // two dependent loads per term; the batch shrinks to what is left of the
    // block, so a short label issues no extra loads) and added in label order.
    constexpr int kListBlock = 64;
    float acc = 0.f;
    const int k0 = d.list_off[q], k1 = d.list_off[q + 1];
    const float *src = d.use_sel ? s.psel + pos * d.nsel : s.p + pos * d.V;
    const int32_t *ids = d.use_sel ? d.list_sel : d.list_tok;
    float blk = 0.f;
    auto batch = [&](auto n, int k) {
        constexpr int N = decltype(n)::value;
        int id[N];
        float x[N];
#pragma unroll
        for (int u = 0; u < N; ++u) id[u] = ids[k + u];
#pragma unroll
        for (int u = 0; u < N; ++u) x[u] = src[id[u]];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            if (!d.use_sel) bad |= !(x[u] >= 0.f);
            blk += d.list_cnt ? x[u] * d.list_cnt[k + u] : x[u];
        }
    };
    for (int kb = k0; kb < k1; kb += kListBlock) {
        const int ke = min(k1, kb + kListBlock);
        blk = 0.f;
        int k = kb;
        for (; k + 8 <= ke; k += 8) batch(std::integral_constant<int, 8>(), k);
        if (k + 4 <= ke) {
            batch(std::integral_constant<int, 4>(), k);
            k += 4;
        }
        if (k + 2 <= ke) {
            batch(std::integral_constant<int, 2>(), k);
            k += 2;
        }
        if (k < ke) batch(std::integral_constant<int, 1>(), k);
        acc += blk;
    }
    return acc;
}

// value of pair q at position pos, with a dense-mask pair's V-chunk partials
// added here in chunk order
__device__ inline float pair_value_direct(const DevTable &d, int q, size_t pos, const EmitSrc &s,
                                          int &bad)
{
    if (d.pair_cls[q] == kDense) {
        const int j = d.pair_aux[q];
        const float *dp = s.dpart + pos * kDenseMax + j;
        const size_t cs = (size_t)s.BLpad * kDenseMax;  // chunk stride
        float acc = 0.f;
        int c = 0;
        // sixteen partials loaded together, then added in chunk order
        for (; c + 16 <= s.n_vchunks; c += 16) {
            float t[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) t[u] = dp[(size_t)(c + u) * cs];
#pragma unroll
            for (int u = 0; u < 16; ++u) acc += t[u];
        }
        for (; c + 4 <= s.n_vchunks; c += 4) {
            float t[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) t[u] = dp[(size_t)(c + u) * cs];
#pragma unroll
            for (int u = 0; u < 4; ++u) acc += t[u];
        }
        for (; c < s.n_vchunks; ++c) acc += dp[(size_t)c * cs];
        return acc;
    }
    return pair_value(d, q, pos, s, bad);
}

// source pointers of pair values for one step (workspace regions of the
// emission reduce)
inline EmitSrc emit_src(const DevTable &d, const Geometry &g, const float *p, uint8_t *ws,
                        const WsLayout &w)
{
    EmitSrc src;
    const int npos = g.B * g.L;
    src.p = p;
    src.dpart = (float *)(ws + w.dpart);
    src.psel = d.use_sel ? (float *)(ws + w.psel) : nullptr;
    src.cutp = (double *)(ws + w.cutp);
    src.n_vchunks = w.n_vchunks;
    src.BLpad = (npos + kDenseTile - 1) / kDenseTile * kDenseTile;
    src.dval = (float *)(ws + w.dval);
    src.ndval = (float *)(ws + w.ndval);
    return src;
}

}  // namespace fa
