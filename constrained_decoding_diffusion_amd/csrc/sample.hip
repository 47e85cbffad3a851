// Top-down exact sampling over the span tree (paperfeed "The scan trick:
// log-depth exact sampling": given both boundary states of a segment, the
// two halves are independent given the midpoint, whose conditional is
// proportional to P_[l,m)[z_l][z_m] P_[m,r)[z_m][z_r]; the midpoints are drawn
// level by level, then every token in parallel; papernotes 关键设计 2: the
// final boundary state first, from its joint marginal with the pinned start).
// The draw rule and the midpoint draws are in sample_draw.h.
#include "sample_draw.h"

namespace fa {
namespace {

// root draw alone (a tree of one leaf, Lpad = 1, L = 1)
__global__ void sample_root(DevTable d, StepView sv, const float *__restrict__ tree,
                            const int32_t *__restrict__ meta, uint64_t seed,
                            int32_t *__restrict__ zc, int32_t *__restrict__ tpair,
                            uint32_t *__restrict__ tdbit, int32_t *__restrict__ status)
{
    const int b = blockIdx.x;
    draw_root(d, sv, tree, meta, seed, b, threadIdx.x, zc, status);
    if (threadIdx.x == 0) {
        const int32_t *z = zc + (size_t)b * (sv.Lpad + 1);
        put_pair(d, z[0], z[1], tpair + b, tdbit + b);
    }
}

__global__ __launch_bounds__(kSubThreads) void sample_levels(
    DevTable d, StepView sv, const float *__restrict__ tree, const int32_t *__restrict__ meta,
    uint64_t seed, int level0, int depth, int32_t *__restrict__ zc, int32_t *__restrict__ tpair,
    uint32_t *__restrict__ tdbit, int32_t *__restrict__ status)
{
    sample_levels_wg(d, sv, tree, meta, seed, level0, depth, zc, tpair, tdbit, status, blockIdx.x);
}

constexpr int kTokThreads = 256;
// a streamed chunk: four float4 groups per thread
static_assert(4 * kTokThreads == kRowChunk4, "dense-pair chunk layout");

// candidates of one token draw: the tokens of the pair (z_i, z_{i+1}) in
// ascending order, weight p[i][v] times the number of edges holding v
struct TokCands {
    int cls, n, base, s0, s1;
    uint32_t dbit;
};

__device__ inline float tok_weight(const DevTable &d, const TokCands &c, const float *prow, int k,
                                   int &sg)
{
    if (c.cls == kList) {
        const float x = prow[d.list_tok[c.base + k]];
        return d.list_cnt ? x * d.list_cnt[c.base + k] : x;
    }
    if (c.cls == kDense) return (d.tokmask[k] & c.dbit) ? prow[k] : 0.f;
    const int v = c.base + k;
    while (sg < c.s1 && d.seg_hi[sg] <= v) ++sg;
    return (sg < c.s1 && d.seg_lo[sg] <= v) ? prow[v] * d.seg_cnt[sg] : 0.f;
}

__device__ inline int seg_cursor(const DevTable &d, const TokCands &c, int k)
{
    if (c.cls != kRange) return 0;
    int lo = c.s0, hi = c.s1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (d.seg_hi[mid] <= c.base + k) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// One workgroup per position.  Pass 1 streams the candidates in chunks
// (each thread a run of consecutive candidates, so loads are coalesced) and
// keeps fp64 chunk sums; the chunk holding u*T is found serially; pass 2
// rescans that chunk only.
// tpair: the pair of (z_i, z_{i+1}) per position, from the midpoint draws.
//
// pre (non-null): the q writer of the same step has already streamed the row
// and left, where pre_ok[position] is set, the wavefront partials of every
// pass-1 chunk of a dense pair (pre[(position * pre_nch + chunk) * 4 + wave],
// summed in the same order as below), so pass 1 is skipped there.
__global__ __launch_bounds__(kTokThreads) void sample_tokens(
    DevTable d, StepView sv, const float *__restrict__ p, uint64_t seed,
    const int32_t *__restrict__ zc, const int32_t *__restrict__ tpair,
    int32_t *__restrict__ tokens, int32_t *__restrict__ status, const double *__restrict__ pre,
    const int32_t *__restrict__ pre_ok, int pre_nch)
{
    const int b = blockIdx.y, i = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *z = zc + (size_t)b * (sv.Lpad + 1);
    const int a = z[i], c = z[i + 1];
    __shared__ double csum[kTokChunksMax];
    __shared__ double wsum[kTokChunksMax][4];
    __shared__ double sh_w[4];
    __shared__ double sh_scan[kTokThreads];
    __shared__ int sh_chunk;
    __shared__ double sh_base, sh_target;
    const int q = tpair[(size_t)b * sv.L + i];
    int32_t *out = tokens + (size_t)b * sv.L + i;
    if (q < 0) {
        if (tid == 0) {
            *out = -1;
            if (a >= 0 && c >= 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
        }
        return;
    }
    const float *prow = p + ((size_t)b * sv.L + i) * d.V;
    TokCands cd;
    cd.cls = d.pair_cls[q];
    cd.base = 0; cd.s0 = 0; cd.s1 = 0; cd.dbit = 0;
    if (cd.cls == kList) {
        cd.base = d.list_off[q];
        cd.n = d.list_off[q + 1] - cd.base;
    } else if (cd.cls == kDense) {
        cd.n = d.V;
        cd.dbit = 1u << d.pair_aux[q];
    } else {
        cd.s0 = d.seg_off[q];
        cd.s1 = d.seg_off[q + 1];
        cd.base = d.seg_lo[cd.s0];
        cd.n = d.seg_hi[cd.s1 - 1] - cd.base;
    }
    // chunk = kTokThreads runs of `per` consecutive candidates (at most 64
    // chunks for row-length candidate sets)
    const bool vec = cd.cls == kDense && (d.V & 3) == 0 && ((uintptr_t)prow & 15) == 0;
    // dense rows up to kTokChunksMax chunks of 4096 tokens stream through the
    // coalesced pass 1 below
    const bool streamed = vec && (long long)cd.n <= (long long)kTokChunksMax * 16 * kTokThreads;
    int per = 4;
    if (streamed) {
        per = 16;
    } else {
        while ((long long)per * kTokThreads * 64 < cd.n && per < 64) per *= 2;
        while ((long long)per * kTokThreads * kTokChunksMax < cd.n) per *= 2;
    }
    const int chunk = per * kTokThreads;
    const int nchunks = (cd.n + chunk - 1) / chunk;
    auto run_sum = [&](int c0) -> double {
        const int k0 = c0 + tid * per;
        double s = 0.0;
        if (vec) {  // dense mask: float4 / uint4 loads, same order as the scalar walk
            for (int k = k0; k < min(k0 + per, cd.n); k += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(prow + k);
                const uint4 m = *reinterpret_cast<const uint4 *>(d.tokmask + k);
                s += (double)((m.x & cd.dbit) ? x.x : 0.f);
                s += (double)((m.y & cd.dbit) ? x.y : 0.f);
                s += (double)((m.z & cd.dbit) ? x.z : 0.f);
                s += (double)((m.w & cd.dbit) ? x.w : 0.f);
            }
            return s;
        }
        int sg = seg_cursor(d, cd, k0);
        for (int k = k0; k < min(k0 + per, cd.n); ++k) s += (double)tok_weight(d, cd, prow, k, sg);
        return s;
    };
    // per-chunk wavefront partials, combined in wavefront order after one
    // barrier
    const size_t pos = (size_t)b * sv.L + i;
    const bool have_pre = streamed && pre && pre_ok[pos];
    if (have_pre) {
        const double *pp = pre + pos * pre_nch * 4;
        for (int ch = tid; ch < nchunks; ch += kTokThreads) {
            wsum[ch][0] = pp[4 * ch];
            wsum[ch][1] = pp[4 * ch + 1];
            wsum[ch][2] = pp[4 * ch + 2];
            wsum[ch][3] = pp[4 * ch + 3];
        }
    } else if (streamed) {
        // chunk ch = float4 groups [1024 ch, 1024 ch + 1024): thread t takes
        // groups 1024 ch + 256 u + t (u < 4), so each load instruction reads
        // 1 KB contiguous per wavefront; the label comes from the pair's own
        // bit array (4 bits per group), and the loads of chunks ch+1 and
        // ch+2 (unconditional, clamped) are in flight while chunk ch is summed
        const float4 *p4 = reinterpret_cast<const float4 *>(prow);
        const uint32_t *bits = d.dense_bits + (size_t)d.pair_aux[q] * d.dense_words;
        const int n4 = d.V >> 2;
        struct Buf {
            float4 x[4];
            uint32_t m[4];
        };
        auto load = [&](Buf &bf, int ch) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = min(ch * kRowChunk4 + u * kTokThreads + tid, n4 - 1);
                bf.x[u] = p4[k];
                bf.m[u] = bits[k >> 3];
            }
        };
        auto chunk_sum = [&](const Buf &bf, int ch) -> double {
            double s = 0.0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k = ch * kRowChunk4 + u * kTokThreads + tid;
                if (k < n4) {
                    const uint32_t m = bf.m[u] >> ((k & 7) * 4);
                    s += (double)((m & 1u) ? bf.x[u].x : 0.f);
                    s += (double)((m & 2u) ? bf.x[u].y : 0.f);
                    s += (double)((m & 4u) ? bf.x[u].z : 0.f);
                    s += (double)((m & 8u) ? bf.x[u].w : 0.f);
                }
            }
            return s;
        };
        auto put = [&](const Buf &bf, int ch) {
            const double s0 = wave_sum_d(chunk_sum(bf, ch));
            if (lane == 0 && ch < nchunks) wsum[ch][wave] = s0;
        };
        Buf A, Bn, C;
        load(A, 0);
        load(Bn, 1);
        for (int ch = 0; ch < nchunks; ch += 3) {
            load(C, ch + 2);
            __builtin_amdgcn_sched_barrier(0);
            put(A, ch);
            __builtin_amdgcn_sched_barrier(0);
            load(A, ch + 3);
            __builtin_amdgcn_sched_barrier(0);
            put(Bn, ch + 1);
            __builtin_amdgcn_sched_barrier(0);
            load(Bn, ch + 4);
            __builtin_amdgcn_sched_barrier(0);
            put(C, ch + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        for (int ch = 0; ch < nchunks; ++ch) {
            const double s = wave_sum_d(run_sum(ch * chunk));
            if (lane == 0) wsum[ch][wave] = s;
        }
    }
    __syncthreads();
    for (int ch = tid; ch < nchunks; ch += kTokThreads)
        csum[ch] = ((wsum[ch][0] + wsum[ch][1]) + wsum[ch][2]) + wsum[ch][3];
    __syncthreads();
    if (tid == 0) {
        double T = 0.0;
        for (int ch = 0; ch < nchunks; ++ch) T += csum[ch];
        int pick = -1;
        double base = 0.0, target = 0.0;
        if (T > 0.0) {
            target = (double)philox_u01(seed, (uint32_t)(sv.b0 + b), (uint32_t)(sv.K + 1), (uint32_t)i) * T;
            double acc = 0.0, acc_last = 0.0;
            int last = -1;
            for (int ch = 0; ch < nchunks; ++ch) {
                if (csum[ch] > 0.0) {
                    last = ch;
                    acc_last = acc;
                    if (acc + csum[ch] > target) {
                        pick = ch;
                        base = acc;
                        break;
                    }
                }
                acc += csum[ch];
            }
            if (pick < 0) {
                pick = last;
                base = acc_last;
            }
        }
        sh_chunk = pick;
        sh_base = base;
        sh_target = target;
    }
    __syncthreads();
    const int ch = sh_chunk;
    if (ch < 0) {
        if (tid == 0) {
            *out = -1;
            atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
        }
        return;
    }
    // pass 2: exclusive scan of the runs of the chosen chunk
    const double part = run_sum(ch * chunk);
    const double inc = wave_incl_scan_d(part, lane);
    if (lane == 63) sh_w[wave] = inc;
    __syncthreads();
    double off = sh_base;
    for (int w = 0; w < wave; ++w) off += sh_w[w];
    sh_scan[tid] = off + inc;
    __syncthreads();
    const double target = sh_target;
    const bool cross = part > 0.0 && off + inc > target;
    const uint64_t bal = __ballot(cross);
    __shared__ int sh_first[4], sh_lastw[4];
    const uint64_t any = __ballot(part > 0.0);
    if (lane == 0) {
        sh_first[wave] = bal ? wave * 64 + __ffsll((unsigned long long)bal) - 1 : 0x7fffffff;
        sh_lastw[wave] = any ? wave * 64 + 63 - __clzll((unsigned long long)any) : -1;
    }
    __syncthreads();
    int tpick = min(min(sh_first[0], sh_first[1]), min(sh_first[2], sh_first[3]));
    if (tpick == 0x7fffffff) tpick = max(max(sh_lastw[0], sh_lastw[1]), max(sh_lastw[2], sh_lastw[3]));
    if (tpick < 0) {  // no mass left in the chunk: cannot happen for a chunk with csum > 0
        if (tid == 0) {
            *out = -1;
            atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
        }
        return;
    }
    if (tid == tpick) {
        double cacc = sh_scan[tid] - part;
        const int k0 = ch * chunk + tid * per;
        int sg = seg_cursor(d, cd, k0);
        int last = -1, pick = -1;
        for (int k = k0; k < min(k0 + per, cd.n); ++k) {
            const float x = tok_weight(d, cd, prow, k, sg);
            cacc += (double)x;
            if (x > 0.f) {
                last = k;
                if (cacc > target) {
                    pick = k;
                    break;
                }
            }
        }
        if (pick < 0) pick = last;
        *out = pick < 0 ? -1 : (cd.cls == kList ? d.list_tok[cd.base + pick] : cd.base + pick);
    }
}

__global__ void sample_finalize(DevTable d, StepView sv, const int32_t *__restrict__ zc,
                                int32_t *__restrict__ states, int32_t *__restrict__ tokens,
                                const int32_t *__restrict__ status)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i > sv.L) return;
    const bool bad = status[b] != 0;
    const int zz = zc[(size_t)b * (sv.Lpad + 1) + i];
    states[(size_t)b * (sv.L + 1) + i] = (bad || zz < 0) ? -1 : d.orig[zz];
    if (i < sv.L && bad) tokens[(size_t)b * sv.L + i] = -1;
}

__global__ void sample_empty(DevTable d, int B, int32_t *__restrict__ states,
                             const int32_t *__restrict__ status)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) states[b] = status[b] ? -1 : d.orig[d.start];
}

}  // namespace

int launch_sample(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                  const int32_t *meta, uint64_t seed, int32_t *states, int32_t *tokens,
                  uint8_t *ws, const WsLayout &w, int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (g.L == 0) {
        sample_empty<<<(g.B + 255) / 256, 256, 0, st>>>(d, g.B, states, status);
        return (int)hipGetLastError();
    }
    int rc = launch_sample_states(d, g, tree, meta, seed, ws, w, status, stream);
    if (rc) return rc;
    return launch_sample_tokens(d, g, p, seed, states, tokens, ws, w, false, status, stream);
}

int launch_sample_states(const DevTable &d, const Geometry &g, const float *tree,
                         const int32_t *meta, uint64_t seed, uint8_t *ws, const WsLayout &w,
                         int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    if (d.leafless && g.K >= 1) sv.pvf = (const float *)(ws + w.pvf);
    int32_t *zc = (int32_t *)(ws + w.zc);
    int32_t *tpair = (int32_t *)(ws + w.tpair);
    uint32_t *tdbit = (uint32_t *)(ws + w.tdbit);
    hipError_t e;
    if (g.K == 0) {  // otherwise the first midpoint launch draws the root
        sample_root<<<g.B, 64, 0, st>>>(d, sv, tree, meta, seed, zc, tpair, tdbit, status);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    for (int level0 = 1; level0 <= g.K; level0 += kSubDepth) {
        const int depth = std::min(kSubDepth, g.K - level0 + 1);
        const int nn0 = 1 << (level0 - 1);
        sample_levels<<<g.B * nn0, kSubThreads, 0, st>>>(d, sv, tree, meta, seed, level0,
                                                                    depth, zc, tpair, tdbit, status);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

int launch_sample_tokens(const DevTable &d, const Geometry &g, const float *p, uint64_t seed,
                         int32_t *states, int32_t *tokens, uint8_t *ws, const WsLayout &w,
                         bool pre, int32_t *status, void *stream, bool finish)
{
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    const int32_t *zc = (const int32_t *)(ws + w.zc);
    const double *tcs = pre ? (const double *)(ws + w.tcs) : nullptr;
    const int32_t *tcs_ok = pre ? (const int32_t *)(ws + w.tcs_ok) : nullptr;
    const int32_t *tpair = (const int32_t *)(ws + w.tpair);
    sample_tokens<<<dim3(g.L, g.B), kTokThreads, 0, st>>>(d, sv, p, seed, zc, tpair, tokens, status,
                                                           tcs, tcs_ok, w.tcs_nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !finish) return (int)e;
    sample_finalize<<<dim3((g.L + 1 + 255) / 256, g.B), 256, 0, st>>>(d, sv, zc, states, tokens,
                                                                      status);
    return (int)hipGetLastError();
}

}  // namespace fa
