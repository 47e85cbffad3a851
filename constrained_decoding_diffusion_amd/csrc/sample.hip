// Top-down exact sampling over the span tree (paperfeed "The scan trick:
// log-depth exact sampling": given both boundary states of a segment, the
// two halves are independent given the midpoint, whose conditional is
// proportional to P_[l,m)[z_l][z_m] P_[m,r)[z_m][z_r]; the midpoints are drawn
// level by level, then every token in parallel; papernotes 关键设计 2: the
// final boundary state first, from its joint marginal with the pinned start).
//
// Every draw is an inverse CDF over ascending candidate ids: the smallest j
// with w_j > 0 and C_j > u T (C the inclusive prefix sum, T its total), u
// from Philox4x32-10 keyed (seed, b, level, node).  A zero-weight candidate
// is never chosen, so every sample is accepted by the automaton.
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

__device__ inline float mant(float x)
{
    int e;
    return frexpf(x, &e);
}

// root: z_Lpad over the accepting states
__global__ void sample_root(DevTable d, StepView sv, const float *__restrict__ tree,
                            const int32_t *__restrict__ meta, uint64_t seed,
                            int32_t *__restrict__ zc, int32_t *__restrict__ status)
{
    const int b = blockIdx.x, lane = threadIdx.x;
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
        const float u = philox_u01(seed, (uint32_t)b, 0u, 0u);
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

// one midpoint level: node n = nn + idx covers [l, r); children 2n (stored as
// is) and 2n+1 (stored transposed): both needed vectors are stored rows
__global__ __launch_bounds__(256) void sample_level(DevTable d, StepView sv,
                                                    const float *__restrict__ tree,
                                                    const int32_t *__restrict__ meta,
                                                    uint64_t seed, int level, int nn,
                                                    int32_t *__restrict__ zc,
                                                    int32_t *__restrict__ status)
{
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= sv.B * nn) return;
    const int b = gw / nn, idx = gw % nn, n = nn + idx;
    const int span = sv.Lpad / nn, l = idx * span, r = l + span, m = l + span / 2;
    int32_t *z = zc + (size_t)b * (sv.Lpad + 1);
    const int zl = z[l], zr = z[r];
    int j = -1;
    if (zl >= 0 && zr >= 0) {
        const float *PL = sv.mat_ptr(tree, b, 2 * n) + (size_t)zl * sv.Sp;
        const float *PR = sv.mat_ptr(tree, b, 2 * n + 1) + (size_t)zr * sv.Sp;
        const int32_t *coL = sv.meta_ptr(meta, b, 2 * n, 1);
        const int32_t *coR = sv.meta_ptr(meta, b, 2 * n + 1, 1);
        auto expo = [&](int k) {
            const float a = PL[k], c = PR[k];
            if (!(a > 0.f) || !(c > 0.f) || coL[k] <= kNeg || coR[k] <= kNeg) return kNeg;
            return fexp(a) + coL[k] + fexp(c) + coR[k];
        };
        int e = kNeg;
        for (int k = lane; k < d.S; k += 64) e = max(e, expo(k));
        const int emax = wave_max_i(e);
        if (emax > kNeg) {
            const float u = philox_u01(seed, (uint32_t)b, (uint32_t)level, (uint32_t)idx);
            j = wave_icdf(d.S, u, lane, [&](int k) {
                const int ek = expo(k);
                return ek > kNeg ? scale2(mant(PL[k]) * mant(PR[k]), ek - emax) : 0.f;
            });
        }
        if (j < 0 && lane == 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
    }
    if (lane == 0) z[m] = j;
}

constexpr int kTokThreads = 256;

__global__ __launch_bounds__(kTokThreads) void sample_tokens(
    DevTable d, StepView sv, const float *__restrict__ p, uint64_t seed,
    const int32_t *__restrict__ zc, int32_t *__restrict__ tokens, int32_t *__restrict__ status)
{
    const int b = blockIdx.y, i = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *z = zc + (size_t)b * (sv.Lpad + 1);
    const int a = z[i], c = z[i + 1];
    __shared__ double sh_part[kTokThreads];
    __shared__ double sh_wtot[4];
    __shared__ int sh_q;
    if (tid == 0) {
        int q = -1;
        if (a >= 0 && c >= 0) {
            int lo = d.row_ptr[a], hi = d.row_ptr[a + 1];
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (d.pair_b[mid] < c) lo = mid + 1;
                else hi = mid;
            }
            if (lo < d.row_ptr[a + 1] && d.pair_b[lo] == c) q = lo;
        }
        sh_q = q;
    }
    __syncthreads();
    const int q = sh_q;
    if (q < 0) {
        if (tid == 0) {
            tokens[(size_t)b * sv.L + i] = -1;
            if (a >= 0 && c >= 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
        }
        return;
    }
    const float *prow = p + ((size_t)b * sv.L + i) * d.V;
    const int cls = d.pair_cls[q];
    // candidate space [0, n) and its weights, ascending token order
    int n, base = 0, s0 = 0, s1 = 0;
    uint32_t dbit = 0;
    if (cls == kList) {
        base = d.list_off[q];
        n = d.list_off[q + 1] - base;
    } else if (cls == kDense) {
        n = d.V;
        dbit = 1u << d.pair_aux[q];
    } else {
        s0 = d.seg_off[q];
        s1 = d.seg_off[q + 1];
        base = d.seg_lo[s0];
        n = d.seg_hi[s1 - 1] - base;
    }
    const int sl = (n + kTokThreads - 1) / kTokThreads;
    const int k0 = min(n, tid * sl), k1 = min(n, k0 + sl);
    // segment cursor for range pairs
    int seg = s0;
    if (cls == kRange) {
        int lo = s0, hi = s1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (d.seg_hi[mid] <= base + k0) lo = mid + 1;
            else hi = mid;
        }
        seg = lo;
    }
    auto weight = [&](int k, int &sg) -> float {
        if (cls == kList) {
            const float x = prow[d.list_tok[base + k]];
            return d.list_cnt ? x * d.list_cnt[base + k] : x;
        }
        if (cls == kDense) return (d.tokmask[k] & dbit) ? prow[k] : 0.f;
        const int v = base + k;
        while (sg < s1 && d.seg_hi[sg] <= v) ++sg;
        if (sg < s1 && d.seg_lo[sg] <= v) return prow[v] * d.seg_cnt[sg];
        return 0.f;
    };
    double part = 0.0;
    {
        int sg = seg;
        for (int k = k0; k < k1; ++k) part += (double)weight(k, sg);
    }
    // block inclusive scan of the thread partials (fp64)
    const double ws = wave_incl_scan_d(part, lane);
    if (lane == 63) sh_wtot[wave] = ws;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += sh_wtot[w];
    const double incl = off + ws;
    sh_part[tid] = incl;
    __syncthreads();
    const double T = sh_part[kTokThreads - 1];
    if (!(T > 0.0)) {
        if (tid == 0) {
            tokens[(size_t)b * sv.L + i] = -1;
            atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
        }
        return;
    }
    const float u = philox_u01(seed, (uint32_t)b, (uint32_t)(sv.K + 1), (uint32_t)i);
    const double target = (double)u * T;
    // first thread whose inclusive prefix passes the target
    const bool cross = part > 0.0 && incl > target;
    const uint64_t bal = __ballot(cross);
    __shared__ int sh_first[4];
    if (lane == 0) sh_first[wave] = bal ? (wave * 64 + __ffsll((unsigned long long)bal) - 1) : 0x7fffffff;
    __syncthreads();
    const int tstar = min(min(sh_first[0], sh_first[1]), min(sh_first[2], sh_first[3]));
    int tpick = tstar;
    if (tstar == 0x7fffffff) {
        // rounding left no crossing: take the last thread with mass
        __shared__ int sh_last[4];
        const uint64_t any = __ballot(part > 0.0);
        if (lane == 0) sh_last[wave] = any ? (wave * 64 + 63 - __clzll((unsigned long long)any)) : -1;
        __syncthreads();
        tpick = max(max(sh_last[0], sh_last[1]), max(sh_last[2], sh_last[3]));
    }
    if (tid == tpick) {
        double cacc = incl - part;
        int last = -1, pick = -1;
        int sg = seg;
        for (int k = k0; k < k1; ++k) {
            const float x = weight(k, sg);
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
        int tok = -1;
        if (pick >= 0) tok = (cls == kList) ? d.list_tok[base + pick] : base + pick;
        tokens[(size_t)b * sv.L + i] = tok;
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
    StepView sv = step_view(g);
    int32_t *zc = (int32_t *)(ws + w.zc);
    sample_root<<<g.B, 64, 0, st>>>(d, sv, tree, meta, seed, zc, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    for (int level = 1; level <= g.K; ++level) {
        const int nn = 1 << (level - 1);
        const int waves = g.B * nn;
        sample_level<<<(waves + 3) / 4, 256, 0, st>>>(d, sv, tree, meta, seed, level, nn, zc, status);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    sample_tokens<<<dim3(g.L, g.B), kTokThreads, 0, st>>>(d, sv, p, seed, zc, tokens, status);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    sample_finalize<<<dim3((g.L + 1 + 255) / 256, g.B), 256, 0, st>>>(d, sv, zc, states, tokens,
                                                                      status);
    return (int)hipGetLastError();
}

}  // namespace fa
