// Live states of every boundary, for span products restricted to them
// (tables compiled with FA_LIVE_STATES).  Under the step's p only the
// states that are reachable from s0 (R_i, through positions 0 .. i-1) and
// can still reach F (C_i, through positions i .. L-1) carry weight: a path
// of the posterior visits live states only, so a product whose two factors
// meet at boundary m sums over the states live at m without changing any
// entry between live states, and the entries it does change (rows or
// columns of dead states) are only ever met by zero forward or backward
// weight.  The restriction is exact (paperfeed summary "What to be
// skeptical about": the |S|^3 cost of the products; here, fewer states per
// contraction where committed positions prune the automaton).
//
// Per batch row one workgroup walks the positions forward for R and one
// backward for C, the state sets as bitsets in LDS; a pair is usable at
// position i when its transition value there is positive (the dense leaf
// entry, or on a table without dense leaves the folded value the products
// consume).  Boundaries past L (identity positions) keep R_L and F.  Then
// per boundary the states in both sets, ascending, padded with -1 to a
// multiple of 64 entries (at least 64).
#include "device_common.h"

namespace fa {
namespace {

constexpr int kLiveThreads = 1024;

__device__ inline bool bit_of(const uint32_t *s, int k) { return (s[k >> 5] >> (k & 31)) & 1u; }

// bits: [B][2][Lpad+1][W] (W = ceil(Sp / 32)); y = 0 forward (R), 1 backward (C)
__global__ __launch_bounds__(kLiveThreads) void live_reach(DevTable d, StepView sv,
                                                           const float *__restrict__ tree,
                                                           const float *__restrict__ pvf,
                                                           uint32_t *__restrict__ bits)
{
    extern __shared__ uint32_t lbs[];  // cur [W] | nxt [W]
    const int W = (sv.Sp + 31) >> 5;
    uint32_t *cur = lbs, *nxt = lbs + W;
    const int b = blockIdx.x, tid = threadIdx.x;
    const bool fwd = blockIdx.y == 0;
    uint32_t *out = bits + ((size_t)b * 2 + blockIdx.y) * (sv.Lpad + 1) * W;
    for (int w = tid; w < W; w += kLiveThreads) cur[w] = 0u;
    __syncthreads();
    if (fwd) {
        if (tid == 0) cur[d.start >> 5] |= 1u << (d.start & 31);
    } else {
        for (int k = tid; k < d.n_acc; k += kLiveThreads) atomicOr(&cur[d.acc[k] >> 5], 1u << (d.acc[k] & 31));
    }
    __syncthreads();
    const int first = fwd ? 0 : sv.L;
    for (int w = tid; w < W; w += kLiveThreads) out[(size_t)first * W + w] = cur[w];
    const int np = d.npairs;
    for (int step = 0; step < sv.L; ++step) {
        const int i = fwd ? step : sv.L - 1 - step;  // position
        for (int w = tid; w < W; w += kLiveThreads) nxt[w] = 0u;
        __syncthreads();
        const int h = sv.Lpad + i;
        const bool tr = stored_transposed(h);
        const float *M = d.leafless ? nullptr : sv.mat_ptr(tree, b, h);
        const float *pv = d.leafless ? pvf + ((size_t)b * sv.L + i) * np : nullptr;
        // entry e of the leaf's stored order: pair order, or column order
        // for a transposed leaf
        for (int e = tid; e < np; e += kLiveThreads) {
            const int q = tr ? d.col_pairs[e] : e;
            const int a = d.pair_a[q], c = d.pair_b[q];
            const float v = d.leafless ? pv[e] : (tr ? M[(size_t)c * sv.Sp + a] : M[(size_t)a * sv.Sp + c]);
            const int from = fwd ? a : c, to = fwd ? c : a;
            if (v > 0.f && bit_of(cur, from)) atomicOr(&nxt[to >> 5], 1u << (to & 31));
        }
        __syncthreads();
        const int ib = fwd ? i + 1 : i;  // boundary of the new set
        for (int w = tid; w < W; w += kLiveThreads) {
            cur[w] = nxt[w];
            out[(size_t)ib * W + w] = nxt[w];
        }
        __syncthreads();
    }
    // boundaries L+1 .. Lpad: R_L forward; F backward (identity positions)
    if (!fwd) {
        for (int w = tid; w < W; w += kLiveThreads) cur[w] = 0u;
        __syncthreads();
        for (int k = tid; k < d.n_acc; k += kLiveThreads) atomicOr(&cur[d.acc[k] >> 5], 1u << (d.acc[k] & 31));
        __syncthreads();
    }
    for (int ib = sv.L + 1; ib <= sv.Lpad; ++ib)
        for (int w = tid; w < W; w += kLiveThreads) out[(size_t)ib * W + w] = cur[w];
}

constexpr int kListThreads = 256;

// live: [B][Lpad+1][Sp] lists; nlive: [B][Lpad+1] counts.  grid (Lpad+1, B)
__global__ __launch_bounds__(kListThreads) void live_lists(StepView sv, const uint32_t *__restrict__ bits,
                                                           int32_t *__restrict__ live,
                                                           int32_t *__restrict__ nlive)
{
    __shared__ int sh_part[kListThreads / 64];
    const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int W = (sv.Sp + 31) >> 5;
    const uint32_t *R = bits + ((size_t)b * 2 * (sv.Lpad + 1) + i) * W;
    const uint32_t *C = bits + (((size_t)b * 2 + 1) * (sv.Lpad + 1) + i) * W;
    int32_t *out = live + ((size_t)b * (sv.Lpad + 1) + i) * sv.Sp;
    int base = 0;
    for (int w0 = 0; w0 < W; w0 += kListThreads) {
        const int w = w0 + tid;
        const uint32_t m = w < W ? (R[w] & C[w]) : 0u;
        const int cnt = __popc(m);
        // exclusive block scan of the counts, in word order
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) sh_part[wave] = incl;
        __syncthreads();
        int off = base + incl - cnt, tot = base;
        for (int k = 0; k < kListThreads / 64; ++k) {
            if (k < wave) off += sh_part[k];
            tot += sh_part[k];
        }
        __syncthreads();  // sh_part is rewritten by the next chunk
        uint32_t r = m;
        while (r) {
            const int j = __ffs(r) - 1;
            out[off++] = w * 32 + j;
            r &= r - 1u;
        }
        base = tot;
    }
    const int npad = max(64, (base + 63) & ~63);
    for (int k = base + tid; k < npad; k += kListThreads) out[k] = -1;
    if (tid == 0) nlive[(size_t)b * (sv.Lpad + 1) + i] = base;
}

}  // namespace

int launch_live_states(const DevTable &d, const Geometry &g, const float *tree, uint8_t *ws,
                       const WsLayout &w, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    const int W = (g.Sp + 31) >> 5;
    uint32_t *bits = (uint32_t *)(ws + w.lbits);
    const size_t lds = (size_t)2 * W * sizeof(uint32_t);
    if (lds > 48 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&live_reach),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
    }
    live_reach<<<dim3(g.B, 2), kLiveThreads, lds, st>>>(d, sv, tree, (const float *)(ws + w.pvf), bits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    live_lists<<<dim3(g.Lpad + 1, g.B), kListThreads, 0, st>>>(sv, bits, (int32_t *)(ws + w.live),
                                                                (int32_t *)(ws + w.nlive));
    return (int)hipGetLastError();
}

}  // namespace fa
