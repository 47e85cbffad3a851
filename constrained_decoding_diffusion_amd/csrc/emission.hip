// Emission reduce: M_i[a][b] = sum_v c(a, v, b) p[i][v] for every position,
// written as dense leaves of the span tree (papernotes 关键设计 1: each
// position's transition matrix sums the mean-field-reweighted emissions over
// the vocabulary; paperfeed "The insight": the |E||V| term).
//
// Two kernels:
//  * emission_stream: one workgroup per position streams the p row once,
//    coalesced, and produces what needs the whole row: the dense-mask pair
//    sums, fp64 prefix sums at every range cut point, and a compact copy of
//    p at the tokens the LIST pairs use.  Runs only for tables with dense or
//    range pairs.
//  * emission_densify: one wavefront per stored leaf row evaluates the pair
//    values of that row and writes the row (Sp floats) in 64-column chunks,
//    zeros included, with its power-of-two row exponent.  Odd leaves are
//    stored transposed, so their stored rows are the columns of M_i.
#include "device_common.h"

namespace fa {
namespace {

constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void emission_stream(
    DevTable d, const float *__restrict__ p, int L, float *__restrict__ dval,
    float *__restrict__ psel, double *__restrict__ cutp, int32_t *__restrict__ status)
{
    const int pos = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *row = p + (size_t)pos * d.V;
    const int nd = d.ndense;
    __shared__ float sh_x[kStreamThreads];
    __shared__ double sh_incl[kStreamThreads];
    __shared__ double sh_wsum[4];
    __shared__ float sh_red[4][kDenseMax];
    __shared__ int sh_bad;
    if (tid == 0) sh_bad = 0;

    float acc[kDenseMax];
#pragma unroll
    for (int j = 0; j < kDenseMax; ++j) acc[j] = 0.f;
    double carry = 0.0;
    int cptr = 0, sptr = 0;
    int bad = 0;
    const bool want_sel = d.use_sel && psel;
    for (int c0 = 0; c0 < d.V; c0 += kStreamThreads) {
        const int v = c0 + tid;
        float x = 0.f;
        if (v < d.V) {
            x = row[v];
            bad |= !(x >= 0.f);
            if (nd) {
                uint32_t m = d.tokmask[v];
#pragma unroll
                for (int j = 0; j < kDenseMax; ++j)
                    if (j < nd) acc[j] += ((m >> j) & 1u) ? x : 0.f;
            }
        }
        if (want_sel) sh_x[tid] = x;
        if (d.ncut) {
            double inc = wave_incl_scan_d((double)x, lane);
            if (lane == 63) sh_wsum[wave] = inc;
            __syncthreads();
            double off = 0.0;
            for (int w = 0; w < wave; ++w) off += sh_wsum[w];
            sh_incl[tid] = off + inc;
            __syncthreads();
            // cut points inside this chunk (sorted, at most one per token)
            const int idx = cptr + tid;
            int c = (idx < d.ncut) ? d.cuts[idx] : 0x7fffffff;
            bool in = c < c0 + kStreamThreads && c < d.V;
            if (in) {
                int k = c - c0;
                cutp[(size_t)pos * d.ncut + idx] = carry + (k > 0 ? sh_incl[k - 1] : 0.0);
            }
            cptr += __syncthreads_count(in);
            carry += sh_incl[kStreamThreads - 1];
            __syncthreads();
        } else if (want_sel) {
            __syncthreads();
        }
        if (want_sel) {
            const int idx = sptr + tid;
            int t = (idx < d.nsel) ? d.sel_tok[idx] : 0x7fffffff;
            bool in = t < c0 + kStreamThreads;
            if (in) psel[(size_t)pos * d.nsel + idx] = sh_x[t - c0];
            sptr += __syncthreads_count(in);
        }
    }
    // cut points equal to V hold the row total
    if (d.ncut)
        for (int idx = cptr + tid; idx < d.ncut; idx += kStreamThreads)
            cutp[(size_t)pos * d.ncut + idx] = carry;
    if (nd) {
#pragma unroll
        for (int j = 0; j < kDenseMax; ++j) {
            if (j < nd) {
                float s = wave_sum(acc[j]);
                if (lane == 0) sh_red[wave][j] = s;
            }
        }
    }
    if (bad) atomicOr(&sh_bad, 1);
    __syncthreads();
    if (tid < nd) {
        float s = ((sh_red[0][tid] + sh_red[1][tid]) + sh_red[2][tid]) + sh_red[3][tid];
        dval[(size_t)pos * nd + tid] = s;
    }
    if (tid == 0 && sh_bad) atomicOr(&status[pos / L], (int)FA_ROW_BADPROB);
}

// value of pair q at position pos
__device__ inline float pair_value(const DevTable &d, int q, size_t pos, const float *p,
                                   const float *dval, const float *psel, const double *cutp,
                                   int &bad)
{
    const int cls = d.pair_cls[q];
    if (cls == kDense) return dval[pos * d.ndense + d.pair_aux[q]];
    if (cls == kRange) {
        double s = 0.0;
        const double *cp = cutp + pos * d.ncut;
        for (int k = d.seg_off[q]; k < d.seg_off[q + 1]; ++k)
            s += (cp[d.seg_hi_cut[k]] - cp[d.seg_lo_cut[k]]) * (double)d.seg_cnt[k];
        return (float)s;
    }
    float s = 0.f;
    const int k0 = d.list_off[q], k1 = d.list_off[q + 1];
    if (d.use_sel) {
        const float *src = psel + pos * d.nsel;
        if (d.list_cnt)
            for (int k = k0; k < k1; ++k) s += src[d.list_sel[k]] * d.list_cnt[k];
        else
            for (int k = k0; k < k1; ++k) s += src[d.list_sel[k]];
    } else {
        const float *src = p + pos * d.V;
        for (int k = k0; k < k1; ++k) {
            float x = src[d.list_tok[k]];
            bad |= !(x >= 0.f);
            s += d.list_cnt ? x * d.list_cnt[k] : x;
        }
    }
    return s;
}

constexpr int kRowsPerWave = 2;
constexpr int kDensifyThreads = 256;

__global__ __launch_bounds__(kDensifyThreads) void emission_densify(
    DevTable d, StepView sv, const float *__restrict__ p, const float *__restrict__ dval,
    const float *__restrict__ psel, const double *__restrict__ cutp, float *__restrict__ tree,
    int32_t *__restrict__ meta, int32_t *__restrict__ status)
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
    int bad = 0;
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
        const int r = (blockIdx.x * 4 + wave) * kRowsPerWave + rr;
        if (r >= sv.Sp) break;
        float *out = M + (size_t)r * sv.Sp;
        int emax = kNeg;
        if (i >= sv.L) {  // identity leaf
            for (int c = lane; c < sv.Sp; c += 64) {
                float x = (c == r && r < d.S) ? 1.f : 0.f;
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
                stage[wave][lane] = 0.f;
                const int k = kp + lane;
                int q = -1, col = 0x7fffffff;
                if (k < k1) {
                    q = tr ? d.col_pairs[k] : k;
                    col = tr ? d.pair_a[q] : d.pair_b[q];
                }
                const bool in = col < cw + 64;
                wave_sync();
                if (in) stage[wave][col - cw] = pair_value(d, q, pos, p, dval, psel, cutp, bad);
                wave_sync();
                float x = stage[wave][lane];
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
    if (bad) atomicOr(&status[b], (int)FA_ROW_BADPROB);
}

}  // namespace

int launch_build_transitions(const DevTable &d, const Geometry &g, const float *p, float *tree,
                             int32_t *meta, uint8_t *ws, const WsLayout &w, int32_t *status,
                             void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    float *dval = (float *)(ws + w.dval);
    float *psel = d.use_sel ? (float *)(ws + w.psel) : nullptr;
    double *cutp = (double *)(ws + w.cutp);
    const int npos = g.B * g.L;
    if (d.ndense > 0 || d.nseg > 0) {
        emission_stream<<<npos, kStreamThreads, 0, st>>>(d, p, g.L, dval, psel, cutp, status);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    StepView sv = step_view(g);
    dim3 grid((g.Sp + 4 * kRowsPerWave - 1) / (4 * kRowsPerWave), g.B * g.Lpad);
    emission_densify<<<grid, kDensifyThreads, 0, st>>>(d, sv, p, dval, psel, cutp, tree, meta,
                                                       status);
    return (int)hipGetLastError();
}

}  // namespace fa
