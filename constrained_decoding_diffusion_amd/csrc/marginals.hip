// Constrained per-token marginals and the remasking confidence (papernotes
// 关键设计 3: the constrained marginal of the sampled token scores which
// positions to commit; paperfeed "Two immediate bonuses": LLaDA keeps the
// highest probability, Dream the lowest entropy).
//
// Forward and backward boundary messages come top-down from the span tree:
// alpha_0 = e_s0, beta_Lpad = 1_F, and for a node [l, r) with midpoint m,
// alpha_m = alpha_l T_[l,m) and beta_m = T_[m,r) beta_r.  Both are a vector
// times a stored matrix (the right child is stored transposed), with the
// vector's own power-of-two exponent.  Then, per position,
//   q[i][v] = p[i][v] sum_{pairs (a,a') holding v} c alpha_i[a] beta_{i+1}[a'] / Z.
#include "device_common.h"

namespace fa {
namespace {

__device__ inline float mant(float x)
{
    int e;
    return frexpf(x, &e);
}

__global__ void marg_init(DevTable d, StepView sv, float *__restrict__ va, int32_t *__restrict__ ea,
                          float *__restrict__ vb, int32_t *__restrict__ eb)
{
    const int b = blockIdx.x;
    float *a0 = va + (size_t)b * (sv.Lpad + 1) * sv.Sp;
    float *bL = vb + ((size_t)b * (sv.Lpad + 1) + sv.Lpad) * sv.Sp;
    for (int s = threadIdx.x; s < sv.Sp; s += blockDim.x) {
        a0[s] = (s == d.start) ? 1.f : 0.f;
        bL[s] = 0.f;
    }
    __syncthreads();
    for (int k = threadIdx.x; k < d.n_acc; k += blockDim.x) bL[d.acc[k]] = 1.f;
    if (threadIdx.x == 0) {
        ea[(size_t)b * (sv.Lpad + 1)] = 0;
        eb[(size_t)b * (sv.Lpad + 1) + sv.Lpad] = 0;
    }
}

constexpr int kVecThreads = 256;

// out = in * T for the consumed stored rows of one node; grid.y enumerates
// (b, node, alpha|beta)
__global__ __launch_bounds__(kVecThreads) void marg_level(DevTable d, StepView sv,
                                                          const float *__restrict__ tree,
                                                          const int32_t *__restrict__ meta,
                                                          int nn, float *__restrict__ va,
                                                          int32_t *__restrict__ ea,
                                                          float *__restrict__ vb,
                                                          int32_t *__restrict__ eb)
{
    extern __shared__ float gsh[];  // [Sp] normalized input weights
    __shared__ int sh_max[4];
    __shared__ int sh_G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int y = blockIdx.y;
    const int beta = y & 1;
    const int bn = y >> 1;
    const int b = bn / nn, idx = bn % nn, n = nn + idx;
    const int span = sv.Lpad / nn, l = idx * span, r = l + span, m = l + span / 2;
    const int h = beta ? 2 * n + 1 : 2 * n;
    const int src = beta ? r : l;
    float *vbase = beta ? vb : va;
    int32_t *ebase = beta ? eb : ea;
    const float *vin = vbase + ((size_t)b * (sv.Lpad + 1) + src) * sv.Sp;
    float *vout = vbase + ((size_t)b * (sv.Lpad + 1) + m) * sv.Sp;
    const int ein = ebase[(size_t)b * (sv.Lpad + 1) + src];
    const float *P = sv.mat_ptr(tree, b, h);
    const int32_t *ro = sv.meta_ptr(meta, b, h, 0);
    const int32_t *co = sv.meta_ptr(meta, b, h, 1);
    const int32_t *rf = sv.meta_ptr(meta, b, h, 2);
    // G = max_a e(in[a]) + ro[a] + rf[a]
    int e = kNeg;
    for (int a = tid; a < d.S; a += kVecThreads) {
        const float x = vin[a];
        const int s = add_exp(ro[a], rf[a]);
        if (x > 0.f && s > kNeg) e = max(e, fexp(x) + s);
    }
    e = wave_max_i(e);
    if (lane == 0) sh_max[wave] = e;
    __syncthreads();
    if (tid == 0) sh_G = max(max(sh_max[0], sh_max[1]), max(sh_max[2], sh_max[3]));
    __syncthreads();
    const int G = sh_G;
    for (int a = tid; a < d.S; a += kVecThreads) {
        const float x = vin[a];
        const int s = add_exp(ro[a], rf[a]);
        gsh[a] = (x > 0.f && s > kNeg && G > kNeg) ? scale2(mant(x), fexp(x) + s - G) : 0.f;
    }
    __syncthreads();
    const int j = blockIdx.x * kVecThreads + tid;
    if (j < sv.Sp) {
        float acc = 0.f;
        if (G > kNeg && j < d.S) {
            const int coj = co[j];
            for (int a = 0; a < d.S; ++a) {
                const float g = gsh[a];
                if (g == 0.f) continue;
                const float x = P[(size_t)a * sv.Sp + j];
                if (x != 0.f) acc += g * scale2(x, coj - rf[a]);
            }
        }
        vout[j] = acc;
    }
    if (blockIdx.x == 0 && tid == 0)
        ebase[(size_t)b * (sv.Lpad + 1) + m] = (G > kNeg && ein > kNeg) ? ein + G : kNeg;
}

// range weights per cut interval: rcut[pos][c] = sum of c*alpha*beta over
// the segments covering [cuts[c], cuts[c+1]); fp64 sweep, exact zero when no
// segment is active
__global__ void marg_rcut(DevTable d, StepView sv, const float *__restrict__ va,
                          const float *__restrict__ vb, float *__restrict__ rcut)
{
    const int pos = blockIdx.x * blockDim.x + threadIdx.x;
    if (pos >= sv.B * sv.L) return;
    const int b = pos / sv.L, i = pos % sv.L;
    const float *al = va + ((size_t)b * (sv.Lpad + 1) + i) * sv.Sp;
    const float *be = vb + ((size_t)b * (sv.Lpad + 1) + i + 1) * sv.Sp;
    double R = 0.0;
    int active = 0;
    float *out = rcut + (size_t)pos * d.ncut;
    for (int c = 0; c < d.ncut; ++c) {
        for (int k = d.cut_off[c]; k < d.cut_off[c + 1]; ++k) {
            const int ev = d.cut_ev[k];
            const int s = ev >> 1;
            const int q = d.seg_pair[s];
            const double w = (double)al[d.pair_a[q]] * (double)be[d.pair_b[q]] * (double)d.seg_cnt[s];
            if (ev & 1) { R -= w; --active; }
            else { R += w; ++active; }
        }
        if (active == 0 || R < 0.0) R = 0.0;
        out[c] = (float)R;
    }
}

constexpr int kQThreads = 256;

__global__ __launch_bounds__(kQThreads) void marg_q(DevTable d, StepView sv,
                                                    const float *__restrict__ p,
                                                    const double *__restrict__ logZ,
                                                    const int32_t *__restrict__ tokens,
                                                    int conf_mode, float *__restrict__ q,
                                                    float *__restrict__ conf,
                                                    const float *__restrict__ va,
                                                    const int32_t *__restrict__ ea,
                                                    const float *__restrict__ vb,
                                                    const int32_t *__restrict__ eb,
                                                    const float *__restrict__ rcut,
                                                    const int32_t *__restrict__ status)
{
    __shared__ float wd[kDenseMax];
    __shared__ double sh_h[4];
    const int b = blockIdx.y, i = blockIdx.x;
    const size_t pos = (size_t)b * sv.L + i;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *prow = p + pos * d.V;
    float *qrow = q ? q + pos * d.V : nullptr;
    const double lz = logZ[b];
    const int e1 = ea[(size_t)b * (sv.Lpad + 1) + i], e2 = eb[(size_t)b * (sv.Lpad + 1) + i + 1];
    const bool ok = status[b] == 0 && lz > -INFINITY && e1 > kNeg && e2 > kNeg;
    if (!ok) {
        if (qrow)
            for (int v = tid; v < d.V; v += kQThreads) qrow[v] = 0.f;
        if (tid == 0) conf[pos] = -INFINITY;
        return;
    }
    const double factor = exp2((double)e1 + (double)e2 - lz * 1.4426950408889634074);
    const float *al = va + ((size_t)b * (sv.Lpad + 1) + i) * sv.Sp;
    const float *be = vb + ((size_t)b * (sv.Lpad + 1) + i + 1) * sv.Sp;
    if (tid < d.ndense) {
        const int qq = d.dense_pair[tid];
        wd[tid] = al[d.pair_a[qq]] * be[d.pair_b[qq]];
    }
    __syncthreads();
    const int tok = tokens ? tokens[pos] : -1;
    int v0 = 0, v1 = d.V;
    if (!qrow && conf_mode == FA_CONF_PROB) {  // only the sampled token is needed
        v0 = tok < 0 ? 0 : tok;
        v1 = tok < 0 ? 0 : tok + 1;
    }
    const float *rc = d.ncut ? rcut + pos * d.ncut : nullptr;
    double hsum = 0.0;
    for (int v = v0 + tid; v < v1; v += kQThreads) {
        float r = 0.f;
        if (d.ndense) {
            const uint32_t msk = d.tokmask[v];
#pragma unroll
            for (int jj = 0; jj < kDenseMax; ++jj)
                if (jj < d.ndense && ((msk >> jj) & 1u)) r += wd[jj];
        }
        if (d.nsel) {
            const int s = d.tok2sel[v];
            if (s >= 0)
                for (int k = d.tm_off[s]; k < d.tm_off[s + 1]; ++k) {
                    const int qq = d.tm_pair[k];
                    const float w = al[d.pair_a[qq]] * be[d.pair_b[qq]];
                    r += d.tm_cnt ? w * d.tm_cnt[k] : w;
                }
        }
        if (rc) {
            const int c = d.tok2cut[v];
            if (c >= 0) r += rc[c];
        }
        const float x = prow[v];
        const float qv = (r > 0.f && x > 0.f) ? (float)((double)x * (double)r * factor) : 0.f;
        if (qrow) qrow[v] = qv;
        if (v == tok && conf_mode == FA_CONF_PROB) conf[pos] = qv;
        if (conf_mode == FA_CONF_NEGENT && qv > 0.f) hsum += (double)qv * log((double)qv);
    }
    if (conf_mode == FA_CONF_NEGENT) {
        hsum = wave_sum_d(hsum);
        if (lane == 0) sh_h[wave] = hsum;
        __syncthreads();
        if (tid == 0) conf[pos] = (float)(((sh_h[0] + sh_h[1]) + sh_h[2]) + sh_h[3]);
    } else if (tid == 0 && tok < 0) {
        conf[pos] = -INFINITY;
    }
}

}  // namespace

int launch_marginals(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                     const int32_t *meta, const double *logZ, const int32_t *tokens,
                     int32_t conf_mode, float *q, float *conf, uint8_t *ws, const WsLayout &w,
                     int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    float *va = (float *)(ws + w.va), *vb = (float *)(ws + w.vb);
    int32_t *ea = (int32_t *)(ws + w.ea), *eb = (int32_t *)(ws + w.eb);
    float *rcut = (float *)(ws + w.rcut);
    marg_init<<<g.B, 256, 0, st>>>(d, sv, va, ea, vb, eb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const size_t lds_vec = (size_t)g.Sp * sizeof(float);
    for (int level = 1; level <= g.K; ++level) {
        const int nn = 1 << (level - 1);
        dim3 grid((g.Sp + kVecThreads - 1) / kVecThreads, g.B * nn * 2);
        marg_level<<<grid, kVecThreads, lds_vec, st>>>(d, sv, tree, meta, nn, va, ea, vb, eb);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    if (d.ncut) {
        const int npos = g.B * g.L;
        marg_rcut<<<(npos + 63) / 64, 64, 0, st>>>(d, sv, va, vb, rcut);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    marg_q<<<dim3(g.L, g.B), kQThreads, 0, st>>>(d, sv, p, logZ, tokens, conf_mode, q,
                                                           conf, va, ea, vb, eb, rcut, status);
    return (int)hipGetLastError();
}

}  // namespace fa
