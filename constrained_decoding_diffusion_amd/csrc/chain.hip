// The serial chain sampler: forward filtering over the positions, then
// backward sampling -- the baseline the log-depth tree replaces (paperfeed
// summary "The scan trick: log-depth exact sampling": a serial
// forward-backward pass needs L dependent steps per denoising step; the
// tree needs log L rounds of batched products; papernotes 消融实验: the
// chain's latency against the tree's).  Same posterior, same leaves (the
// dense per-position matrices of fa_build_transitions), other draws:
//   a_0 = e_{s0}; e_i = the exponent of max a_i; a_{i+1} = (a_i 2^-e_i) M_i
//   (one launch per position: the L dependent steps);
//   log Z = ln 2 sum_{i<L} e_i + ln sum_{f in F} a_L[f];
//   z_L ~ a_L[f] over f in F, then z_i ~ a_i[a] M_i[a][z_{i+1}] for
//   i = L-1 .. 0 (one serial walk per row), u keyed (seed, b, K+2, i);
//   tokens as in the tree sampler, u keyed (seed, b, K+1, i).
// The scale of a_i does not change its draw (the inverse CDF normalizes).
// With the marginals, backward messages follow (one launch per position):
//   b_L = 1_F; e'_i = the exponent of max b_i; b_i = M_i (b_{i+1} 2^-e'_{i+1});
// alpha_i = a_i 2^(e_0 + .. + e_{i-1}) and beta_i = b_i 2^(e'_{i+1} + .. + e'_L)
// then feed the marginal writer of the tree path.
#include "sample_draw.h"

namespace fa {
namespace {

constexpr int kChainThreads = 256;

__global__ void chain_init(DevTable d, StepView sv, float *__restrict__ va)
{
    const int b = blockIdx.y;
    const int a = blockIdx.x * blockDim.x + threadIdx.x;
    if (a < sv.Sp) va[(size_t)b * (sv.Lpad + 1) * sv.Sp + a] = a == d.start ? 1.f : 0.f;
}

// One step of a message chain over this workgroup's kChainCols outputs, for
// every row: out = (x 2^-e) A with e the exponent of max x (recorded at the
// input vector's slot of ex).  Forward (a_{i+1} = a_i M_i): x = a_i, A = M_i.
// Backward (b_i = M_i b_{i+1}): x = b_{i+1}, A = M_i^T.  When a stored row
// of leaf i is a row of A (M_i stored as is going forward, a transposed
// leaf going backward) thread t sums rows r = t / 16 + 16 k (k ascending)
// for the four outputs 4 (t % 16) .. +3; otherwise stored row c is output c
// and thread t sums entries r = t % 4 + 4 k of stored row t / 4.  The
// partial sums are added in a fixed order, so the result does not depend
// on timing.
constexpr int kChainCols = 64;

__device__ void chain_msg_step(const DevTable &d, const StepView &sv, const float *__restrict__ tree,
                               int i, bool backward, float *__restrict__ v, int32_t *__restrict__ ex)
{
    extern __shared__ __align__(16) float xh[];  // [Sp] x scaled by 2^-e (0 past S)
    __shared__ int sh_e[kChainThreads / 64];
    __shared__ __align__(16) float4 part[kChainThreads];
    const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Sp = sv.Sp, S = d.S;
    const int src = backward ? i + 1 : i, dst = backward ? i : i + 1;
    const float *xin = v + ((size_t)b * (sv.Lpad + 1) + src) * Sp;
    float *out = v + ((size_t)b * (sv.Lpad + 1) + dst) * Sp;
    int e = kNeg;
    for (int a = tid; a < Sp; a += kChainThreads) {
        const float x = a < S ? xin[a] : 0.f;
        xh[a] = x;
        e = max(e, fexp(x));
    }
    e = wave_max_i(e);
    if (lane == 0) sh_e[wave] = e;
    __syncthreads();
    e = max(max(sh_e[0], sh_e[1]), max(sh_e[2], sh_e[3]));
    for (int a = tid; a < Sp; a += kChainThreads) xh[a] = e > kNeg ? ldexpf(xh[a], -e) : 0.f;
    __syncthreads();
    if (blockIdx.x == 0 && tid == 0) ex[(size_t)b * (sv.Lpad + 1) + src] = e;
    const int h = sv.Lpad + i;
    const float *M = sv.mat_ptr(tree, b, h);
    const int c0 = blockIdx.x * kChainCols;  // Sp is a multiple of kChainCols
    const bool rows_of_A = backward ? stored_transposed(h) : !stored_transposed(h);
    if (rows_of_A) {
        const int cg = tid & 15, rs = tid >> 4;
        const int c = c0 + 4 * cg;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int r = rs; r < S; r += 16) {
            const float4 m = *reinterpret_cast<const float4 *>(M + (size_t)r * Sp + c);
            const float x = xh[r];
            acc.x += x * m.x;
            acc.y += x * m.y;
            acc.z += x * m.z;
            acc.w += x * m.w;
        }
        part[tid] = acc;
        __syncthreads();
        if (tid < 16) {
            float4 t = part[tid];
            for (int r = 1; r < 16; ++r) {
                const float4 u = part[16 * r + tid];
                t.x += u.x;
                t.y += u.y;
                t.z += u.z;
                t.w += u.w;
            }
            *reinterpret_cast<float4 *>(out + c0 + 4 * tid) = t;
        }
    } else {
        // stored row c is output c; its entries past S are zero
        const int c = c0 + (tid >> 2), qd = tid & 3;
        const float4 *mr = reinterpret_cast<const float4 *>(M + (size_t)c * Sp);
        const float4 *x4 = reinterpret_cast<const float4 *>(xh);
        float acc = 0.f;
        for (int k = qd; k < Sp / 4; k += 4) {
            const float4 m = mr[k], x = x4[k];
            acc += x.x * m.x + x.y * m.y + x.z * m.z + x.w * m.w;
        }
        float *ps = reinterpret_cast<float *>(part);
        ps[tid] = acc;
        __syncthreads();
        if (tid < kChainCols) out[c0 + tid] = ((ps[4 * tid] + ps[4 * tid + 1]) + ps[4 * tid + 2]) + ps[4 * tid + 3];
    }
}

// a_{i+1} = (a_i 2^-e_i) M_i, e_i into ea[i]: one launch per position
__global__ __launch_bounds__(kChainThreads) void chain_forward(DevTable d, StepView sv,
                                                               const float *__restrict__ tree, int i,
                                                               float *__restrict__ va,
                                                               int32_t *__restrict__ ea)
{
    chain_msg_step(d, sv, tree, i, false, va, ea);
}

// b_i = M_i (b_{i+1} 2^-e'_{i+1}), e'_{i+1} into eb[i+1]: one launch per
// position, i = L-1 .. 0
__global__ __launch_bounds__(kChainThreads) void chain_backward_msg(DevTable d, StepView sv,
                                                                    const float *__restrict__ tree,
                                                                    int i, float *__restrict__ vb,
                                                                    int32_t *__restrict__ eb)
{
    chain_msg_step(d, sv, tree, i, true, vb, eb);
}

// b_L = 1 on the accepting states
__global__ void chain_binit(DevTable d, StepView sv, float *__restrict__ vb)
{
    const int b = blockIdx.y;
    const int a = blockIdx.x * blockDim.x + threadIdx.x;
    if (a >= sv.Sp) return;
    bool acc = false;
    for (int k = 0; k < d.n_acc; ++k) acc |= d.acc[k] == a;
    vb[((size_t)b * (sv.Lpad + 1) + sv.L) * sv.Sp + a] = acc ? 1.f : 0.f;
}

// The messages' step exponents become each vector's own exponent, as the
// marginal writer reads them: alpha_i = a_i 2^(e_0 + .. + e_{i-1}) and
// beta_i = b_i 2^(e'_{i+1} + .. + e'_L); kNeg from a vanished vector on.
// One thread per row.
__global__ void chain_cumexp(StepView sv, int32_t *__restrict__ ea, int32_t *__restrict__ eb)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= sv.B) return;
    int32_t *fa = ea + (size_t)b * (sv.Lpad + 1);
    int32_t *fb = eb + (size_t)b * (sv.Lpad + 1);
    int acc = 0;
    bool dead = false;
    for (int i = 0; i <= sv.L; ++i) {
        const int step = i < sv.L ? fa[i] : 0;
        fa[i] = dead ? kNeg : acc;
        if (i < sv.L) {
            if (step <= kNeg) dead = true;
            else acc += step;
        }
    }
    acc = 0;
    dead = false;
    for (int i = sv.L; i >= 0; --i) {
        const int step = i >= 1 ? fb[i] : 0;
        fb[i] = dead ? kNeg : acc;
        if (i >= 1) {
            if (step <= kNeg) dead = true;
            else acc += step;
        }
    }
}

// log Z per row (one wavefront); infeasible rows flagged
__global__ __launch_bounds__(64) void chain_logz(DevTable d, StepView sv, const float *__restrict__ va,
                                                 const int32_t *__restrict__ ea,
                                                 double *__restrict__ logZ, int32_t *__restrict__ status)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    const float *aL = va + ((size_t)b * (sv.Lpad + 1) + sv.L) * sv.Sp;
    double s = 0.0;
    for (int k = lane; k < d.n_acc; k += 64) s += (double)aL[d.acc[k]];
    s = wave_sum_d(s);
    if (lane == 0) {
        long long es = 0;
        bool dead = false;
        for (int i = 0; i < sv.L; ++i) {
            const int e = ea[(size_t)b * (sv.Lpad + 1) + i];
            dead |= e <= kNeg;
            es += e;
        }
        const bool ok = status[b] == 0 && !dead && s > 0.0;
        logZ[b] = ok ? (double)es * 0.69314718055994530942 + log(s) : -INFINITY;
        if (!ok && status[b] == 0) atomicOr(&status[b], (int)FA_ROW_INFEASIBLE);
    }
}

// backward sampling of one row (one wavefront, L + 1 dependent draws); each
// position's pair is recorded for the token draws
__global__ __launch_bounds__(64) void chain_backward(DevTable d, StepView sv,
                                                     const float *__restrict__ tree,
                                                     const float *__restrict__ va, uint64_t seed,
                                                     int32_t *__restrict__ zc,
                                                     int32_t *__restrict__ tpair,
                                                     uint32_t *__restrict__ tdbit,
                                                     int32_t *__restrict__ status)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    const int Sp = sv.Sp, L = sv.L;
    const uint32_t lev = (uint32_t)sv.K + 2u;
    int32_t *z = zc + (size_t)b * (sv.Lpad + 1);
    for (int k = lane; k <= L; k += 64) z[k] = -1;
    for (int k = lane; k < L; k += 64) {
        tpair[(size_t)b * L + k] = -1;
        tdbit[(size_t)b * L + k] = 0u;
    }
    if (status[b] != 0) return;
    const float *aL = va + ((size_t)b * (sv.Lpad + 1) + L) * Sp;
    int j = wave_icdf(d.n_acc, philox_u01(seed, (uint32_t)(sv.b0 + b), lev, (uint32_t)L), lane,
                      [&](int k) { return aL[d.acc[k]]; });
    int zn = j >= 0 ? d.acc[j] : -1;
    if (lane == 0) z[L] = zn;
    for (int i = L - 1; i >= 0 && zn >= 0; --i) {
        const float *ai = va + ((size_t)b * (sv.Lpad + 1) + i) * Sp;
        const int h = sv.Lpad + i;
        const float *M = sv.mat_ptr(tree, b, h);
        const bool tr = stored_transposed(h);
        const int zi = wave_icdf(d.S, philox_u01(seed, (uint32_t)(sv.b0 + b), lev, (uint32_t)i), lane, [&](int a) {
            const float m = tr ? M[(size_t)zn * Sp + a] : M[(size_t)a * Sp + zn];
            return ai[a] * m;
        });
        if (lane == 0) {
            z[i] = zi;
            if (zi >= 0) put_pair(d, zi, zn, tpair + (size_t)b * L + i, tdbit + (size_t)b * L + i);
        }
        zn = zi;
    }
    if (lane == 0 && zn < 0) atomicOr(&status[b], (int)FA_ROW_UNDERFLOW);
}

// L = 0: the empty string, accepted when the start state is accepting
__global__ void chain_empty(DevTable d, int B, double *__restrict__ logZ,
                           int32_t *__restrict__ states, int32_t *__restrict__ status)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    bool acc = false;
    for (int a = 0; a < d.n_acc; ++a) acc |= d.acc[a] == d.start;
    const bool ok = acc && status[b] == 0;
    logZ[b] = ok ? 0.0 : -INFINITY;
    states[b] = ok ? d.orig[d.start] : -1;
    if (!acc) atomicOr(&status[b], (int)FA_ROW_INFEASIBLE);
}

}  // namespace

int launch_chain_sample(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                        uint64_t seed, double *logZ, int32_t *states, int32_t *tokens,
                        uint8_t *ws, const WsLayout &w, int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (g.L == 0) {
        chain_empty<<<(g.B + 255) / 256, 256, 0, st>>>(d, g.B, logZ, states, status);
        return (int)hipGetLastError();
    }
    StepView sv = step_view(g);
    float *va = (float *)(ws + w.va);
    int32_t *ea = (int32_t *)(ws + w.ea);
    chain_init<<<dim3((g.Sp + 255) / 256, g.B), 256, 0, st>>>(d, sv, va);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const size_t lds = (size_t)g.Sp * sizeof(float);
    if (lds > 48 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chain_forward),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
    }
    const dim3 fgrid(g.Sp / kChainCols, g.B);
    for (int i = 0; i < g.L; ++i) {
        chain_forward<<<fgrid, kChainThreads, lds, st>>>(d, sv, tree, i, va, ea);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    chain_logz<<<g.B, 64, 0, st>>>(d, sv, va, ea, logZ, status);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    chain_backward<<<g.B, 64, 0, st>>>(d, sv, tree, va, seed, (int32_t *)(ws + w.zc),
                                       (int32_t *)(ws + w.tpair), (uint32_t *)(ws + w.tdbit),
                                       status);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    return launch_sample_tokens(d, g, p, seed, states, tokens, ws, w, false, status, stream);
}

int launch_chain_sample_marginals(const DevTable &d, const Geometry &g, const float *p,
                                  const float *tree, uint64_t seed, int32_t conf_mode,
                                  double *logZ, int32_t *states, int32_t *tokens, float *q,
                                  float *conf, uint8_t *ws, const WsLayout &w, int32_t *status,
                                  void *stream)
{
    int rc = launch_chain_sample(d, g, p, tree, seed, logZ, states, tokens, ws, w, status, stream);
    if (rc || g.L == 0) return rc;
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    float *vb = (float *)(ws + w.vb);
    int32_t *ea = (int32_t *)(ws + w.ea), *eb = (int32_t *)(ws + w.eb);
    chain_binit<<<dim3((g.Sp + 255) / 256, g.B), 256, 0, st>>>(d, sv, vb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const size_t lds = (size_t)g.Sp * sizeof(float);
    if (lds > 48 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chain_backward_msg),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
    }
    const dim3 grid(g.Sp / kChainCols, g.B);
    for (int i = g.L - 1; i >= 0; --i) {
        chain_backward_msg<<<grid, kChainThreads, lds, st>>>(d, sv, tree, i, vb, eb);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    chain_cumexp<<<(g.B + 63) / 64, 64, 0, st>>>(sv, ea, eb);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    return launch_marg_from_messages(d, g, p, logZ, tokens, conf_mode, q, conf, ws, w, status,
                                     stream);
}

}  // namespace fa
