// Span tree: bottom-up 2^k-span transition products, level by level, as
// batched fp32 MFMA matrix products (paperfeed "The scan trick: log-depth
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
#include "device_common.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;        // output tile (rows and columns)
constexpr int kBK = 32;          // K step staged in LDS
constexpr int kLdk = kBK + 4;    // padded LDS row (floats)
constexpr int kGemmThreads = 256;

__global__ void tree_init_rf(StepView sv, int32_t *__restrict__ meta)
{
    // rf of every internal node of every row: kNeg (filled by atomicMax)
    const size_t per_row = (size_t)(sv.Lpad - 1) * sv.Sp;
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

__device__ inline void load8(const float *src, float4 &a, float4 &b)
{
    a = *reinterpret_cast<const float4 *>(src);
    b = *reinterpret_cast<const float4 *>(src + 4);
}

__device__ inline float4 fold4(float4 x, int4 c, int rfrow)
{
    x.x = scale2(x.x, c.x - rfrow);
    x.y = scale2(x.y, c.y - rfrow);
    x.z = scale2(x.z, c.z - rfrow);
    x.w = scale2(x.w, c.w - rfrow);
    return x;
}

// One 64x64 output tile of D = X Y^T for node n of row b.
__global__ __launch_bounds__(kGemmThreads) void span_gemm(StepView sv, float *__restrict__ tree,
                                                          int32_t *__restrict__ meta, int n0,
                                                          int nn)
{
    const int Sp = sv.Sp;
    const int tiles = Sp / kTile;
    const int tm = (blockIdx.x / tiles) * kTile, tn = (blockIdx.x % tiles) * kTile;
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

    __shared__ __align__(16) float Fs[kTile][kLdk];
    __shared__ __align__(16) float Gs[kTile][kLdk];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = tid >> 2, lk = (tid & 3) * 8;
    const int rfFrow = rfF[tm + lrow], rfGrow = rfG[tn + lrow];
    const float *Frow = F + (size_t)(tm + lrow) * Sp;
    const float *Grow = G + (size_t)(tn + lrow) * Sp;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
    const int l32 = lane & 31, half = lane >> 5;

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    float4 f0, f1, g0, g1;
    load8(Frow + lk, f0, f1);
    load8(Grow + lk, g0, g1);
    for (int k0 = 0; k0 < Sp; k0 += kBK) {
        const int4 cf0 = *reinterpret_cast<const int4 *>(coF + k0 + lk);
        const int4 cf1 = *reinterpret_cast<const int4 *>(coF + k0 + lk + 4);
        const int4 cg0 = *reinterpret_cast<const int4 *>(coG + k0 + lk);
        const int4 cg1 = *reinterpret_cast<const int4 *>(coG + k0 + lk + 4);
        __syncthreads();
        *reinterpret_cast<float4 *>(&Fs[lrow][lk]) = fold4(f0, cf0, rfFrow);
        *reinterpret_cast<float4 *>(&Fs[lrow][lk + 4]) = fold4(f1, cf1, rfFrow);
        *reinterpret_cast<float4 *>(&Gs[lrow][lk]) = fold4(g0, cg0, rfGrow);
        *reinterpret_cast<float4 *>(&Gs[lrow][lk + 4]) = fold4(g1, cg1, rfGrow);
        __syncthreads();
        if (k0 + kBK < Sp) {
            load8(Frow + k0 + kBK + lk, f0, f1);
            load8(Grow + k0 + kBK + lk, g0, g1);
        }
#pragma unroll
        for (int t = 0; t < kBK / 2; t += 4) {
            const float4 a = *reinterpret_cast<const float4 *>(&Fs[wr + l32][half * (kBK / 2) + t]);
            const float4 c = *reinterpret_cast<const float4 *>(&Gs[wc + l32][half * (kBK / 2) + t]);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, c.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, c.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, c.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, c.w, acc, 0, 0, 0);
        }
    }
    // epilogue: store, row fold normalizer, outer scales
    const int j = tn + wc + l32;
    const int coDj = add_exp(roG[j], rfG[j]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = tm + wr + (r >> 2) * 8 + half * 4 + (r & 3);
        const float x = acc[r];
        D[(size_t)i * Sp + j] = x;
        int e = (x > 0.f && coDj > kNeg) ? fexp(x) + coDj : kNeg;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) e = max(e, __shfl_xor(e, o));
        if (l32 == 0 && e > kNeg) atomicMax(&rfD[i], e);
    }
    if (blockIdx.x % tiles == 0 && tid < kTile) roD[tm + tid] = add_exp(roF[tm + tid], rfF[tm + tid]);
    if (blockIdx.x / tiles == 0 && tid < kTile) coD[tn + tid] = add_exp(roG[tn + tid], rfG[tn + tid]);
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

}  // namespace

int launch_span_tree(const DevTable &d, const Geometry &g, float *tree, int32_t *meta,
                     double *logZ, int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (g.L == 0) {
        tree_logz_empty<<<(g.B + 255) / 256, 256, 0, st>>>(d, g.B, logZ, status);
        return (int)hipGetLastError();
    }
    StepView sv = step_view(g);
    if (g.Lpad > 1) {
        const size_t total = (size_t)g.B * (g.Lpad - 1) * g.Sp;
        const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
        tree_init_rf<<<blocks, 256, 0, st>>>(sv, meta);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    const int tiles = g.Sp / kTile;
    for (int k = 1; k <= g.K; ++k) {
        const int n0 = g.Lpad >> k, nn = n0;
        dim3 grid(tiles * tiles, g.B * nn);
        span_gemm<<<grid, kGemmThreads, 0, st>>>(sv, tree, meta, n0, nn);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    tree_logz<<<g.B, 64, 0, st>>>(d, sv, tree, meta, logZ, status);
    return (int)hipGetLastError();
}

}  // namespace fa
