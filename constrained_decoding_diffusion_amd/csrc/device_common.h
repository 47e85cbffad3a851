// Device helpers shared by the gfx950 kernels: the counter-based generator,
// power-of-two exponent arithmetic, wavefront-64 reductions and scans, and
// the tree/meta indexing of a step.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_internal.h"

namespace fa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- Philox
// Philox4x32-10 from its published description (Salmon et al., "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC'11): ten rounds; in each, words 0
// and 2 are multiplied by two fixed odd constants, the high product halves
// are mixed with words 1 and 3 and the round key, the low halves move to
// words 1 and 3; the key advances by two Weyl increments between rounds.
// The first output word gives u = (r0 >> 8) * 2^-24, exact in fp32.
__device__ inline float philox_u01(uint64_t seed, uint32_t b, uint32_t level, uint32_t node)
{
    uint32_t c0 = b, c1 = level, c2 = node, c3 = 0u;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t m0 = 0xD2511F53u, m1 = 0xCD9E8D57u;
        uint32_t hi0 = __umulhi(m0, c0), lo0 = m0 * c0;
        uint32_t hi1 = __umulhi(m1, c2), lo1 = m1 * c2;
        uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return (float)(c0 >> 8) * (1.0f / 16777216.0f);
}

// ---------------------------------------------------------- exponents
// e such that x = f 2^e with f in [0.5, 1); kNeg for x == 0.
__device__ inline int fexp(float x)
{
    if (!(x > 0.f)) return kNeg;
    int e;
    frexpf(x, &e);
    return e;
}

// a float4 load with the non-temporal hint: for streamed inputs read once
// per kernel (p), which then do not displace cached tables; on gfx950 a plain
// read of p ran at 5.9 TB/s, a non-temporal one at 6.8 TB/s
__device__ inline float4 load_nt(const float *src)
{
    typedef float f32x4n __attribute__((ext_vector_type(4)));
    const f32x4n x = __builtin_nontemporal_load(reinterpret_cast<const f32x4n *>(src));
    return make_float4(x.x, x.y, x.z, x.w);
}

// sum of two exponents, saturating at kNeg (an all-zero row or column)
__device__ inline int add_exp(int a, int b)
{
    if (a <= kNeg || b <= kNeg) return kNeg;
    int s = a + b;
    return s < kNeg ? kNeg : s;
}

__device__ inline float scale2(float x, int e)
{
    if (x == 0.f) return 0.f;
    if (e < -400) return 0.f;
    if (e > 400) e = 400;
    return ldexpf(x, e);
}

// ------------------------------------------------------- wave primitives
// orders LDS traffic between the lanes of one wavefront
__device__ inline void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ inline double wave_sum_d(double x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// mantissa of x in [0.5, 1) (x > 0): x = mant(x) 2^e
__device__ inline float mant(float x)
{
    int e;
    return frexpf(x, &e);
}

// index of the pair (a, c) in the table's row-sorted pair list, or -1
__device__ inline int pair_index(const DevTable &d, int a, int c)
{
    if (a < 0 || c < 0) return -1;
    int lo = d.row_ptr[a], hi = d.row_ptr[a + 1];
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (d.pair_b[mid] < c) lo = mid + 1;
        else hi = mid;
    }
    return (lo < d.row_ptr[a + 1] && d.pair_b[lo] == c) ? lo : -1;
}

__device__ inline int wave_sum_i(int x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ inline int wave_max_i(int x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}

__device__ inline float wave_max_f(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// inclusive scan over the 64 lanes
__device__ inline float wave_incl_scan(float x, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        float y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

__device__ inline double wave_incl_scan_d(double x, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        double y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

// -------------------------------------------------------------- indexing
struct StepView {
    int32_t B, L, Lpad, K, Sp;
    int32_t b0;  // batch row of this launch's row 0: draws are keyed by b0 + b
    size_t mat;
    // folded leaf pair values when the table keeps no dense leaves (the
    // leaf-level midpoint draws read them instead), else nullptr
    const float *pvf = nullptr;
    __device__ size_t node(int b, int h) const { return (size_t)b * 2 * Lpad + h; }
    __device__ float *mat_ptr(float *tree, int b, int h) const { return tree + node(b, h) * mat; }
    __device__ const float *mat_ptr(const float *tree, int b, int h) const
    {
        return tree + node(b, h) * mat;
    }
    // which: 0 row scale ro, 1 column scale co, 2 row fold normalizer rf
    __device__ int32_t *meta_ptr(int32_t *meta, int b, int h, int which) const
    {
        return meta + (node(b, h) * 3 + which) * (size_t)Sp;
    }
    __device__ const int32_t *meta_ptr(const int32_t *meta, int b, int h, int which) const
    {
        return meta + (node(b, h) * 3 + which) * (size_t)Sp;
    }
};

inline StepView step_view(const Geometry &g)
{
    StepView s;
    s.B = g.B;
    s.b0 = g.b0;
    s.L = g.L;
    s.Lpad = g.Lpad;
    s.K = g.K;
    s.Sp = g.Sp;
    s.mat = g.mat;
    return s;
}

// stored orientation of heap node h: odd nodes >= 3 (right children) are
// stored transposed
__host__ __device__ inline bool stored_transposed(int h) { return (h & 1) && h >= 3; }

}  // namespace fa
