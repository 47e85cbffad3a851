// The remasking step between denoising steps (papernotes 关键设计 3: the
// constrained marginal of a position's sampled token is the confidence that
// decides which positions are committed; paperfeed "Two immediate bonuses":
// LLaDA commits its highest-probability positions, Dream its lowest-entropy
// ones).  Per row, of the n positions still masked, the k = ceil(n /
// steps_left) with the largest confidence (ties: the lower position first)
// are committed to their sampled tokens: committed[b][i] = 1, and p[b][i][.]
// becomes one-hot at the token, which is how the next step sees them.
#include "device_common.h"

namespace fa {
namespace {

constexpr int kCommitThreads = 256;

// One workgroup per row.  Each position gets a 64-bit key: for a masked
// position (not committed, a sampled token) the confidence mapped to an
// order-preserving integer and complemented (so larger confidence sorts
// first; NaN is read as -inf) above the position (so ties go to the lower
// position), for any other position all ones.  The keys are sorted in LDS
// by a bitonic network over the next power of two >= L (O(L log^2 L)), and
// the first k keys name the committed positions.  A flagged row commits
// nothing.
__device__ inline uint32_t ordered_bits(float c)
{
    const uint32_t u = __float_as_uint(c == c ? c : -INFINITY);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending as c ascends
}

__global__ __launch_bounds__(kCommitThreads) void commit_select(
    int L, int Lp2, const float *__restrict__ conf, const int32_t *__restrict__ tokens,
    int steps_left, int32_t *__restrict__ committed, int32_t *__restrict__ fresh,
    const int32_t *__restrict__ status)
{
    extern __shared__ unsigned long long keys[];  // [Lp2] keys | [L] selected flags
    int *sel = reinterpret_cast<int *>(keys + Lp2);
    __shared__ int sh_n[kCommitThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t row = (size_t)b * L;
    const bool flagged = status && status[b] != 0;
    int n = 0;
    for (int i = tid; i < Lp2; i += kCommitThreads) {
        unsigned long long key = ~0ull;
        if (i < L) {
            const bool m = !flagged && committed[row + i] == 0 && tokens[row + i] >= 0;
            if (m) key = ((unsigned long long)(~ordered_bits(conf[row + i])) << 32) | (uint32_t)i;
            n += m;
            sel[i] = 0;
        }
        keys[i] = key;
    }
    n = wave_sum_i(n);
    if (lane == 0) sh_n[wave] = n;
    __syncthreads();
    n = 0;
    for (int w = 0; w < kCommitThreads / 64; ++w) n += sh_n[w];
    const int k = steps_left <= 1 ? n : (n + steps_left - 1) / steps_left;
    // bitonic sort, ascending: stage (size, stride); each thread takes the
    // pairs (i, i ^ stride) with i < i ^ stride
    for (int size = 2; size <= Lp2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < Lp2 / 2; t += kCommitThreads) {
                const int i = 2 * t - (t & (stride - 1));  // bit `stride` of i clear
                const int j = i + stride;
                const bool up = (i & size) == 0;
                const unsigned long long a = keys[i], c = keys[j];
                if ((a > c) == up) {
                    keys[i] = c;
                    keys[j] = a;
                }
            }
            __syncthreads();
        }
    }
    for (int r = tid; r < k; r += kCommitThreads) sel[(int)(keys[r] & 0xffffffffu)] = 1;
    __syncthreads();
    for (int i = tid; i < L; i += kCommitThreads) {
        const int take = sel[i];
        fresh[row + i] = take;
        if (take) committed[row + i] = 1;
    }
}

// p rows of the positions committed by commit_select: one-hot at the token
__global__ __launch_bounds__(kCommitThreads) void commit_onehot(
    int L, int V, const int32_t *__restrict__ fresh, const int32_t *__restrict__ tokens,
    float *__restrict__ p)
{
    const size_t pos = (size_t)blockIdx.y * L + blockIdx.x;
    if (!fresh[pos]) return;
    const int tok = tokens[pos];
    float *row = p + pos * V;
    if ((V & 3) == 0 && ((uintptr_t)row & 15) == 0) {
        float4 *r4 = reinterpret_cast<float4 *>(row);
        for (int k = threadIdx.x; k < V / 4; k += kCommitThreads) {
            const int v = 4 * k;
            r4[k] = make_float4(v == tok ? 1.f : 0.f, v + 1 == tok ? 1.f : 0.f,
                                v + 2 == tok ? 1.f : 0.f, v + 3 == tok ? 1.f : 0.f);
        }
    } else {
        for (int v = threadIdx.x; v < V; v += kCommitThreads) row[v] = v == tok ? 1.f : 0.f;
    }
}

}  // namespace

int launch_commit(int B, int L, int V, const float *conf, const int32_t *tokens, int steps_left,
                  int32_t *committed, int32_t *fresh, float *p, const int32_t *status,
                  void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    int Lp2 = 1;
    while (Lp2 < L) Lp2 <<= 1;
    const size_t lds = (size_t)Lp2 * sizeof(unsigned long long) + (size_t)L * sizeof(int);
    hipError_t e;
    if (lds > 48 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&commit_select),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
    }
    commit_select<<<B, kCommitThreads, lds, st>>>(L, Lp2, conf, tokens, steps_left, committed,
                                                  fresh, status);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    commit_onehot<<<dim3(L, B), kCommitThreads, 0, st>>>(L, V, fresh, tokens, p);
    return (int)hipGetLastError();
}

}  // namespace fa
