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

// One workgroup per row.  Masked positions (not committed, a sampled token)
// and their confidence (NaN read as -inf) go to LDS; each masked position's
// rank is the number of masked positions with a larger confidence, or an
// equal one and a lower index, and it is committed when its rank is below k.
// A flagged row commits nothing.
__global__ __launch_bounds__(kCommitThreads) void commit_select(
    int L, const float *__restrict__ conf, const int32_t *__restrict__ tokens, int steps_left,
    int32_t *__restrict__ committed, int32_t *__restrict__ fresh,
    const int32_t *__restrict__ status)
{
    extern __shared__ float cs[];  // [L] confidence | [L] masked flags
    int *mk = reinterpret_cast<int *>(cs + L);
    __shared__ int sh_n[kCommitThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t row = (size_t)b * L;
    const bool flagged = status && status[b] != 0;
    int n = 0;
    for (int i = tid; i < L; i += kCommitThreads) {
        const bool m = !flagged && committed[row + i] == 0 && tokens[row + i] >= 0;
        const float c = conf[row + i];
        cs[i] = c == c ? c : -INFINITY;
        mk[i] = m;
        n += m;
    }
    n = wave_sum_i(n);
    if (lane == 0) sh_n[wave] = n;
    __syncthreads();
    n = 0;
    for (int w = 0; w < kCommitThreads / 64; ++w) n += sh_n[w];
    const int k = steps_left <= 1 ? n : (n + steps_left - 1) / steps_left;
    for (int i = tid; i < L; i += kCommitThreads) {
        int take = 0;
        if (mk[i]) {
            const float ci = cs[i];
            int rank = 0;
            for (int j = 0; j < L; ++j)
                rank += mk[j] && (cs[j] > ci || (cs[j] == ci && j < i));
            take = rank < k;
        }
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
    const size_t lds = (size_t)L * (sizeof(float) + sizeof(int));
    hipError_t e;
    if (lds > 48 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&commit_select),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
    }
    commit_select<<<B, kCommitThreads, lds, st>>>(L, conf, tokens, steps_left, committed, fresh,
                                                  status);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    commit_onehot<<<dim3(L, B), kCommitThreads, 0, st>>>(L, V, fresh, tokens, p);
    return (int)hipGetLastError();
}

}  // namespace fa
