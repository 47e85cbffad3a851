// Measurement hook, not part of the method: plain streaming kernels whose
// rates are the achievable HBM ceilings the step's kernels are compared
// with (a read-only pass, and a copy).  Each workgroup walks its own
// contiguous chunk as float4 with non-temporal loads (and stores): the read
// with 256 threads and eight loads in flight per thread, the copy with 1024
// threads and four (the fastest of the patterns measured: grid-stride,
// per-workgroup chunks, 256 to 1024 threads, 4 to 16 loads in flight, with
// and without the non-temporal hints; the read rate does not depend on the
// form, the copy is about 10% faster with 1024 threads than with 256).
#include "device_common.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;  // float4 loads in flight per thread
constexpr int kCopyThreads = 1024;
constexpr int kCopyInFlight = 4;

typedef float f32x4p __attribute__((ext_vector_type(4)));

// every float4 of src read once (streaming loads), each workgroup over its
// own contiguous chunk; one partial sum per workgroup goes to dst so that
// the loads are live
__global__ __launch_bounds__(kProbeThreads) void probe_read(const f32x4p *__restrict__ src,
                                                            size_t n4, float *__restrict__ dst)
{
    const size_t per = (n4 + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n4 ? lo + per : n4;
    f32x4p acc = {0.f, 0.f, 0.f, 0.f};
    size_t i = lo + threadIdx.x;
    for (; i + (kProbeInFlight - 1) * kProbeThreads < hi; i += kProbeInFlight * kProbeThreads) {
        f32x4p v[kProbeInFlight];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) acc += v[u];
    }
    for (; i < hi; i += kProbeThreads) acc += __builtin_nontemporal_load(src + i);
    float a = (acc.x + acc.y) + (acc.z + acc.w);
    __shared__ float part[kProbeThreads / kWave];
    for (int o = kWave / 2; o > 0; o >>= 1) a += __shfl_xor(a, o);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.f;
        for (int k = 0; k < kProbeThreads / kWave; ++k) s += part[k];
        dst[blockIdx.x] = s;
    }
}

// dst = src over contiguous chunks per workgroup, streaming loads and stores
__global__ __launch_bounds__(kCopyThreads) void probe_copy(const f32x4p *__restrict__ src,
                                                           f32x4p *__restrict__ dst, size_t n4)
{
    const size_t per = (n4 + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n4 ? lo + per : n4;
    size_t i = lo + threadIdx.x;
    for (; i + (kCopyInFlight - 1) * kCopyThreads < hi; i += kCopyInFlight * kCopyThreads) {
        f32x4p v[kCopyInFlight];
#pragma unroll
        for (int u = 0; u < kCopyInFlight; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * kCopyThreads);
#pragma unroll
        for (int u = 0; u < kCopyInFlight; ++u)
            __builtin_nontemporal_store(v[u], dst + i + u * kCopyThreads);
    }
    for (; i < hi; i += kCopyThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace
}  // namespace fa

using namespace fa;

extern "C" int fa_probe_bandwidth(int32_t mode, const void *src, void *dst, size_t bytes,
                                  int32_t blocks, fa_stream_t stream)
{
    if (!src || !dst || blocks < 1 || blocks > (1 << 20)) return FA_EINVAL;
    if ((bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return FA_EINVAL;
    const size_t n4 = bytes / 16;
    hipStream_t st = (hipStream_t)stream;
    if (mode == FA_PROBE_READ) {
        probe_read<<<blocks, kProbeThreads, 0, st>>>((const f32x4p *)src, n4, (float *)dst);
    } else if (mode == FA_PROBE_COPY) {
        probe_copy<<<blocks, kCopyThreads, 0, st>>>((const f32x4p *)src, (f32x4p *)dst, n4);
    } else {
        return FA_EINVAL;
    }
    return hipGetLastError() == hipSuccess ? FA_OK : FA_EHIP;
}
