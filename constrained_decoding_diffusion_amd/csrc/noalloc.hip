// fa_span_tree_noalloc: the span tree of fa_span_tree for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops and
// harnesses that forbid hipMalloc).  The only scratch memory the span tree
// uses, the split-K partial tiles of its upper levels, lives here in a
// file-scope device array instead of the caller's workspace.  Every other
// buffer is the caller's, as in fa_span_tree, and the kernels are the same.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "fa_internal.h"

using namespace fa;

namespace {

// Each GPU the library runs on holds its own copy of this array until the
// process ends.  Host code never passes the array's name to a kernel (on
// the host it is a stand-in, not a device address): it takes the address of
// the current device's copy from hipGetSymbolAddress once per device and
// passes that.
constexpr size_t kScratchBytes = FA_SPAN_TREE_NOALLOC_MAX_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[kMaxDevices] = {};

// address of the current device's copy of `scratch`, looked up on the first
// call on that device (with that device current)
int scratch_of_current_device(uint8_t **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FA_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_ETOOBIG;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_EHIP;
        g_scratch_ptr[dev] = (uint8_t *)ptr;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

}  // namespace

extern "C" int fa_span_tree_noalloc(const fa_table *t, int32_t B, int32_t L, float *tree,
                                    int32_t *meta, double *logZ, int32_t *row_status,
                                    fa_stream_t stream)
{
    if (!t) return FA_EINVAL;
    // a first level formed from the pair values reads what this step's
    // fa_build_transitions left in the caller's workspace: fa_span_tree only
    if (t->h.first_sparse || t->h.first_pairs) return FA_EINVAL;
    if (!t->h.dev) return FA_ESTATE;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    if (B == 0) return FA_OK;
    if (!logZ || !row_status) return FA_EINVAL;
    if (L > 0 && (!tree || !meta)) return FA_EINVAL;
    // the partial tiles go to offset 0 of the scratch array; nothing else of
    // the workspace is touched on a table with a dense first level.  The
    // split rule bounds them by 2^20 floats (see fa.h); the check guards
    // that bound should the rule change.  Row chunks run in turn on the
    // stream and reuse the array.
    uint8_t *ptr = nullptr;
    // the live-state lists need workspace: this form runs the products over
    // every state (the same results)
    DevTable d = t->h.device_view();
    d.live_states = 0;
    for (int32_t k = 0; k < ck.count; ++k) {
        const int32_t b0 = k * ck.rows;
        Geometry g;
        make_geometry(t->h, std::min(ck.rows, B - b0), L, &g);
        g.b0 = b0;
        size_t kp = 0;
        for (int level = 1; level <= g.K; ++level) {
            const int s = tree_ksplit(g, level);
            if (s > 1) kp = std::max(kp, (size_t)g.B * (g.Lpad >> level) * s * g.mat * sizeof(float));
        }
        if (kp > kScratchBytes) return FA_ETOOBIG;
        if (!ptr)
            if (int rc = scratch_of_current_device(&ptr)) return rc;
        WsLayout ws{};
        ws.kpart = 0;
        const size_t mrow = 2 * (size_t)g.Lpad;
        const int rc = launch_span_tree(d, g, tree ? tree + mrow * g.mat * b0 : tree,
                                        meta ? meta + mrow * 3 * g.Sp * b0 : meta, ptr, ws,
                                        logZ + b0, row_status + b0, stream);
        if (rc) return FA_EHIP;
    }
    return FA_OK;
}
