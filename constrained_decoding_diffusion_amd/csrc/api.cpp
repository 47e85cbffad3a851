// C-ABI entry points of one constrained denoising step: argument checks,
// geometry, workspace layout, then the kernel launchers.  Nothing here
// allocates device memory or synchronizes.
#include <hip/hip_runtime_api.h>

#include "fa_internal.h"

using namespace fa;

namespace {

int ready(const fa_table *t)
{
    if (!t) return FA_EINVAL;
    if (!t->h.dev) return FA_ESTATE;
    return FA_OK;
}

int hip_rc(int e) { return e == 0 ? FA_OK : FA_EHIP; }

bool conf_mode_ok(int32_t m)
{
    return m == FA_CONF_PROB || m == FA_CONF_NEGENT || m == FA_CONF_UNCONSTRAINED;
}

// the score whose path computes q: the unconstrained score runs the PROB path
int32_t base_mode(int32_t m) { return m == FA_CONF_UNCONSTRAINED ? FA_CONF_PROB : m; }

int sample_marginals_base(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                          const int32_t *meta, const double *logZ, uint64_t seed,
                          int32_t conf_mode, int32_t *states, int32_t *tokens, float *q,
                          float *conf, uint8_t *wb, const WsLayout &w, int32_t *row_status,
                          fa_stream_t stream);

struct ProfHook {
    int which = FA_PROF_NONE;
    hipEvent_t start = nullptr, stop = nullptr;
};
thread_local ProfHook g_prof;

}  // namespace

namespace fa {

int prof_mark(int which, bool begin, void *stream)
{
    if (which == FA_PROF_NONE || g_prof.which != which) return 0;
    return (int)hipEventRecord(begin ? g_prof.start : g_prof.stop, (hipStream_t)stream);
}

}  // namespace fa

extern "C" int fa_profile_kernel(int32_t which, void *start_event, void *stop_event)
{
    if (which < FA_PROF_NONE || which > FA_PROF_MARG_Q) return FA_EINVAL;
    if (which != FA_PROF_NONE && (!start_event || !stop_event)) return FA_EINVAL;
    g_prof.which = which;
    g_prof.start = (hipEvent_t)start_event;
    g_prof.stop = (hipEvent_t)stop_event;
    return FA_OK;
}

extern "C" int fa_table_upload(fa_table *t, void *dev_buf, size_t bytes, fa_stream_t stream)
{
    if (!t || !dev_buf || bytes < t->h.image.size()) return FA_EINVAL;
    if (((uintptr_t)dev_buf & 255u) != 0) return FA_EINVAL;
    hipError_t e = hipMemcpyAsync(dev_buf, t->h.image.data(), t->h.image.size(),
                                  hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return FA_EHIP;
    t->h.dev = dev_buf;
    t->h.dev_bytes = bytes;
    return FA_OK;
}

extern "C" int fa_build_transitions(const fa_table *t, const float *p, int32_t B, int32_t L,
                                    float *tree, int32_t *meta, void *ws, size_t ws_bytes,
                                    int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    if (B == 0 || L == 0) return FA_OK;
    WsLayout w = ws_layout(t->h, g);
    if (!p || !tree || !meta || !row_status || !ws || ws_bytes < w.total) return FA_EINVAL;
    return hip_rc(launch_build_transitions(t->h.device_view(), g, p, tree, meta, (uint8_t *)ws, w,
                                           row_status, stream));
}

extern "C" int fa_span_tree(const fa_table *t, int32_t B, int32_t L, float *tree, int32_t *meta,
                            void *ws, size_t ws_bytes, double *logZ, int32_t *row_status,
                            fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    if (B == 0) return FA_OK;
    if (!logZ || !row_status) return FA_EINVAL;
    WsLayout w = ws_layout(t->h, g);
    if (L > 0 && (!tree || !meta || !ws || ws_bytes < w.total)) return FA_EINVAL;
    return hip_rc(launch_span_tree(t->h.device_view(), g, tree, meta, (uint8_t *)ws, w, logZ,
                                   row_status, stream));
}

extern "C" int fa_sample(const fa_table *t, const float *p, int32_t B, int32_t L, const float *tree,
                         const int32_t *meta, uint64_t seed, int32_t *states, int32_t *tokens,
                         void *ws, size_t ws_bytes, int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    if (B == 0) return FA_OK;
    WsLayout w = ws_layout(t->h, g);
    if (!states || !row_status || !ws || ws_bytes < w.total) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !meta || !tokens)) return FA_EINVAL;
    return hip_rc(launch_sample(t->h.device_view(), g, p, tree, meta, seed, states, tokens,
                                (uint8_t *)ws, w, row_status, stream));
}

extern "C" int fa_marginals(const fa_table *t, const float *p, int32_t B, int32_t L,
                            const float *tree, const int32_t *meta, const double *logZ,
                            const int32_t *tokens, int32_t conf_mode, float *q, float *conf,
                            void *ws, size_t ws_bytes, int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    if (!conf_mode_ok(conf_mode)) return FA_EINVAL;
    if (B == 0 || L == 0) return FA_OK;
    WsLayout w = ws_layout(t->h, g);
    if (!p || !tree || !meta || !logZ || !conf || !row_status || !ws || ws_bytes < w.total)
        return FA_EINVAL;
    if (conf_mode != FA_CONF_NEGENT && !tokens) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    // the unconstrained score takes the PROB path for q, then its own conf
    int rc2 = launch_marginals(d, g, p, tree, meta, logZ, tokens, base_mode(conf_mode), q, conf,
                               (uint8_t *)ws, w, row_status, stream);
    if (!rc2 && conf_mode == FA_CONF_UNCONSTRAINED)
        rc2 = launch_conf_unconstrained(d, g, p, tokens, row_status, conf, stream);
    return hip_rc(rc2);
}

extern "C" int fa_sample_marginals(const fa_table *t, const float *p, int32_t B, int32_t L,
                                   const float *tree, const int32_t *meta, const double *logZ,
                                   uint64_t seed, int32_t conf_mode, int32_t *states,
                                   int32_t *tokens, float *q, float *conf, void *ws,
                                   size_t ws_bytes, int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    if (!conf_mode_ok(conf_mode)) return FA_EINVAL;
    if (B == 0) return FA_OK;
    WsLayout w = ws_layout(t->h, g);
    if (!states || !row_status || !ws || ws_bytes < w.total) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !meta || !logZ || !tokens || !conf)) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    rc = sample_marginals_base(d, g, p, tree, meta, logZ, seed, base_mode(conf_mode), states,
                               tokens, q, conf, (uint8_t *)ws, w, row_status, stream);
    if (!rc && L > 0 && conf_mode == FA_CONF_UNCONSTRAINED)
        rc = launch_conf_unconstrained(d, g, p, tokens, row_status, conf, stream);
    return hip_rc(rc);
}

namespace {

// fa_sample_marginals for the PROB and NEGENT scores; returns 0 or a
// hipError_t value
int sample_marginals_base(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                          const int32_t *meta, const double *logZ, uint64_t seed,
                          int32_t conf_mode, int32_t *states, int32_t *tokens, float *q,
                          float *conf, uint8_t *wb, const WsLayout &w, int32_t *row_status,
                          fa_stream_t stream)
{
    const int32_t L = g.L;
    int rc;
    if (L == 0 || !marg_joint_ok(d, g, p, q, conf_mode, w)) {
        rc = launch_sample(d, g, p, tree, meta, seed, states, tokens, wb, w, row_status, stream);
        if (rc || L == 0) return rc;
        return launch_marginals(d, g, p, tree, meta, logZ, tokens, conf_mode, q, conf, wb, w,
                                row_status, stream);
    }
    // midpoints riding on the message pass; q with the draws' chunk sums;
    // the token draws; the confidence of the drawn tokens and the rows the
    // draws flagged
    rc = 0;
    if (g.K == 0) rc = launch_sample_states(d, g, tree, meta, seed, wb, w, row_status, stream);
    if (!rc)
        rc = launch_marg_pass(d, g, p, tree, meta, wb, w, stream, g.K >= 1, seed, row_status);
    if (!rc)
        rc = launch_marg_out(d, g, p, logZ, nullptr, conf_mode, q, conf, wb, w, 1, row_status,
                             stream, nullptr);
    if (!rc)
        rc = launch_sample_tokens(d, g, p, seed, states, tokens, wb, w, true, row_status, stream,
                                  false);
    if (!rc)
        rc = launch_marg_out(d, g, p, logZ, tokens, conf_mode, q, conf, wb, w, 2, row_status,
                             stream, states);
    return rc;
}

}  // namespace

extern "C" int fa_chain_sample(const fa_table *t, const float *p, int32_t B, int32_t L,
                               const float *tree, uint64_t seed, double *logZ, int32_t *states,
                               int32_t *tokens, void *ws, size_t ws_bytes, int32_t *row_status,
                               fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    // the chain reads every position's dense matrix
    if (t->h.leafless && L > 1) return FA_EINVAL;
    if (B == 0) return FA_OK;
    WsLayout w = ws_layout(t->h, g);
    if (!logZ || !states || !row_status || !ws || ws_bytes < w.total) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !tokens)) return FA_EINVAL;
    return hip_rc(launch_chain_sample(t->h.device_view(), g, p, tree, seed, logZ, states, tokens,
                                      (uint8_t *)ws, w, row_status, stream));
}

extern "C" int fa_map_sizes(const fa_table *t, int32_t B, int32_t L, size_t *tree_bytes,
                            size_t *ws_bytes)
{
    if (!t) return FA_EINVAL;
    if (t->h.nseg() > 0) return FA_EINVAL;  // range labels: no range-maximum structure
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    if (tree_bytes) *tree_bytes = g.tree_floats * sizeof(double);
    if (ws_bytes) *ws_bytes = map_ws_layout(t->h, g).total;
    return FA_OK;
}

extern "C" int fa_map_decode(const fa_table *t, const float *p, int32_t B, int32_t L,
                             double *tree, void *ws, size_t ws_bytes, double *logmax,
                             int32_t *states, int32_t *tokens, int32_t *row_status,
                             fa_stream_t stream)
{
    if (t && t->h.nseg() > 0) return FA_EINVAL;
    int rc = ready(t);
    if (rc) return rc;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    if (!grid_fits(g)) return FA_ETOOBIG;
    if (B == 0) return FA_OK;
    MapWs w = map_ws_layout(t->h, g);
    if (!logmax || !states || !row_status) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !tokens || !ws || ws_bytes < w.total)) return FA_EINVAL;
    return hip_rc(launch_map_decode(t->h.device_view(), g, p, tree, (uint8_t *)ws, w, logmax,
                                    states, tokens, row_status, stream));
}

extern "C" int fa_commit(int32_t B, int32_t L, int32_t V, const float *conf,
                         const int32_t *tokens, int32_t steps_left, int32_t *committed,
                         int32_t *fresh, float *p, const int32_t *row_status, fa_stream_t stream)
{
    if (B < 0 || L < 0 || V < 1 || steps_left < 1) return FA_EINVAL;
    if (L > kCommitMaxL || B > 65535) return FA_ETOOBIG;
    if (B == 0 || L == 0) return FA_OK;
    if (!conf || !tokens || !committed || !fresh || !p) return FA_EINVAL;
    return hip_rc(launch_commit(B, L, V, conf, tokens, steps_left, committed, fresh, p, row_status,
                                stream));
}

extern "C" const char *fa_strerror(int code)
{
    switch (code) {
    case FA_OK: return "ok";
    case FA_EINVAL: return "invalid argument (size, id, range, pointer or workspace)";
    case FA_ENOTDET: return "automaton flagged deterministic has two edges for one (state, token)";
    case FA_ETOOBIG: return "size exceeds what the kernels index";
    case FA_EHIP: return "HIP call or kernel launch failed";
    case FA_ESTATE: return "table not uploaded";
    default: return "unknown error";
    }
}
