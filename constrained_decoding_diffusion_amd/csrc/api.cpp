// C-ABI entry points of one constrained denoising step: argument checks,
// geometry, workspace layout, then the kernel launchers.  Nothing here
// allocates device memory or synchronizes.
#include <hip/hip_runtime_api.h>

#include <algorithm>

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

namespace {

// a row offset of a caller buffer (null stays null)
template <class T>
T *rows(T *ptr, size_t per_row, int32_t b0)
{
    return ptr ? ptr + per_row * (size_t)b0 : ptr;
}

// runs fn(b0, geometry of the chunk, workspace of the chunk) for every row
// chunk of a step, in order; stops at the first failure
template <class Fn>
int each_chunk(const HostTable &h, int32_t B, int32_t L, const StepChunks &ck, uint8_t *ws, Fn fn)
{
    for (int32_t k = 0; k < ck.count; ++k) {
        const int32_t b0 = k * ck.rows;
        Geometry gc;
        make_geometry(h, std::min(ck.rows, B - b0), L, &gc);
        gc.b0 = b0;
        if (int rc = fn(b0, gc, ws ? ws + (size_t)k * ck.slot : ws)) return rc;
    }
    return 0;
}

size_t ws_need(const StepChunks &ck) { return (size_t)ck.count * ck.slot; }

}  // namespace

extern "C" int fa_build_transitions(const fa_table *t, const float *p, int32_t B, int32_t L,
                                    float *tree, int32_t *meta, void *ws, size_t ws_bytes,
                                    int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    if (B == 0 || L == 0) return FA_OK;
    if (!p || !tree || !meta || !row_status || !ws || ws_bytes < ws_need(ck)) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        return launch_build_transitions(d, g, rows(p, (size_t)L * d.V, b0),
                                        rows(tree, 2 * (size_t)g.Lpad * g.mat, b0),
                                        rows(meta, 6 * (size_t)g.Lpad * g.Sp, b0), wsc,
                                        ws_layout(t->h, g), rows(row_status, 1, b0), stream);
    }));
}

extern "C" int fa_span_tree(const fa_table *t, int32_t B, int32_t L, float *tree, int32_t *meta,
                            void *ws, size_t ws_bytes, double *logZ, int32_t *row_status,
                            fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    if (B == 0) return FA_OK;
    if (!logZ || !row_status) return FA_EINVAL;
    if (L > 0 && (!tree || !meta || !ws || ws_bytes < ws_need(ck))) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        return launch_span_tree(d, g, rows(tree, 2 * (size_t)g.Lpad * g.mat, b0),
                                rows(meta, 6 * (size_t)g.Lpad * g.Sp, b0), wsc, ws_layout(t->h, g),
                                rows(logZ, 1, b0), rows(row_status, 1, b0), stream);
    }));
}

extern "C" int fa_sample(const fa_table *t, const float *p, int32_t B, int32_t L, const float *tree,
                         const int32_t *meta, uint64_t seed, int32_t *states, int32_t *tokens,
                         void *ws, size_t ws_bytes, int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    if (B == 0) return FA_OK;
    if (!states || !row_status || !ws || ws_bytes < ws_need(ck)) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !meta || !tokens)) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        // a chunk's row b draws with the keys of batch row b0 + b
        return launch_sample(d, g, rows(p, (size_t)L * d.V, b0),
                             rows(tree, 2 * (size_t)g.Lpad * g.mat, b0),
                             rows(meta, 6 * (size_t)g.Lpad * g.Sp, b0), seed,
                             rows(states, (size_t)L + 1, b0), rows(tokens, (size_t)L, b0), wsc,
                             ws_layout(t->h, g), rows(row_status, 1, b0), stream);
    }));
}

extern "C" int fa_marginals(const fa_table *t, const float *p, int32_t B, int32_t L,
                            const float *tree, const int32_t *meta, const double *logZ,
                            const int32_t *tokens, int32_t conf_mode, float *q, float *conf,
                            void *ws, size_t ws_bytes, int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    if (!conf_mode_ok(conf_mode)) return FA_EINVAL;
    if (B == 0 || L == 0) return FA_OK;
    if (!p || !tree || !meta || !logZ || !conf || !row_status || !ws || ws_bytes < ws_need(ck))
        return FA_EINVAL;
    if (conf_mode != FA_CONF_NEGENT && !tokens) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        const float *pc = rows(p, (size_t)L * d.V, b0);
        const int32_t *tc = rows(tokens, (size_t)L, b0);
        float *cc = rows(conf, (size_t)L, b0);
        int32_t *sc = rows(row_status, 1, b0);
        // the unconstrained score takes the PROB path for q, then its own conf
        int r = launch_marginals(d, g, pc, rows(tree, 2 * (size_t)g.Lpad * g.mat, b0),
                                 rows(meta, 6 * (size_t)g.Lpad * g.Sp, b0), rows(logZ, 1, b0), tc,
                                 base_mode(conf_mode), rows(q, (size_t)L * d.V, b0), cc, wsc,
                                 ws_layout(t->h, g), sc, stream);
        if (!r && conf_mode == FA_CONF_UNCONSTRAINED)
            r = launch_conf_unconstrained(d, g, pc, tc, sc, cc, stream);
        return r;
    }));
}

extern "C" int fa_sample_marginals(const fa_table *t, const float *p, int32_t B, int32_t L,
                                   const float *tree, const int32_t *meta, const double *logZ,
                                   uint64_t seed, int32_t conf_mode, int32_t *states,
                                   int32_t *tokens, float *q, float *conf, void *ws,
                                   size_t ws_bytes, int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    if (!conf_mode_ok(conf_mode)) return FA_EINVAL;
    if (B == 0) return FA_OK;
    if (!states || !row_status || !ws || ws_bytes < ws_need(ck)) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !meta || !logZ || !tokens || !conf)) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        const float *pc = rows(p, (size_t)L * d.V, b0);
        int32_t *tc = rows(tokens, (size_t)L, b0);
        float *cc = rows(conf, (size_t)L, b0);
        int32_t *sc = rows(row_status, 1, b0);
        int r = sample_marginals_base(d, g, pc, rows(tree, 2 * (size_t)g.Lpad * g.mat, b0),
                                      rows(meta, 6 * (size_t)g.Lpad * g.Sp, b0), rows(logZ, 1, b0),
                                      seed, base_mode(conf_mode), rows(states, (size_t)L + 1, b0), tc,
                                      rows(q, (size_t)L * d.V, b0), cc, wsc, ws_layout(t->h, g), sc,
                                      stream);
        if (!r && L > 0 && conf_mode == FA_CONF_UNCONSTRAINED)
            r = launch_conf_unconstrained(d, g, pc, tc, sc, cc, stream);
        return r;
    }));
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
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    // the chain reads every position's dense matrix
    if (t->h.leafless && L > 1) return FA_EINVAL;
    if (B == 0) return FA_OK;
    if (!logZ || !states || !row_status || !ws || ws_bytes < ws_need(ck)) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !tokens)) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        return launch_chain_sample(d, g, rows(p, (size_t)L * d.V, b0),
                                   rows(tree, 2 * (size_t)g.Lpad * g.mat, b0), seed,
                                   rows(logZ, 1, b0), rows(states, (size_t)L + 1, b0),
                                   rows(tokens, (size_t)L, b0), wsc, ws_layout(t->h, g),
                                   rows(row_status, 1, b0), stream);
    }));
}

extern "C" int fa_chain_sample_marginals(const fa_table *t, const float *p, int32_t B, int32_t L,
                                         const float *tree, uint64_t seed, int32_t conf_mode,
                                         double *logZ, int32_t *states, int32_t *tokens, float *q,
                                         float *conf, void *ws, size_t ws_bytes,
                                         int32_t *row_status, fa_stream_t stream)
{
    int rc = ready(t);
    if (rc) return rc;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, false, &ck)) return grc;
    if (!conf_mode_ok(conf_mode)) return FA_EINVAL;
    if (t->h.leafless && L > 1) return FA_EINVAL;
    if (B == 0) return FA_OK;
    if (!logZ || !states || !row_status || !ws || ws_bytes < ws_need(ck)) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !tokens || !conf)) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        const float *pc = rows(p, (size_t)L * d.V, b0);
        int32_t *tc = rows(tokens, (size_t)L, b0);
        float *cc = rows(conf, (size_t)L, b0);
        int32_t *sc = rows(row_status, 1, b0);
        int r = launch_chain_sample_marginals(
            d, g, pc, rows(tree, 2 * (size_t)g.Lpad * g.mat, b0), seed, base_mode(conf_mode),
            rows(logZ, 1, b0), rows(states, (size_t)L + 1, b0), tc, rows(q, (size_t)L * d.V, b0), cc,
            wsc, ws_layout(t->h, g), sc, stream);
        if (!r && L > 0 && conf_mode == FA_CONF_UNCONSTRAINED)
            r = launch_conf_unconstrained(d, g, pc, tc, sc, cc, stream);
        return r;
    }));
}

extern "C" int fa_map_sizes(const fa_table *t, int32_t B, int32_t L, size_t *tree_bytes,
                            size_t *ws_bytes)
{
    if (!t) return FA_EINVAL;
    // range labels: the per-position range-maximum structure must fit one workgroup's LDS
    if (t->h.nseg() > 0 && map_range_lds(t->h.ncut()) > kMapRangeLdsMax) return FA_ETOOBIG;
    Geometry g;
    if (int grc = make_geometry(t->h, B, L, &g)) return grc;
    StepChunks ck;
    if (int rc = plan_chunks(t->h, B, L, true, &ck)) return rc;
    if (tree_bytes) *tree_bytes = g.tree_floats * sizeof(double);
    if (ws_bytes) *ws_bytes = std::max<size_t>(ws_need(ck), 256);
    return FA_OK;
}

extern "C" int fa_map_decode(const fa_table *t, const float *p, int32_t B, int32_t L,
                             double *tree, void *ws, size_t ws_bytes, double *logmax,
                             int32_t *states, int32_t *tokens, int32_t *row_status,
                             fa_stream_t stream)
{
    if (t && t->h.nseg() > 0 && map_range_lds(t->h.ncut()) > kMapRangeLdsMax) return FA_ETOOBIG;
    int rc = ready(t);
    if (rc) return rc;
    StepChunks ck;
    if (int grc = plan_chunks(t->h, B, L, true, &ck)) return grc;
    if (B == 0) return FA_OK;
    if (!logmax || !states || !row_status) return FA_EINVAL;
    if (L > 0 && (!p || !tree || !tokens || !ws || ws_bytes < ws_need(ck))) return FA_EINVAL;
    const DevTable d = t->h.device_view();
    return hip_rc(each_chunk(t->h, B, L, ck, (uint8_t *)ws, [&](int32_t b0, const Geometry &g,
                                                                 uint8_t *wsc) {
        return launch_map_decode(d, g, rows(p, (size_t)L * d.V, b0),
                                 rows(tree, 2 * (size_t)g.Lpad * g.mat, b0), wsc,
                                 map_ws_layout(t->h, g), rows(logmax, 1, b0),
                                 rows(states, (size_t)L + 1, b0), rows(tokens, (size_t)L, b0),
                                 rows(row_status, 1, b0), stream);
    }));
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
