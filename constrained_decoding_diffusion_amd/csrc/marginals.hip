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
#include "pair_value.h"
#include "sample_draw.h"

namespace fa {
namespace {

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

// out = in * T for the consumed stored rows of one node.  grid.x: column
// blocks of CW columns; grid.y: (b, node, alpha|beta).  The rows are dealt
// to the 16 wavefronts of the workgroup; their partial sums are added in
// wavefront order.
constexpr int kMsgThreads = 1024;
constexpr int kMsgWaves = kMsgThreads / 64;
constexpr int kMsgU = 4;  // rows per wavefront per load group

//
// md: midpoint draws riding on the launch (the joint call): md.nwg
// workgroups in the first rows of blockIdx.y, column block 0, so that they
// are dispatched first; the products follow.
template <int CW>
__global__ __launch_bounds__(kMsgThreads) void marg_level(
    DevTable d, StepView sv, const float *__restrict__ tree, const int32_t *__restrict__ meta,
    int nn, float *__restrict__ va, int32_t *__restrict__ ea, float *__restrict__ vb,
    int32_t *__restrict__ eb, int top, MidDraws md)
{
    if ((int)blockIdx.y < md.nwg) {
        if (blockIdx.x == 0) mid_draws_wg(d, sv, md, (int)blockIdx.y);
        return;
    }
    constexpr int PER = CW / 64;  // columns per lane: 4 or 1
    extern __shared__ float gsh[];  // [Sp] normalized input weights, then [Sp] row folds
    int *rsh = reinterpret_cast<int *>(gsh + sv.Sp);
    __shared__ int sh_max[kMsgWaves];
    __shared__ float red[kMsgWaves][CW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cb = blockIdx.x, prod = (int)blockIdx.y - md.nwg;
    const int beta = prod & 1;
    const int bn = prod >> 1;
    const int b = bn / nn, idx = bn % nn, n = nn + idx;
    const int span = sv.Lpad / nn, l = idx * span, r = l + span, m = l + span / 2;
    const int h = beta ? 2 * n + 1 : 2 * n;
    const int src = beta ? r : l;
    float *vbase = beta ? vb : va;
    int32_t *ebase = beta ? eb : ea;
    const float *vin = vbase + ((size_t)b * (sv.Lpad + 1) + src) * sv.Sp;
    float *vout = vbase + ((size_t)b * (sv.Lpad + 1) + m) * sv.Sp;
    if (top) {
        // the top level builds its input, the boundary vector alpha_0 = e_start
        // or beta_Lpad = 1 on F (exponent 0), in LDS; column block 0 also
        // stores it for the later passes
        for (int a = tid; a < sv.Sp; a += kMsgThreads) gsh[a] = 0.f;
        __syncthreads();
        if (beta) {
            for (int k = tid; k < d.n_acc; k += kMsgThreads) gsh[d.acc[k]] = 1.f;
        } else if (tid == 0) {
            gsh[d.start] = 1.f;
        }
        __syncthreads();
        if (cb == 0) {
            float *bound = vbase + ((size_t)b * (sv.Lpad + 1) + src) * sv.Sp;
            for (int a = tid; a < sv.Sp; a += kMsgThreads) bound[a] = gsh[a];
            if (tid == 0) ebase[(size_t)b * (sv.Lpad + 1) + src] = 0;
        }
    }
    const int ein = top ? 0 : ebase[(size_t)b * (sv.Lpad + 1) + src];
    const float *P = sv.mat_ptr(tree, b, h);
    const int32_t *ro = sv.meta_ptr(meta, b, h, 0);
    const int32_t *co = sv.meta_ptr(meta, b, h, 1);
    const int32_t *rf = sv.meta_ptr(meta, b, h, 2);
    // G = max_a e(in[a]) + ro[a] + rf[a]; the per-row exponents go to LDS
    int e = kNeg;
    for (int a = tid; a < d.S; a += kMsgThreads) {
        const float x = top ? gsh[a] : vin[a];
        const int s = add_exp(ro[a], rf[a]);
        rsh[a] = s;
        gsh[a] = x;
        if (x > 0.f && s > kNeg) e = max(e, fexp(x) + s);
    }
    e = wave_max_i(e);
    if (lane == 0) sh_max[wave] = e;
    __syncthreads();
    int G = kNeg;
    for (int w = 0; w < kMsgWaves; ++w) G = max(G, sh_max[w]);
    // normalized input weights g[a] and the row fold rf[a] (replaces the
    // row exponent slot)
    for (int a = tid; a < d.S; a += kMsgThreads) {
        const float x = gsh[a];
        const int s = rsh[a];
        gsh[a] = (x > 0.f && s > kNeg && G > kNeg) ? scale2(mant(x), fexp(x) + s - G) : 0.f;
        rsh[a] = rf[a];
    }
    __syncthreads();
    const int j0 = cb * CW + PER * lane;
    const bool colok = j0 < sv.Sp && G > kNeg;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
    if (colok) {
        int cj[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) cj[k] = co[j0 + k];
        // rows a = wave + 16 t of this wavefront, in groups of kMsgU whose
        // loads are unconditional (clamped) and issued one group ahead.  A
        // row with zero input weight adds +0: its consumed entries are at
        // most 1 (the row fold) and an all-zero row stays zero, so every
        // row is summed, in order, with no data-dependent branch.
        const int na = (d.S - wave + kMsgWaves - 1) / kMsgWaves;
        struct Grp {
            float4 y[kMsgU];
        };
        auto ld = [&](Grp &gr, int t) {
#pragma unroll
            for (int u = 0; u < kMsgU; ++u) {
                const int a = min(wave + (t + u) * kMsgWaves, d.S - 1);
                const float *row = P + (size_t)a * sv.Sp + j0;
                if constexpr (PER == 4) gr.y[u] = *reinterpret_cast<const float4 *>(row);
                else gr.y[u].x = row[0];
            }
        };
        auto use = [&](const Grp &gr, int t) {
#pragma unroll
            for (int u = 0; u < kMsgU; ++u) {
                const int a = min(wave + (t + u) * kMsgWaves, d.S - 1);
                const float g = (t + u < na) ? gsh[a] : 0.f;
                const int ra = rsh[a];
                acc[0] += g * scale2(gr.y[u].x, cj[0] - ra);
                if constexpr (PER == 4) {
                    acc[1] += g * scale2(gr.y[u].y, cj[1] - ra);
                    acc[2] += g * scale2(gr.y[u].z, cj[2] - ra);
                    acc[3] += g * scale2(gr.y[u].w, cj[3] - ra);
                }
            }
        };
        Grp A, B;
        ld(A, 0);
        for (int t = 0; t < na; t += 2 * kMsgU) {
            ld(B, t + kMsgU);
            use(A, t);
            ld(A, t + 2 * kMsgU);
            use(B, t + kMsgU);
        }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) red[wave][PER * lane + k] = acc[k];
    __syncthreads();
    for (int c = tid; c < CW; c += kMsgThreads) {
        const int j = cb * CW + c;
        if (j >= sv.Sp) continue;
        float s = 0.f;
        for (int w = 0; w < kMsgWaves; ++w) s += red[w][c];
        vout[j] = s;
    }
    if (cb == 0 && tid == 0)
        ebase[(size_t)b * (sv.Lpad + 1) + m] = (G > kNeg && ein > kNeg) ? ein + G : kNeg;
}

// range weights per cut interval: rcut[pos][c] = sum of c*alpha*beta over
// the segments covering [cuts[c], cuts[c+1]), in fp64, exactly zero where no
// segment is active.  One workgroup per position walks the cuts in tiles of
// kRcutTile: each thread takes kRcutPer consecutive cuts of the tile and
// sums their events (one load each of the event's states and signed count;
// alpha and beta come from LDS), a block scan of the active-segment counts
// marks the cuts where no segment is active, and a segmented fp64 scan
// restarts the weight sum at exactly zero there (a rounding residue never
// carries past such a cut); a sum rounded below zero is written as zero.
constexpr int kRcutThreads = 256;
constexpr int kRcutPer = 8;
constexpr int kRcutTile = kRcutThreads * kRcutPer;

// segmented sum: (x, reset) o (y, reset') = (reset' ? y : x + y, reset | reset')
struct SegSum {
    double x;
    int reset;
};

__device__ inline SegSum seg_combine(SegSum a, SegSum b)
{
    return SegSum{b.reset ? b.x : a.x + b.x, a.reset | b.reset};
}

__global__ __launch_bounds__(kRcutThreads) void marg_rcut(DevTable d, StepView sv,
                                                          const float *__restrict__ va,
                                                          const float *__restrict__ vb,
                                                          float *__restrict__ rcut, int ab_lds)
{
    extern __shared__ float abs_[];  // alpha [Sp] | beta [Sp] when ab_lds
    __shared__ int sh_cnt[kRcutThreads];
    __shared__ double sh_x[kRcutThreads];
    __shared__ int sh_r[kRcutThreads];
    __shared__ int sh_act;
    __shared__ double sh_carry;
    const int pos = blockIdx.x;
    const int tid = threadIdx.x;
    const int b = pos / sv.L, i = pos % sv.L;
    const float *alg = va + ((size_t)b * (sv.Lpad + 1) + i) * sv.Sp;
    const float *beg = vb + ((size_t)b * (sv.Lpad + 1) + i + 1) * sv.Sp;
    const float *al = alg, *be = beg;
    if (ab_lds) {
        for (int a = tid; a < d.S; a += kRcutThreads) {
            abs_[a] = alg[a];
            abs_[sv.Sp + a] = beg[a];
        }
        al = abs_;
        be = abs_ + sv.Sp;
    }
    if (tid == 0) {
        sh_act = 0;
        sh_carry = 0.0;
    }
    float *out = rcut + (size_t)pos * d.ncut;
    for (int t0 = 0; t0 < d.ncut; t0 += kRcutTile) {
        __syncthreads();  // alpha/beta staged; the previous tile's carry is final
        const int c0 = min(t0 + tid * kRcutPer, d.ncut), c1 = min(c0 + kRcutPer, d.ncut);
        const int k0 = d.cut_off[c0];
        int off[kRcutPer + 1];
#pragma unroll
        for (int j = 0; j <= kRcutPer; ++j) off[j] = d.cut_off[min(c0 + j, c1)];
        // per cut: signed weight sum and count change of its events
        double dw[kRcutPer];
        int dc[kRcutPer];
        int dsum = 0;
#pragma unroll
        for (int j = 0; j < kRcutPer; ++j) {
            double w = 0.0;
            int cnt = 0;
            for (int k = off[j]; k < off[j + 1]; ++k) {
                const float sw = d.ev_w[k];
                w += (double)al[d.ev_a[k]] * (double)be[d.ev_b[k]] * (double)sw;
                cnt += sw < 0.f ? -1 : 1;
            }
            dw[j] = w;
            dc[j] = cnt;
            dsum += cnt;
        }
        (void)k0;
        // active count before this thread's cuts: exclusive block scan + the tile's carry-in
        sh_cnt[tid] = dsum;
        __syncthreads();
        for (int o = 1; o < kRcutThreads; o <<= 1) {
            const int v = tid >= o ? sh_cnt[tid - o] : 0;
            __syncthreads();
            sh_cnt[tid] += v;
            __syncthreads();
        }
        const int act0 = sh_act + sh_cnt[tid] - dsum;
        // this thread's segmented sum over its cuts
        SegSum mine{0.0, 0};
        {
            int act = act0;
#pragma unroll
            for (int j = 0; j < kRcutPer; ++j) {
                act += dc[j];
                mine.x += dw[j];
                if (c0 + j < c1 && act == 0) mine = SegSum{0.0, 1};
            }
        }
        sh_x[tid] = mine.x;
        sh_r[tid] = mine.reset;
        __syncthreads();
        for (int o = 1; o < kRcutThreads; o <<= 1) {
            SegSum v{0.0, 0};
            const bool has = tid >= o;
            if (has) v = SegSum{sh_x[tid - o], sh_r[tid - o]};
            __syncthreads();
            if (has) {
                const SegSum r = seg_combine(v, SegSum{sh_x[tid], sh_r[tid]});
                sh_x[tid] = r.x;
                sh_r[tid] = r.reset;
            }
            __syncthreads();
        }
        // carry into this thread: the previous tile's running sum combined
        // with the runs before it in this tile
        const SegSum before = tid > 0 ? seg_combine(SegSum{sh_carry, 0}, SegSum{sh_x[tid - 1], sh_r[tid - 1]})
                                      : SegSum{sh_carry, 0};
        double R = before.x;
        int act = act0;
#pragma unroll
        for (int j = 0; j < kRcutPer; ++j) {
            if (c0 + j < c1) {
                act += dc[j];
                R += dw[j];
                if (act == 0) R = 0.0;
                out[c0 + j] = R > 0.0 ? (float)R : 0.f;
            }
        }
        __syncthreads();  // every thread has read sh_carry / sh_act of this tile
        if (tid == kRcutThreads - 1) {
            sh_carry = seg_combine(SegSum{sh_carry, 0}, SegSum{sh_x[tid], sh_r[tid]}).x;
            sh_act = act0 + dsum;
        }
    }
}

constexpr int kQThreads = 256;
constexpr size_t kQLdsMax = 64 * 1024;  // LDS lookup tables of the streaming q writer

// LIST weight of selected token s: sum over its token-major entries
__device__ inline float list_weight(const DevTable &d, int s, const float *al, const float *be)
{
    float r = 0.f;
    for (int k = d.tm_off[s]; k < d.tm_off[s + 1]; ++k) {
        const int qq = d.tm_pair[k];
        const float w = al[d.pair_a[qq]] * be[d.pair_b[qq]];
        r += d.tm_cnt ? w * d.tm_cnt[k] : w;
    }
    return r;
}

// nparts (1 or kQParts) workgroups per position each stream their share of
// the p row once and write that part of the q row (short batches take
// kQParts parts: a position per workgroup would leave most of the chip
// idle); with FA_CONF_NEGENT and several parts each leaves its q ln q sum in
// hpart for marg_negent_sum.
// The dense-mask pairs' weight of a token is read from NG 256-entry tables
// indexed by the bytes of its mask word; with SELBIT, tokens held by
// token-list pairs carry a flag bit and add their precomputed weight (LIST
// only tables look every token up instead); RANGES adds the weight of the
// token's cut interval.  The feature set is a template so the per-token
// path has no branches beyond the rare token-list lookups.
template <int NG, bool SELBIT, bool LISTALL, bool RANGES>
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
                                                    double *__restrict__ hpart, int nparts,
                                                    const int32_t *__restrict__ status)
{
    __shared__ float lut[NG > 0 ? NG : 1][256];
    __shared__ float rsel[(SELBIT || LISTALL) ? kSelMax : 1];
    __shared__ double sh_h[4];
    const int b = blockIdx.y, i = blockIdx.x / nparts, part = blockIdx.x % nparts;
    const size_t pos = (size_t)b * sv.L + i;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *prow = p + pos * d.V;
    float *qrow = q ? q + pos * d.V : nullptr;
    // this part's tokens: a quarter of the float4 groups (or of the tokens)
    const int n4 = d.V >> 2;
    const int per4 = (n4 + nparts - 1) / nparts;
    const int k_lo = min(part * per4, n4), k_hi = min(k_lo + per4, n4);
    const int perv = (d.V + nparts - 1) / nparts;
    const int v_lo = min(part * perv, d.V), v_hi = min(v_lo + perv, d.V);
    const double lz = logZ[b];
    const int e1 = ea[(size_t)b * (sv.Lpad + 1) + i], e2 = eb[(size_t)b * (sv.Lpad + 1) + i + 1];
    const bool ok = status[b] == 0 && lz > -INFINITY && e1 > kNeg && e2 > kNeg;
    const bool negent = conf_mode == FA_CONF_NEGENT;
    if (!ok) {
        if (qrow)
            for (int v = v_lo + tid; v < v_hi; v += kQThreads) qrow[v] = 0.f;
        if (tid == 0 && part == 0) conf[pos] = -INFINITY;
        if (tid == 0 && negent && nparts > 1) hpart[pos * kQParts + part] = -INFINITY;
        return;
    }
    const double factor = exp2((double)e1 + (double)e2 - lz * 1.4426950408889634074);
    const float *al = va + ((size_t)b * (sv.Lpad + 1) + i) * sv.Sp;
    const float *be = vb + ((size_t)b * (sv.Lpad + 1) + i + 1) * sv.Sp;
    const int nd = d.ndense;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float s = 0.f;
        for (int bit = 0; bit < 8; ++bit) {
            const int j = 8 * g + bit;
            if (j < nd && ((tid >> bit) & 1)) {
                const int qq = d.dense_pair[j];
                s += al[d.pair_a[qq]] * be[d.pair_b[qq]];
            }
        }
        lut[g][tid] = s;
    }
    const bool sel_lds = d.nsel > 0 && d.nsel <= kSelMax;
    if (SELBIT || LISTALL)
        if (sel_lds)
            for (int s = tid; s < d.nsel; s += kQThreads) rsel[s] = list_weight(d, s, al, be);
    __syncthreads();
    const float *rc = RANGES ? rcut + pos * d.ncut : nullptr;
    const int tok = tokens ? tokens[pos] : -1;
    auto list_r = [&](int v) -> float {
        const int s = d.tok2sel[v];
        if (s < 0) return 0.f;
        return sel_lds ? rsel[s] : list_weight(d, s, al, be);
    };
    auto weight_r = [&](int v, uint32_t m) -> float {
        float r = 0.f;
        if constexpr (NG > 0) r = lut[0][m & 255u];
        if constexpr (NG > 1) r += lut[1][(m >> 8) & 255u];
        if constexpr (NG > 2) r += lut[2][(m >> 16) & 255u];
        if constexpr (NG > 3) r += lut[3][(m >> 24) & 255u];
        if constexpr (SELBIT) {
            if (m & kSelBit) r += list_r(v);
        }
        if constexpr (LISTALL) r += list_r(v);
        if constexpr (RANGES) {
            const int c = d.tok2cut[v];
            if (c >= 0) r += rc[c];
        }
        return r;
    };
    auto qval = [&](float x, float r) -> float {
        return (r > 0.f && x > 0.f) ? (float)((double)x * (double)r * factor) : 0.f;
    };
    if (!qrow && !negent) {
        // only the sampled token's marginal is needed
        if (tid == 0 && part == 0)
            conf[pos] = tok >= 0 ? qval(prow[tok], weight_r(tok, NG > 0 || SELBIT ? d.tokmask[tok] : 0u))
                                 : -INFINITY;
        return;
    }
    double hsum = 0.0;
    float tokq = -INFINITY;
    bool have_tok = false;
    if ((d.V & 3) == 0) {
        constexpr int U = 4;  // float4 groups in flight per thread
        const uint4 *m4 = reinterpret_cast<const uint4 *>(d.tokmask);
        float4 *q4 = reinterpret_cast<float4 *>(qrow);
        for (int k0 = k_lo + tid; k0 < k_hi; k0 += U * kQThreads) {
            float4 x[U];
            uint4 mm[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = min(k0 + u * kQThreads, k_hi - 1);
                x[u] = load_nt(prow + 4 * (size_t)k);
                if constexpr (NG > 0 || SELBIT) mm[u] = m4[k];
                else mm[u] = make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + u * kQThreads;
                const int v = 4 * min(k, k_hi - 1);  // in-bounds tokens for the lookups
                float4 o;
                o.x = qval(x[u].x, weight_r(v, mm[u].x));
                o.y = qval(x[u].y, weight_r(v + 1, mm[u].y));
                o.z = qval(x[u].z, weight_r(v + 2, mm[u].z));
                o.w = qval(x[u].w, weight_r(v + 3, mm[u].w));
                if (k < k_hi) {
                    if (q4) q4[k] = o;
                    if (tok >= v && tok < v + 4) {
                        have_tok = true;
                        tokq = tok == v ? o.x : tok == v + 1 ? o.y : tok == v + 2 ? o.z : o.w;
                    }
                    if (negent) {
                        if (o.x > 0.f) hsum += (double)o.x * log((double)o.x);
                        if (o.y > 0.f) hsum += (double)o.y * log((double)o.y);
                        if (o.z > 0.f) hsum += (double)o.z * log((double)o.z);
                        if (o.w > 0.f) hsum += (double)o.w * log((double)o.w);
                    }
                }
            }
        }
    } else {
        for (int v = v_lo + tid; v < v_hi; v += kQThreads) {
            const float o = qval(prow[v], weight_r(v, NG > 0 || SELBIT ? d.tokmask[v] : 0u));
            if (qrow) qrow[v] = o;
            if (v == tok) {
                have_tok = true;
                tokq = o;
            }
            if (negent && o > 0.f) hsum += (double)o * log((double)o);
        }
    }
    if (negent) {
        hsum = wave_sum_d(hsum);
        if (lane == 0) sh_h[wave] = hsum;
        __syncthreads();
        const double h = ((sh_h[0] + sh_h[1]) + sh_h[2]) + sh_h[3];
        if (tid == 0) {
            if (nparts > 1) hpart[pos * kQParts + part] = h;
            else conf[pos] = (float)h;
        }
    } else {
        if (have_tok) conf[pos] = tokq;
        if (tid == 0 && part == 0 && tok < 0) conf[pos] = -INFINITY;
    }
}

// Per-position pair weights alpha_i[a] beta_{i+1}[a'] that the q writer
// looks up: pw[pos][j] for dense-mask pair j (0 past ndense), then
// pw[pos][32 + s] = the summed weight of the token-list pairs holding
// sel_tok[s].  One workgroup per position: the weights of all token-major
// entries are formed in parallel into LDS (chunks of kPwChunk entries), then
// each token's entries are summed in entry order.
constexpr int kPwThreads = 512;
constexpr int kPwUnroll = 4;
constexpr int kPwChunk = 8192;

// The weights of one position from its two vectors (global or LDS); wsh:
// LDS scratch of min(n_tm, kPwChunk) + nl floats.  All kPwThreads threads
// call it.
__device__ void pair_weights(const DevTable &d, const float *al, const float *be, int nl,
                             float *__restrict__ out, float *wsh)
{
    const int tid = threadIdx.x;
    if (tid < kDenseMax) {
        float w = 0.f;
        if (tid < d.ndense) {
            const int qq = d.dense_pair[tid];
            w = al[d.pair_a[qq]] * be[d.pair_b[qq]];
        }
        out[tid] = w;
    }
    if (nl == 0) return;
    const int cap = min(d.n_tm, kPwChunk);
    float *rs = wsh + cap;
    for (int s = tid; s < nl; s += kPwThreads) rs[s] = 0.f;
    for (int c0 = 0; c0 < d.n_tm; c0 += kPwChunk) {
        const int c1 = min(d.n_tm, c0 + kPwChunk);
        __syncthreads();
        // kPwUnroll entries per thread in flight: index loads first (clamped,
        // unconditional), then the message gathers
        for (int k0 = c0; k0 < c1; k0 += kPwThreads * kPwUnroll) {
            int ka[kPwUnroll], kb[kPwUnroll];
            float kc[kPwUnroll];
#pragma unroll
            for (int u = 0; u < kPwUnroll; ++u) {
                const int k = min(k0 + u * kPwThreads + tid, c1 - 1);
                ka[u] = d.tm_a[k];
                kb[u] = d.tm_b[k];
                kc[u] = d.tm_cnt ? d.tm_cnt[k] : 1.f;
            }
#pragma unroll
            for (int u = 0; u < kPwUnroll; ++u) {
                const int k = k0 + u * kPwThreads + tid;
                const float w = al[ka[u]] * be[kb[u]];
                if (k < c1) wsh[k - c0] = d.tm_cnt ? w * kc[u] : w;
            }
        }
        __syncthreads();
        for (int s = tid; s < nl; s += kPwThreads) {
            const int k0 = max(d.tm_off[s], c0), k1 = min(d.tm_off[s + 1], c1);
            float r = rs[s];
            for (int k = k0; k < k1; ++k) r += wsh[k - c0];
            rs[s] = r;
        }
    }
    for (int s = tid; s < nl; s += kPwThreads) out[kDenseMax + s] = rs[s];
}

__global__ __launch_bounds__(kPwThreads) void marg_pairw(DevTable d, StepView sv,
                                                         const float *__restrict__ va,
                                                         const float *__restrict__ vb, int nl,
                                                         int ld, float *__restrict__ pw)
{
    extern __shared__ float wsh[];  // [min(n_tm, kPwChunk)] entry weights | [nl] sums
    const int pos = blockIdx.x;
    const int b = pos / sv.L, i = pos % sv.L;
    const float *al = va + ((size_t)b * (sv.Lpad + 1) + i) * sv.Sp;
    const float *be = vb + ((size_t)b * (sv.Lpad + 1) + i + 1) * sv.Sp;
    pair_weights(d, al, be, nl, pw + (size_t)pos * ld, wsh);
}

// Streaming q writer (V % 4 == 0, lookup tables in LDS).  kQParts
// workgroups per position, consecutive in the grid, each over one
// contiguous part of the row (adjacent workgroups stream adjacent memory);
// each thread handles U float4 groups per iteration.  Every global
// load of the loop is unconditional (clamped index) and issued one iteration
// ahead, and the per-token weight reads LDS only: the dense-mask lookup
// table, the token-list weights (found in the token's 256-token bucket of
// the sorted token-list tokens when the mask's flag bit marks the token, or
// through tok2sel), and the range weights at each cut.
//
// The parts are whole chunks of kRowChunk4 float4 groups, so iteration `it`
// of a part covers one chunk of the token sampler's streamed pass.  SAMP
// (the joint call): tdbit holds the dense-mask bit of the pair the
// position's token draw uses (0 when it is not a dense pair); for a dense
// pair each wavefront also sums its masked p over each chunk, in the sampler's order
// (u ascending, then x, y, z, w), and stores the sum in tcs, and part 0 sets
// tcs_ok for the position (tokens is then unused: marg_conf_tok writes the
// confidence after the draws).  The sums cost registers; the joint variants
// are held to 128 VGPRs (four wavefronts per SIMD, a few spills), which
// streams faster than three wavefronts per SIMD without spills.
template <int NG, bool SELBIT, bool LISTALL, bool RANGES, bool SAMP>
__global__ __launch_bounds__(kQThreads)
__attribute__((amdgpu_waves_per_eu(SAMP && !LISTALL ? 4 : 1))) void marg_q_stream(
    DevTable d, StepView sv, const float *__restrict__ p, const double *__restrict__ logZ,
    const int32_t *__restrict__ tokens, int conf_mode, float *__restrict__ q,
    float *__restrict__ conf, const int32_t *__restrict__ ea, const int32_t *__restrict__ eb,
    const float *__restrict__ pw, int pw_ld, const float *__restrict__ rcut,
    double *__restrict__ hpart, const int32_t *__restrict__ status,
    const uint32_t *__restrict__ tdbit, double *__restrict__ tcs, int32_t *__restrict__ tcs_ok,
    int tcs_nch)
{
    constexpr bool LISTS = SELBIT || LISTALL;
    constexpr bool MASK = NG > 0 || SELBIT;
    static_assert(!SAMP || NG > 0, "the token draws' sums read the dense mask");
    extern __shared__ float dyn[];  // rsel [nsel] | selk [nsel] | slb [V/256 + 2] | rcl [ncut]
    __shared__ float lut[NG > 0 ? NG : 1][256];
    __shared__ double sh_h[4];
    const int b = blockIdx.y, i = blockIdx.x / kQParts, part = blockIdx.x % kQParts;
    const size_t pos = (size_t)b * sv.L + i;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *prow = p + pos * d.V;
    float *qrow = q ? q + pos * d.V : nullptr;
    // this part's float4 groups [k_lo, k_hi) of the row: whole chunks
    const int n4 = d.V >> 2;
    const int nch = (n4 + kRowChunk4 - 1) / kRowChunk4;
    const int per = (nch + kQParts - 1) / kQParts * kRowChunk4;
    const int k_lo = min(n4, part * per), k_hi = min(n4, k_lo + per);
    const double lz = logZ[b];
    const int e1 = ea[(size_t)b * (sv.Lpad + 1) + i], e2 = eb[(size_t)b * (sv.Lpad + 1) + i + 1];
    const bool ok = status[b] == 0 && lz > -INFINITY && e1 > kNeg && e2 > kNeg;
    const bool negent = conf_mode == FA_CONF_NEGENT;
    if (!ok) {
        if (qrow)
            for (int v = 4 * k_lo + tid; v < 4 * k_hi; v += kQThreads) qrow[v] = 0.f;
        if (tid == 0 && negent) hpart[pos * kQParts + part] = -INFINITY;
        if (tid == 0 && part == 0) conf[pos] = -INFINITY;
        if (SAMP && tid == 0 && part == 0) tcs_ok[pos] = 0;
        return;
    }
    const double factor = exp2((double)e1 + (double)e2 - lz * 1.4426950408889634074);
    const float *pwr = pw + pos * pw_ld;
    float *rsel = dyn;
    int *selk = reinterpret_cast<int *>(dyn + (LISTS ? d.nsel : 0));
    const int nslb = SELBIT ? d.V / 256 + 2 : 0;
    int *slb = selk + (SELBIT ? d.nsel : 0);
    float *rcl = dyn + (LISTS ? d.nsel : 0) + (SELBIT ? d.nsel + nslb : 0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float sm = 0.f;
        for (int bit = 0; bit < 8; ++bit)
            if ((tid >> bit) & 1) sm += pwr[8 * g + bit];
        lut[g][tid] = sm;
    }
    if (LISTS)
        for (int k = tid; k < d.nsel; k += kQThreads) {
            rsel[k] = pwr[kDenseMax + k];
            if (SELBIT) selk[k] = d.sel_tok[k];
        }
    if (SELBIT)
        for (int k = tid; k < nslb; k += kQThreads) slb[k] = d.sel_lb[k];
    if (RANGES)
        for (int c = tid; c < d.ncut; c += kQThreads) rcl[c] = rcut[pos * d.ncut + c];
    const uint32_t dbit = SAMP ? tdbit[pos] : 0u;
    if (SAMP && tid == 0 && part == 0) tcs_ok[pos] = dbit != 0u;
    __syncthreads();
    const int tok = tokens ? tokens[pos] : -1;
    auto weight_r = [&](int v, uint32_t m, int sl, int c) -> float {
        float r = 0.f;
        if constexpr (NG > 0) r = lut[0][m & 255u];
        if constexpr (NG > 1) r += lut[1][(m >> 8) & 255u];
        if constexpr (NG > 2) r += lut[2][(m >> 16) & 255u];
        if constexpr (NG > 3) r += lut[3][(m >> 24) & 255u];
        if constexpr (SELBIT) {
            if (m & kSelBit) {
                // v is a token-list token: its index is found inside its
                // 256-token bucket (usually the first entry)
                int lo = slb[v >> 8];
                const int hi = slb[(v >> 8) + 1];
                while (lo < hi && selk[lo] < v) ++lo;
                r += rsel[min(lo, d.nsel - 1)];
            }
        }
        if constexpr (LISTALL) {
            if (sl >= 0) r += rsel[sl];
        }
        if constexpr (RANGES) {
            if (c >= 0) r += rcl[c];
        }
        return r;
    };
    auto qval = [&](float x, float r) -> float {
        return (r > 0.f && x > 0.f) ? (float)((double)x * (double)r * factor) : 0.f;
    };
    if (!qrow && !negent) {
        // only the sampled token's marginal is needed
        if (tid == 0 && part == 0) {
            float o = -INFINITY;
            if (tok >= 0)
                o = qval(prow[tok], weight_r(tok, MASK ? d.tokmask[tok] : 0u,
                                             LISTALL ? d.tok2sel[tok] : -1,
                                             RANGES ? d.tok2cut[tok] : -1));
            conf[pos] = o;
        }
        return;
    }
    constexpr int U = 4;
    constexpr int kPer = U * kQThreads;  // float4 groups per iteration
    const uint4 *m4 = reinterpret_cast<const uint4 *>(d.tokmask);
    const int4 *s4 = reinterpret_cast<const int4 *>(d.tok2sel);
    const int4 *c4 = reinterpret_cast<const int4 *>(d.tok2cut);
    float4 *q4 = reinterpret_cast<float4 *>(qrow);
    const int iters = (k_hi - k_lo + kPer - 1) / kPer;
    struct Buf {
        float4 x[U];
        uint4 m[U];
        int4 sl[U];
        int4 c[U];
    };
    auto load = [&](Buf &bf, int it) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = min(k_lo + it * kPer + u * kQThreads + tid, k_hi - 1);
            bf.x[u] = load_nt(prow + 4 * (size_t)k);
            if constexpr (MASK) bf.m[u] = m4[k];
            if constexpr (LISTALL) bf.sl[u] = s4[k];
            if constexpr (RANGES) bf.c[u] = c4[k];
        }
    };
    double hsum = 0.0;
    float tokq = -INFINITY;
    bool have_tok = false;
    static_assert(kPer == kRowChunk4, "one chunk of the token draws per iteration");
    double *tcs_row = SAMP ? tcs + (pos * tcs_nch + k_lo / kRowChunk4) * 4 + wave : nullptr;
    auto compute = [&](const Buf &bf, int it) {
        double ts = 0.0;  // the token draw's chunk sum (SAMP)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k_lo + it * kPer + u * kQThreads + tid;
            const int v = 4 * min(k, k_hi - 1);
            const uint4 m = MASK ? bf.m[u] : make_uint4(0u, 0u, 0u, 0u);
            const int4 sl = LISTALL ? bf.sl[u] : make_int4(-1, -1, -1, -1);
            const int4 c = RANGES ? bf.c[u] : make_int4(-1, -1, -1, -1);
            float4 o;
            o.x = qval(bf.x[u].x, weight_r(v, m.x, sl.x, c.x));
            o.y = qval(bf.x[u].y, weight_r(v + 1, m.y, sl.y, c.y));
            o.z = qval(bf.x[u].z, weight_r(v + 2, m.z, sl.z, c.z));
            o.w = qval(bf.x[u].w, weight_r(v + 3, m.w, sl.w, c.w));
            if (k < k_hi) {
                // plain stores: with p read non-temporally here and in the
                // emission reduce, streaming q through the caches measured
                // 22 us faster per launch (14 us per step) than non-temporal
                // stores
                if (q4) q4[k] = o;
                if (tok >= v && tok < v + 4) {
                    have_tok = true;
                    tokq = tok == v ? o.x : tok == v + 1 ? o.y : tok == v + 2 ? o.z : o.w;
                }
                if (negent) {
                    if (o.x > 0.f) hsum += (double)o.x * log((double)o.x);
                    if (o.y > 0.f) hsum += (double)o.y * log((double)o.y);
                    if (o.z > 0.f) hsum += (double)o.z * log((double)o.z);
                    if (o.w > 0.f) hsum += (double)o.w * log((double)o.w);
                }
                if constexpr (SAMP) {
                    ts += (double)((m.x & dbit) ? bf.x[u].x : 0.f);
                    ts += (double)((m.y & dbit) ? bf.x[u].y : 0.f);
                    ts += (double)((m.z & dbit) ? bf.x[u].z : 0.f);
                    ts += (double)((m.w & dbit) ? bf.x[u].w : 0.f);
                }
            }
        }
        if constexpr (SAMP) {
            if (dbit) {
                const double w = wave_sum_d(ts);
                if (lane == 0 && it < iters) tcs_row[4 * it] = w;
            }
        }
    };
    if (k_hi > k_lo) {
        Buf A, Bn;
        load(A, 0);
        // iteration it sits in A (even) or Bn (odd); loads past the part
        // re-read its last group and an odd count gets one empty iteration
        for (int it = 0; it < iters; it += 2) {
            load(Bn, it + 1);
            compute(A, it);
            load(A, it + 2);
            compute(Bn, it + 1);
        }
    }
    if (negent) {
        hsum = wave_sum_d(hsum);
        if (lane == 0) sh_h[wave] = hsum;
        __syncthreads();
        if (tid == 0) hpart[pos * kQParts + part] = ((sh_h[0] + sh_h[1]) + sh_h[2]) + sh_h[3];
    } else {
        if (have_tok) conf[pos] = tokq;
        if (tid == 0 && part == 0 && tok < 0) conf[pos] = -INFINITY;
    }
}

// NEGENT confidence of the streaming q writer: the parts' fp64 sums of
// q ln q, added in part order (a failed row's parts hold -inf)
__global__ void marg_negent_sum(int npos, const double *__restrict__ hpart,
                                float *__restrict__ conf)
{
    const int pos = blockIdx.x * blockDim.x + threadIdx.x;
    if (pos >= npos) return;
    double s = 0.0;
    for (int k = 0; k < kQParts; ++k) s += hpart[(size_t)pos * kQParts + k];
    conf[pos] = (float)s;
}

// Finish of the joint call, after the token draws (streaming writer tables,
// no ranges).  One wavefront per position.  Rows flagged since the q writer
// ran get what the writer gives a flagged row (q = 0, conf = -inf, q ln q
// parts -inf); otherwise, for FA_CONF_PROB, lane 0 recomputes the sampled
// token's q from the pair weights in global memory with the additions of the
// writer's lookup tables in the same order (per byte of the mask, its set
// bits ascending from 0; the bytes' sums in byte order; then the token-list
// weight), so conf equals the writer's value bit for bit.
//
// It also finishes the sampler's outputs as sample_finalize does: states in
// original ids (-1 for a flagged row) and -1 tokens for a flagged row.
template <int NG, bool SELBIT, bool LISTALL>
__global__ __launch_bounds__(64) void marg_conf_tok(
    DevTable d, StepView sv, const float *__restrict__ p, const double *__restrict__ logZ,
    int32_t *__restrict__ tokens, int conf_mode, float *__restrict__ q,
    float *__restrict__ conf, const int32_t *__restrict__ ea, const int32_t *__restrict__ eb,
    const float *__restrict__ pw, int pw_ld, double *__restrict__ hpart,
    const int32_t *__restrict__ status, const int32_t *__restrict__ zc,
    int32_t *__restrict__ states)
{
    const int b = blockIdx.y, i = blockIdx.x, lane = threadIdx.x;
    const size_t pos = (size_t)b * sv.L + i;
    const bool flagged = status[b] != 0;
    if (lane == 1 || (lane == 2 && i == sv.L - 1)) {  // states i and, for the last, L
        const int k = lane == 1 ? i : sv.L;
        const int zz = zc[(size_t)b * (sv.Lpad + 1) + k];
        states[(size_t)b * (sv.L + 1) + k] = (flagged || zz < 0) ? -1 : d.orig[zz];
    }
    const double lz = logZ[b];
    const int e1 = ea[(size_t)b * (sv.Lpad + 1) + i], e2 = eb[(size_t)b * (sv.Lpad + 1) + i + 1];
    const bool ok = status[b] == 0 && lz > -INFINITY && e1 > kNeg && e2 > kNeg;
    const bool negent = conf_mode == FA_CONF_NEGENT;
    if (!ok) {
        if (q) {
            float *qrow = q + pos * d.V;
            for (int v = lane; v < d.V; v += 64) qrow[v] = 0.f;
        }
        if (negent && lane < kQParts) hpart[pos * kQParts + lane] = -INFINITY;
        if (lane == 0) {
            conf[pos] = -INFINITY;
            if (flagged) tokens[pos] = -1;
        }
        return;
    }
    if (negent || lane != 0) return;
    const int tok = tokens[pos];
    float o = -INFINITY;
    if (tok >= 0) {
        const float *pwr = pw + pos * pw_ld;
        const uint32_t m = (NG > 0 || SELBIT) ? d.tokmask[tok] : 0u;
        float r = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint32_t byte = (m >> (8 * g)) & 255u;
            float sm = 0.f;
            for (int bit = 0; bit < 8; ++bit)
                if ((byte >> bit) & 1u) sm += pwr[8 * g + bit];
            r = g == 0 ? sm : r + sm;
        }
        if (SELBIT && (m & kSelBit)) {
            int lo = 0, hi = d.nsel - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (d.sel_tok[mid] < tok) lo = mid + 1;
                else hi = mid;
            }
            r += pwr[kDenseMax + lo];
        }
        if (LISTALL) {
            const int sl = d.tok2sel[tok];
            if (sl >= 0) r += pwr[kDenseMax + sl];
        }
        const double factor = exp2((double)e1 + (double)e2 - lz * 1.4426950408889634074);
        const float x = p[pos * d.V + tok];
        o = (r > 0.f && x > 0.f) ? (float)((double)x * (double)r * factor) : 0.f;
    }
    conf[pos] = o;
}

// Leaf level of the message pass without reading the leaves.  Each leaf
// holds only the automaton's pairs, whose values are recomputed from the
// emission workspace: a one-token list pair reads p (or its compact copy),
// every other pair the value the leaf writer stored for it, so the values are
// bit-identical to the leaf entries.  One workgroup
// per (leaf pair, alpha|beta): the input weights are normalized as in
// marg_level (leaf scales: ro = co = 0, row fold rf); every thread loads its
// (at most PER) leaf entries and their values at once, and each
// term g[in] * v * 2^-rf[in] goes to LDS in output-grouped order (column
// order for alpha through a row-major leaf, pair order for beta through a
// transposed one); each output state then adds its own segment in order.
// Leaf entries per thread: the smallest of 14, 24, 40 that holds the
// table's pairs.  Fewer held entries take fewer registers, and more
// workgroups fit on a CU at once (69 registers at 14: three per CU, against
// two at 24), which matters because the launch has more workgroups than fit
// (fewer than 14 entries take no fewer registers).
constexpr int kLeafMsgThreads = 512;
constexpr int kLeafMsgPerMax = 40;
constexpr int kLeafMsgMax = kLeafMsgThreads * kLeafMsgPerMax;
static_assert(kLeafMsgMax == kLeafMsgMaxPairs,
              "the table compiler's leafless decision assumes marg_leaf takes this many pairs");

//
// pw (non-null): each workgroup also writes the q writer's pair weights of
// one position (pair_weights; marg_pairw is then not launched): the alpha
// workgroup of leaves (l, l+1) those of position l+1 (alpha_{l+1} its own
// output, beta_{l+2} from the level above), the beta workgroup those of
// position l (alpha_l from the level above, beta_{l+1} its own output).
// md: midpoint draws riding on the launch, md.nwg workgroups before the
// products.
static_assert(kLeafMsgThreads == kPwThreads, "the leaf workgroups run pair_weights");
static_assert(kLeafMsgThreads >= kSubThreads && kMsgThreads >= kSubThreads,
              "message-pass workgroups can carry a midpoint subtree");

template <int PER>
__global__ __launch_bounds__(kLeafMsgThreads) void marg_leaf(
    DevTable d, StepView sv, EmitSrc src, const int32_t *__restrict__ meta,
    float *__restrict__ va, int32_t *__restrict__ ea, float *__restrict__ vb,
    int32_t *__restrict__ eb, float *__restrict__ pw, int pw_nl, int pw_ld, MidDraws md)
{
    if ((int)blockIdx.x < md.nwg) {  // midpoint draws riding on the launch, dispatched first
        mid_draws_wg(d, sv, md, (int)blockIdx.x);
        return;
    }
    // [own output, Sp, with pw] | terms [npairs] | g [S] | rf [S]; after the
    // leaf product the terms region holds pair_weights' scratch
    extern __shared__ float lsh[];
    float *own = lsh;
    float *term = lsh + (pw ? sv.Sp : 0);
    float *gsh = term + d.npairs;
    int *rsh = reinterpret_cast<int *>(gsh + d.S);
    __shared__ int sh_max[kLeafMsgThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nn = sv.Lpad >> 1;
    const int prod = (int)blockIdx.x - md.nwg, beta = prod & 1, bn = prod >> 1;
    const int b = bn / nn, idx = bn % nn;
    const int l = 2 * idx, m = l + 1;
    const int i = beta ? l + 1 : l;  // position of the leaf
    const int h = sv.Lpad + i;
    const int srcpos = beta ? l + 2 : l;
    const bool real = i < sv.L;
    const size_t pos = (size_t)b * sv.L + min(i, max(sv.L - 1, 0));
    float *vbase = beta ? vb : va;
    int32_t *ebase = beta ? eb : ea;
    const float *vin = vbase + ((size_t)b * (sv.Lpad + 1) + srcpos) * sv.Sp;
    float *vout = vbase + ((size_t)b * (sv.Lpad + 1) + m) * sv.Sp;
    const int ein = ebase[(size_t)b * (sv.Lpad + 1) + srcpos];
    const int32_t *rf = sv.meta_ptr(meta, b, h, 2);
    // this thread's leaf entries and their values, all loads issued together
    // (clamped, unconditional)
    const int np = d.npairs;
    const int32_t *erc = beta ? d.ent_n_rc : d.ent_t_rc;
    const int32_t *esrc = beta ? d.ent_n_src : d.ent_t_src;
    const float *direct = d.use_sel ? src.psel + pos * d.nsel : src.p + pos * d.V;
    // indirect pairs read the values the leaf writer stored for them
    const float *indv = src.ndval + pos * d.n_ind;
    int prc[PER];
    float pval[PER];
    if (real && np > 0) {
        int pcode[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int k = min(tid + u * kLeafMsgThreads, np - 1);
            prc[u] = erc[k];
            pcode[u] = esrc[k];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const float xd = direct[max(pcode[u], 0)];
            const float xi = indv[max(-1 - pcode[u], 0)];
            pval[u] = pcode[u] >= 0 ? xd : xi;
        }
    }
    int e = kNeg;
    for (int a = tid; a < d.S; a += kLeafMsgThreads) {
        const float x = vin[a];
        const int sr = rf[a];
        rsh[a] = sr;
        gsh[a] = x;
        if (x > 0.f && sr > kNeg) e = max(e, fexp(x) + sr);
    }
    e = wave_max_i(e);
    if (lane == 0) sh_max[wave] = e;
    __syncthreads();
    int G = kNeg;
    for (int w = 0; w < kLeafMsgThreads / 64; ++w) G = max(G, sh_max[w]);
    for (int a = tid; a < d.S; a += kLeafMsgThreads) {
        const float x = gsh[a];
        const int sr = rsh[a];
        gsh[a] = (x > 0.f && sr > kNeg && G > kNeg) ? scale2(mant(x), fexp(x) + sr - G) : 0.f;
    }
    __syncthreads();
    if (!real) {  // identity leaf: v = 1 on the diagonal
        for (int j = tid; j < sv.Sp; j += kLeafMsgThreads) {
            const float o = j < d.S ? gsh[j] * scale2(1.f, -rsh[j]) : 0.f;
            vout[j] = o;
            if (pw) own[j] = o;
        }
    } else {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int k = tid + u * kLeafMsgThreads;
            if (k < np) {
                const int in = prc[u] & 0xffff;
                term[k] = gsh[in] * scale2(pval[u], -rsh[in]);
            }
        }
        __syncthreads();
        const int32_t *seg = beta ? d.row_ptr : d.col_ptr;
        for (int j = tid; j < sv.Sp; j += kLeafMsgThreads) {
            float acc = 0.f;
            if (j < d.S)
                for (int k = seg[j]; k < seg[j + 1]; ++k) acc += term[k];
            const float o = G > kNeg ? acc : 0.f;
            vout[j] = o;
            if (pw) own[j] = o;
        }
    }
    if (tid == 0)
        ebase[(size_t)b * (sv.Lpad + 1) + m] = (G > kNeg && ein > kNeg) ? ein + G : kNeg;
    // the weights of position l (beta) or l+1 (alpha), a real position
    const int wpos = beta ? l : l + 1;
    if (pw && wpos < sv.L) {
        __syncthreads();  // own complete; the terms region is free
        const size_t vrow = (size_t)b * (sv.Lpad + 1);
        const float *al = beta ? va + (vrow + l) * sv.Sp : own;
        const float *be = beta ? own : vb + (vrow + l + 2) * sv.Sp;
        pair_weights(d, al, be, pw_nl, pw + ((size_t)b * sv.L + wpos) * pw_ld, term);
    }
}

}  // namespace

namespace {

// the leaf level straight from pair values when the leaf entries exist
// (Sp < 65536) and their terms fit in LDS
bool sparse_leaf_ok(const DevTable &d, const Geometry &g)
{
    return g.K >= 1 && leaf_level_from_pairs(d.npairs, d.S, g.Sp);
}

// dynamic LDS of marg_leaf, with or without the pair weights
size_t leaf_lds(const DevTable &d, const Geometry &g, const WsLayout &w, bool pw)
{
    const size_t leaf = (size_t)d.npairs + 2 * (size_t)d.S;
    if (!pw) return leaf * 4;
    const size_t pws = (size_t)std::min(d.n_tm, kPwChunk) + w.pw_nl;
    return ((size_t)g.Sp + std::max(leaf, pws)) * 4;
}

// the leaf level writes the pair weights (and marg_pairw is not launched)
bool leaf_writes_pw(const DevTable &d, const Geometry &g, const WsLayout &w)
{
    return sparse_leaf_ok(d, g) && g.L > 0 && leaf_lds(d, g, w, true) <= kSparseLdsMax;
}

}  // namespace

int launch_marginals(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                     const int32_t *meta, const double *logZ, const int32_t *tokens,
                     int32_t conf_mode, float *q, float *conf, uint8_t *ws, const WsLayout &w,
                     int32_t *status, void *stream)
{
    int rc = launch_marg_pass(d, g, p, tree, meta, ws, w, stream, false, 0, status);
    if (rc) return rc;
    return launch_marg_out(d, g, p, logZ, tokens, conf_mode, q, conf, ws, w, 0, status, stream,
                           nullptr);
}

int launch_marg_pass(const DevTable &d, const Geometry &g, const float *p, const float *tree,
                     const int32_t *meta, uint8_t *ws, const WsLayout &w, void *stream,
                     bool ride, uint64_t seed, int32_t *status)
{
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    if (d.leafless && g.K >= 1) sv.pvf = (const float *)(ws + w.pvf);   // the riding leaf-level draws
    float *va = (float *)(ws + w.va), *vb = (float *)(ws + w.vb);
    int32_t *ea = (int32_t *)(ws + w.ea), *eb = (int32_t *)(ws + w.eb);
    float *rcut = (float *)(ws + w.rcut);
    const size_t lds = (size_t)g.Sp * (sizeof(float) + sizeof(int));
    const bool sparse_leaf = sparse_leaf_ok(d, g);
    // a leafless table wrote no dense leaves: its leaf level must take the pairs
    if (d.leafless && g.K >= 1 && !sparse_leaf) return (int)hipErrorInvalidValue;
    // the boundary vectors: built by the top marg_level launch, else here
    const bool init_in_top = g.K >= 1 && !(g.K == 1 && sparse_leaf);
    hipError_t e;
    if (!init_in_top) {
        marg_init<<<g.B, 256, 0, st>>>(d, sv, va, ea, vb, eb);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    if (lds > 48 * 1024) {  // large automata: allow the dynamic LDS the kernels need
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&marg_level<256>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&marg_level<64>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
    }
    // the midpoint launches (kSubDepth levels each) ride on the last ones of
    // the message pass, which take longer than they do; both depend only on
    // the tree, and the launches of each chain stay in order
    const int nmid = (g.K + kSubDepth - 1) / kSubDepth;
    auto draws_for = [&](int level) {
        MidDraws m{tree, meta, seed, 0, 0, 0, (int32_t *)(ws + w.zc), (int32_t *)(ws + w.tpair),
                   (uint32_t *)(ws + w.tdbit), status};
        const int j = level - (g.K - nmid + 1);
        if (ride && j >= 0 && j < nmid) {
            m.level0 = 1 + j * kSubDepth;
            m.depth = std::min(kSubDepth, g.K - m.level0 + 1);
            m.nwg = g.B << (m.level0 - 1);
        }
        return m;
    };
    for (int level = 1; level <= g.K; ++level) {
        const int nn = 1 << (level - 1);
        const int products = g.B * nn * 2;
        const MidDraws md = draws_for(level);
        if (level == g.K && sparse_leaf) {
            const bool wpw = leaf_writes_pw(d, g, w);
            const size_t llds = leaf_lds(d, g, w, wpw);
            float *pw = wpw ? (float *)(ws + w.pw) : nullptr;
            const EmitSrc src = emit_src(d, g, p, ws, w);
            auto leaf = [&](auto kernel) -> hipError_t {
                if (llds > 48 * 1024) {
                    const hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                                             (int)llds);
                    if (a != hipSuccess) return a;
                }
                kernel<<<products + md.nwg, kLeafMsgThreads, llds, st>>>(d, sv, src, meta, va, ea, vb, eb,
                                                                       pw, w.pw_nl, w.pw_ld, md);
                return hipGetLastError();
            };
            const int np = d.npairs;
            if (np <= kLeafMsgThreads * 14) e = leaf(&marg_leaf<14>);
            else if (np <= kLeafMsgThreads * 24) e = leaf(&marg_leaf<24>);
            else e = leaf(&marg_leaf<kLeafMsgPerMax>);
            if (e != hipSuccess) return (int)e;
            continue;
        }
        const int top = level == 1 && init_in_top;
        if (products * ((g.Sp + 255) / 256) >= 256) {
            dim3 grid((g.Sp + 255) / 256, products + md.nwg);
            marg_level<256><<<grid, kMsgThreads, lds, st>>>(d, sv, tree, meta, nn, va, ea, vb, eb, top,
                                                            md);
        } else {
            dim3 grid((g.Sp + 63) / 64, products + md.nwg);
            marg_level<64><<<grid, kMsgThreads, lds, st>>>(d, sv, tree, meta, nn, va, ea, vb, eb, top,
                                                           md);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    if (d.ncut) {
        const int npos = g.B * g.L;
        const size_t ab = (size_t)2 * g.Sp * sizeof(float);
        const int ab_lds = ab <= 48 * 1024;
        marg_rcut<<<npos, kRcutThreads, ab_lds ? ab : 0, st>>>(d, sv, va, vb, rcut, ab_lds);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

namespace {

// rsel [nsel] | selk [nsel] and its 256-token index (selbit) | rcl [ncut]
size_t q_stream_lds(const DevTable &d)
{
    return (d.nsel > 0 ? (size_t)d.nsel * (d.selbit ? 8 : 4) : 0) +
           (d.nsel > 0 && d.selbit ? ((size_t)d.V / 256 + 2) * 4 : 0) +
           (d.ncut > 0 ? (size_t)d.ncut * 4 : 0);
}

// streaming q writer: float4 rows and every lookup table in LDS
bool q_streamed(const DevTable &d, const float *p, const float *q, const WsLayout &w)
{
    const bool aligned = ((uintptr_t)p & 15) == 0 && ((uintptr_t)q & 15) == 0;
    return (d.V & 3) == 0 && aligned && q_stream_lds(d) <= kQLdsMax &&
           (d.nsel == 0 || w.pw_nl == d.nsel);
}

}  // namespace

namespace {

// the unconstrained score: the denoiser's probability of the sampled token,
// -inf on flagged rows (as the constrained score gives them)
__global__ void conf_unconstrained(const float *__restrict__ p, int V, int L, long long npos,
                                   const int32_t *__restrict__ tokens,
                                   const int32_t *__restrict__ status, float *__restrict__ conf)
{
    const long long pos = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (pos >= npos) return;
    const int b = (int)(pos / L);
    const int tok = tokens[pos];
    conf[pos] = (status[b] == 0 && tok >= 0 && tok < V) ? p[pos * V + tok] : -INFINITY;
}

}  // namespace

int launch_conf_unconstrained(const DevTable &d, const Geometry &g, const float *p,
                              const int32_t *tokens, const int32_t *status, float *conf,
                              void *stream)
{
    const long long npos = (long long)g.B * g.L;
    if (npos == 0) return 0;
    conf_unconstrained<<<(unsigned)((npos + 255) / 256), 256, 0, (hipStream_t)stream>>>(
        p, d.V, g.L, npos, tokens, status, conf);
    return (int)hipGetLastError();
}

bool marg_joint_ok(const DevTable &d, const Geometry &g, const float *p, const float *q,
                   int32_t conf_mode, const WsLayout &w)
{
    // the token draws stream dense rows of at most kTokChunksMax chunks; the
    // q writer streams the row only when it writes q or sums q ln q
    return g.L > 0 && d.ndense > 0 && q_streamed(d, p, q, w) &&
           (q != nullptr || conf_mode == FA_CONF_NEGENT) && w.tcs_nch <= kTokChunksMax;
}

int launch_marg_from_messages(const DevTable &d, const Geometry &g, const float *p,
                              const double *logZ, const int32_t *tokens, int32_t conf_mode,
                              float *q, float *conf, uint8_t *ws, const WsLayout &w,
                              int32_t *status, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    const float *va = (const float *)(ws + w.va), *vb = (const float *)(ws + w.vb);
    hipError_t e;
    if (d.ncut) {
        float *rcut = (float *)(ws + w.rcut);
        const int npos = g.B * g.L;
        const size_t ab = (size_t)2 * g.Sp * sizeof(float);
        const int ab_lds = ab <= 48 * 1024;
        marg_rcut<<<npos, kRcutThreads, ab_lds ? ab : 0, st>>>(d, sv, va, vb, rcut, ab_lds);
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    // the streaming writer's pair weights: on tables whose tree path forms
    // them in the message pass's leaf level, the plain writer does not
    if (q_streamed(d, p, q, w) && leaf_writes_pw(d, g, w)) {
        const size_t plds = w.pw_nl ? ((size_t)std::min(d.n_tm, kPwChunk) + w.pw_nl) * 4 : 0;
        if (plds > 48 * 1024) {
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&marg_pairw),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)plds);
            if (e != hipSuccess) return (int)e;
        }
        marg_pairw<<<g.B * g.L, kPwThreads, plds, st>>>(d, sv, va, vb, w.pw_nl, w.pw_ld,
                                                         (float *)(ws + w.pw));
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return launch_marg_out(d, g, p, logZ, tokens, conf_mode, q, conf, ws, w, 0, status, stream,
                           nullptr);
}

int launch_marg_out(const DevTable &d, const Geometry &g, const float *p, const double *logZ,
                    const int32_t *tokens, int32_t conf_mode, float *q, float *conf, uint8_t *ws,
                    const WsLayout &w, int mode, int32_t *status, void *stream, int32_t *states)
{
    hipStream_t st = (hipStream_t)stream;
    StepView sv = step_view(g);
    float *va = (float *)(ws + w.va), *vb = (float *)(ws + w.vb);
    int32_t *ea = (int32_t *)(ws + w.ea), *eb = (int32_t *)(ws + w.eb);
    float *rcut = (float *)(ws + w.rcut);
    hipError_t e;
    // the generic writer: kQParts workgroups per position on short batches
    const int qparts = g.B * g.L < 1024 ? kQParts : 1;
    const dim3 qgrid(g.L * qparts, g.B);
    const int ng = (d.ndense + 7) / 8;
    const bool listall = d.nsel > 0 && !d.selbit;
    const bool ranges = d.ncut > 0;
    const size_t qlds = q_stream_lds(d);
    const bool streamed = q_streamed(d, p, q, w);
    if (mode != 0 && !(streamed && ng > 0 && !ranges)) return (int)hipErrorInvalidValue;
    if (streamed) {
        const int npos = g.B * g.L;
        float *pw = (float *)(ws + w.pw);
        double *hpart = (double *)(ws + w.hpart);
        const uint32_t *tdbit = (const uint32_t *)(ws + w.tdbit);
        double *tcs = mode == 1 ? (double *)(ws + w.tcs) : nullptr;
        int32_t *tcs_ok = mode == 1 ? (int32_t *)(ws + w.tcs_ok) : nullptr;
        const dim3 sgrid(g.L * kQParts, g.B);
        if (mode != 2 && !leaf_writes_pw(d, g, w)) {  // else the leaf level wrote them
            const size_t plds = w.pw_nl ? ((size_t)std::min(d.n_tm, kPwChunk) + w.pw_nl) * 4 : 0;
            if (plds > 48 * 1024) {
                e = hipFuncSetAttribute(reinterpret_cast<const void *>(&marg_pairw),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)plds);
                if (e != hipSuccess) return (int)e;
            }
            marg_pairw<<<npos, kPwThreads, plds, st>>>(d, sv, va, vb, w.pw_nl, w.pw_ld, pw);
            e = hipGetLastError();
            if (e != hipSuccess) return (int)e;
        }
        if (mode == 2) {
            const dim3 cgrid(g.L, g.B);
#define FA_MARG_CT(NG, SB, LA)                                                                 \
    marg_conf_tok<NG, SB, LA><<<cgrid, 64, 0, st>>>(d, sv, p, logZ, (int32_t *)tokens, conf_mode, \
                                                    q, conf, ea, eb, pw, w.pw_ld, hpart, status, \
                                                    (const int32_t *)(ws + w.zc), states)
            if (d.selbit) {
                if (ng == 1) FA_MARG_CT(1, true, false);
                else if (ng == 2) FA_MARG_CT(2, true, false);
                else if (ng == 3) FA_MARG_CT(3, true, false);
                else FA_MARG_CT(4, true, false);
            } else if (listall) {
                FA_MARG_CT(4, false, true);
            } else {
                if (ng == 1) FA_MARG_CT(1, false, false);
                else if (ng == 2) FA_MARG_CT(2, false, false);
                else if (ng == 3) FA_MARG_CT(3, false, false);
                else FA_MARG_CT(4, false, false);
            }
#undef FA_MARG_CT
            e = hipGetLastError();
            if (e != hipSuccess) return (int)e;
            if (conf_mode == FA_CONF_NEGENT)
                marg_negent_sum<<<(npos + 255) / 256, 256, 0, st>>>(npos, hpart, conf);
            return (int)hipGetLastError();
        }
        const bool samp = mode == 1;
#define FA_MARG_QS_K(NG, SB, LA, RG, SA)                                                          \
    do {                                                                                          \
        auto kern = &marg_q_stream<NG, SB, LA, RG, SA>;                                           \
        if (qlds > 48 * 1024) {                                                                   \
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),                         \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)qlds);       \
            if (e != hipSuccess) return (int)e;                                                   \
        }                                                                                         \
        e = (hipError_t)prof_mark(FA_PROF_MARG_Q, true, stream);                                  \
        if (e != hipSuccess) return (int)e;                                                       \
        kern<<<sgrid, kQThreads, qlds, st>>>(d, sv, p, logZ, tokens, conf_mode, q, conf, ea, eb, \
                                             pw, w.pw_ld, rcut, hpart, status, tdbit, tcs, tcs_ok,\
                                             w.tcs_nch);                                          \
    } while (0)
#define FA_MARG_QS(NG, SB, LA, RG)                                                                \
    do {                                                                                          \
        if (samp) FA_MARG_QS_K(NG, SB, LA, RG, true);                                             \
        else FA_MARG_QS_K(NG, SB, LA, RG, false);                                                 \
    } while (0)
#define FA_MARG_QS0(NG, SB, LA, RG) FA_MARG_QS_K(NG, SB, LA, RG, false)
        if (ranges) {
            if (listall) FA_MARG_QS0(0, false, true, true);
            else FA_MARG_QS0(0, false, false, true);
        } else if (ng == 0) {
            if (listall) FA_MARG_QS0(0, false, true, false);
            else FA_MARG_QS0(0, false, false, false);
        } else if (d.selbit) {
            if (ng == 1) FA_MARG_QS(1, true, false, false);
            else if (ng == 2) FA_MARG_QS(2, true, false, false);
            else if (ng == 3) FA_MARG_QS(3, true, false, false);
            else FA_MARG_QS(4, true, false, false);
        } else if (listall) {
            FA_MARG_QS(4, false, true, false);
        } else {
            if (ng == 1) FA_MARG_QS(1, false, false, false);
            else if (ng == 2) FA_MARG_QS(2, false, false, false);
            else if (ng == 3) FA_MARG_QS(3, false, false, false);
            else FA_MARG_QS(4, false, false, false);
        }
#undef FA_MARG_QS
#undef FA_MARG_QS0
#undef FA_MARG_QS_K
        e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
        const int pe = prof_mark(FA_PROF_MARG_Q, false, stream);
        if (pe) return pe;
        // mode 1 leaves the confidence to mode 2
        if (conf_mode == FA_CONF_NEGENT && mode != 1) {
            marg_negent_sum<<<(npos + 255) / 256, 256, 0, st>>>(npos, hpart, conf);
            e = hipGetLastError();
        }
        return (int)e;
    }
    double *hpart = (double *)(ws + w.hpart);
    e = (hipError_t)prof_mark(FA_PROF_MARG_Q, true, stream);
    if (e != hipSuccess) return (int)e;
#define FA_MARG_Q(NG, SB, LA, RG)                                                              \
    marg_q<NG, SB, LA, RG><<<qgrid, kQThreads, 0, st>>>(d, sv, p, logZ, tokens, conf_mode, q,  \
                                                        conf, va, ea, vb, eb, rcut, hpart, qparts, status)
    if (ranges) {
        if (listall) FA_MARG_Q(0, false, true, true);
        else FA_MARG_Q(0, false, false, true);
    } else if (ng == 0) {
        if (listall) FA_MARG_Q(0, false, true, false);
        else FA_MARG_Q(0, false, false, false);
    } else if (d.selbit) {
        if (ng == 1) FA_MARG_Q(1, true, false, false);
        else if (ng == 2) FA_MARG_Q(2, true, false, false);
        else if (ng == 3) FA_MARG_Q(3, true, false, false);
        else FA_MARG_Q(4, true, false, false);
    } else if (listall) {  // 32 dense pairs leave no flag bit for token-list tokens
        FA_MARG_Q(4, false, true, false);
    } else {
        if (ng == 1) FA_MARG_Q(1, false, false, false);
        else if (ng == 2) FA_MARG_Q(2, false, false, false);
        else if (ng == 3) FA_MARG_Q(3, false, false, false);
        else FA_MARG_Q(4, false, false, false);
    }
#undef FA_MARG_Q
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const int pe = prof_mark(FA_PROF_MARG_Q, false, stream);
    if (pe) return pe;
    if (conf_mode == FA_CONF_NEGENT && qparts > 1) {
        const int npos = g.B * g.L;
        marg_negent_sum<<<(npos + 255) / 256, 256, 0, st>>>(npos, hpart, conf);
        e = hipGetLastError();
    }
    return (int)e;
}

}  // namespace fa
