"""Shared helpers of the GPU parity tests: run one step through the C ABI
and compare it with the fp64 oracle.

Tolerances (fp32 path against the fp64 oracle):
  log Z:      |d| <= 1e-4 * max(1, |log Z|)
  marginals:  |d| <= 1e-4 * q_oracle + 1e-12 per entry, and sum_v |d| <= 1e-4
              per position (the absolute floor sits far below anything a
              draw can resolve: u has 24 bits)
  draws:      bit-exact under shared uniforms, except NEAR draws whose
              uniform lies within 1e-6 of a CDF boundary between the two
              choices (oracle replay verifier)
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

LOGZ_RTOL = 1e-4
Q_RTOL = 1e-4
Q_ATOL = 1e-12
Q_L1 = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w, conf_mode=0, write_q=True, table=None, p_dev=None, joint=True):
    import torch
    import constrained_decoding_diffusion_amd as fa
    tb = table or fa.Table.from_automaton(w.aut)
    p = p_dev if p_dev is not None else torch.from_numpy(w.p).cuda()
    bufs = fa.step(tb, p, w.seed, conf_mode=conf_mode, write_q=write_q, joint=joint)
    torch.cuda.synchronize()
    out = dict(table=tb, bufs=bufs,
               logZ=bufs.logZ.cpu().numpy(), status=bufs.status.cpu().numpy(),
               states=bufs.states.cpu().numpy(), tokens=bufs.tokens.cpu().numpy()[:, :w.L],
               conf=bufs.conf.cpu().numpy()[:, :w.L])
    out["q"] = bufs.q.cpu().numpy() if (write_q and bufs.q is not None) else None
    return out


def leaf(w, g, b, i):
    """GPU leaf of position i of row b as a dense M over compact states."""
    tb = g["table"]
    Sp, S = tb.info["Sp"], tb.info["S"]
    Lpad = 1 << max(0, (w.L - 1).bit_length())
    h = Lpad + i
    tree = g["bufs"].tree.view(w.B, 2 * Lpad, Sp, Sp)
    M = tree[b, h].cpu().numpy().astype(np.float64)
    if h % 2 == 1 and h >= 3:
        M = M.T
    return M[:S, :S]


def check_row(w, g, b, orc=None, q_positions=None, check_q=True, conf_mode=0):
    """Compare row b of a GPU step with the oracle; returns the replay report."""
    orc = orc or oracle.Oracle(w.aut)
    W = orc.edge_weights(w.p[b])
    fb = orc.forward_backward(W)
    if fb["status"] != oracle.OK:
        assert g["status"][b] & 1, f"row {b}: oracle infeasible, GPU status {g['status'][b]}"
        assert g["logZ"][b] == -np.inf
        assert (g["states"][b] == -1).all() and (g["tokens"][b] == -1).all()
        return None
    assert g["status"][b] == 0, f"row {b}: GPU status {g['status'][b]}"
    lz = fb["logZ"]
    assert abs(g["logZ"][b] - lz) <= LOGZ_RTOL * max(1.0, abs(lz)), (b, g["logZ"][b], lz)
    rep = orc.replay(w.p[b], W, w.seed, b, g["states"][b], g["tokens"][b])
    assert rep["status"] == oracle.OK, rep
    assert rep["hard"] == 0, f"row {b}: replay {rep}"
    if check_q:
        pos = np.arange(w.L) if q_positions is None else np.asarray(q_positions)
        q, lognorm, conf = orc.marginals(w.p[b], fb, pos, g["tokens"][b], conf_mode)
        if g["q"] is not None:
            qg = g["q"][b, pos].astype(np.float64)
            err = np.abs(qg - q)
            bad = err > Q_RTOL * q + Q_ATOL
            assert not bad.any(), (f"row {b}: {bad.sum()} q entries out of tolerance, worst "
                                   f"{np.max(err - Q_RTOL * q)} at {np.argwhere(bad)[:5]}")
            assert (err.sum(axis=1) <= Q_L1).all()
        cg = g["conf"][b, pos].astype(np.float64)
        if conf_mode == 0:
            np.testing.assert_allclose(cg, conf, rtol=1e-4, atol=1e-12)
        elif conf_mode == 2:   # p at the sampled token: a copy of an fp32 value
            np.testing.assert_array_equal(cg, conf)
        else:
            np.testing.assert_allclose(cg, conf, rtol=1e-4, atol=1e-6)
    return rep


LEAF_RTOL = 1e-5
LEAF_BIAS = 1e-6


def check_leaves(w, g, b, positions, orc=None):
    """Every leaf entry within LEAF_RTOL of the oracle's M_i, and no
    systematic drift: the mass-weighted relative error of each leaf,
    sum(M_gpu - M) / sum(M), averaged over the positions, stays within
    LEAF_BIAS.  A drift compounds along the chain of products (-2e-6 per
    position reached 1e-4 in the marginals after 16 positions), so it is
    checked on its own."""
    tb = g["table"]
    orc = orc or oracle.Oracle(w.aut)
    if tb.info["leafless"] and w.L > 1:
        # no dense leaves: their values are checked through the first-level
        # nodes, each the product of two leaves, with the drift bound of two
        check_span_nodes(w, g, b, orc, level=1)
        return
    orig = tb.orig
    W = orc.edge_weights(w.p[b])
    drift = []
    for i in positions:
        M = orc.dense_M(W, i)[np.ix_(orig, orig)]
        Mg = leaf(w, g, b, i)
        np.testing.assert_allclose(Mg, M, rtol=LEAF_RTOL, atol=1e-30)
        if M.sum() > 0:
            drift.append(float((Mg - M).sum() / M.sum()))
    if drift:
        bias = float(np.mean(drift))
        assert abs(bias) <= LEAF_BIAS, f"row {b}: leaf drift {bias:.3g}"


NODE_RTOL = 3e-5


def span_node(w, g, b, n):
    """Tree node n of row b as the true span matrix over compact states
    (stored values times 2^ro per row and 2^co per column, right children
    transposed back)."""
    tb = g["table"]
    Sp, S = tb.info["Sp"], tb.info["S"]
    Lpad = 1 << max(0, (w.L - 1).bit_length())
    tree = g["bufs"].tree.view(w.B, 2 * Lpad, Sp, Sp)
    meta = g["bufs"].meta[: w.B * 2 * Lpad * 3 * Sp].view(w.B, 2 * Lpad, 3, Sp)
    D = tree[b, n].cpu().numpy().astype(np.float64)
    ro = meta[b, n, 0].cpu().numpy().astype(np.float64)
    co = meta[b, n, 1].cpu().numpy().astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        T = D * np.exp2(ro)[:, None] * np.exp2(co)[None, :]
    T[D == 0] = 0.0
    if n % 2 == 1 and n >= 3:
        T = T.T
    return T[:S, :S]


def check_span_nodes(w, g, b, orc, level=1):
    """Every node of one tree level (spans of 2^level positions) against the
    product of the oracle's M_i over its span: entries within NODE_RTOL, and
    the mass-weighted relative error sum(P_gpu - P) / sum(P), averaged over
    the nodes, within 2^level * LEAF_BIAS (each leaf may carry LEAF_BIAS)."""
    tb = g["table"]
    orig = tb.orig
    S = len(orig)
    Lpad = 1 << max(0, (w.L - 1).bit_length())
    span = 1 << level
    if Lpad < span:
        return
    W = orc.edge_weights(w.p[b])

    def M(i):
        if i >= w.L:
            return np.eye(S)
        return orc.dense_M(W, i)[np.ix_(orig, orig)]

    drift = []
    for j in range(Lpad // span):
        want = M(span * j)
        for i in range(span * j + 1, span * j + span):
            want = want @ M(i)
        got = span_node(w, g, b, Lpad // span + j)
        scale = want.max(axis=1, keepdims=True)
        err = np.abs(got - want)
        bad = err > NODE_RTOL * want + 1e-30 * scale
        assert not bad.any(), (f"row {b} node {Lpad // span + j}: {bad.sum()} entries off, worst "
                               f"rel {np.max(err / np.maximum(want, 1e-300))}")
        if span * j < w.L and want.sum() > 0:
            drift.append(float((got - want).sum() / want.sum()))
    if drift:
        bias = float(np.mean(drift))
        assert abs(bias) <= span * LEAF_BIAS, f"row {b} level {level}: drift {bias:.3g}"
