"""GPU parity of the serial chain sampler (fa_chain_sample: forward
filtering, then backward sampling) against the fp64 oracle: log Z, and every
state and token draw replayed by the oracle's FFBS verifier under the same
keyed uniforms (bit-exact except NEAR draws, whose uniform lies within 1e-6
of every CDF boundary between the two choices); and of the chain's whole
forward-backward step (fa_chain_sample_marginals): q and the confidence from
its two message chains against the oracle's marginals."""
import numpy as np
import pytest

import oracle
from synth import configs
from tests import parity as PT
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


def run_chain(w, table=None):
    import torch
    import constrained_decoding_diffusion_amd as fa
    tb = table or fa.Table.from_automaton(w.aut, first_level="dense")
    p = torch.from_numpy(w.p).cuda()
    bufs = fa.chain_step(tb, p, w.seed)
    torch.cuda.synchronize()
    return dict(table=tb, logZ=bufs.logZ.cpu().numpy(), status=bufs.status.cpu().numpy(),
                states=bufs.states.cpu().numpy(), tokens=bufs.tokens.cpu().numpy()[:, :w.L])


def check_chain_row(w, g, b, orc):
    W = orc.edge_weights(w.p[b])
    fb = orc.forward_backward(W)
    if fb["status"] != oracle.OK:
        assert g["status"][b] & 1, f"row {b}: oracle infeasible, GPU status {g['status'][b]}"
        assert g["logZ"][b] == -np.inf
        assert (g["states"][b] == -1).all() and (g["tokens"][b] == -1).all()
        return None
    assert g["status"][b] == 0, f"row {b}: status {g['status'][b]}"
    lz = fb["logZ"]
    assert abs(g["logZ"][b] - lz) <= PT.LOGZ_RTOL * max(1.0, abs(lz)), (b, g["logZ"][b], lz)
    rep = orc.chain_verify(w.p[b], W, fb, w.seed, b, g["states"][b], g["tokens"][b])
    assert rep["status"] == oracle.OK and rep["hard"] == 0, f"row {b}: {rep}"
    if rep["near"] == 0:
        st, tk, s2 = orc.chain_sample(w.p[b], W, fb, w.seed, b)
        np.testing.assert_array_equal(g["states"][b], st)
        np.testing.assert_array_equal(g["tokens"][b], tk)
    return rep


@pytest.mark.parametrize("name", list(CASES))
def test_chain_parity(name):
    w = CASES[name]()
    PT.log(f"[chain] {name}: {w.describe()}")
    g = run_chain(w)
    orc = oracle.Oracle(w.aut)
    near = draws = 0
    for b in range(w.B):
        rep = check_chain_row(w, g, b, orc)
        near += rep["near"] if rep else 0
        draws += rep["draws"] if rep else 0
    PT.log(f"[chain] {name}: ok, near {near} of {draws}")
    assert near <= 0.01 * max(draws, 1)


def test_chain_refuses_leafless_tables_and_flags_rows():
    import torch
    import constrained_decoding_diffusion_amd as fa
    w = CASES["range-small"]()
    tb = fa.Table.from_automaton(w.aut)
    if tb.info["leafless"]:
        with pytest.raises(fa.FaError) as ei:
            fa.chain_step(tb, torch.from_numpy(w.p).cuda(), 1)
        assert ei.value.code == 1
    w = configs.make(2, B=3, L=16)
    aut = w.aut
    first = set()
    for e in range(aut.E):
        if aut.src[e] == aut.start:
            first |= set(aut.edge_label(e).tolist())
    bad = next(v for v in range(aut.V) if v not in first)
    w.p[1, 0] = 0.0
    w.p[1, 0, bad] = 1.0
    w.p[2, 5, int(aut.label_tok[0])] = np.nan
    g = run_chain(w)
    check_chain_row(w, g, 0, oracle.Oracle(aut))
    assert g["status"][1] & 1 and g["status"][2] & 4
    for b in (1, 2):
        assert g["logZ"][b] == -np.inf
        assert (g["states"][b] == -1).all() and (g["tokens"][b] == -1).all()
    # L = 0
    tb = fa.Table.from_automaton(configs.make(1).aut)
    bufs = fa.chain_step(tb, torch.zeros((2, 0, 12), dtype=torch.float32, device="cuda"), 1)
    torch.cuda.synchronize()
    assert (bufs.logZ.cpu().numpy() == -np.inf).all()


def test_chain_and_tree_agree_on_log_z():
    """Both samplers of one posterior: log Z within the parity tolerance of
    each other, and (the same law) each accepted by its own replay."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    w = CASES["json-small"]()
    tb = fa.Table.from_automaton(w.aut, first_level="dense")
    g = run_chain(w, table=tb)
    bt = fa.step(tb, torch.from_numpy(w.p).cuda(), w.seed)
    torch.cuda.synchronize()
    np.testing.assert_allclose(g["logZ"], bt.logZ.cpu().numpy(), rtol=2e-5, atol=1e-6)


def test_chain_json_like_full():
    w = configs.make(3)
    PT.log(f"[chain-full] {w.describe()}")
    g = run_chain(w)
    PT.log(f"[chain-full] gpu done, logZ {g['logZ']}")
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        rep = check_chain_row(w, g, b, orc)
        PT.log(f"[chain-full] row {b}: ok ({rep})")


def run_chain_marg(w, table=None, conf_mode=0, write_q=True):
    """fa_chain_sample_marginals: the chain's states, tokens and log Z, and
    the marginals from its forward and backward message chains."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    tb = table or fa.Table.from_automaton(w.aut, first_level="dense")
    p = torch.from_numpy(w.p).cuda()
    bufs = fa.chain_step(tb, p, w.seed, marginals=True, conf_mode=conf_mode, write_q=write_q)
    torch.cuda.synchronize()
    return dict(table=tb, logZ=bufs.logZ.cpu().numpy(), status=bufs.status.cpu().numpy(),
                states=bufs.states.cpu().numpy(), tokens=bufs.tokens.cpu().numpy()[:, :w.L],
                conf=bufs.conf.cpu().numpy()[:, :w.L],
                q=bufs.q.cpu().numpy() if write_q else None)


def check_chain_marginals(w, g, b, orc, positions=None, conf_mode=0):
    """Row b's q and conf against the oracle's, at the tree path's tolerances."""
    W = orc.edge_weights(w.p[b])
    fb = orc.forward_backward(W)
    if fb["status"] != oracle.OK:
        if g["q"] is not None:
            assert (g["q"][b] == 0).all()
        assert (g["conf"][b] == -np.inf).all()
        return
    pos = np.arange(w.L) if positions is None else np.asarray(positions)
    q, _, conf = orc.marginals(w.p[b], fb, pos, g["tokens"][b], conf_mode)
    if g["q"] is not None:
        qg = g["q"][b, pos].astype(np.float64)
        err = np.abs(qg - q)
        bad = err > PT.Q_RTOL * q + PT.Q_ATOL
        assert not bad.any(), (f"row {b}: {bad.sum()} q entries out of tolerance, worst "
                               f"{np.max(err - PT.Q_RTOL * q)} at {np.argwhere(bad)[:5]}")
        assert (err.sum(axis=1) <= PT.Q_L1).all()
    cg = g["conf"][b, pos].astype(np.float64)
    if conf_mode == 0:
        np.testing.assert_allclose(cg, conf, rtol=1e-4, atol=1e-12)
    else:
        np.testing.assert_allclose(cg, conf, rtol=1e-4, atol=1e-6)


@pytest.mark.parametrize("name", list(CASES))
def test_chain_marginals_parity(name):
    w = CASES[name]()
    PT.log(f"[chain-marg] {name}: {w.describe()}")
    g = run_chain_marg(w)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        check_chain_row(w, g, b, orc)
        check_chain_marginals(w, g, b, orc)
    PT.log(f"[chain-marg] {name}: ok")


@pytest.mark.parametrize("name", ["real-number", "json-small", "nfa-small"])
def test_chain_marginals_negentropy_and_no_q(name):
    w = CASES[name]()
    PT.log(f"[chain-marg-negent] {name}")
    orc = oracle.Oracle(w.aut)
    g = run_chain_marg(w, conf_mode=1, write_q=False)
    for b in range(w.B):
        check_chain_marginals(w, g, b, orc, conf_mode=1)


def test_chain_marginals_flagged_rows_and_tree_agreement():
    """Flagged rows come out as on the tree path; on a feasible table the
    chain's q agrees with the tree step's within the parity tolerance."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    w = configs.make(2, B=3, L=16)
    aut = w.aut
    first = set()
    for e in range(aut.E):
        if aut.src[e] == aut.start:
            first |= set(aut.edge_label(e).tolist())
    bad = next(v for v in range(aut.V) if v not in first)
    w.p[1, 0] = 0.0
    w.p[1, 0, bad] = 1.0
    w.p[2, 5, int(aut.label_tok[0])] = np.nan
    g = run_chain_marg(w)
    orc = oracle.Oracle(aut)
    check_chain_row(w, g, 0, orc)
    check_chain_marginals(w, g, 0, orc)
    for b in (1, 2):
        assert g["logZ"][b] == -np.inf
        assert (g["q"][b] == 0).all() and (g["conf"][b] == -np.inf).all()
    w = CASES["json-small"]()
    tb = fa.Table.from_automaton(w.aut, first_level="dense")
    g = run_chain_marg(w, table=tb)
    bt = fa.step(tb, torch.from_numpy(w.p).cuda(), w.seed)
    torch.cuda.synchronize()
    qt = bt.q.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g["q"] - qt) <= 2 * PT.Q_RTOL * qt + PT.Q_ATOL)


def test_chain_marginals_json_like_full():
    w = configs.make(3)
    PT.log(f"[chain-marg-full] {w.describe()}")
    g = run_chain_marg(w)
    orc = oracle.Oracle(w.aut)
    rng = np.random.default_rng(5)
    for b in range(w.B):
        check_chain_row(w, g, b, orc)
        pos = np.sort(rng.choice(w.L, 12, replace=False))
        check_chain_marginals(w, g, b, orc, positions=pos)
        PT.log(f"[chain-marg-full] row {b}: ok")
