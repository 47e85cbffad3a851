"""GPU parity of the serial chain sampler (fa_chain_sample: forward
filtering, then backward sampling) against the fp64 oracle: log Z, and every
state and token draw replayed by the oracle's FFBS verifier under the same
keyed uniforms (bit-exact except NEAR draws, whose uniform lies within 1e-6
of every CDF boundary between the two choices)."""
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
