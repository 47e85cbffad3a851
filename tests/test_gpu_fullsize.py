"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: log Z of every row, every draw replayed by the oracle, and
marginals and leaves at sampled positions."""
import numpy as np
import pytest

import oracle
from synth import configs
from tests import parity as PT

pytestmark = pytest.mark.gpu


def _sampled_positions(L, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(L, size=min(k, L), replace=False))


def test_json_like_full():
    w = configs.make(3)
    PT.log(f"[full] {w.describe()}")
    g = PT.run_gpu(w)
    PT.log(f"[full] json-like: gpu done, logZ {g['logZ']}")
    orc = oracle.Oracle(w.aut)
    near = 0
    for b in range(w.B):
        pos = _sampled_positions(w.L, 16, 100 + b)
        rep = PT.check_row(w, g, b, orc, q_positions=pos)
        near += rep["near"]
        PT.check_leaves(w, g, b, pos[:3], orc)
        PT.log(f"[full] json-like row {b}: ok ({rep})")
    # NEAR draws are allowed; they should stay rare
    assert near <= 0.01 * 4 * 2 * w.L


def test_json_like_full_negentropy():
    """The entropy confidence at full size (q not written), checked at
    sampled positions of every row, with every draw replayed."""
    w = configs.make(3)
    PT.log("[full] json-like, entropy confidence, no q")
    g = PT.run_gpu(w, conf_mode=1, write_q=False)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        pos = _sampled_positions(w.L, 4, 400 + b)
        rep = PT.check_row(w, g, b, orc, q_positions=pos, conf_mode=1)
        PT.log(f"[full] json-like negent row {b}: ok ({rep})")


def test_random_nfa_full():
    w = configs.make(5)
    PT.log(f"[full] {w.describe()}")
    g = PT.run_gpu(w)
    PT.log(f"[full] nfa: gpu done, logZ {g['logZ']}")
    orc = oracle.Oracle(w.aut)
    rep = PT.check_row(w, g, 0, orc, q_positions=_sampled_positions(w.L, 12, 7))
    PT.log(f"[full] nfa row 0: ok ({rep})")


@pytest.mark.timeout(300)
def test_range_dfa_full():
    # the full range workload: generation of p (16 x 512 x 151,936) dominates
    PT.log("[full] range DFA: generating inputs")
    w = configs.make(4)
    PT.log(f"[full] {w.describe()}")
    g = PT.run_gpu(w)
    PT.log(f"[full] range DFA: gpu done, status {g['status'].tolist()}")
    assert (g["status"] == 0).all()
    orc = oracle.Oracle(w.aut)
    for b in (0, w.B - 1):
        rep = PT.check_row(w, g, b, orc, q_positions=_sampled_positions(w.L, 8, 300 + b))
        PT.log(f"[full] range DFA row {b}: ok ({rep})")
