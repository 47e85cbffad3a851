"""GPU parity of the sparse span levels: the level-1 products formed from the
pair values (row combination over pairs (a, k), (k, c)) instead of dense
matrix products, and the level-2 products likewise over the two-step
pattern.  Every workload of the step parity suite runs with the sparse forms
forced; the whole step is checked against the fp64 oracle, and the level-1
and level-2 nodes against the oracle's products of 2 and 4 leaves."""
import numpy as np
import pytest

import oracle
from tests import parity as PT
from synth import automata as A
from synth import configs
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


def _check_level1(w, g, b, orc, level=1):
    PT.check_span_nodes(w, g, b, orc, level=level)


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_first_level_parity(name):
    import constrained_decoding_diffusion_amd as fa
    w = CASES[name]()
    tb = fa.Table.from_automaton(w.aut, first_level="sparse")
    assert tb.info["first_sparse"] == 1
    PT.log(f"[first-level] {name}: {w.describe()}, first-level work {tb.info['first_work']}")
    g = PT.run_gpu(w, table=tb)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        PT.check_row(w, g, b, orc)
    _check_level1(w, g, 0, orc)
    if w.B > 1:
        _check_level1(w, g, w.B - 1, orc)
    PT.log(f"[first-level] {name}: ok")


@pytest.mark.parametrize("name", ["json-small", "random-dfa-L3", "nfa-small"])
def test_sparse_and_dense_first_level_agree(name):
    """Both forms of the first level give the same draws where no uniform
    sits near a boundary, and log Z within the parity tolerance."""
    import constrained_decoding_diffusion_amd as fa
    w = CASES[name]()
    gs = PT.run_gpu(w, table=fa.Table.from_automaton(w.aut, first_level="sparse"))
    gd = PT.run_gpu(w, table=fa.Table.from_automaton(w.aut, first_level="dense"))
    assert gd["table"].info["first_sparse"] == 0
    np.testing.assert_allclose(gs["logZ"], gd["logZ"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(gs["q"], gd["q"], rtol=2e-4, atol=1e-10)
    # a draw may differ only where its uniform lies within the fp32 noise
    # of a boundary; the oracle replay in the parity test bounds those
    same = (gs["tokens"] == gd["tokens"]).mean()
    assert same > 0.99, same


def _nfa_wide():
    # more than 1024 states: rows of both sparse levels span two 1024-column
    # windows
    aut = configs._draw(lambda r: A.random_nfa(r, 1500, 3000, 9000, 8, 12.0), 8201, 8)
    return configs.from_automaton(aut, 1, 8, "normal4", 0, 8300, "nfa wide")


def _nfa_mid():
    # 513..1024 states: rows walk two 512-column windows
    aut = configs._draw(lambda r: A.random_nfa(r, 700, 3000, 5000, 8, 12.0), 8401, 8)
    return configs.from_automaton(aut, 2, 8, "normal4", 0, 8500, "nfa mid")


SECOND = dict(CASES, **{"nfa-wide": _nfa_wide, "nfa-mid": _nfa_mid})


@pytest.mark.parametrize("name", list(SECOND))
def test_sparse_second_level_parity(name):
    import constrained_decoding_diffusion_amd as fa
    w = SECOND[name]()
    tb = fa.Table.from_automaton(w.aut, first_level="sparse2")
    assert tb.info["first_sparse"] == 1 and tb.info["second_sparse"] == 1
    PT.log(f"[second-level] {name}: {w.describe()}, two-step pairs {tb.info['pairs2']}, "
           f"work {tb.info['second_work']}")
    g = PT.run_gpu(w, table=tb)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        PT.check_row(w, g, b, orc)
    _check_level1(w, g, 0, orc, level=1)
    _check_level1(w, g, 0, orc, level=2)
    PT.log(f"[second-level] {name}: ok")
