"""Span products over the live states (tables compiled with FA_LIVE_STATES):
the step against the fp64 oracle, and against the same table without the
restriction, on workloads whose committed positions prune the automaton and
whose products run on 256x256 tiles (Sp = 256, at least 256 products per
level): a range DFA without dense leaves (the reachability pass reads the
folded pair values) and a json-like DFA with dense leaves."""
import numpy as np
import pytest

import oracle
from synth import automata as A
from synth import configs
from synth.live_states import live_states
from tests import parity as PT

pytestmark = pytest.mark.gpu


def _range_live():
    aut = configs._draw(lambda r: A.range_dfa(r, S=250, V=5000, edges_per_state=16), 9101, 512)
    return configs.from_automaton(aut, 2, 512, "normal4_zipf", 256, 9200, "range DFA, live states")


def _json_live():
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=240, V=20000, pool=256, string_size=13000),
                        9301, 512)
    return configs.from_automaton(aut, 2, 512, "normal4_zipf", 256, 9400, "json-like, live states")


CASES = {"range": _range_live, "json": _json_live}


@pytest.mark.parametrize("name", list(CASES))
def test_live_states_parity(name):
    import constrained_decoding_diffusion_amd as fa
    w = CASES[name]()
    tb = fa.Table.from_automaton(w.aut, live_states=True)
    assert tb.info["live_states"] == 1 and tb.info["Sp"] == 256
    live = [live_states(w.aut, w.p[b]).sum(axis=1) for b in range(w.B)]
    PT.log(f"[live] {name}: {w.describe()}, leafless {tb.info['leafless']}, live states per boundary "
           f"{[round(float(x.mean()), 1) for x in live]} of {w.aut.S}")
    assert max(float(x.mean()) for x in live) < 0.75 * w.aut.S  # the restricted products are taken
    g = PT.run_gpu(w, table=tb)
    orc = oracle.Oracle(w.aut)
    near = draws = 0
    for b in range(w.B):
        rep = PT.check_row(w, g, b, orc)
        near += rep["near"] if rep else 0
        draws += rep["draws"] if rep else 0
    PT.log(f"[live] {name}: ok, near {near} of {draws}")
    assert near <= 0.01 * max(draws, 1)


@pytest.mark.parametrize("name", list(CASES))
def test_live_states_match_unrestricted(name):
    """The same step without the restriction: log Z within the parity
    tolerance of the restricted one (the sums differ only in rounding
    order), and the sampled tokens equal except where a draw's uniform sits
    at a boundary.  (Its q is not compared: on the json-like input the
    unrestricted messages lose the live states' weight at a few positions,
    where states that can no longer reach F carry more than 2^126 times
    their mass; the restricted step's q matches the oracle above.)"""
    import constrained_decoding_diffusion_amd as fa
    w = CASES[name]()
    g1 = PT.run_gpu(w, table=fa.Table.from_automaton(w.aut, live_states=True))
    g0 = PT.run_gpu(w, table=fa.Table.from_automaton(w.aut))
    np.testing.assert_allclose(g1["logZ"], g0["logZ"], rtol=2e-5, atol=1e-6)
    same = (g1["tokens"] == g0["tokens"]).mean()
    PT.log(f"[live] {name}: tokens equal at {100 * same:.2f}% of positions")
    assert same > 0.99
