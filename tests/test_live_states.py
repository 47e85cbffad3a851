"""The live-state analysis of the synthetic inputs (synth/live_states.py),
against sets worked out by hand on the real-number DFA and the single-string
automaton."""
import numpy as np

from synth import automata as A
from synth.live_states import live_arithmetic, live_states


def _sets(live):
    return [set(np.nonzero(row)[0].tolist()) for row in live]


def test_real_number_dfa_uniform():
    # uniform p: after one token the int state (1) and the dot state (2) can
    # still reach an accepting state; after two only int (1) and frac (3); at
    # the end the accepting states reached, 1 and 3
    aut = A.real_number_dfa()
    p = np.full((3, 12), 1.0 / 12, dtype=np.float32)
    assert _sets(live_states(aut, p)) == [{0}, {1, 2}, {1, 3}, {1, 3}]


def test_real_number_dfa_committed_dot():
    # a one-hot '.' at position 0 leaves one live state per boundary
    aut = A.real_number_dfa()
    p = np.full((3, 12), 1.0 / 12, dtype=np.float32)
    p[0] = 0.0
    p[0, A.REAL_DOT] = 1.0
    assert _sets(live_states(aut, p)) == [{0}, {2}, {3}, {3}]


def test_single_string_and_arithmetic():
    aut = A.single_string_automaton([0, 1, 2, 3], 4)
    p = np.full((4, 4), 0.25, dtype=np.float32)
    live = live_states(aut, p)
    assert _sets(live) == [{0}, {1}, {2}, {3}, {4}]
    # every product of the four-position tree touches one live state per
    # boundary: 3 products of 1 multiply-add against 3 * 5^3 dense
    assert live_arithmetic(live, aut.S) == 3 / (3 * 5 ** 3)
