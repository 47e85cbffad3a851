"""GPU parity of greedy (MAP) constrained decoding (fa_map_decode) against
the fp64 oracle: every decision replayed by the oracle (the final state, the
midpoints and the tokens must be the oracle's except where two candidates
tie to fp64 rounding, which the replay counts as NEAR), the log-max within
1e-9 relative (both sides sum fp64 logs, in different orders), and the
decoded string accepted with exactly that log-probability."""
import numpy as np
import pytest

import oracle
from synth import automata as A
from synth import configs
from tests import parity as PT
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu

LOGMAX_RTOL = 1e-9


def run_map(w, table=None):
    import torch
    import constrained_decoding_diffusion_amd as fa
    tb = table or fa.Table.from_automaton(w.aut)
    p = torch.from_numpy(w.p).cuda()
    bufs = fa.map_decode(tb, p)
    torch.cuda.synchronize()
    return dict(table=tb, logmax=bufs.logmax.cpu().numpy(), status=bufs.status.cpu().numpy(),
                states=bufs.states.cpu().numpy(), tokens=bufs.tokens.cpu().numpy()[:, :w.L])


def check_map_row(w, g, b, orc):
    Wm = orc.map_weights(w.p[b])
    s_o, t_o, lm_o, st_o = orc.map_tree(w.p[b], Wm)
    if st_o != oracle.OK:
        assert g["status"][b] & 1, f"row {b}: oracle infeasible, GPU status {g['status'][b]}"
        assert g["logmax"][b] == -np.inf
        assert (g["states"][b] == -1).all() and (g["tokens"][b] == -1).all()
        return None
    assert g["status"][b] == 0, f"row {b}: status {g['status'][b]}"
    lm = g["logmax"][b]
    assert abs(lm - lm_o) <= LOGMAX_RTOL * max(1.0, abs(lm_o)), (b, lm, lm_o)
    rep = orc.map_verify(w.p[b], Wm, g["states"][b], g["tokens"][b])
    assert rep["status"] == oracle.OK and rep["hard"] == 0, f"row {b}: {rep}"
    if rep["near"] == 0:
        np.testing.assert_array_equal(g["states"][b], s_o)
        np.testing.assert_array_equal(g["tokens"][b], t_o)
    # the decoded string: an accepting path of it, and its log-probability
    st, tk = g["states"][b], g["tokens"][b]
    assert st[0] == w.aut.start and st[-1] in set(w.aut.accept.tolist())
    for i in range(w.L):
        assert orc.edge_count(int(st[i]), int(tk[i]), int(st[i + 1])) > 0, (b, i)
    own = float(np.log(w.p[b][np.arange(w.L), tk].astype(np.float64)).sum())
    assert abs(own - lm_o) <= LOGMAX_RTOL * max(1.0, abs(lm_o))
    return rep


MAP_CASES = list(CASES)


@pytest.mark.parametrize("name", MAP_CASES)
def test_map_parity(name):
    w = CASES[name]()
    PT.log(f"[map] {name}: {w.describe()}")
    g = run_map(w)
    orc = oracle.Oracle(w.aut)
    near = dec = 0
    for b in range(w.B):
        rep = check_map_row(w, g, b, orc)
        near += rep["near"] if rep else 0
        dec += rep["decisions"] if rep else 0
    PT.log(f"[map] {name}: ok, near {near} of {dec}")
    assert near <= 0.01 * max(dec, 1)


def test_map_special_automata():
    rng = np.random.default_rng(12)
    V, L = 300, 19
    p = rng.normal(0, 2, (2, L, V))
    p = np.exp(p - p.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    p[1, 4, 7] = p[1, 4, 9] = p[1, 4].max() + np.float32(0.05)   # an exact tie: token 7
    uni = A.universal_automaton(V)
    w = configs.Workload(uni.name, uni, p, 2, L, 1, [])
    PT.log("[map] universal automaton")
    g = run_map(w)
    np.testing.assert_array_equal(g["tokens"], np.argmax(p, -1))
    assert g["tokens"][1, 4] == 7
    for b in range(2):
        check_map_row(w, g, b, oracle.Oracle(uni))
    word = rng.integers(0, V, L)
    one = A.single_string_automaton(word, V)
    w = configs.Workload(one.name, one, p, 2, L, 1, [])
    PT.log("[map] single-string automaton")
    g = run_map(w)
    np.testing.assert_array_equal(g["tokens"], np.stack([word, word]))
    for b in range(2):
        check_map_row(w, g, b, oracle.Oracle(one))


def test_map_tie_rule_two_token_example():
    """p = 1/2 everywhere: three accepted strings tie; the smallest-id rule
    gives "11" through states 0, 1, 1 (hand-derived)."""
    aut = A.two_token_real_dfa()
    p = np.full((1, 2, 2), 0.5, np.float32)
    w = configs.Workload(aut.name, aut, p, 1, 2, 1, [])
    g = run_map(w)
    np.testing.assert_array_equal(g["states"][0], [0, 1, 1])
    np.testing.assert_array_equal(g["tokens"][0], [0, 0])
    assert g["logmax"][0] == pytest.approx(2 * np.log(0.5), abs=1e-15)


def test_map_flagged_rows_and_empty():
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
    w.p[1, 0, bad] = 1.0                        # infeasible
    w.p[2, 5, int(aut.label_tok[0])] = np.nan   # bad probability
    PT.log("[map] flagged rows")
    g = run_map(w)
    orc = oracle.Oracle(aut)
    check_map_row(w, g, 0, orc)
    assert g["status"][1] & 1 and g["logmax"][1] == -np.inf
    assert g["status"][2] & 4 and g["logmax"][2] == -np.inf
    for b in (1, 2):
        assert (g["states"][b] == -1).all() and (g["tokens"][b] == -1).all()
    # L = 0: the empty string; the real-number start state is not accepting
    tb = fa.Table.from_automaton(configs.make(1).aut)
    bufs = fa.map_decode(tb, torch.zeros((2, 0, 12), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert (bufs.logmax.cpu().numpy() == -np.inf).all() and (bufs.status.cpu().numpy() & 1).all()
    # B = 0: nothing to do
    fa.map_decode(tb, torch.zeros((0, 6, 12), dtype=torch.float32, device="cuda"))


def _hand_range_nfa():
    """Three states over 50 tokens with range labels: pair (0, 1) holds two
    parallel edges whose ranges overlap (segments of counts 1 and 2), pair
    (0, 2) overlaps pair (0, 1), and tokens 38, 39 and 46-49 lie in no
    segment (38 and 39 inside an elementary interval between cut points)."""
    edges = [(0, 1, np.array([5, 10, 20, 30])), (0, 2, np.array([8, 15])),
             (0, 1, np.array([25, 35])), (1, 1, np.array([0, 38])), (1, 2, np.array([44, 46])),
             (2, 0, np.array([40, 45])), (2, 2, np.array([1, 3]))]
    return A._pack(3, 50, 0, [1, 2], edges, ranges=True, dfa=False, name="hand range NFA")


def test_map_range_labels_by_hand():
    """Range labels through the per-position range-maximum structure: rows
    of a hand-built range NFA decode like the oracle; a NaN at a token in no
    segment leaves its row unflagged, one inside a segment flags it."""
    aut = _hand_range_nfa()
    rng = np.random.default_rng(77)
    B, L = 4, 13
    p = rng.normal(0, 2, (B, L, aut.V))
    p = np.exp(p - p.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    p[0, 2, 39] = np.nan      # in no segment
    p[1, 3, 7] = np.nan       # in pair (0, 1)'s first segment
    w = configs.Workload(aut.name, aut, p, B, L, 1, [])
    g = run_map(w)
    orc = oracle.Oracle(aut)
    for b in (0, 2, 3):
        check_map_row(w, g, b, orc)
    assert g["status"][1] & 4 and g["logmax"][1] == -np.inf
    assert (g["states"][1] == -1).all() and (g["tokens"][1] == -1).all()


def test_map_range_universal_and_ties():
    """The universal automaton as one range [0, V): the decoded tokens are the
    per-position argmax of p, the smaller id on an exact tie."""
    V, L = 3000, 21
    rng = np.random.default_rng(78)
    p = rng.normal(0, 2, (2, L, V))
    p = np.exp(p - p.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    p[0, 5, 1234] = p[0, 5, 2345] = p[0, 5].max() + np.float32(0.05)
    aut = A._pack(1, V, 0, [0], [(0, 0, np.array([0, V]))], ranges=True, name="universal range")
    w = configs.Workload(aut.name, aut, p, 2, L, 1, [])
    g = run_map(w)
    np.testing.assert_array_equal(g["tokens"], np.argmax(p, -1))
    assert g["tokens"][0, 5] == 1234
    expect = np.log(p.max(-1).astype(np.float64)).sum(-1)
    np.testing.assert_allclose(g["logmax"], expect, rtol=LOGMAX_RTOL)


def test_map_range_dfa_full_vocabulary():
    """The range DFA of S = 1024 over V = 151,936 (16 ranges per state: about
    29,500 cut points, every level of the block table in use) at a short
    length, row for row against the oracle."""
    import constrained_decoding_diffusion_amd as fa
    aut = configs._draw(lambda r: A.range_dfa(r, S=1024, V=151936), 7801, 12)
    w = configs.from_automaton(aut, 2, 12, "normal4_zipf", 0, 7802, "range DFA S 1024, L 12")
    tb = fa.Table.from_automaton(w.aut)
    PT.log(f"[map] {w.describe()}, cuts {tb.info['cuts']}")
    assert tb.info["cuts"] > 20000
    g = run_map(w, table=tb)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        rep = check_map_row(w, g, b, orc)
        PT.log(f"[map] range DFA row {b}: ok ({rep})")


def _map_tree(fa, torch, w, first_level):
    tb = fa.Table.from_automaton(w.aut, first_level=first_level)
    p = torch.from_numpy(w.p).cuda()
    bufs = fa.map_decode(tb, p)
    torch.cuda.synchronize()
    Lpad = 1 << max(0, (w.L - 1).bit_length())
    Sp = tb.info["Sp"]
    tree = bufs.tree[: w.B * 2 * Lpad * Sp * Sp].view(w.B, 2 * Lpad, Sp, Sp)
    return tb, [tree[:, 1:Lpad].cpu().numpy(), bufs.logmax.cpu().numpy(), bufs.states.cpu().numpy(),
                bufs.tokens.cpu().numpy(), bufs.status.cpu().numpy()]


@pytest.mark.parametrize("name", ["json-small", "random-dfa", "range-small", "nfa-small",
                                  "hand-range", "odd-length"])
def test_map_sparse_first_level_equals_dense(name):
    """The first max-plus level formed over the pairs (map_sparse1) against
    the dense products: every internal node of the tree, the log-max, the
    states and the tokens equal bit for bit (each term is the same fp64 add,
    and the maximum does not depend on the order)."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    if name == "hand-range":
        aut = _hand_range_nfa()
        rng = np.random.default_rng(79)
        p = rng.dirichlet(np.ones(aut.V), (3, 11)).astype(np.float32)
        w = configs.Workload(aut.name, aut, p, 3, 11, 1, [])
    elif name == "odd-length":
        w = configs.make(2, B=2, L=13)   # identity leaves past the sequence end
    else:
        w = CASES[name]()
    ts, rs = _map_tree(fa, torch, w, "sparse")
    td, rd = _map_tree(fa, torch, w, "dense")
    assert ts.info["map_first_sparse"] == 1 and td.info["map_first_sparse"] == 0
    PT.log(f"[map] {name}: sparse first level against dense, {w.describe()}")
    for a, b_, what in zip(rs, rd, ("internal nodes", "log-max", "states", "tokens", "status")):
        np.testing.assert_array_equal(a, b_, err_msg=what)


def test_map_determinism_and_repeat():
    w = CASES["json-small"]()
    g1 = run_map(w)
    g2 = run_map(w, table=g1["table"])
    for k in ("logmax", "states", "tokens", "status"):
        np.testing.assert_array_equal(g1[k], g2[k])


def test_map_json_like_full():
    w = configs.make(3)
    PT.log(f"[map-full] {w.describe()}")
    g = run_map(w)
    PT.log(f"[map-full] gpu done, logmax {g['logmax']}")
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        rep = check_map_row(w, g, b, orc)
        PT.log(f"[map-full] row {b}: ok ({rep})")
