"""Pins of the fp64 oracle against facts fixed independently of it:
published Philox known-answer vectors, hand-derived closed forms, special
automata that reduce to textbook results, an integer path-count DP, a
library chain product, and brute-force enumeration of all V^L strings."""
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from synth import automata as A
from tests import bruteforce as BF

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(name):
    out = {}
    for line in open(os.path.join(GOLD, name)):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        out[k] = v
    return out


def _softmax(x):
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


# ------------------------------------------------------------------ Philox
def test_philox_known_answers():
    for line in open(os.path.join(GOLD, "philox4x32_10_kat.txt")):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(t, 16) for t in line.split()]
        out = oracle.philox4x32_10(w[0:4], w[4:6])
        assert list(out) == w[6:10]


def test_uniform_definition():
    seed = 0x123456789ABCDEF
    for (b, lev, node) in [(0, 0, 0), (3, 2, 7), (1, 9, 255)]:
        r = oracle.philox4x32_10([b, lev, node, 0], [seed & 0xffffffff, seed >> 32])
        u = oracle.uniform(seed, b, lev, node)
        assert u == (int(r[0]) >> 8) / 2.0 ** 24
        assert 0.0 <= u < 1.0


# -------------------------------------------------------------- closed forms
def test_two_token_example_closed_form():
    g = _read_kv("two_token_real_example.txt")
    aut = A.two_token_real_dfa()
    p = np.full((2, 2), 0.5, np.float32)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    fb = orc.forward_backward(W)
    assert fb["status"] == oracle.OK
    assert np.exp(fb["logZ"]) == pytest.approx(float(g["Z"][0]), rel=1e-14)
    q, lognorm, _ = orc.marginals(p, fb)
    for i in range(2):
        assert q[i, 1] == pytest.approx(float(g["q_dot"][0]), rel=1e-13)
        assert q[i, 0] == pytest.approx(float(g["q_one"][0]), rel=1e-13)
    np.testing.assert_allclose(lognorm, fb["logZ"], rtol=0, atol=1e-13)
    # samples: uniform over the three accepted strings, never ".."
    accepted = {tuple(map(int, s.split(","))) for s in g["accepted"]}
    counts = {s: 0 for s in accepted}
    n = 6000
    for seed in range(n):
        st, tk, status = orc.sample_tree(p, W, seed, 0)
        assert status == oracle.OK
        t = tuple(int(x) for x in tk)
        assert t in accepted
        counts[t] += 1
    chi2 = sum((c - n / 3) ** 2 / (n / 3) for c in counts.values())
    assert stats.chi2.sf(chi2, 2) > 1e-4


def test_real_number_uniform_closed_form():
    g = _read_kv("real_number_uniform.txt")
    aut = A.real_number_dfa()
    L = 6
    p = np.full((L, 12), 1.0 / 12.0, np.float32)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    fb = orc.forward_backward(W)
    # p is fp32(1/12): the closed form holds for the fp32 value of 1/12
    p12 = float(np.float32(1.0 / 12.0))
    Z = int(g["count"][0]) * p12 ** L
    assert np.exp(fb["logZ"]) == pytest.approx(Z, rel=1e-13)
    assert float(g["Z"][0]) == pytest.approx(int(g["count"][0]) / 12.0 ** 6, rel=1e-15)
    q, _, _ = orc.marginals(p, fb)
    np.testing.assert_allclose(q[:, 10], float(g["q_dot"][0]), rtol=1e-12)
    np.testing.assert_allclose(q[:, :10], float(g["q_digit"][0]), rtol=1e-12)
    np.testing.assert_allclose(q[:, 11], float(g["q_pad"][0]), atol=0)


def test_universal_automaton_reduces_to_unconstrained():
    rng = np.random.default_rng(7)
    V, L = 9, 13
    p = _softmax(rng.normal(0, 2, (L, V))).astype(np.float32)
    aut = A.universal_automaton(V)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    fb = orc.forward_backward(W)
    pd = p.astype(np.float64)
    assert fb["logZ"] == pytest.approx(np.log(pd.sum(axis=1)).sum(), abs=1e-12)
    q, _, _ = orc.marginals(p, fb)
    np.testing.assert_allclose(q, pd / pd.sum(axis=1, keepdims=True), rtol=1e-12)
    # token draws are plain inverse-CDF draws of p under the level K+1 keys
    seed = 99
    st, tk, status = orc.sample_tree(p, W, seed, 0)
    K = int(np.ceil(np.log2(L)))
    for i in range(L):
        u = oracle.uniform(seed, 0, K + 1, i)
        c = np.cumsum(pd[i])
        assert tk[i] == int(np.flatnonzero(c > u * c[-1])[0])
    assert (st == 0).all()


def test_single_string_automaton():
    rng = np.random.default_rng(3)
    V, L = 7, 11
    word = rng.integers(0, V, L)
    p = _softmax(rng.normal(0, 1, (L, V))).astype(np.float32)
    aut = A.single_string_automaton(word, V)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    fb = orc.forward_backward(W)
    assert fb["logZ"] == pytest.approx(np.log(p.astype(np.float64)[np.arange(L), word]).sum(),
                                       abs=1e-12)
    for seed in range(5):
        st, tk, _ = orc.sample_tree(p, W, seed, 0)
        np.testing.assert_array_equal(tk, word)
        np.testing.assert_array_equal(st, np.arange(L + 1))


def test_counting_mode_matches_integer_path_count():
    # p == 1 everywhere: Z is the number of accepting (path, string) pairs
    rng = np.random.default_rng(11)
    aut = A.random_nfa(rng, 6, 5, 14, 2, 2.0)
    L = 12
    p = np.ones((L, aut.V), np.float32)
    orc = oracle.Oracle(aut)
    fb = orc.forward_backward(orc.edge_weights(p))
    # integer DP over states: number of (string, path) pairs
    cnt = [0] * aut.S
    cnt[aut.start] = 1
    for _ in range(L):
        nxt = [0] * aut.S
        for e in range(aut.E):
            nxt[aut.dst[e]] += cnt[aut.src[e]] * int(aut.edge_label(e).size)
        cnt = nxt
    total = sum(cnt[f] for f in aut.accept)
    assert total > 0
    assert np.exp(fb["logZ"]) == pytest.approx(float(total), rel=1e-12)


def test_chain_product_matches_library_multi_dot():
    rng = np.random.default_rng(5)
    aut = A.random_nfa(rng, 7, 6, 20, 3, 2.5)
    L = 9
    p = _softmax(rng.normal(0, 2, (L, aut.V))).astype(np.float32)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    # dense count tensor c[a, v, b] from the raw edge list, contracted with p
    c = np.zeros((aut.S, aut.V, aut.S))
    for e in range(aut.E):
        c[aut.src[e], aut.edge_label(e), aut.dst[e]] += 1.0
    Ms = [np.einsum("avb,v->ab", c, p[i].astype(np.float64)) for i in range(L)]
    for i in range(L):
        np.testing.assert_allclose(orc.dense_M(W, i), Ms[i], rtol=1e-13, atol=1e-300)
    prod = np.linalg.multi_dot(Ms)
    Z = prod[aut.start, aut.accept].sum()
    fb = orc.forward_backward(W)
    assert fb["logZ"] == pytest.approx(np.log(Z), abs=1e-12)


def test_range_sums_match_direct_summation():
    rng = np.random.default_rng(2)
    aut = A.tiny_range_automaton(rng, 5, 300, 12, dfa=False)
    p = _softmax(rng.normal(0, 4, (4, aut.V))).astype(np.float32)
    W = oracle.Oracle(aut).edge_weights(p)
    for i in range(4):
        for e in range(aut.E):
            direct = sum(float(p[i, v]) for v in aut.edge_label(e))
            assert W[i, e] == pytest.approx(direct, rel=1e-12, abs=1e-300)


def test_forward_backward_invariant():
    rng = np.random.default_rng(4)
    aut = A.random_dfa(rng, 12, 40, 3, 0.4)
    L = 30
    p = _softmax(rng.normal(0, 3, (L, aut.V))).astype(np.float32)
    orc = oracle.Oracle(aut)
    fb = orc.forward_backward(orc.edge_weights(p))
    assert fb["status"] == oracle.OK
    for i in range(L + 1):
        z = np.log(fb["alpha"][i] @ fb["beta"][i]) + fb["alog"][i] + fb["blog"][i]
        assert z == pytest.approx(fb["logZ"], abs=1e-10)
    q, lognorm, _ = orc.marginals(p, fb)
    np.testing.assert_allclose(q.sum(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(lognorm, fb["logZ"], atol=1e-10)


def test_infeasible_row():
    aut = A.single_string_automaton([1, 2, 3], 5)
    p = np.full((3, 5), 0.2, np.float32)
    p[1] = 0.0
    p[1, 4] = 1.0  # committed token that contradicts the only accepted string
    orc = oracle.Oracle(aut)
    fb = orc.forward_backward(orc.edge_weights(p))
    assert fb["status"] == oracle.INFEASIBLE
    assert fb["logZ"] == -np.inf


# ------------------------------------------------------------ brute force
def _tiny_family():
    out = []
    for k in range(4):
        rng = np.random.default_rng(100 + k)
        out.append((A.random_dfa(rng, 5, 4, 2, 0.6), 5))
    for k in range(3):
        rng = np.random.default_rng(200 + k)
        aut = A.random_nfa(rng, 4, 4, 10, 2, 2.0)
        # a parallel edge with an overlapping label: path counts > 1
        aut = A._pack(aut.S, aut.V, aut.start, aut.accept.tolist(),
                      [(int(aut.src[e]), int(aut.dst[e]), aut.edge_label(e)) for e in range(aut.E)]
                      + [(int(aut.src[0]), int(aut.dst[0]), aut.edge_label(0))],
                      dfa=False, name="tiny NFA + parallel edge")
        out.append((aut, 5))
    for k in range(2):
        rng = np.random.default_rng(300 + k)
        out.append((A.tiny_range_automaton(rng, 4, 5, 8, dfa=(k == 0)), 5))
    out.append((A.real_number_dfa(), 4))
    return out


@pytest.mark.parametrize("idx", range(10))
def test_oracle_vs_bruteforce(idx):
    aut, L = _tiny_family()[idx]
    rng = np.random.default_rng(500 + idx)
    p = _softmax(rng.normal(0, 1.5, (L, aut.V))).astype(np.float32)
    X, prob, Z, q_bf = BF.distribution(aut, p)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    fb = orc.forward_backward(W)
    if Z == 0:
        assert fb["status"] == oracle.INFEASIBLE
        return
    assert fb["logZ"] == pytest.approx(np.log(Z), abs=1e-12)
    q, _, _ = orc.marginals(p, fb)
    np.testing.assert_allclose(q, q_bf, atol=1e-12)
    # chi-square of the tree-order sampler and of FFBS against the exact law
    n = 20000
    idx_of = {tuple(x): j for j, x in enumerate(X.tolist())}
    ctr_tree = np.zeros(X.shape[0])
    ctr_ffbs = np.zeros(X.shape[0])
    urng = np.random.default_rng(900 + idx)
    for s in range(n):
        st, tk, status = orc.sample_tree(p, W, 10_000 + s, 0)
        assert status == oracle.OK
        ctr_tree[idx_of[tuple(int(t) for t in tk)]] += 1
        st2, tk2, status2 = orc.ffbs(p, W, fb, urng.random(2 * L + 1))
        assert status2 == oracle.OK
        ctr_ffbs[idx_of[tuple(int(t) for t in tk2)]] += 1
    assert ctr_tree[prob == 0].sum() == 0
    exp = prob * n
    keep = exp >= 5
    for ctr in (ctr_tree, ctr_ffbs):
        obs = np.append(ctr[keep], ctr[~keep].sum())
        ex = np.append(exp[keep], exp[~keep].sum())
        if ex[-1] < 5:
            obs[-2] += obs[-1]; ex[-2] += ex[-1]
            obs, ex = obs[:-1], ex[:-1]
        chi2 = ((obs - ex) ** 2 / ex).sum()
        assert stats.chi2.sf(chi2, len(ex) - 1) > 1e-4


def test_replay_accepts_own_samples_and_flags_planted_error():
    rng = np.random.default_rng(8)
    aut = A.random_dfa(rng, 10, 30, 3, 0.3)
    L = 21
    p = _softmax(rng.normal(0, 2, (L, aut.V))).astype(np.float32)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    st, tk, status = orc.sample_tree(p, W, 77, 2)
    assert status == oracle.OK
    rep = orc.replay(p, W, 77, 2, st, tk)
    assert rep["hard"] == 0 and rep["near"] == 0
    assert rep["draws"] == 1 + (32 - 1) + L  # root + Lpad-1 midpoints + L tokens
    # planted mistake: a token outside the sampled edge's label
    bad = tk.copy()
    lab = set()
    for e in range(aut.E):
        if aut.src[e] == st[4] and aut.dst[e] == st[5]:
            lab |= set(aut.edge_label(e).tolist())
    bad[4] = next(v for v in range(aut.V) if v not in lab)
    rep2 = orc.replay(p, W, 77, 2, st, bad)
    assert rep2["hard"] >= 1
    # planted mistake: a different final state
    bad_st = st.copy()
    bad_st[-1] = next(s for s in range(aut.S) if s != st[-1])
    assert orc.replay(p, W, 77, 2, bad_st, tk)["hard"] >= 1


def test_samples_accepted_and_states_follow_delta():
    from synth import configs
    for k in (1, 2):
        w = configs.make(k)
        orc = oracle.Oracle(w.aut)
        delta = {}
        for e in range(w.aut.E):
            for v in w.aut.edge_label(e):
                delta[(int(w.aut.src[e]), int(v))] = int(w.aut.dst[e])
        for b in range(w.B):
            W = orc.edge_weights(w.p[b])
            st, tk, status = orc.sample_tree(w.p[b], W, w.seed, b)
            assert status == oracle.OK
            s = w.aut.start
            for i in range(w.L):
                s = delta[(s, int(tk[i]))]
                assert s == st[i + 1]
            assert s in set(w.aut.accept.tolist())
            for pos, toks in w.commits[b:b + 1]:
                np.testing.assert_array_equal(tk[pos], toks)


def test_commit_topk_worked_examples():
    """The remasking selection on hand-worked rows: k = ceil(masked / steps
    left), highest confidence first, ties to the lower position, NaN last,
    positions without a token or already committed skipped, flagged rows
    untouched, and the last step commits everything left."""
    nan, ninf = float("nan"), float("-inf")
    conf = np.array([[0.5, 0.9, 0.9, 0.1],      # 4 masked, k = 2: the two 0.9 (ties by position)
                     [0.5, 0.9, 0.7, 0.1],      # position 1 committed: 3 masked, k = 2 -> 2, 0
                     [nan, 0.2, ninf, 0.3],     # NaN counts as -inf; k = 2 -> 3, 1
                     [0.9, 0.8, 0.7, 0.6],      # flagged row: nothing
                     [0.1, 0.2, 0.3, 0.4]])     # position 3 has no token: 3 masked, k = 2 -> 2, 1
    tokens = np.array([[3, 1, 4, 1], [5, 9, 2, 6], [5, 3, 5, 8], [9, 7, 9, 3], [2, 3, 8, -1]])
    committed = np.zeros((5, 4), np.int32)
    committed[1, 1] = 1
    status = np.array([0, 0, 0, 4, 0])
    new, fresh = oracle.commit_topk(conf, tokens, committed, status, steps_left=2)
    np.testing.assert_array_equal(fresh, [[0, 1, 1, 0], [1, 0, 1, 0], [0, 1, 0, 1], [0, 0, 0, 0],
                                          [0, 1, 1, 0]])
    np.testing.assert_array_equal(new, fresh + committed)
    # the last step commits every masked position with a token
    new1, fresh1 = oracle.commit_topk(conf, tokens, committed, status, steps_left=1)
    np.testing.assert_array_equal(fresh1, [[1, 1, 1, 1], [1, 0, 1, 1], [1, 1, 1, 1], [0, 0, 0, 0],
                                           [1, 1, 1, 0]])
    # NaN and -inf tie as -inf: position order decides between them
    _, f3 = oracle.commit_topk(np.array([[nan, ninf, 0.0]]), np.array([[1, 1, 1]]),
                               np.zeros((1, 3), np.int32), None, steps_left=2)
    np.testing.assert_array_equal(f3, [[1, 0, 1]])


# ------------------------------------------------------------- confidence
@pytest.mark.parametrize("idx", range(10))
def test_confidence_vs_bruteforce(idx):
    """Both confidence scores against the brute-force law: PROB is the exact
    q at the sampled token, NEGENT is sum_v q ln q of the exact q (0 ln 0 =
    0), at every position of the tiny family."""
    aut, L = _tiny_family()[idx]
    rng = np.random.default_rng(700 + idx)
    p = _softmax(rng.normal(0, 1.5, (L, aut.V))).astype(np.float32)
    X, prob, Z, q_bf = BF.distribution(aut, p)
    if Z == 0:
        return
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    fb = orc.forward_backward(W)
    for seed in (1, 2, 3):
        _, tk, status = orc.sample_tree(p, W, seed, 0)
        assert status == oracle.OK
        _, _, conf = orc.marginals(p, fb, None, tk, 0)
        np.testing.assert_allclose(conf, q_bf[np.arange(L), tk], rtol=1e-12, atol=1e-15)
    with np.errstate(divide="ignore", invalid="ignore"):
        h = np.where(q_bf > 0, q_bf * np.log(q_bf), 0.0).sum(axis=1)
    _, _, conf1 = orc.marginals(p, fb, None, None, 1)
    np.testing.assert_allclose(conf1, h, rtol=1e-11, atol=1e-14)
    assert (conf1 <= 0).all()


def test_negentropy_closed_forms():
    """sum_v q ln q at every position of the two hand-derived examples."""
    g2 = _read_kv("two_token_real_example.txt")
    aut = A.two_token_real_dfa()
    p = np.full((2, 2), 0.5, np.float32)
    orc = oracle.Oracle(aut)
    fb = orc.forward_backward(orc.edge_weights(p))
    _, _, conf = orc.marginals(p, fb, None, None, 1)
    np.testing.assert_allclose(conf, float(g2["negent"][0]), rtol=1e-13)
    g6 = _read_kv("real_number_uniform.txt")
    aut = A.real_number_dfa()
    p = np.full((6, 12), 1.0 / 12.0, np.float32)
    orc = oracle.Oracle(aut)
    fb = orc.forward_backward(orc.edge_weights(p))
    _, _, conf = orc.marginals(p, fb, None, None, 1)
    np.testing.assert_allclose(conf, float(g6["negent"][0]), rtol=1e-12)
    # the PROB score of a digit / a dot at every position is its closed-form q
    tk = np.array([3, 10, 0, 10, 9, 1], np.int32)
    _, _, conf0 = orc.marginals(p, fb, None, tk, 0)
    want = np.where(tk == 10, float(g6["q_dot"][0]), float(g6["q_digit"][0]))
    np.testing.assert_allclose(conf0, want, rtol=1e-12)
    # the unconstrained score ignores the automaton: fp32(1/12) for any token
    _, _, conf2 = orc.marginals(p, fb, None, tk, 2)
    np.testing.assert_array_equal(conf2, float(np.float32(1.0 / 12.0)))


# ------------------------------------------------------ replay NEAR / HARD
def test_judge_draw_hand_built():
    """The verifier's split on hand-built weight vectors: a differing choice
    is NEAR only when every CDF boundary between the two choices lies within
    1e-6 of u; 5e-5 away is HARD and counts as fp32-margin; a zero-weight
    choice, a choice past the candidates, or a real-weight candidate between
    the two choices is HARD."""
    u = 0.375
    for d, verdict, margin in ((5e-7, 1, 0), (-5e-7, 1, 0), (5e-5, 2, 1), (-5e-5, 2, 1),
                               (5e-3, 2, 0)):
        # two candidates, boundary C_0 / T = u + d
        w = np.array([u + d, 1.0 - (u + d)])
        mine = 0 if d > 0 else 1
        other = 1 - mine
        assert oracle.judge_draw(w, u, mine) == (mine, 0, 0)
        assert oracle.judge_draw(w, u, other) == (mine, verdict, margin)
    # zero-weight candidates between the two choices share the boundary: NEAR
    w = np.array([u + 5e-7, 0.0, 0.0, 1.0 - u - 5e-7])
    assert oracle.judge_draw(w, u, 3) == (0, 1, 0)
    # a zero-weight choice is HARD however close the boundary
    assert oracle.judge_draw(w, u, 1)[1] == 2
    assert oracle.judge_draw(w, u, 2)[1] == 2
    # a choice past the candidate list is HARD
    assert oracle.judge_draw(w, u, 4)[1] == 2
    # first boundary at u + 5e-7, but a candidate of weight 0.3 lies between
    # the two choices: the second boundary is far from u, so HARD
    w = np.array([u + 5e-7, 0.3, 1.0 - u - 0.3 - 5e-7])
    assert oracle.judge_draw(w, u, 0) == (0, 0, 0)
    assert oracle.judge_draw(w, u, 2)[1] == 2
    assert oracle.judge_draw(w, u, 1) == (0, 1, 0)
    # vanishing weights: the oracle has no choice, any claim is HARD
    assert oracle.judge_draw(np.zeros(3), u, 0)[0:2] == (-1, 2)


def _u_from_philox(seed, b, level, node):
    """u from the published Philox4x32-10 (pinned above by its known-answer
    vectors): first output word of counter (b, level, node, 0) under the key
    (seed low, seed high), top 24 bits scaled by 2^-24."""
    r = oracle.philox4x32_10([b, level, node, 0], [seed & 0xFFFFFFFF, seed >> 32])
    return (int(r[0]) >> 8) / float(1 << 24)


def test_replay_near_and_hard_on_a_token_draw():
    """End to end through the replay walker: the universal automaton with one
    position (Lpad = 1, K = 0, the token stage is level 1, node 0) and p set
    so that the boundary between tokens 0 and 2 sits just above u; the
    middle token gets weight 0 or a real weight."""
    aut = A.universal_automaton(3)
    seed = 0xC0FFEE
    u = _u_from_philox(seed, 0, 1, 0)
    assert 0.01 < u < 0.98
    orc = oracle.Oracle(aut)
    states = np.zeros(2, np.int32)
    # want = (hard, near, margin) counts of the replay
    for d, mid, want in ((5e-7, 0.0, (0, 1, 0)), (5e-5, 0.0, (1, 0, 1)), (3e-3, 0.0, (1, 0, 0)),
                         (5e-7, 0.2, (1, 0, 0))):
        x = np.float32(u + d)
        m = np.float32(mid)
        p = np.array([[x, m, np.float32(1.0) - x - m]], np.float32)
        W = orc.edge_weights(p)
        st, tk, status = orc.sample_tree(p, W, seed, 0)
        assert status == oracle.OK and tk[0] == 0
        rep = orc.replay(p, W, seed, 0, states, np.array([2], np.int32))
        assert (rep["hard"], rep["near"], rep["margin"]) == want, (d, mid, rep)
        assert rep["draws"] == 2  # the root over F = {0}, then the token


def _two_state_dfa():
    # state 0: token 0 -> 0, token 1 -> 1;  state 1: token 2 -> 0, tokens
    # 0 and 1 -> 1;  accepting {0, 1}
    edges = [(0, 0, [0]), (0, 1, [1]), (1, 0, [2]), (1, 1, [0, 1])]
    return A._pack(2, 3, 0, [0, 1], edges, name="two-state DFA")


@pytest.mark.parametrize("L", [4, 3, 8])
def test_tree_sampler_by_hand(L):
    """Every draw of the tree-order sampler recomputed by hand: the
    transition matrices from the raw edge list, span products by numpy,
    inverse CDFs over ascending ids, and the uniforms keyed (b, level, heap
    index - 2^(level-1)) for the midpoints, (b, 0, 0) for the final state and
    (b, K+1, i) for the tokens."""
    aut = _two_state_dfa()
    rng = np.random.default_rng(41)
    p = _softmax(rng.normal(0, 1, (L, aut.V))).astype(np.float32)
    c = np.zeros((aut.S, aut.V, aut.S))
    for e in range(aut.E):
        c[aut.src[e], aut.edge_label(e), aut.dst[e]] += 1.0
    Lpad = 1 << (L - 1).bit_length()
    K = Lpad.bit_length() - 1
    M = [np.einsum("avb,v->ab", c, p[i].astype(np.float64)) if i < L else np.eye(aut.S)
         for i in range(Lpad)]

    def span(l, r):
        out = np.eye(aut.S)
        for i in range(l, r):
            out = out @ M[i]
        return out

    def icdf(w, u):
        C = np.cumsum(w)
        return int(np.flatnonzero((C > u * C[-1]) & (w > 0))[0])

    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    for seed in (5, 6, 2 ** 40 + 9):
        for b in (0, 3):
            z = [-1] * (Lpad + 1)
            z[0] = aut.start
            F = sorted(aut.accept.tolist())
            root = span(0, Lpad)[z[0]]
            z[Lpad] = F[icdf(np.array([root[f] for f in F]), _u_from_philox(seed, b, 0, 0))]
            for lev in range(1, K + 1):
                width = Lpad >> (lev - 1)
                for heap in range(1 << (lev - 1), 1 << lev):
                    node = heap - (1 << (lev - 1))
                    l, r = node * width, node * width + width
                    m = (l + r) // 2
                    w = span(l, m)[z[l]] * span(m, r)[:, z[r]]
                    z[m] = icdf(w, _u_from_philox(seed, b, lev, node))
            tk = []
            for i in range(L):
                w = p[i].astype(np.float64) * c[z[i], :, z[i + 1]]
                tk.append(icdf(w, _u_from_philox(seed, b, K + 1, i)))
            st, to, status = orc.sample_tree(p, W, seed, b)
            assert status == oracle.OK
            np.testing.assert_array_equal(st, z[:L + 1])
            np.testing.assert_array_equal(to, tk)


# --------------------------------------------------------- MAP decoding
@pytest.mark.parametrize("idx", range(10))
def test_map_vs_bruteforce(idx):
    """The most probable accepted string of the tiny family by enumeration:
    log-max from the serial Viterbi and from the tree, and the tree's string
    equal to the enumerated argmax (unique for these continuous p), its
    states a path of that string through the automaton."""
    aut, L = _tiny_family()[idx]
    rng = np.random.default_rng(1500 + idx)
    p = _softmax(rng.normal(0, 1.5, (L, aut.V))).astype(np.float32)
    X = BF.all_strings(aut.V, L)
    paths = BF.path_counts(aut, X)
    logp = np.zeros(X.shape[0])
    for i in range(L):
        logp += np.log(p[i, X[:, i]].astype(np.float64))
    orc = oracle.Oracle(aut)
    Wm = orc.map_weights(p)
    lv, st_v = orc.viterbi(Wm)
    states, tokens, lt, st_t = orc.map_tree(p, Wm)
    if not (paths > 0).any():
        assert st_v == oracle.INFEASIBLE and st_t == oracle.INFEASIBLE
        return
    acc = np.flatnonzero(paths > 0)
    order = acc[np.argsort(-logp[acc])]
    assert logp[order[0]] - logp[order[1]] > 1e-9  # a unique maximum
    assert lv == pytest.approx(logp[order[0]], abs=1e-12)
    assert lt == pytest.approx(logp[order[0]], abs=1e-12)
    np.testing.assert_array_equal(tokens, X[order[0]])
    # the states are an accepting path of the tokens
    assert states[0] == aut.start and states[-1] in set(aut.accept.tolist())
    for i in range(L):
        assert orc.edge_count(int(states[i]), int(tokens[i]), int(states[i + 1])) > 0


def test_map_viterbi_matches_tree_on_larger_automata():
    for k, (aut, L) in enumerate([(A.random_dfa(np.random.default_rng(31), 20, 60, 3, 0.3), 37),
                                  (A.random_nfa(np.random.default_rng(32), 25, 50, 120, 4, 6.0), 29)]):
        p = _softmax(np.random.default_rng(33 + k).normal(0, 3, (L, aut.V))).astype(np.float32)
        orc = oracle.Oracle(aut)
        Wm = orc.map_weights(p)
        lv, st = orc.viterbi(Wm)
        states, tokens, lt, st2 = orc.map_tree(p, Wm)
        assert st == st2 == oracle.OK
        assert lt == pytest.approx(lv, abs=1e-9)
        # the decoded string's own log-probability is the maximum
        assert np.log(p[np.arange(L), tokens].astype(np.float64)).sum() == pytest.approx(lv, abs=1e-9)
        rep = orc.map_verify(p, Wm, states, tokens)
        assert rep["hard"] == 0 and rep["near"] == 0
        assert rep["decisions"] == 1 + ((1 << (L - 1).bit_length()) - 1) + L


def test_map_special_automata():
    rng = np.random.default_rng(34)
    V, L = 9, 13
    p = _softmax(rng.normal(0, 2, (L, V))).astype(np.float32)
    p[3, 2] = p[3, 5] = p[3].max() + np.float32(0.1)   # an exact tie: the smaller id wins
    orc = oracle.Oracle(A.universal_automaton(V))
    states, tokens, lm, st = orc.map_tree(p, orc.map_weights(p))
    np.testing.assert_array_equal(tokens, np.argmax(p, axis=1))
    assert tokens[3] == 2
    assert lm == pytest.approx(np.log(p.max(axis=1).astype(np.float64)).sum(), abs=1e-12)
    word = rng.integers(0, V, L)
    orc = oracle.Oracle(A.single_string_automaton(word, V))
    states, tokens, lm, st = orc.map_tree(p, orc.map_weights(p))
    np.testing.assert_array_equal(tokens, word)
    np.testing.assert_array_equal(states, np.arange(L + 1))
    assert lm == pytest.approx(np.log(p[np.arange(L), word].astype(np.float64)).sum(), abs=1e-12)


def test_map_tie_rule_by_hand():
    g = _read_kv("map_two_token_tie.txt")
    aut = A.two_token_real_dfa()
    p = np.full((2, 2), 0.5, np.float32)
    orc = oracle.Oracle(aut)
    states, tokens, lm, st = orc.map_tree(p, orc.map_weights(p))
    np.testing.assert_array_equal(states, [int(x) for x in g["states"]])
    np.testing.assert_array_equal(tokens, [int(x) for x in g["tokens"]])
    assert lm == pytest.approx(float(g["logmax"][0]), abs=1e-15)


def test_map_verify_flags_planted_mistakes():
    rng = np.random.default_rng(35)
    aut = A.random_dfa(rng, 10, 30, 3, 0.4)
    L = 21
    p = _softmax(rng.normal(0, 2, (L, aut.V))).astype(np.float32)
    orc = oracle.Oracle(aut)
    Wm = orc.map_weights(p)
    states, tokens, lm, st = orc.map_tree(p, Wm)
    assert st == oracle.OK
    assert orc.map_verify(p, Wm, states, tokens)["hard"] == 0
    # a token of the same edge with a lower probability: HARD
    lab = [v for v in range(aut.V) if orc.edge_count(int(states[4]), v, int(states[5])) > 0]
    worse = [v for v in lab if p[4, v] < p[4, tokens[4]]]
    if worse:
        bad = tokens.copy()
        bad[4] = worse[0]
        assert orc.map_verify(p, Wm, states, bad)["hard"] == 1
    # an equally probable token of the same edge: NEAR, not HARD
    if len(lab) > 1:
        other = next(v for v in lab if v != tokens[4])
        p2 = p.copy()
        p2[4, other] = p2[4, tokens[4]]
        Wm2 = orc.map_weights(p2)
        s2, t2, _, _ = orc.map_tree(p2, Wm2)
        alt = t2.copy()
        alt[4] = other if t2[4] != other else tokens[4]
        r = orc.map_verify(p2, Wm2, s2, alt)
        assert r["hard"] == 0 and r["near"] == 1
    # a different, non-optimal final state: HARD
    bad_st = states.copy()
    bad_st[-1] = next(f for f in aut.accept.tolist() if f != states[-1]) if aut.accept.size > 1 else 0
    assert orc.map_verify(p, Wm, bad_st, tokens)["hard"] >= 1


# ------------------------------------------------- chain (FFBS) replay
def test_chain_verify_accepts_own_draws_and_flags_planted_mistakes():
    """The chain sampler (FFBS with keyed uniforms) replayed by its verifier:
    its own draws pass; a state that cannot precede the next one, a token
    outside its edge's label, and a different final state are HARD.  (FFBS
    itself is pinned against enumeration by the chi-square test above.)"""
    rng = np.random.default_rng(36)
    aut = A.random_dfa(rng, 10, 30, 3, 0.3)
    L = 21
    p = _softmax(rng.normal(0, 2, (L, aut.V))).astype(np.float32)
    orc = oracle.Oracle(aut)
    W = orc.edge_weights(p)
    fb = orc.forward_backward(W)
    seed = 4242
    st, tk, status = orc.chain_sample(p, W, fb, seed, 1)
    assert status == oracle.OK
    rep = orc.chain_verify(p, W, fb, seed, 1, st, tk)
    assert rep["status"] == oracle.OK and rep["hard"] == 0 and rep["near"] == 0
    assert rep["draws"] == (L + 1) + L
    # a token outside the label of its edge
    bad = tk.copy()
    lab = {v for v in range(aut.V) if orc.edge_count(int(st[6]), v, int(st[7])) > 0}
    bad[6] = next(v for v in range(aut.V) if v not in lab)
    assert orc.chain_verify(p, W, fb, seed, 1, st, bad)["hard"] >= 1
    # a state with no edge into the next state
    bst = st.copy()
    preds = {int(aut.src[e]) for e in range(aut.E) if aut.dst[e] == st[9]}
    bst[8] = next(s for s in range(aut.S) if s not in preds)
    assert orc.chain_verify(p, W, fb, seed, 1, bst, tk)["hard"] >= 1
    # another final state
    fst = st.copy()
    fst[-1] = next(f for f in aut.accept.tolist() if f != st[-1]) if aut.accept.size > 1 else 0
    assert orc.chain_verify(p, W, fb, seed, 1, fst, tk)["hard"] >= 1
    # the keyed chain sample is accepted and pins z_0 = s0
    assert st[0] == aut.start and st[-1] in set(aut.accept.tolist())
