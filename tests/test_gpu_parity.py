"""GPU parity of one constrained step (C ABI) against the fp64 oracle on
small seeded workloads that span several tiles and ragged tails."""
import numpy as np
import pytest

import oracle
from synth import automata as A
from synth import configs
from tests import parity as PT

pytestmark = pytest.mark.gpu


def _json_small():
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=200, V=20000, pool=256, string_size=13000),
                        7001, 37)
    return configs.from_automaton(aut, 3, 37, "normal4_zipf", 0, 7100, "json-like small")


def _range_small():
    aut = configs._draw(lambda r: A.range_dfa(r, S=150, V=5000, edges_per_state=16), 7201, 29)
    return configs.from_automaton(aut, 2, 29, "normal4_zipf", 14, 7300, "range small")


def _nfa_small():
    def build(r):
        a = A.random_nfa(r, 300, 2000, 3000, 8, 12.0)
        # parallel edges with overlapping labels: path counts above one
        extra = [(int(a.src[e]), int(a.dst[e]), a.edge_label(e)[: max(1, a.edge_label(e).size // 2)])
                 for e in range(0, a.E, 7)]
        edges = [(int(a.src[e]), int(a.dst[e]), a.edge_label(e)) for e in range(a.E)] + extra
        return A._pack(a.S, a.V, 0, a.accept.tolist(), edges, dfa=False, name="random NFA small")
    aut = configs._draw(build, 7401, 21)
    return configs.from_automaton(aut, 2, 21, "normal4", 0, 7500, "nfa small")


def _json_odd_v():
    # V % 4 != 0: scalar dense-mask loads, the chunked token draw and the
    # general q writer
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=120, V=9999, pool=128, string_size=6000),
                        7601, 23)
    return configs.from_automaton(aut, 2, 23, "normal4_zipf", 3, 7700, "json-like odd V")


def _json_many_list_tokens():
    # more than 64 token-list tokens per V chunk: their copy is gathered from p
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=96, V=20000, pool=6000, max_struct=64,
                                                  string_size=12000), 7801, 19)
    return configs.from_automaton(aut, 3, 19, "normal4_zipf", 0, 7900, "json-like many list tokens")


def _json_32_dense():
    # 32 dense-mask pairs: no flag bit is left for token-list tokens
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=400, V=8000, string_frac=0.1, pool=200,
                                                  string_size=5000), 8001, 17)
    return configs.from_automaton(aut, 2, 17, "normal4_zipf", 2, 8100, "json-like 32 dense")


def _json_split_k():
    # Sp = 512 and one row: the top tree levels' few tiles are split along K
    # and added by the reduce kernel
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=480, V=20000, pool=256, string_size=13000),
                        7001, 37)
    return configs.from_automaton(aut, 1, 37, "normal4_zipf", 0, 8200, "json-like split K")


CASES = {
    "real-number": lambda: configs.make(1),
    "random-dfa": lambda: configs.make(2),
    "json-small": _json_small,
    "range-small": _range_small,
    "nfa-small": _nfa_small,
    "real-L1": lambda: configs.make(1, L=1),
    "random-dfa-L3": lambda: configs.make(2, L=3, B=2),
    "json-odd-V": _json_odd_v,
    "json-many-list-tokens": _json_many_list_tokens,
    "json-32-dense": _json_32_dense,
    "json-split-K": _json_split_k,
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_parity(name):
    w = CASES[name]()
    PT.log(f"[parity] {name}: {w.describe()}")
    g = PT.run_gpu(w)
    PT.log(f"[parity] {name}: gpu done, status {g['status']}")
    orc = oracle.Oracle(w.aut)
    near = draws = 0
    for b in range(w.B):
        rep = PT.check_row(w, g, b, orc)
        near += rep["near"] if rep else 0
        draws += rep["draws"] if rep else 0
    if w.aut.S <= 400:
        PT.check_leaves(w, g, 0, range(w.L), orc)
    PT.log(f"[parity] {name}: ok, near draws {near} of {draws}")
    # NEAR draws (u within 1e-6 of every boundary between the two choices)
    # are exempt from bit-exactness; they must stay rare
    assert near <= 0.01 * draws


@pytest.mark.parametrize("name", ["real-number", "json-small"])
def test_negentropy_confidence(name):
    w = CASES[name]()
    PT.log(f"[parity-negent] {name}")
    g = PT.run_gpu(w, conf_mode=1)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        PT.check_row(w, g, b, orc, conf_mode=1)


@pytest.mark.parametrize("conf_mode", [0, 1])
def test_confidence_without_q(conf_mode):
    """The confidence with q not written, against the oracle's confidence
    (and the draws against its replay), in both modes."""
    w = _json_small()
    PT.log(f"[parity] conf without q, mode {conf_mode}")
    g = PT.run_gpu(w, conf_mode=conf_mode, write_q=False)
    assert g["q"] is None
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        PT.check_row(w, g, b, orc, conf_mode=conf_mode)
    g2 = PT.run_gpu(w, conf_mode=conf_mode, write_q=True, table=g["table"])
    np.testing.assert_array_equal(g["tokens"], g2["tokens"])
    np.testing.assert_array_equal(g["conf"], g2["conf"])


@pytest.mark.parametrize("name", ["json-small", "random-dfa", "range-small", "nfa-small"])
@pytest.mark.parametrize("joint", [True, False])
def test_unconstrained_confidence(name, joint):
    """FA_CONF_UNCONSTRAINED: conf is p at the sampled token (bit for bit),
    -inf on flagged rows; draws, log Z and q are those of the PROB call."""
    w = CASES[name]()
    PT.log(f"[parity-mf] {name} joint {joint}")
    g = PT.run_gpu(w, conf_mode=2, joint=joint)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        PT.check_row(w, g, b, orc, conf_mode=2)
    rows = np.arange(w.B)[:, None]
    np.testing.assert_array_equal(g["conf"], w.p[rows, np.arange(w.L)[None, :], g["tokens"]])
    g0 = PT.run_gpu(w, conf_mode=0, joint=joint, table=g["table"])
    for k in ("status", "logZ", "states", "tokens", "q"):
        np.testing.assert_array_equal(g[k], g0[k], err_msg=k)


def test_special_automata():
    rng = np.random.default_rng(12)
    V, L = 300, 19
    p = rng.normal(0, 2, (2, L, V))
    p = np.exp(p - p.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    for aut in (A.universal_automaton(V), A.single_string_automaton(rng.integers(0, V, L), V)):
        w = configs.Workload(aut.name, aut, p, 2, L, 31337, [])
        PT.log(f"[parity] {aut.name}")
        g = PT.run_gpu(w)
        orc = oracle.Oracle(aut)
        for b in range(2):
            PT.check_row(w, g, b, orc)


def test_infeasible_row_is_flagged():
    w = configs.make(2, B=2, L=16)
    # row 1: a committed token no state can emit from the start state
    aut = w.aut
    first = set()
    for e in range(aut.E):
        if aut.src[e] == aut.start:
            first |= set(aut.edge_label(e).tolist())
    bad = next(v for v in range(aut.V) if v not in first)
    w.p[1, 0] = 0.0
    w.p[1, 0, bad] = 1.0
    PT.log("[parity] infeasible row")
    g = PT.run_gpu(w)
    orc = oracle.Oracle(aut)
    PT.check_row(w, g, 0, orc)
    assert g["status"][1] & 1
    assert g["logZ"][1] == -np.inf
    assert (g["states"][1] == -1).all() and (g["tokens"][1] == -1).all()
    assert (g["q"][1] == 0).all() and (g["conf"][1] == -np.inf).all()


@pytest.mark.parametrize("joint", [True, False])
def test_underflow_is_flagged(joint):
    """A draw whose candidates all weigh zero while log Z is finite, forced
    from the host: after the span tree, row 1's left child of the root is
    cleared, so the first midpoint draw of that row finds no weight.  The row
    is flagged FA_ROW_UNDERFLOW and gets the flagged outputs; log Z keeps the
    value the tree gave; the other rows match an untouched step bit for bit."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    w = _json_small()
    tb = fa.Table.from_automaton(w.aut)
    PT.log(f"[parity] underflow, joint {joint}")
    ref = PT.run_gpu(w, table=tb, joint=joint)
    dev = torch.device("cuda")
    p = torch.from_numpy(w.p).to(dev)
    bufs = fa.StepBuffers(tb, w.B, w.L, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    bufs.status.zero_()
    fa.build_transitions(tb, p, bufs, st)
    fa.span_tree(tb, bufs, st)
    Lpad = 1 << (w.L - 1).bit_length()
    Sp = tb.info["Sp"]
    bufs.tree.view(w.B, 2 * Lpad, Sp, Sp)[1, 2].zero_()
    if joint:
        fa.sample_marginals(tb, p, bufs, w.seed, fa.FA_CONF_PROB, st, write_q=True)
    else:
        fa.sample(tb, p, bufs, w.seed, st)
        fa.marginals(tb, p, bufs, fa.FA_CONF_PROB, st, write_q=True)
    torch.cuda.synchronize()
    status = bufs.status.cpu().numpy()
    states, tokens = bufs.states.cpu().numpy(), bufs.tokens.cpu().numpy()[:, :w.L]
    q, conf = bufs.q.cpu().numpy(), bufs.conf.cpu().numpy()[:, :w.L]
    logZ = bufs.logZ.cpu().numpy()
    PT.log(f"[parity] underflow: status {status}")
    assert status[1] == fa.FA_ROW_UNDERFLOW
    assert (states[1] == -1).all() and (tokens[1] == -1).all()
    assert (q[1] == 0).all() and (conf[1] == -np.inf).all()
    assert logZ[1] == ref["logZ"][1]
    for b in (0, 2):
        assert status[b] == 0
        for k, got in (("states", states), ("tokens", tokens), ("q", q), ("conf", conf), ("logZ", logZ)):
            np.testing.assert_array_equal(got[b], ref[k][b], err_msg=f"{k} row {b}")


def test_bad_probability_is_flagged():
    w = configs.make(2, B=2, L=8)
    w.p[0, 3, int(w.aut.label_tok[0])] = np.nan  # a token some label holds
    PT.log("[parity] bad probability")
    g = PT.run_gpu(w)
    assert g["status"][0] & 4
    assert g["logZ"][0] == -np.inf
    assert (g["tokens"][0] == -1).all()
    PT.check_row(w, g, 1, oracle.Oracle(w.aut))


@pytest.mark.parametrize("name", ["real-number", "json-small", "json-32-dense", "json-odd-V",
                                  "json-many-list-tokens", "range-small", "nfa-small"])
@pytest.mark.parametrize("conf_mode,write_q", [(0, True), (1, True), (1, False), (0, False)])
def test_joint_call_matches_separate_calls(name, conf_mode, write_q):
    """fa_sample_marginals (token draws fed by the q writer's pass where it
    applies) gives bit-for-bit what fa_sample then fa_marginals give."""
    w = CASES[name]()
    PT.log(f"[joint] {name} conf_mode {conf_mode} q {write_q}")
    g1 = PT.run_gpu(w, conf_mode=conf_mode, write_q=write_q, joint=True)
    g2 = PT.run_gpu(w, conf_mode=conf_mode, write_q=write_q, table=g1["table"], joint=False)
    for k in ("status", "logZ", "states", "tokens", "conf") + (("q",) if write_q else ()):
        np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)


def test_joint_call_flagged_rows():
    """Rows flagged before the draws (infeasible, bad probability) come out of
    the joint call exactly as out of the separate calls."""
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
    PT.log("[joint] flagged rows")
    for conf_mode in (0, 1):
        g1 = PT.run_gpu(w, conf_mode=conf_mode, joint=True)
        g2 = PT.run_gpu(w, conf_mode=conf_mode, table=g1["table"], joint=False)
        for k in ("status", "logZ", "states", "tokens", "q", "conf"):
            np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)
        assert g1["status"][1] & 1 and g1["status"][2] & 4


def test_joint_call_on_another_stream():
    """The joint call on a non-default stream (every launch of the call,
    the midpoint draws riding on the message pass included, goes to the
    caller's stream) gives what it gives on the default stream."""
    import torch
    w = _json_small()
    PT.log("[joint] non-default stream")
    g1 = PT.run_gpu(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g2 = PT.run_gpu(w, table=g1["table"])
    for k in ("status", "logZ", "states", "tokens", "q", "conf"):
        np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)


def test_determinism_bitwise():
    w = _json_small()
    PT.log("[parity] determinism")
    g1 = PT.run_gpu(w)
    g2 = PT.run_gpu(w, table=g1["table"])
    for k in ("logZ", "states", "tokens", "q", "conf"):
        np.testing.assert_array_equal(g1[k], g2[k])
    Sp = g1["table"].info["Sp"]
    Lpad = 1 << (w.L - 1).bit_length()
    # heap node 0 is unused; every other node is written by the step, the
    # leaves (Lpad ..) only on a table that keeps dense leaves
    last = Lpad if g1["table"].info["leafless"] else 2 * Lpad
    t1 = g1["bufs"].tree.view(w.B, 2 * Lpad, Sp, Sp)[:, 1:last].cpu().numpy()
    t2 = g2["bufs"].tree.view(w.B, 2 * Lpad, Sp, Sp)[:, 1:last].cpu().numpy()
    np.testing.assert_array_equal(t1, t2)


def test_empty_inputs():
    import torch
    import constrained_decoding_diffusion_amd as fa
    w = configs.make(1)
    tb = fa.Table.from_automaton(w.aut)
    PT.log("[parity] empty inputs")
    # B = 0: every call is a no-op
    p0 = torch.zeros((0, 6, 12), dtype=torch.float32, device="cuda")
    fa.step(tb, p0, 1)
    # L = 0: the empty string is rejected (start state not accepting)
    pz = torch.zeros((2, 0, 12), dtype=torch.float32, device="cuda")
    bufs = fa.step(tb, pz, 1)
    torch.cuda.synchronize()
    assert (bufs.logZ.cpu().numpy() == -np.inf).all()
    assert (bufs.status.cpu().numpy() & 1).all()
    assert (bufs.states.cpu().numpy() == -1).all()


def test_misaligned_probabilities():
    """p at a 4-byte offset from a 16-byte boundary takes the scalar load
    paths; the step still matches the oracle."""
    import torch
    w = _json_small()
    PT.log("[parity] misaligned p")
    base = torch.empty(w.p.size + 1, dtype=torch.float32, device="cuda")
    p = base[1:].view(w.p.shape)
    p.copy_(torch.from_numpy(w.p))
    assert p.data_ptr() % 16 != 0
    g = PT.run_gpu(w, p_dev=p)
    orc = oracle.Oracle(w.aut)
    for b in range(w.B):
        PT.check_row(w, g, b, orc)


def test_probe_bandwidth_hook():
    """The measurement hook's copy reproduces its source and its read pass
    sums every element once (partial sums per workgroup)."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    stream = torch.cuda.current_stream().cuda_stream
    src = torch.arange(1 << 20, dtype=torch.float32, device="cuda") % 97
    dst = torch.zeros_like(src)
    fa.probe_bandwidth(fa.FA_PROBE_COPY, src, dst, src.numel() * 4, 1024, stream)
    part = torch.zeros(1024, dtype=torch.float32, device="cuda")
    fa.probe_bandwidth(fa.FA_PROBE_READ, src, part, src.numel() * 4, 1024, stream)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert abs(float(part.double().sum()) - float(src.double().sum())) <= 1e-6 * float(src.double().sum())
