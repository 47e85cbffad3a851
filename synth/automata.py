"""Seeded synthetic finite automata.

Every builder returns an :class:`Automaton`: states, vocabulary size, start
state, accepting states and an edge list whose labels are either explicit
token lists or half-open token ranges.  Nothing here evaluates the
constrained distribution; these are inputs only.

Shapes follow the pages' workloads: a real-number automaton (the length-2
example of "Why constrained decoding breaks for diffusion LMs", enlarged), a
JSON-like automaton (function-calling constraints of "The evidence"), and a
large random NFA sized like the Spider SQL automaton (~10k states, ~100k
edges; "Arbitrary schedules and NFAs" and "What to be skeptical about").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Automaton:
    S: int
    V: int
    start: int
    accept: np.ndarray  # int32 [n_accept]
    src: np.ndarray  # int32 [E]
    dst: np.ndarray  # int32 [E]
    label_off: np.ndarray  # int64 [E+1] offsets into label_tok
    label_tok: np.ndarray  # int32: token ids, or flat (lo, hi) pairs if ranges
    ranges: bool = False
    dfa: bool = True
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def E(self) -> int:
        return int(self.src.shape[0])

    def edge_label(self, e: int) -> np.ndarray:
        """Explicit sorted token ids of edge ``e`` (ranges are expanded)."""
        seg = self.label_tok[self.label_off[e]:self.label_off[e + 1]]
        if not self.ranges:
            return np.asarray(seg, dtype=np.int64)
        parts = [np.arange(seg[2 * j], seg[2 * j + 1], dtype=np.int64)
                 for j in range(seg.shape[0] // 2)]
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def _pack(S, V, start, accept, edges, *, ranges=False, dfa=True, name="", meta=None):
    """edges: list of (src, dst, int array of tokens or flat range pairs)."""
    src = np.array([e[0] for e in edges], dtype=np.int32)
    dst = np.array([e[1] for e in edges], dtype=np.int32)
    lens = np.array([len(e[2]) for e in edges], dtype=np.int64)
    off = np.zeros(len(edges) + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    tok = (np.concatenate([np.asarray(e[2], dtype=np.int32) for e in edges])
           if edges else np.zeros(0, np.int32))
    return Automaton(S=S, V=V, start=start, accept=np.asarray(sorted(accept), dtype=np.int32),
                     src=src, dst=dst, label_off=off, label_tok=tok.astype(np.int32),
                     ranges=ranges, dfa=dfa, name=name, meta=meta or {})


def _group_by_pair(S, tok_dst):
    """tok_dst: dict state -> (tokens array, destinations array) -> edge list
    with one edge per (src, dst) pair carrying the sorted tokens."""
    edges = []
    for s in range(S):
        if s not in tok_dst:
            continue
        toks, dsts = tok_dst[s]
        order = np.lexsort((toks, dsts))
        toks, dsts = toks[order], dsts[order]
        if toks.size == 0:
            continue
        cut = np.flatnonzero(np.diff(dsts)) + 1
        for t_seg, d_seg in zip(np.split(toks, cut), np.split(dsts, cut)):
            edges.append((s, int(d_seg[0]), np.sort(t_seg)))
    return edges


# ---------------------------------------------------------------- real numbers
REAL_DIGITS = tuple(range(10))
REAL_DOT = 10
REAL_PAD = 11


def real_number_dfa() -> Automaton:
    """Five-state DFA for real numbers over digits 0-9, '.' (10) and pad (11).

    States: 0 start, 1 int-digits, 2 dot seen (no digit yet), 3 digits after a
    dot or a dot after digits, 4 reject sink.  Accepting: {1, 3}.  Accepts a
    string with at least one digit and at most one dot, so both "1." and ".1"
    are legal and ".." is not.  Pad leads to the sink from every state.
    """
    d = np.array(REAL_DIGITS)
    dot = np.array([REAL_DOT])
    pad = np.array([REAL_PAD])
    allv = np.arange(12)
    edges = [
        (0, 1, d), (0, 2, dot), (0, 4, pad),
        (1, 1, d), (1, 3, dot), (1, 4, pad),
        (2, 3, d), (2, 4, dot), (2, 4, pad),
        (3, 3, d), (3, 4, dot), (3, 4, pad),
        (4, 4, allv),
    ]
    # merge the two (2,4) and (3,4) edges so the DFA has one edge per pair
    merged = {}
    for s, t, lab in edges:
        merged.setdefault((s, t), []).append(np.asarray(lab))
    edges = [(s, t, np.sort(np.concatenate(v))) for (s, t), v in sorted(merged.items())]
    return _pack(5, 12, 0, [1, 3], edges, name="real-number DFA S=5 V=12")


def two_token_real_dfa() -> Automaton:
    """The pages' length-2 example over the two tokens '1' (0) and '.' (1):
    the same real-number DFA restricted to one digit and no pad."""
    edges = [(0, 1, [0]), (0, 2, [1]), (1, 1, [0]), (1, 3, [1]),
             (2, 3, [0]), (2, 4, [1]), (3, 3, [0]), (3, 4, [1]), (4, 4, [0, 1])]
    return _pack(5, 2, 0, [1, 3], edges, name="two-token real-number DFA")


# ------------------------------------------------------------ special shapes
def universal_automaton(V: int) -> Automaton:
    """One accepting state with a self-loop on every token: accepts V^L."""
    return _pack(1, V, 0, [0], [(0, 0, np.arange(V))], name=f"universal V={V}")


def single_string_automaton(word, V: int) -> Automaton:
    """Chain DFA accepting exactly ``word``."""
    L = len(word)
    edges = [(i, i + 1, [int(word[i])]) for i in range(L)]
    return _pack(L + 1, V, 0, [L], edges, name=f"single-string L={L}")


# ------------------------------------------------------------ random families
def random_dfa(rng: np.random.Generator, S: int, V: int, n_accept: int, density: float,
               name="") -> Automaton:
    """Each state gets round(density*V) distinct tokens, each sent to a
    uniform destination; ``n_accept`` uniform accepting states."""
    k = max(1, int(round(density * V)))
    tok_dst = {}
    for s in range(S):
        toks = rng.choice(V, size=k, replace=False)
        dsts = rng.integers(0, S, size=k)
        tok_dst[s] = (toks.astype(np.int64), dsts.astype(np.int64))
    accept = rng.choice(S, size=n_accept, replace=False)
    edges = _group_by_pair(S, tok_dst)
    return _pack(S, V, 0, accept.tolist(), edges, name=name or f"random DFA S={S} V={V}")


def random_nfa(rng: np.random.Generator, S: int, V: int, E: int, n_accept: int,
               mean_label: float, name="") -> Automaton:
    """Uniform src/dst with replacement (parallel edges allowed); label size
    ~ Geometric(1/mean_label) on {1,2,...} capped at V; tokens uniform without
    replacement within an edge."""
    src = rng.integers(0, S, size=E)
    dst = rng.integers(0, S, size=E)
    sizes = np.minimum(rng.geometric(1.0 / mean_label, size=E), V)
    edges = []
    for e in range(E):
        k = int(sizes[e])
        if k * 4 < V:
            toks = np.unique(rng.integers(0, V, size=2 * k + 8))
            while toks.size < k:
                toks = np.unique(np.concatenate([toks, rng.integers(0, V, size=k)]))
            toks = rng.permutation(toks)[:k]
        else:
            toks = rng.choice(V, size=k, replace=False)
        edges.append((int(src[e]), int(dst[e]), np.sort(toks)))
    accept = rng.choice(S, size=n_accept, replace=False)
    return _pack(S, V, 0, accept.tolist(), edges, dfa=False,
                 name=name or f"random NFA S={S} E={E}")


def json_like_dfa(rng: np.random.Generator, S=256, V=151936, string_frac=0.1, pool=256,
                  max_struct=64, string_size=100_000, n_accept=4) -> Automaton:
    """JSON-schema-like DFA.

    round(string_frac*S) string states are drawn from 1..S-1; the rest are
    structural.  A pool of ``pool`` distinct token ids is shared by the
    structural states; its first id is the quote token q*.  A structural state
    has k ~ U{1..max_struct} pool tokens, each to a uniform destination.  A
    string state self-loops on ``string_size`` random tokens from V minus q*
    and sends q* to a uniform structural state.  Accepting states are
    structural.
    """
    n_str = int(round(string_frac * S))
    string_states = np.sort(rng.choice(np.arange(1, S), size=n_str, replace=False))
    is_str = np.zeros(S, bool)
    is_str[string_states] = True
    structural = np.flatnonzero(~is_str)
    pool_ids = rng.choice(V, size=pool, replace=False)
    q_star = int(pool_ids[0])
    non_q = np.delete(np.arange(V), q_star)
    edges = []
    for s in range(S):
        if is_str[s]:
            toks = np.sort(rng.choice(non_q, size=string_size, replace=False))
            qdst = int(rng.choice(structural))
            edges.append((s, s, toks))
            edges.append((s, qdst, np.array([q_star])))
        else:
            k = int(rng.integers(1, max_struct + 1))
            toks = rng.choice(pool_ids, size=k, replace=False).astype(np.int64)
            dsts = rng.integers(0, S, size=k).astype(np.int64)
            edges.extend(_group_by_pair(S, {s: (toks, dsts)}))
    edges.sort(key=lambda e: (e[0], e[1]))
    accept = rng.choice(structural, size=n_accept, replace=False)
    return _pack(S, V, 0, accept.tolist(), edges,
                 name=f"json-like DFA S={S} V={V}",
                 meta={"string_states": string_states, "q_star": q_star, "pool": pool_ids})


def range_dfa(rng: np.random.Generator, S=1024, V=151936, edges_per_state=16,
              n_accept=4) -> Automaton:
    """Batch-throughput DFA with contiguous range labels: per state,
    2*edges_per_state distinct sorted cut points in [0, V] give the ranges
    [c0,c1), [c2,c3), ... each to a uniform destination."""
    edges = []
    for s in range(S):
        cuts = np.sort(rng.choice(V + 1, size=2 * edges_per_state, replace=False))
        dsts = rng.integers(0, S, size=edges_per_state)
        for j in range(edges_per_state):
            edges.append((s, int(dsts[j]), np.array([cuts[2 * j], cuts[2 * j + 1]])))
    accept = rng.choice(S, size=n_accept, replace=False)
    return _pack(S, V, 0, accept.tolist(), edges, ranges=True,
                 name=f"range DFA S={S} V={V}")


def tiny_range_automaton(rng: np.random.Generator, S: int, V: int, E: int, dfa: bool) -> Automaton:
    """Small automaton with 1-2 random ranges per edge (possibly overlapping
    within an NFA)."""
    edges = []
    if dfa:
        for s in range(S):
            cuts = np.sort(rng.choice(V + 1, size=4, replace=False))
            d = rng.integers(0, S, size=2)
            if d[0] == d[1]:
                edges.append((s, int(d[0]), np.array([cuts[0], cuts[1], cuts[2], cuts[3]])))
            else:
                edges.append((s, int(d[0]), np.array([cuts[0], cuts[1]])))
                edges.append((s, int(d[1]), np.array([cuts[2], cuts[3]])))
    else:
        # one or two disjoint sorted ranges per edge; parallel edges may overlap
        for _ in range(E):
            n_rng = 1 if rng.random() < 0.7 or V < 4 else 2
            cuts = np.sort(rng.choice(V + 1, size=2 * n_rng, replace=False))
            edges.append((int(rng.integers(0, S)), int(rng.integers(0, S)), cuts))
    accept = rng.choice(S, size=max(1, S // 3), replace=False)
    return _pack(S, V, 0, accept.tolist(), edges, ranges=True, dfa=dfa,
                 name=f"tiny range {'DFA' if dfa else 'NFA'} S={S} V={V}")


# ---------------------------------------------------------------- reachability
def accepting_reach_sets(aut: Automaton, L: int):
    """R[j] = boolean mask of states that reach an accepting state in exactly
    j steps over edges with non-empty labels (input-side witness helper)."""
    R = np.zeros((L + 1, aut.S), bool)
    R[0, aut.accept] = True
    nonempty = np.diff(aut.label_off) > 0
    if aut.ranges:
        for e in np.flatnonzero(nonempty):
            seg = aut.label_tok[aut.label_off[e]:aut.label_off[e + 1]]
            nonempty[e] = bool(np.any(seg[1::2] > seg[0::2]))
    src = aut.src[nonempty]
    dst = aut.dst[nonempty]
    for j in range(1, L + 1):
        R[j, src[R[j - 1, dst]]] = True
    return R


def witness(aut: Automaton, L: int, rng: np.random.Generator):
    """A random accepted string of length L: walk from the start taking a
    uniform edge whose destination still reaches an accepting state in the
    remaining number of steps, then a uniform token of its label."""
    R = accepting_reach_sets(aut, L)
    if not R[L, aut.start]:
        return None
    out = np.zeros(L, np.int64)
    s = aut.start
    out_edges = {}
    for e in range(aut.E):
        out_edges.setdefault(int(aut.src[e]), []).append(e)
    for i in range(L):
        cands = [e for e in out_edges.get(s, [])
                 if R[L - i - 1, aut.dst[e]] and aut.edge_label(e).size > 0]
        e = cands[int(rng.integers(0, len(cands)))]
        lab = aut.edge_label(e)
        out[i] = lab[int(rng.integers(0, lab.size))]
        s = int(aut.dst[e])
    return out
