"""Live states of a workload: per sequence row and boundary i, the states
reachable from the start state by i tokens of nonzero probability that can
still reach an accepting state with the remaining tokens.  Only these states
carry weight in the constrained posterior, so the counts bound what
position-dependent reachability masks could save: a span product over
[l, r) with midpoint m needs only live(l) x live(m) x live(r) multiply-adds.

This is an analysis of the synthetic inputs (numpy, host only); it holds none
of the sampler's arithmetic.

    python -m synth.live_states            # presets 2..5, rows 0 and B-1
"""
from __future__ import annotations

import sys

import numpy as np

from . import configs


def _label_index(aut):
    """Per label entry its edge, and the entries' token ids or [lo, hi) ranges."""
    counts = np.diff(aut.label_off)
    if aut.ranges:
        npair = counts // 2
        edge = np.repeat(np.arange(aut.E), npair)
        lo = aut.label_tok[0::2].astype(np.int64)
        hi = aut.label_tok[1::2].astype(np.int64)
        return edge, lo, hi
    edge = np.repeat(np.arange(aut.E), counts)
    tok = aut.label_tok.astype(np.int64)
    return edge, tok, tok + 1


def usable_edges(aut, support, index=None):
    """Bool [E]: edges whose label holds a token of `support` (sorted ids)."""
    edge, lo, hi = index if index is not None else _label_index(aut)
    if support.size == aut.V:
        return np.diff(aut.label_off) > 0
    # a label entry [lo, hi) holds a support token iff one lies in it
    first = np.searchsorted(support, lo, side="left")
    hit = first < np.searchsorted(support, hi, side="left")
    out = np.zeros(aut.E, dtype=bool)
    out[edge[hit]] = True
    return out


def live_states(aut, p_row):
    """Bool [L+1, S] for one row of probabilities p_row [L, V]."""
    L = p_row.shape[0]
    index = _label_index(aut)
    use = [usable_edges(aut, np.nonzero(p_row[i] > 0)[0], index) for i in range(L)]
    fwd = np.zeros((L + 1, aut.S), dtype=bool)
    fwd[0, aut.start] = True
    for i in range(L):
        e = use[i] & fwd[i, aut.src]
        fwd[i + 1, aut.dst[e]] = True
    bwd = np.zeros((L + 1, aut.S), dtype=bool)
    bwd[L, aut.accept] = True
    for i in range(L - 1, -1, -1):
        e = use[i] & bwd[i + 1, aut.dst]
        bwd[i, aut.src[e]] = True
    return fwd & bwd


def live_arithmetic(live, S):
    """Multiply-adds of the span tree's products restricted to live states,
    as a fraction of the dense S^3 per product (boundaries past L count
    every state: the identity leaves keep them)."""
    n = live.sum(axis=1).astype(np.float64)
    L = live.shape[0] - 1
    Lpad = 1 << max(0, (L - 1).bit_length())
    cnt = np.full(Lpad + 1, float(S))
    cnt[:L + 1] = n
    live_ops = dense_ops = 0.0
    span = 2
    while span <= Lpad:
        for l in range(0, Lpad, span):
            live_ops += cnt[l] * cnt[l + span // 2] * cnt[l + span]
            dense_ops += float(S) ** 3
        span *= 2
    return live_ops / dense_ops


def main(presets=(2, 3, 4, 5)):
    for k in presets:
        w = configs.make(k)
        for b in sorted({0, w.B - 1}):
            live = live_states(w.aut, w.p[b])
            n = live.sum(axis=1)
            print(f"preset {k} ({w.name}) row {b}: S={w.aut.S} L={w.L}: live states per boundary "
                  f"mean {n.mean():.1f} ({100 * n.mean() / w.aut.S:.1f}%), min {n.min()}, "
                  f"{int((n < 0.9 * w.aut.S).sum())} of {w.L + 1} boundaries below 90%; "
                  f"live products need {100 * live_arithmetic(live, w.aut.S):.1f}% of the dense arithmetic",
                  flush=True)


if __name__ == "__main__":
    main(tuple(int(x) for x in sys.argv[1:]) or (2, 3, 4, 5))
