"""Named synthetic workloads.

Five presets mirror the workloads the sampler is measured on; every preset
can be shrunk (B, L, S, V) for tests.  Seeds: automaton 1000+k, logits
2000+k, commits and witness 3000+k, sampler seed 4000+k for preset k; if the
start state cannot reach an accepting state in exactly L steps the automaton
is re-drawn with the next seed.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import automata as A
from .probs import make_probs, make_probs_device


@dataclass
class Workload:
    name: str
    aut: A.Automaton
    p: np.ndarray  # fp32 [B, L, V]
    B: int
    L: int
    seed: int  # sampler seed
    commits: list

    def describe(self) -> str:
        a = self.aut
        return (f"{self.name}: {a.name}, S={a.S} V={a.V} E={a.E} "
                f"{'ranges ' if a.ranges else ''}{'DFA' if a.dfa else 'NFA'}, B={self.B} L={self.L}")


def _feasible(aut, L):
    return bool(A.accepting_reach_sets(aut, L)[L, aut.start])


def _draw(builder, seed, L, tries=16):
    for t in range(tries):
        aut = builder(np.random.Generator(np.random.PCG64(seed + t)))
        if _feasible(aut, L):
            return aut
    raise RuntimeError("no feasible automaton")


def make(k: int, *, B=None, L=None, S=None, V=None, E=None, device=None) -> Workload:
    """Preset k in 1..5, optionally shrunk.  With a device, p is drawn there
    (make_probs_device: the same distribution, other numbers) and the
    workload's p is a cuda tensor instead of a numpy array."""
    if k == 1:
        B, L = B or 1, L or 6
        aut = A.real_number_dfa()
        kind, n_commit = "normal2", 2
        name = "real-number DFA"
    elif k == 2:
        B, L, S, V = B or 4, L or 64, S or 32, V or 1024
        aut = _draw(lambda r: A.random_dfa(r, S, V, 4, 0.3), 1000 + k, L)
        kind, n_commit = "gumbel3", int(round(0.2 * L))
        name = "random DFA"
    elif k == 3:
        B, L, S, V = B or 4, L or 256, S or 256, V or 151936
        string_size = min(100_000, int(round(V * 100_000 / 151936)))
        aut = _draw(lambda r: A.json_like_dfa(r, S=S, V=V, pool=min(256, V // 4),
                                              string_size=string_size), 1000 + k, L)
        kind, n_commit = "normal4_zipf", 0
        name = "json-like DFA"
    elif k == 4:
        B, L, S, V = B or 16, L or 512, S or 1024, V or 151936
        aut = _draw(lambda r: A.range_dfa(r, S=S, V=V), 1000 + k, L)
        kind, n_commit = "normal4_zipf", L // 2
        name = "range DFA"
    elif k == 5:
        B, L, S, V, E = B or 1, L or 64, S or 10000, V or 151936, E or 100_000
        aut = _draw(lambda r: A.random_nfa(r, S, V, E, 16, 50.0), 1000 + k, L)
        kind, n_commit = "normal4", 0
        name = "random NFA"
    else:
        raise ValueError(k)
    if device is None:
        p, commits = make_probs(aut, B, L, kind, n_commit, 2000 + k, 3000 + k)
    else:
        p, commits = make_probs_device(aut, B, L, kind, n_commit, 2000 + k, 3000 + k, device)
    return Workload(name=name, aut=aut, p=p, B=B, L=L, seed=4000 + k, commits=commits)


def from_automaton(aut: A.Automaton, B: int, L: int, kind: str, n_commit: int, seed: int,
                   name: str = "") -> Workload:
    p, commits = make_probs(aut, B, L, kind, n_commit, seed + 1, seed + 2)
    return Workload(name=name or aut.name, aut=aut, p=p, B=B, L=L, seed=seed + 3,
                    commits=commits)
