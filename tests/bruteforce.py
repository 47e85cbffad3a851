"""Brute-force enumeration of all V^L strings of a tiny automaton.

Independent of the oracle: the number of accepting paths of every string is
counted by an integer dynamic program over the raw edge list, and the
constrained distribution is weight(x) = prod_i p[i, x_i] * paths(x) / Z
(DFA: paths(x) is 0 or 1; NFA: the number of accepting paths).
"""
from __future__ import annotations

import itertools

import numpy as np


def label_sets(aut):
    return [set(aut.edge_label(e).tolist()) for e in range(aut.E)]


def all_strings(V: int, L: int) -> np.ndarray:
    return np.array(list(itertools.product(range(V), repeat=L)), dtype=np.int64).reshape(-1, L)


def path_counts(aut, X: np.ndarray) -> np.ndarray:
    """paths(x) for every row x of X (int64)."""
    N, L = X.shape
    labs = label_sets(aut)
    member = np.zeros((aut.E, aut.V), dtype=np.int64)
    for e, s in enumerate(labs):
        member[e, list(s)] = 1
    vec = np.zeros((N, aut.S), dtype=np.int64)
    vec[:, aut.start] = 1
    for i in range(L):
        nxt = np.zeros_like(vec)
        m = member[:, X[:, i]]  # [E, N]
        for e in range(aut.E):
            nxt[:, aut.dst[e]] += vec[:, aut.src[e]] * m[e]
        vec = nxt
    return vec[:, aut.accept].sum(axis=1)


def distribution(aut, p: np.ndarray):
    """For one batch row p [L, V]: (strings, probabilities, Z, q [L, V])."""
    L, V = p.shape
    X = all_strings(V, L)
    paths = path_counts(aut, X)
    w = np.ones(X.shape[0])
    pd = p.astype(np.float64)
    for i in range(L):
        w *= pd[i, X[:, i]]
    w *= paths
    Z = w.sum()
    prob = w / Z if Z > 0 else w
    q = np.zeros((L, V))
    for i in range(L):
        np.add.at(q[i], X[:, i], prob)
    return X, prob, Z, q
