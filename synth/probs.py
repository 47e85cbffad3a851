"""Seeded per-position token probabilities p[b, i, v] (fp32).

Logits are drawn in fp64, soft-maxed in fp64 and cast to fp32.  Committed
positions (tokens a denoiser has already unmasked) are one-hot rows on the
tokens of an accepted witness string, so the constraint stays feasible.
"""
from __future__ import annotations

import numpy as np

from .automata import Automaton, witness


def _softmax_rows(x: np.ndarray) -> np.ndarray:
    x = x - x.max(axis=-1, keepdims=True)
    np.exp(x, out=x)
    x /= x.sum(axis=-1, keepdims=True)
    return x


def logits_rows(rng: np.random.Generator, kind: str, n: int, V: int) -> np.ndarray:
    """n rows of fp64 logits of the named distribution."""
    if kind == "normal2":
        return rng.normal(0.0, 2.0, size=(n, V))
    if kind == "normal4":
        return rng.normal(0.0, 4.0, size=(n, V))
    if kind == "gumbel3":
        return 3.0 * rng.gumbel(0.0, 1.0, size=(n, V))
    if kind == "normal4_zipf":
        # the token id plays the role of the Zipf rank: bias -1.1*ln(v+1)
        bias = -1.1 * np.log(np.arange(V, dtype=np.float64) + 1.0)
        return rng.normal(0.0, 4.0, size=(n, V)) + bias
    if kind == "uniform":
        return np.zeros((n, V))
    raise ValueError(kind)


def make_probs(aut: Automaton, B: int, L: int, kind: str, n_commit: int,
               seed_logits: int, seed_commit: int, chunk_rows: int = 64):
    """Return (p fp32 [B,L,V], commits list of (positions, tokens) per row)."""
    V = aut.V
    p = np.empty((B, L, V), dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(seed_logits))
    for b in range(B):
        for i0 in range(0, L, chunk_rows):
            n = min(chunk_rows, L - i0)
            p[b, i0:i0 + n] = _softmax_rows(logits_rows(rng, kind, n, V)).astype(np.float32)
    commits = []
    if n_commit > 0:
        crng = np.random.Generator(np.random.PCG64(seed_commit))
        for b in range(B):
            w = witness(aut, L, crng)
            if w is None:
                raise ValueError("automaton accepts no string of length L")
            pos = np.sort(crng.choice(L, size=min(n_commit, L), replace=False))
            p[b, pos] = 0.0
            p[b, pos, w[pos]] = 1.0
            commits.append((pos, w[pos]))
    return p, commits


def make_probs_device(aut: Automaton, B: int, L: int, kind: str, n_commit: int,
                      seed_logits: int, seed_commit: int, device):
    """The same distribution as make_probs, drawn on the device (torch's
    generator there, so not the same numbers): fp64 logits, fp64 softmax,
    cast to fp32, then the committed positions one-hot on the tokens of an
    accepted witness string (chosen on the host exactly as make_probs does).
    For workloads whose p is too large to draw and copy from the host
    quickly.  Returns (p cuda fp32 [B, L, V], commits)."""
    import torch
    V = aut.V
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_logits)
    p = torch.empty((B, L, V), dtype=torch.float32, device=device)
    bias = None
    if kind == "normal4_zipf":
        bias = -1.1 * torch.log(torch.arange(V, dtype=torch.float64, device=device) + 1.0)
    for b in range(B):
        if kind in ("normal2", "normal4", "normal4_zipf"):
            sd = 2.0 if kind == "normal2" else 4.0
            x = torch.randn((L, V), dtype=torch.float64, device=device, generator=gen) * sd
            if bias is not None:
                x += bias
        elif kind == "uniform":
            x = torch.zeros((L, V), dtype=torch.float64, device=device)
        else:
            raise ValueError(kind)
        p[b] = torch.softmax(x, dim=-1).to(torch.float32)
    commits = []
    if n_commit > 0:
        crng = np.random.Generator(np.random.PCG64(seed_commit))
        for b in range(B):
            w = witness(aut, L, crng)
            if w is None:
                raise ValueError("automaton accepts no string of length L")
            pos = np.sort(crng.choice(L, size=min(n_commit, L), replace=False))
            pt = torch.from_numpy(pos).to(device)
            p[b, pt] = 0.0
            p[b, pt, torch.from_numpy(w[pos]).to(device)] = 1.0
            commits.append((pos, w[pos]))
    return p, commits
