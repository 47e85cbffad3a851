"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.  Holds no part of the sampler's arithmetic."""
from .automata import Automaton  # noqa: F401
from . import automata, probs, configs  # noqa: F401
