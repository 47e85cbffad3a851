"""Finite-automaton-constrained sampling for one denoising step of a
diffusion language model, on AMD MI355X (gfx950).

The C ABI (include/fa.h, libfa.so) does the work; this package marshals
arguments.  See ``_fa.step`` for one whole step.
"""
from ._fa import (  # noqa: F401
    FA_CONF_NEGENT, FA_CONF_PROB, FA_CONF_UNCONSTRAINED, FA_DFA, FA_FIRST_LEVEL_DENSE, FA_FIRST_LEVEL_PAIRS, FA_FIRST_LEVEL_SPARSE, FA_SECOND_LEVEL_SPARSE, FA_LIVE_STATES,
    FA_LABEL_RANGES, FA_NFA, FA_NO_TRIM,
    FA_PROBE_COPY, FA_PROBE_READ,
    FA_PROF_EMISSION_DENSE, FA_PROF_MARG_Q, FA_PROF_NONE, FA_PROF_TREE_LEVEL1,
    FA_ROW_BADPROB, FA_ROW_INFEASIBLE, FA_ROW_UNDERFLOW, FaError, MapBuffers, StepBuffers, Table,
    build_transitions, chain_sample, chain_sample_marginals, chain_step, commit, generate, lib, map_decode, marginals, probe_bandwidth, profile_kernel, sample, sample_marginals,
    span_tree, span_tree_noalloc, step,
)
