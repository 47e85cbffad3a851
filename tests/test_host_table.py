"""Host-side tests of libfa.so (no GPU): every symbol fa.h declares is
exported, the automaton compiler validates its input, checks determinism,
trims dead states, and sizes the step buffers."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import constrained_decoding_diffusion_amd as fa
from constrained_decoding_diffusion_amd import _fa
from synth import automata as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"fa_compile_table", "fa_build_transitions", "fa_span_tree", "fa_sample",
            "fa_marginals"} <= set(names)
    lib = C.CDLL(_fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_fa.EXPORTS)


def _compile(S, V, start, accept, edges, flags=fa.FA_DFA):
    src = np.array([e[0] for e in edges], np.int32)
    dst = np.array([e[1] for e in edges], np.int32)
    off = np.zeros(len(edges) + 1, np.int64)
    off[1:] = np.cumsum([len(e[2]) for e in edges])
    tok = np.concatenate([np.asarray(e[2], np.int32) for e in edges]) if edges else np.zeros(0, np.int32)
    return fa.Table(S, V, start, accept, src, dst, off, tok, flags)


def _code(fn):
    with pytest.raises(fa.FaError) as ei:
        fn()
    return ei.value.code


@pytest.mark.parametrize("case", [
    dict(S=0, V=3, start=0, accept=[0], edges=[]),
    dict(S=2, V=3, start=2, accept=[0], edges=[]),
    dict(S=2, V=3, start=0, accept=[5], edges=[]),
    dict(S=2, V=3, start=0, accept=[1], edges=[(0, 2, [1])]),
    dict(S=2, V=3, start=0, accept=[1], edges=[(0, 1, [3])]),
    dict(S=2, V=3, start=0, accept=[1], edges=[(0, 1, [-1])]),
    dict(S=2, V=0, start=0, accept=[1], edges=[]),
])
def test_invalid_ids_rejected(case):
    assert _code(lambda: _compile(**case)) == _fa.FA_EINVAL


def test_invalid_ranges_and_flags():
    R = fa.FA_DFA | fa.FA_LABEL_RANGES
    assert _code(lambda: _compile(2, 10, 0, [1], [(0, 1, [5, 3])], R)) == _fa.FA_EINVAL
    assert _code(lambda: _compile(2, 10, 0, [1], [(0, 1, [5])], R)) == _fa.FA_EINVAL
    assert _code(lambda: _compile(2, 10, 0, [1], [(0, 1, [0, 11])], R)) == _fa.FA_EINVAL
    assert _code(lambda: _compile(2, 10, 0, [1], [(0, 1, [0, 5, 3, 7])], R)) == _fa.FA_EINVAL
    assert _code(lambda: _compile(2, 10, 0, [1], [(0, 1, [1])], fa.FA_DFA | fa.FA_NFA)) == _fa.FA_EINVAL
    assert _code(lambda: _compile(2, 10, 0, [1], [(0, 1, [1])], 1 << 10)) == _fa.FA_EINVAL
    # the sparse second level needs the sparse first level
    assert _code(lambda: _compile(2, 10, 0, [1], [(0, 1, [1])], fa.FA_DFA | fa.FA_FIRST_LEVEL_DENSE
                                  | fa.FA_SECOND_LEVEL_SPARSE)) == _fa.FA_EINVAL
    # decreasing label offsets
    with pytest.raises(fa.FaError):
        fa.Table(2, 10, 0, [1], [0], [1], np.array([0, -1], np.int64), np.zeros(0, np.int32), 1)


def test_first_level_flags_and_choice():
    """The first span level's form: forced either way, both at once
    rejected, and the automatic choice by the work ratio (a chain of states
    with one successor each is sparse; a complete graph is dense)."""
    edges = [(s, s + 1, [s % 7]) for s in range(39)]
    chain = lambda f: _compile(40, 10, 0, [39], edges, fa.FA_DFA | f)
    assert chain(0).info["first_sparse"] == 1
    assert chain(0).info["first_work"] == 38      # pairs (a, k), (k, c) sharing k
    assert chain(fa.FA_FIRST_LEVEL_DENSE).info["first_sparse"] == 0
    assert chain(fa.FA_FIRST_LEVEL_SPARSE).info["first_sparse"] == 1
    both = fa.FA_FIRST_LEVEL_SPARSE | fa.FA_FIRST_LEVEL_DENSE
    assert _code(lambda: chain(both)) == _fa.FA_EINVAL
    full = [(a, b, [a * 64 + b]) for a in range(64) for b in range(64)]
    t = _compile(64, 4096, 0, [63], full, fa.FA_DFA)
    assert t.info["first_work"] == 64 ** 3 and t.info["first_sparse"] == 0
    # the two-step pattern of a chain: pairs (s, s + 2); its work per product
    # is one multiply-add per pair (s, s + 2) followed by (s + 2, s + 4)
    t2 = chain(fa.FA_FIRST_LEVEL_SPARSE | fa.FA_SECOND_LEVEL_SPARSE)
    assert t2.info["second_sparse"] == 1
    assert t2.info["pairs2"] == 38 and t2.info["second_work"] == 36
    assert chain(fa.FA_FIRST_LEVEL_DENSE).info["second_sparse"] == 0
    # no dense leaves once the first level is sparse and every leaf reader
    # can take the pair values
    assert chain(0).info["leafless"] == 1
    assert chain(fa.FA_FIRST_LEVEL_DENSE).info["leafless"] == 0
    # the sparse form keeps the row pointers and column exponents in LDS,
    # which bounds its states
    big = [(s, s + 1, [0]) for s in range(16400)]
    assert _code(lambda: _compile(16401, 2, 0, [16400], big,
                                  fa.FA_DFA | fa.FA_FIRST_LEVEL_SPARSE)) == _fa.FA_ETOOBIG
    assert _compile(16401, 2, 0, [16400], big, fa.FA_DFA).info["first_sparse"] == 0


def test_pair_staged_first_level():
    """The dense first level staged from the pair values: chosen when the
    sparse form's work is too large and the table allows it (Sp a multiple
    of 256, the pairs fit the pair-value leaf level, no live states); such a
    table keeps no dense leaves.  Forced where it cannot run: FA_ETOOBIG, or
    FA_EINVAL with FA_LIVE_STATES or another first-level flag."""
    S, fan = 200, 40
    edges = [(s, (13 * s + 17 * j + 1) % S, [s * fan + j]) for s in range(S) for j in range(fan)]
    mk = lambda f: _compile(S, S * fan, 0, [S - 1], edges, fa.FA_DFA | f)
    t = mk(0)
    assert t.info["Sp"] == 256 and t.info["first_work"] > 256 ** 3 // 256
    assert t.info["first_pairs"] == 1 and t.info["first_sparse"] == 0 and t.info["leafless"] == 1
    assert mk(fa.FA_FIRST_LEVEL_PAIRS).info["first_pairs"] == 1
    dense = mk(fa.FA_FIRST_LEVEL_DENSE)
    assert dense.info["first_pairs"] == 0 and dense.info["leafless"] == 0
    assert mk(fa.FA_FIRST_LEVEL_SPARSE).info["first_pairs"] == 0
    live = mk(fa.FA_LIVE_STATES)
    assert live.info["first_pairs"] == 0 and live.info["leafless"] == 0
    assert _code(lambda: mk(fa.FA_FIRST_LEVEL_PAIRS | fa.FA_LIVE_STATES)) == _fa.FA_EINVAL
    assert _code(lambda: mk(fa.FA_FIRST_LEVEL_PAIRS | fa.FA_FIRST_LEVEL_DENSE)) == _fa.FA_EINVAL
    # Sp = 64: no 256x256 tiles
    chain = [(s, s + 1, [s % 7]) for s in range(39)]
    assert _code(lambda: _compile(40, 10, 0, [39], chain, fa.FA_DFA | fa.FA_FIRST_LEVEL_PAIRS)) \
        == _fa.FA_ETOOBIG
    assert _compile(40, 10, 0, [39], chain, fa.FA_DFA).info["first_pairs"] == 0


def test_determinism_check():
    edges = [(0, 1, [3, 4]), (0, 2, [4, 5]), (1, 1, [0]), (2, 2, [0])]
    assert _code(lambda: _compile(3, 6, 0, [1, 2], edges, fa.FA_DFA)) == _fa.FA_ENOTDET
    t = _compile(3, 6, 0, [1, 2], edges, fa.FA_NFA)
    assert t.info["pairs"] == 4
    R = fa.FA_DFA | fa.FA_LABEL_RANGES
    assert _code(lambda: _compile(3, 9, 0, [1], [(0, 1, [0, 5]), (0, 2, [4, 6])], R)) == _fa.FA_ENOTDET
    assert _compile(3, 9, 0, [1], [(0, 1, [0, 4]), (0, 2, [4, 6])], R).info["range_pairs"] == 1


def test_repeated_label_tokens_count_once():
    t = _compile(2, 5, 0, [1], [(0, 1, [2, 2, 3]), (1, 1, [1])], fa.FA_DFA)
    assert t.info["list_entries"] == 3


def test_trimming_and_state_map():
    # 0 -> 2 -> 4 (accepting); 1 unreachable; 3 dead (cannot reach 4)
    edges = [(0, 2, [0]), (2, 4, [1]), (1, 4, [0]), (0, 3, [2]), (3, 3, [2]), (4, 4, [0])]
    t = _compile(5, 3, 0, [4], edges)
    assert t.info["S"] == 3 and t.info["S_orig"] == 5
    np.testing.assert_array_equal(t.orig, [0, 2, 4])
    assert t.info["pairs"] == 3 and t.info["n_accept"] == 1
    t2 = _compile(5, 3, 0, [4], edges, fa.FA_DFA | fa.FA_NO_TRIM)
    assert t2.info["S"] == 5 and t2.info["pairs"] == 6
    # empty accepting set: only the start state survives, nothing is feasible
    t3 = _compile(5, 3, 0, [], edges)
    assert t3.info["S"] == 1 and t3.info["pairs"] == 0 and t3.info["n_accept"] == 0


def test_label_classes():
    rng = np.random.default_rng(0)
    aut = A.json_like_dfa(rng, S=64, V=40000, pool=64, string_size=20000)
    t = fa.Table.from_automaton(aut)
    n_str = len(aut.meta["string_states"])
    assert t.info["dense_pairs"] == n_str
    assert t.info["use_sel"] == 1
    # NFA with overlapping parallel edges: counts > 1 keep the pair a token list
    edges = [(0, 1, np.arange(5000)), (0, 1, np.arange(4000, 9000)), (1, 1, [0])]
    t2 = _compile(2, 10000, 0, [1], edges, fa.FA_NFA)
    assert t2.info["dense_pairs"] == 0 and t2.info["list_entries"] == 9001 - 1 + 1


def test_range_pairs_merge_parallel_edges():
    R = fa.FA_NFA | fa.FA_LABEL_RANGES
    # two parallel ranges overlapping on [4, 6): three segments, counts 1, 2, 1
    t = _compile(2, 10, 0, [1], [(0, 1, [0, 6]), (0, 1, [4, 9]), (1, 1, [0, 10])], R)
    assert t.info["range_pairs"] == 2
    assert t.info["segments"] == 4
    assert t.info["cuts"] == 5  # 0, 4, 6, 9, 10


def test_map_range_structure_limit():
    """MAP decoding over range labels keeps one position's interval maxima and
    their block table in 160 KB of LDS: 35,420 cut points fit, 35,422 do not
    (FA_ETOOBIG from the sizes and from the decode call, before any launch)."""
    R = fa.FA_DFA | fa.FA_LABEL_RANGES
    lib = _fa.lib()
    for k, ok in ((17710, True), (17711, False)):
        lab = np.stack([2 * np.arange(k), 2 * np.arange(k) + 1], 1).ravel()
        t = _compile(1, 40000, 0, [0], [(0, 0, lab)], R)
        assert t.info["cuts"] == 2 * k
        tb, wb = C.c_size_t(), C.c_size_t()
        rc = lib.fa_map_sizes(t.handle, 1, 8, C.byref(tb), C.byref(wb))
        assert rc == (_fa.FA_OK if ok else _fa.FA_ETOOBIG)
        if not ok:
            rc = lib.fa_map_decode(t.handle, None, 1, 8, None, None, 0, None, None, None, None,
                                   None)
            assert rc == _fa.FA_ETOOBIG


def test_sizes_and_limits():
    t = fa.Table.from_automaton(A.real_number_dfa())
    Sp = t.info["Sp"]
    tree, meta, ws = t.sizes(3, 6)
    assert tree == 3 * 2 * 8 * Sp * Sp * 4
    assert meta == 3 * 2 * 8 * 3 * Sp * 4
    assert ws > 0
    assert t.sizes(0, 6)[0] == 0
    # a batch beyond one launch's grid runs in row chunks, each with its own
    # workspace slot: 40000 rows of Lpad 8 take 10 chunks of 4095 rows
    tb1, mb1, wb1 = t.sizes(4095, 6)
    tbn, mbn, wbn = t.sizes(40000, 6)
    assert tbn == 40000 * 2 * 8 * Sp * Sp * 4 and mbn == 40000 * 2 * 8 * 3 * Sp * 4
    assert wbn >= 10 * wb1
    # one row must fit: 2 Lpad <= 65535
    t.sizes(1, 16384)
    with pytest.raises(fa.FaError) as ei:
        t.sizes(1, 16385)
    assert ei.value.code == _fa.FA_ETOOBIG
    # lengths at and far beyond the kernels' 24-bit position fields are
    # rejected before any geometry is formed (no overflow of the padded length)
    for L in (1 << 24, (1 << 30) + 1, 2 ** 31 - 1):
        with pytest.raises(fa.FaError) as ei:
            t.sizes(1, L)
        assert ei.value.code == _fa.FA_ETOOBIG
    with pytest.raises(fa.FaError) as ei:
        t.sizes(1, -1)
    assert ei.value.code == _fa.FA_EINVAL
    rc = _fa.lib().fa_span_tree(t.handle, 1, 2 ** 31 - 1, None, None, None, 0, None, None, None)
    assert rc in (_fa.FA_ETOOBIG, _fa.FA_ESTATE)


def test_step_calls_need_an_uploaded_table():
    t = fa.Table.from_automaton(A.real_number_dfa())
    rc = _fa.lib().fa_build_transitions(t.handle, None, 1, 6, None, None, None, 0, None, None)
    assert rc == _fa.FA_ESTATE
    rc = _fa.lib().fa_span_tree(None, 1, 6, None, None, None, 0, None, None, None)
    assert rc == _fa.FA_EINVAL
    rc = _fa.lib().fa_sample_marginals(t.handle, None, 1, 6, None, None, None, C.c_uint64(1), 0,
                                       None, None, None, None, None, 0, None, None)
    assert rc == _fa.FA_ESTATE
    rc = _fa.lib().fa_sample_marginals(None, None, 1, 6, None, None, None, C.c_uint64(1), 0,
                                       None, None, None, None, None, 0, None, None)
    assert rc == _fa.FA_EINVAL


def test_commit_argument_checks():
    """fa_commit rejects bad sizes before launching anything."""
    lib = _fa.lib()
    call = lambda B, L, V, steps: lib.fa_commit(B, L, V, None, None, steps, None, None, None,
                                                None, None)
    assert call(1, 9000, 10, 1) == _fa.FA_ETOOBIG
    assert call(1, 16, 10, 0) == _fa.FA_EINVAL
    assert call(1, 16, 0, 1) == _fa.FA_EINVAL
    assert call(-1, 16, 10, 1) == _fa.FA_EINVAL
    assert call(1, 16, 10, 1) == _fa.FA_EINVAL  # buffers missing
    assert call(0, 16, 10, 1) == _fa.FA_OK      # nothing to do
    assert call(2, 0, 10, 1) == _fa.FA_OK


def test_profile_hook_arguments():
    lib = _fa.lib()
    assert lib.fa_profile_kernel(_fa.FA_PROF_NONE, None, None) == _fa.FA_OK
    assert lib.fa_profile_kernel(_fa.FA_PROF_MARG_Q, None, None) == _fa.FA_EINVAL
    assert lib.fa_profile_kernel(99, None, None) == _fa.FA_EINVAL
    assert lib.fa_profile_kernel(-1, None, None) == _fa.FA_EINVAL
    # a set hook with no GPU work issued is cleared again
    fake = C.c_void_p(0x1000)
    assert lib.fa_profile_kernel(_fa.FA_PROF_EMISSION_DENSE, fake, fake) == _fa.FA_OK
    assert lib.fa_profile_kernel(_fa.FA_PROF_NONE, None, None) == _fa.FA_OK


def test_noalloc_span_tree_argument_checks():
    """fa_span_tree_noalloc refuses, before launching anything, a table whose
    first span level reads the emission workspace, and a table not uploaded."""
    lib = _fa.lib()
    aut = A.random_dfa(np.random.default_rng(3), 12, 40, 3, 0.4)
    sparse = fa.Table.from_automaton(aut, first_level="sparse")
    assert sparse.info["first_sparse"] == 1
    call = lambda t, B, L: lib.fa_span_tree_noalloc(t, B, L, None, None, None, None, None)
    assert call(sparse.handle, 1, 8) == _fa.FA_EINVAL
    dense = fa.Table.from_automaton(aut, first_level="dense")
    assert call(dense.handle, 1, 8) == _fa.FA_ESTATE
    assert call(None, 1, 8) == _fa.FA_EINVAL
    assert _fa.FA_SPAN_TREE_NOALLOC_MAX_BYTES == 8 << 20
