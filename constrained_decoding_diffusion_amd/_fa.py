"""ctypes binding of libfa.so: argument marshalling only.

Every step of the sampler runs in the library's HIP kernels; torch is used
for device memory and the current stream.  Importing works without a GPU
(the table compiler is host code); the step calls need one.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK, FA_EINVAL, FA_ENOTDET, FA_ETOOBIG, FA_EHIP, FA_ESTATE = range(6)
FA_ROW_INFEASIBLE, FA_ROW_UNDERFLOW, FA_ROW_BADPROB = 1, 2, 4
FA_DFA, FA_NFA, FA_LABEL_RANGES, FA_NO_TRIM = 1, 2, 4, 8
FA_FIRST_LEVEL_SPARSE, FA_FIRST_LEVEL_DENSE, FA_SECOND_LEVEL_SPARSE = 16, 32, 64
FA_LIVE_STATES = 128
FA_FIRST_LEVEL_PAIRS = 256
FA_CONF_PROB, FA_CONF_NEGENT, FA_CONF_UNCONSTRAINED = 0, 1, 2
FA_PROF_NONE, FA_PROF_EMISSION_DENSE, FA_PROF_TREE_LEVEL1, FA_PROF_MARG_Q = range(4)
FA_PROBE_READ, FA_PROBE_COPY = 0, 1

EXPORTS = ["fa_compile_table", "fa_table_upload", "fa_table_destroy", "fa_table_info",
           "fa_table_state_map", "fa_sizes", "fa_build_transitions", "fa_span_tree", "fa_sample",
           "fa_marginals", "fa_sample_marginals", "fa_commit", "fa_strerror", "fa_profile_kernel",
           "fa_span_tree_noalloc", "fa_probe_bandwidth", "fa_map_sizes", "fa_map_decode",
           "fa_chain_sample", "fa_chain_sample_marginals"]
FA_SPAN_TREE_NOALLOC_MAX_BYTES = 8 << 20


class FaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {lib().fa_strerror(code).decode()} (code {code})")
        self.code = code


_lib = None


def lib():
    """Load libfa.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(the sampler has no CPU path)")
    # torch first: the HIP runtime torch ships is then the one libfa binds
    # to, so device pointers and streams from torch are valid in the library
    import torch  # noqa: F401
    L = C.CDLL(LIB_PATH)
    P, I32, I64, U32, U64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64, C.c_size_t
    L.fa_compile_table.argtypes = [I32, I32, I32, P, I32, I64, P, P, P, P, U32, P, P]
    L.fa_table_upload.argtypes = [P, P, SZ, P]
    L.fa_table_destroy.argtypes = [P]
    L.fa_table_destroy.restype = None
    L.fa_table_info.argtypes = [P, P, I32]
    L.fa_table_state_map.argtypes = [P, P]
    L.fa_sizes.argtypes = [P, I32, I32, P, P, P]
    L.fa_build_transitions.argtypes = [P, P, I32, I32, P, P, P, SZ, P, P]
    L.fa_span_tree.argtypes = [P, I32, I32, P, P, P, SZ, P, P, P]
    L.fa_span_tree_noalloc.argtypes = [P, I32, I32, P, P, P, P, P]
    L.fa_sample.argtypes = [P, P, I32, I32, P, P, U64, P, P, P, SZ, P, P]
    L.fa_marginals.argtypes = [P, P, I32, I32, P, P, P, P, I32, P, P, P, SZ, P, P]
    L.fa_sample_marginals.argtypes = [P, P, I32, I32, P, P, P, U64, I32, P, P, P, P, P, SZ, P, P]
    L.fa_commit.argtypes = [I32, I32, I32, P, P, I32, P, P, P, P, P]
    L.fa_profile_kernel.argtypes = [I32, P, P]
    L.fa_probe_bandwidth.argtypes = [I32, P, P, SZ, I32, P]
    L.fa_map_sizes.argtypes = [P, I32, I32, P, P]
    L.fa_chain_sample.argtypes = [P, P, I32, I32, P, U64, P, P, P, P, SZ, P, P]
    L.fa_chain_sample_marginals.argtypes = [P, P, I32, I32, P, U64, I32, P, P, P, P, P, P, SZ, P, P]
    L.fa_map_decode.argtypes = [P, P, I32, I32, P, P, SZ, P, P, P, P, P]
    L.fa_strerror.argtypes = [C.c_int]
    L.fa_strerror.restype = C.c_char_p
    for fn in EXPORTS:
        if fn != "fa_table_destroy" and fn != "fa_strerror":
            getattr(L, fn).restype = C.c_int
    _lib = L
    return L


def _check(fn: str, rc: int):
    if rc != FA_OK:
        raise FaError(fn, rc)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


INFO_KEYS = ["S", "Sp", "start", "n_accept", "pairs", "list_pairs", "dense_pairs", "range_pairs",
             "list_entries", "segments", "cuts", "sel_tokens", "use_sel", "V", "S_orig",
             "first_sparse", "first_work", "second_sparse", "second_work", "pairs2", "leafless",
             "leaf_msg_pairs", "live_states", "first_pairs", "map_first_sparse"]


class Table:
    """A compiled automaton (host handle); ``upload`` places its image in a
    torch uint8 device buffer owned by this object."""

    def __init__(self, S, V, start, accept, src, dst, label_off, label_tok, flags):
        self._arr = [np.ascontiguousarray(accept, np.int32), np.ascontiguousarray(src, np.int32),
                     np.ascontiguousarray(dst, np.int32), np.ascontiguousarray(label_off, np.int64),
                     np.ascontiguousarray(label_tok, np.int32)]
        acc, s, d, off, tok = self._arr
        h = C.c_void_p()
        nbytes = C.c_size_t()
        rc = lib().fa_compile_table(S, V, start, _np_ptr(acc), acc.size, s.size, _np_ptr(s),
                                    _np_ptr(d), _np_ptr(off), _np_ptr(tok), flags, C.byref(h),
                                    C.byref(nbytes))
        _check("fa_compile_table", rc)
        self.handle = h
        self.device_bytes = nbytes.value
        self.buf = None
        info = np.zeros(len(INFO_KEYS), np.int64)
        _check("fa_table_info", lib().fa_table_info(h, _np_ptr(info), len(INFO_KEYS)))
        self.info = dict(zip(INFO_KEYS, (int(x) for x in info)))
        orig = np.zeros(self.info["S"], np.int32)
        _check("fa_table_state_map", lib().fa_table_state_map(h, _np_ptr(orig)))
        self.orig = orig

    @classmethod
    def from_automaton(cls, aut, flags=None, first_level="auto", live_states=False):
        """first_level: "auto" (the library's choice), "sparse" (first span
        level from the pair values), "sparse2" (also the second level, from
        the two-step pattern), "dense" (dense matrix products over dense
        leaves) or "pairs" (dense matrix products whose operands are staged
        from the pair values; no dense leaves).
        live_states: FA_LIVE_STATES (span products over the states live at
        their midpoint under each step's p)."""
        if flags is None:
            flags = (FA_DFA if aut.dfa else FA_NFA) | (FA_LABEL_RANGES if aut.ranges else 0)
        if live_states:
            flags |= FA_LIVE_STATES
        flags |= {"auto": 0, "sparse": FA_FIRST_LEVEL_SPARSE,
                  "dense": FA_FIRST_LEVEL_DENSE, "pairs": FA_FIRST_LEVEL_PAIRS,
                  "sparse2": FA_FIRST_LEVEL_SPARSE | FA_SECOND_LEVEL_SPARSE}[first_level]
        return cls(aut.S, aut.V, aut.start, aut.accept, aut.src, aut.dst, aut.label_off,
                   aut.label_tok, flags)

    def upload(self, device="cuda"):
        import torch
        self.buf = torch.empty(max(self.device_bytes, 256), dtype=torch.uint8, device=device)
        stream = torch.cuda.current_stream(self.buf.device).cuda_stream
        _check("fa_table_upload", lib().fa_table_upload(self.handle, C.c_void_p(self.buf.data_ptr()),
                                                        self.buf.numel(), C.c_void_p(stream)))
        return self

    def sizes(self, B: int, L: int):
        t, m, w = C.c_size_t(), C.c_size_t(), C.c_size_t()
        _check("fa_sizes", lib().fa_sizes(self.handle, B, L, C.byref(t), C.byref(m), C.byref(w)))
        return t.value, m.value, w.value

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.fa_table_destroy(h)
            self.handle = None


def _ptr(t):
    return C.c_void_p(0 if t is None else t.data_ptr())


class StepBuffers:
    """Device buffers of one constrained step (batch B, length L)."""

    def __init__(self, table: Table, B: int, L: int, want_q=True, device="cuda"):
        import torch
        tb, mb, wb = table.sizes(B, L)
        self.B, self.L = B, L
        self.tree = torch.empty(max(tb // 4, 1), dtype=torch.float32, device=device)
        self.meta = torch.empty(max(mb // 4, 1), dtype=torch.int32, device=device)
        self.ws = torch.empty(max(wb, 256), dtype=torch.uint8, device=device)
        self.logZ = torch.empty(B, dtype=torch.float64, device=device)
        self.status = torch.zeros(B, dtype=torch.int32, device=device)
        self.states = torch.empty((B, L + 1), dtype=torch.int32, device=device)
        self.tokens = torch.empty((B, max(L, 1)), dtype=torch.int32, device=device)
        self.conf = torch.empty((B, max(L, 1)), dtype=torch.float32, device=device)
        self.q = None
        if want_q:
            self.q = torch.empty((B, L, table.info["V"]), dtype=torch.float32, device=device)


def build_transitions(table: Table, p, bufs: StepBuffers, stream):
    _check("fa_build_transitions", lib().fa_build_transitions(
        table.handle, _ptr(p), bufs.B, bufs.L, _ptr(bufs.tree), _ptr(bufs.meta), _ptr(bufs.ws),
        bufs.ws.numel(), _ptr(bufs.status), C.c_void_p(stream)))


def span_tree(table: Table, bufs: StepBuffers, stream):
    _check("fa_span_tree", lib().fa_span_tree(
        table.handle, bufs.B, bufs.L, _ptr(bufs.tree), _ptr(bufs.meta), _ptr(bufs.ws),
        bufs.ws.numel(), _ptr(bufs.logZ), _ptr(bufs.status), C.c_void_p(stream)))


def span_tree_noalloc(table: Table, bufs: StepBuffers, stream):
    """fa_span_tree_noalloc: the span tree with its scratch in the library's
    own device array (bufs.ws is not used)."""
    _check("fa_span_tree_noalloc", lib().fa_span_tree_noalloc(
        table.handle, bufs.B, bufs.L, _ptr(bufs.tree), _ptr(bufs.meta), _ptr(bufs.logZ),
        _ptr(bufs.status), C.c_void_p(stream)))


def sample(table: Table, p, bufs: StepBuffers, seed: int, stream):
    _check("fa_sample", lib().fa_sample(
        table.handle, _ptr(p), bufs.B, bufs.L, _ptr(bufs.tree), _ptr(bufs.meta),
        C.c_uint64(seed), _ptr(bufs.states), _ptr(bufs.tokens), _ptr(bufs.ws), bufs.ws.numel(),
        _ptr(bufs.status), C.c_void_p(stream)))


def marginals(table: Table, p, bufs: StepBuffers, conf_mode: int, stream, write_q=True):
    _check("fa_marginals", lib().fa_marginals(
        table.handle, _ptr(p), bufs.B, bufs.L, _ptr(bufs.tree), _ptr(bufs.meta), _ptr(bufs.logZ),
        _ptr(bufs.tokens), conf_mode, _ptr(bufs.q if write_q else None), _ptr(bufs.conf),
        _ptr(bufs.ws), bufs.ws.numel(), _ptr(bufs.status), C.c_void_p(stream)))


def sample_marginals(table: Table, p, bufs: StepBuffers, seed: int, conf_mode: int, stream,
                     write_q=True):
    _check("fa_sample_marginals", lib().fa_sample_marginals(
        table.handle, _ptr(p), bufs.B, bufs.L, _ptr(bufs.tree), _ptr(bufs.meta), _ptr(bufs.logZ),
        C.c_uint64(seed), conf_mode, _ptr(bufs.states), _ptr(bufs.tokens),
        _ptr(bufs.q if write_q else None), _ptr(bufs.conf), _ptr(bufs.ws), bufs.ws.numel(),
        _ptr(bufs.status), C.c_void_p(stream)))


def commit(p, bufs: StepBuffers, committed, fresh, steps_left: int, stream):
    """The remasking step (fa_commit) on the step's confidence and tokens:
    committed and fresh are cuda int32 [B, L]; committed rows of p become
    one-hot."""
    B, L, V = p.shape
    _check("fa_commit", lib().fa_commit(
        B, L, V, _ptr(bufs.conf), _ptr(bufs.tokens), steps_left, _ptr(committed), _ptr(fresh),
        _ptr(p), _ptr(bufs.status), C.c_void_p(stream)))


def generate(table: Table, p, T: int, seed: int, conf_mode: int = FA_CONF_PROB, bufs=None,
             on_step=None):
    """A synthetic T-step denoising generation on torch's current stream: p
    (cuda float32 [B, L, V], updated in place) holds the model's per-position
    probabilities; each step is one constrained step (seed + t) followed by
    the remasking step with T - t steps left, so after T steps every position
    is committed and p is one-hot at the generated tokens.  on_step(t, bufs,
    committed, fresh), if given, is called after each step's commit.  Returns
    (bufs, committed)."""
    import torch
    B, L, V = p.shape
    if bufs is None:
        bufs = StepBuffers(table, B, L, want_q=True, device=p.device)
    committed = torch.zeros((B, max(L, 1)), dtype=torch.int32, device=p.device)
    fresh = torch.zeros_like(committed)
    stream = torch.cuda.current_stream(p.device).cuda_stream
    for t in range(T):
        step(table, p, seed + t, bufs, conf_mode=conf_mode)
        commit(p, bufs, committed, fresh, T - t, stream)
        if on_step is not None:
            on_step(t, bufs, committed, fresh)
    return bufs, committed


def chain_sample(table: Table, p, bufs: StepBuffers, seed: int, stream):
    """fa_chain_sample: the serial chain sampler on the leaves in bufs.tree
    (after build_transitions); writes bufs.logZ, states, tokens."""
    _check("fa_chain_sample", lib().fa_chain_sample(
        table.handle, _ptr(p), bufs.B, bufs.L, _ptr(bufs.tree), C.c_uint64(seed), _ptr(bufs.logZ),
        _ptr(bufs.states), _ptr(bufs.tokens), _ptr(bufs.ws), bufs.ws.numel(), _ptr(bufs.status),
        C.c_void_p(stream)))


def chain_sample_marginals(table: Table, p, bufs: StepBuffers, seed: int, conf_mode: int, stream,
                           write_q=True):
    """fa_chain_sample_marginals: the chain sampler, backward messages and
    the marginals from the two message chains (after build_transitions)."""
    _check("fa_chain_sample_marginals", lib().fa_chain_sample_marginals(
        table.handle, _ptr(p), bufs.B, bufs.L, _ptr(bufs.tree), C.c_uint64(seed), conf_mode,
        _ptr(bufs.logZ), _ptr(bufs.states), _ptr(bufs.tokens), _ptr(bufs.q if write_q else None),
        _ptr(bufs.conf), _ptr(bufs.ws), bufs.ws.numel(), _ptr(bufs.status), C.c_void_p(stream)))


def chain_step(table: Table, p, seed: int, bufs: StepBuffers = None, marginals=False,
               conf_mode: int = FA_CONF_PROB, write_q=True):
    """The emission reduce and the chain sampler on torch's current stream
    (the serial baseline of step()'s sampling half); with marginals, the
    whole serial forward-backward step (q and conf as well)."""
    import torch
    B, L, V = p.shape
    if table.buf is None:
        table.upload(p.device)
    if bufs is None:
        bufs = StepBuffers(table, B, L, want_q=marginals and write_q, device=p.device)
    stream = torch.cuda.current_stream(p.device).cuda_stream
    bufs.status.zero_()
    build_transitions(table, p, bufs, stream)
    if marginals:
        chain_sample_marginals(table, p, bufs, seed, conf_mode, stream, write_q=write_q)
    else:
        chain_sample(table, p, bufs, seed, stream)
    return bufs


class MapBuffers:
    """Device buffers of MAP decoding (batch B, length L)."""

    def __init__(self, table: Table, B: int, L: int, device="cuda"):
        import torch
        t, w = C.c_size_t(), C.c_size_t()
        _check("fa_map_sizes", lib().fa_map_sizes(table.handle, B, L, C.byref(t), C.byref(w)))
        self.B, self.L = B, L
        self.tree = torch.empty(max(t.value // 8, 1), dtype=torch.float64, device=device)
        self.ws = torch.empty(max(w.value, 256), dtype=torch.uint8, device=device)
        self.logmax = torch.empty(B, dtype=torch.float64, device=device)
        self.status = torch.zeros(B, dtype=torch.int32, device=device)
        self.states = torch.empty((B, L + 1), dtype=torch.int32, device=device)
        self.tokens = torch.empty((B, max(L, 1)), dtype=torch.int32, device=device)


def map_decode(table: Table, p, bufs: "MapBuffers" = None):
    """Greedy constrained decoding (fa_map_decode) on torch's current stream:
    p cuda float32 [B, L, V].  Returns the buffers (logmax, states, tokens,
    status)."""
    import torch
    B, L, V = p.shape
    if V != table.info["V"]:
        raise ValueError(f"p has V={V}, table has V={table.info['V']}")
    if not p.is_cuda or p.dtype != torch.float32 or not p.is_contiguous():
        raise ValueError("p must be a contiguous cuda float32 tensor")
    if table.buf is None:
        table.upload(p.device)
    if bufs is None:
        bufs = MapBuffers(table, B, L, device=p.device)
    stream = torch.cuda.current_stream(p.device).cuda_stream
    bufs.status.zero_()
    _check("fa_map_decode", lib().fa_map_decode(
        table.handle, _ptr(p), B, L, _ptr(bufs.tree), _ptr(bufs.ws), bufs.ws.numel(),
        _ptr(bufs.logmax), _ptr(bufs.states), _ptr(bufs.tokens), _ptr(bufs.status),
        C.c_void_p(stream)))
    return bufs


def probe_bandwidth(mode: int, src, dst, nbytes: int, blocks: int, stream):
    """Measurement hook: one plain read (FA_PROBE_READ) or copy
    (FA_PROBE_COPY) kernel over nbytes of the cuda tensors src/dst."""
    _check("fa_probe_bandwidth", lib().fa_probe_bandwidth(mode, _ptr(src), _ptr(dst), nbytes,
                                                          blocks, C.c_void_p(stream)))


def profile_kernel(which: int, start_event=None, stop_event=None):
    """Measurement hook: bracket the launches of one kernel with two HIP
    events (raw hipEvent_t handles as ints), FA_PROF_NONE to clear."""
    _check("fa_profile_kernel", lib().fa_profile_kernel(which, C.c_void_p(start_event or 0),
                                                        C.c_void_p(stop_event or 0)))


def step(table: Table, p, seed: int, bufs: StepBuffers = None, conf_mode: int = FA_CONF_PROB,
         write_q: bool = True, joint: bool = True):
    """One constrained denoising step on torch's current stream: emission
    reduce, span tree, sampling, marginals.  p: cuda float32 [B, L, V].
    joint: sampling and marginals through fa_sample_marginals (one pass over
    p less when the draws can share the q writer's pass); else fa_sample then
    fa_marginals.  Both give the same outputs."""
    import torch
    B, L, V = p.shape
    if V != table.info["V"]:
        raise ValueError(f"p has V={V}, table has V={table.info['V']}")
    if not p.is_cuda or p.dtype != torch.float32 or not p.is_contiguous():
        raise ValueError("p must be a contiguous cuda float32 tensor")
    if table.buf is None:
        table.upload(p.device)
    if bufs is None:
        bufs = StepBuffers(table, B, L, want_q=write_q, device=p.device)
    stream = torch.cuda.current_stream(p.device).cuda_stream
    bufs.status.zero_()
    build_transitions(table, p, bufs, stream)
    span_tree(table, bufs, stream)
    wq = write_q and bufs.q is not None
    if joint:
        sample_marginals(table, p, bufs, seed, conf_mode, stream, write_q=wq)
    else:
        sample(table, p, bufs, seed, stream)
        marginals(table, p, bufs, conf_mode, stream, write_q=wq)
    return bufs
