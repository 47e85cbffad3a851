"""ctypes front end of the serial fp64 oracle (oracle.c).

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, INFEASIBLE, UNDERFLOW, BADARG = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Aut(C.Structure):
    _fields_ = [("S", C.c_int32), ("V", C.c_int32), ("start", C.c_int32),
                ("n_accept", C.c_int32), ("accept", C.c_void_p), ("E", C.c_int64),
                ("src", C.c_void_p), ("dst", C.c_void_p), ("label_off", C.c_void_p),
                ("label_tok", C.c_void_p), ("ranges", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        P = C.c_void_p
        _lib.or_philox4x32_10.argtypes = [P, P, P]
        _lib.or_uniform.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, C.c_uint32]
        _lib.or_uniform.restype = C.c_double
        _lib.or_edge_weights.argtypes = [P, P, C.c_int32, P]
        _lib.or_dense_M.argtypes = [P, P, C.c_int32, P]
        _lib.or_forward_backward.argtypes = [P, P, C.c_int32, P, P, P, P, P]
        _lib.or_marginals.argtypes = [P, P, C.c_int32, P, P, P, P, P, C.c_int32, P, P, P,
                                      C.c_int32, P]
        _lib.or_sample_tree.argtypes = [P, P, P, C.c_int32, C.c_uint64, C.c_uint32, P, P]
        _lib.or_replay_verify.argtypes = [P, P, P, C.c_int32, C.c_uint64, C.c_uint32, P, P, P]
        _lib.or_ffbs.argtypes = [P, P, P, C.c_int32, P, P, P, P]
        _lib.or_judge_draw.argtypes = [P, C.c_int32, C.c_double, C.c_int32, P]
        _lib.or_ffbs_verify.argtypes = [P, P, P, C.c_int32, P, C.c_uint64, C.c_uint32, P, P, P]
        _lib.or_map_weights.argtypes = [P, P, C.c_int32, P]
        _lib.or_viterbi.argtypes = [P, P, C.c_int32, P]
        _lib.or_map_tree.argtypes = [P, P, P, C.c_int32, P, P, P]
        _lib.or_map_verify.argtypes = [P, P, P, C.c_int32, P, P, P]
        _lib.or_edge_count.argtypes = [P, C.c_int32, C.c_int32, C.c_int32]
        _lib.or_edge_count.restype = C.c_int32
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, b: int, level: int, node: int) -> float:
    return lib().or_uniform(seed, b, level, node)


def judge_draw(w, u: float, chosen: int):
    """One draw judged as the replay verifier judges it: returns (the
    oracle's choice, verdict 0 same / 1 NEAR / 2 HARD, fp32-margin flag)."""
    w = np.ascontiguousarray(w, np.float64)
    out = np.zeros(3, np.int32)
    lib().or_judge_draw(_ptr(w), w.size, float(u), int(chosen), _ptr(out))
    return int(out[0]), int(out[1]), int(out[2])


class Oracle:
    """Oracle bound to one automaton (original state ids, raw edge list)."""

    def __init__(self, aut):
        self.aut = aut
        self._keep = [np.ascontiguousarray(aut.accept, np.int32),
                      np.ascontiguousarray(aut.src, np.int32),
                      np.ascontiguousarray(aut.dst, np.int32),
                      np.ascontiguousarray(aut.label_off, np.int64),
                      np.ascontiguousarray(aut.label_tok, np.int32)]
        acc, src, dst, off, tok = self._keep
        self._s = _Aut(aut.S, aut.V, aut.start, acc.size, acc.ctypes.data, aut.E,
                       src.ctypes.data, dst.ctypes.data, off.ctypes.data, tok.ctypes.data,
                       1 if aut.ranges else 0)
        self._sp = C.cast(C.pointer(self._s), C.c_void_p)

    # p: fp32 [L, V] for one batch row
    def edge_weights(self, p: np.ndarray) -> np.ndarray:
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        W = np.zeros((L, self.aut.E), np.float64)
        lib().or_edge_weights(self._sp, _ptr(p), L, _ptr(W))
        return W

    def dense_M(self, W: np.ndarray, i: int) -> np.ndarray:
        M = np.zeros((self.aut.S, self.aut.S), np.float64)
        lib().or_dense_M(self._sp, _ptr(np.ascontiguousarray(W)), i, _ptr(M))
        return M

    def forward_backward(self, W: np.ndarray):
        L = W.shape[0]
        S = self.aut.S
        alpha = np.zeros((L + 1, S)); beta = np.zeros((L + 1, S))
        alog = np.zeros(L + 1); blog = np.zeros(L + 1)
        logZ = np.zeros(1)
        st = lib().or_forward_backward(self._sp, _ptr(np.ascontiguousarray(W)), L, _ptr(alpha),
                                       _ptr(alog), _ptr(beta), _ptr(blog), _ptr(logZ))
        return dict(alpha=alpha, alog=alog, beta=beta, blog=blog, logZ=float(logZ[0]),
                    status=int(st))

    def marginals(self, p, fb, positions=None, tokens=None, conf_mode=0):
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        pos = np.ascontiguousarray(np.arange(L) if positions is None else positions, np.int32)
        q = np.zeros((pos.size, self.aut.V))
        lognorm = np.zeros(pos.size)
        conf = np.zeros(pos.size)
        tok = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
        st = lib().or_marginals(self._sp, _ptr(p), L, _ptr(fb["alpha"]), _ptr(fb["alog"]),
                                _ptr(fb["beta"]), _ptr(fb["blog"]), _ptr(pos), pos.size, _ptr(q),
                                _ptr(lognorm), None if tok is None else _ptr(tok), conf_mode,
                                _ptr(conf))
        if st != OK:
            raise RuntimeError(f"or_marginals status {st}")
        return q, lognorm, conf

    def sample_tree(self, p, W, seed: int, b: int):
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        states = np.full(L + 1, -1, np.int32)
        tokens = np.full(L, -1, np.int32)
        st = lib().or_sample_tree(self._sp, _ptr(p), _ptr(np.ascontiguousarray(W)), L, seed, b,
                                  _ptr(states), _ptr(tokens))
        return states, tokens, int(st)

    def replay(self, p, W, seed: int, b: int, states, tokens):
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        rep = np.zeros(5, np.int64)
        st = lib().or_replay_verify(self._sp, _ptr(p), _ptr(np.ascontiguousarray(W)), L, seed, b,
                                    _ptr(np.ascontiguousarray(states, np.int32)),
                                    _ptr(np.ascontiguousarray(tokens, np.int32)), _ptr(rep))
        return dict(status=int(st), draws=int(rep[0]), hard=int(rep[1]), near=int(rep[2]),
                    margin=int(rep[3]), first_hard=int(rep[4]))

    def ffbs(self, p, W, fb, u):
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        states = np.full(L + 1, -1, np.int32)
        tokens = np.full(L, -1, np.int32)
        st = lib().or_ffbs(self._sp, _ptr(p), _ptr(np.ascontiguousarray(W)), L, _ptr(fb["alpha"]),
                           _ptr(np.ascontiguousarray(u, np.float64)), _ptr(states), _ptr(tokens))
        return states, tokens, int(st)

    # ---- the serial chain sampler (forward filtering, backward sampling)
    @staticmethod
    def chain_uniforms(seed: int, b: int, L: int):
        """The uniforms of the chain sampler's draws in the order or_ffbs
        takes them: z_L, z_{L-1} .. z_0 at level K+2 (node = state index),
        then the tokens at level K+1 (node = position)."""
        K = (1 << max(0, (L - 1).bit_length())).bit_length() - 1
        u = [uniform(seed, b, K + 2, L)] + [uniform(seed, b, K + 2, i) for i in range(L - 1, -1, -1)]
        return np.array(u + [uniform(seed, b, K + 1, i) for i in range(L)], np.float64)

    def chain_sample(self, p, W, fb, seed: int, b: int):
        """FFBS with the chain sampler's keyed uniforms: (states, tokens, status)."""
        return self.ffbs(p, W, fb, self.chain_uniforms(seed, b, np.asarray(p).shape[0]))

    def chain_verify(self, p, W, fb, seed: int, b: int, states, tokens):
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        rep = np.zeros(5, np.int64)
        st = lib().or_ffbs_verify(self._sp, _ptr(p), _ptr(np.ascontiguousarray(W)), L,
                                  _ptr(fb["alpha"]), seed, b,
                                  _ptr(np.ascontiguousarray(states, np.int32)),
                                  _ptr(np.ascontiguousarray(tokens, np.int32)), _ptr(rep))
        return dict(status=int(st), draws=int(rep[0]), hard=int(rep[1]), near=int(rep[2]),
                    margin=int(rep[3]), first_hard=int(rep[4]))

    # ---- MAP (greedy) decoding
    def map_weights(self, p: np.ndarray) -> np.ndarray:
        """Wm[i, e] = max of p[i, v] over the label of edge e (0 if empty)."""
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        Wm = np.zeros((L, self.aut.E), np.float64)
        lib().or_map_weights(self._sp, _ptr(p), L, _ptr(Wm))
        return Wm

    def viterbi(self, Wm) -> tuple:
        """Serial Viterbi: (log-max, status)."""
        out = np.zeros(1)
        st = lib().or_viterbi(self._sp, _ptr(np.ascontiguousarray(Wm)), Wm.shape[0], _ptr(out))
        return float(out[0]), int(st)

    def map_tree(self, p, Wm):
        """Tree-order MAP decoding: (states [L+1], tokens [L], log-max, status)."""
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        states = np.full(L + 1, -1, np.int32)
        tokens = np.full(L, -1, np.int32)
        lm = np.zeros(1)
        st = lib().or_map_tree(self._sp, _ptr(p), _ptr(np.ascontiguousarray(Wm)), L,
                               _ptr(states), _ptr(tokens), _ptr(lm))
        return states, tokens, float(lm[0]), int(st)

    def map_verify(self, p, Wm, states, tokens):
        p = np.ascontiguousarray(p, np.float32)
        L = p.shape[0]
        rep = np.zeros(5, np.int64)
        st = lib().or_map_verify(self._sp, _ptr(p), _ptr(np.ascontiguousarray(Wm)), L,
                                 _ptr(np.ascontiguousarray(states, np.int32)),
                                 _ptr(np.ascontiguousarray(tokens, np.int32)), _ptr(rep))
        return dict(status=int(st), decisions=int(rep[0]), hard=int(rep[1]), near=int(rep[2]),
                    first_hard=int(rep[4]))

    def edge_count(self, a: int, v: int, b: int) -> int:
        return int(lib().or_edge_count(self._sp, a, v, b))


def step(aut, p: np.ndarray, seed: int, rows=None, q_positions=None, conf_mode=0):
    """Oracle for one constrained step over the rows of p [B, L, V]: log Z,
    tree-order samples, and marginals at q_positions (all positions if None;
    an empty list skips them).  Returns a list of per-row dicts."""
    orc = Oracle(aut)
    B = p.shape[0]
    out = []
    for b in (range(B) if rows is None else rows):
        W = orc.edge_weights(p[b])
        fb = orc.forward_backward(W)
        d = dict(b=b, W=W, fb=fb, logZ=fb["logZ"], status=fb["status"])
        if fb["status"] == OK:
            st, tk, s2 = orc.sample_tree(p[b], W, seed, b)
            d.update(states=st, tokens=tk, sample_status=s2)
            if q_positions is None or len(q_positions):
                q, ln, conf = orc.marginals(p[b], fb, q_positions, tk, conf_mode)
                d.update(q=q, lognorm=ln, conf=conf)
        out.append(d)
    return out


def commit_topk(conf, tokens, committed, status, steps_left: int):
    """The remasking step written out (papernotes 关键设计 3: the confidence
    of each position's sampled token decides which positions are committed).
    Per row b with status[b] == 0: the masked positions are those with
    committed == 0 and a sampled token (>= 0); with n of them, the first
    k = ceil(n / steps_left) (all n when steps_left == 1) in the order of
    decreasing confidence, ties by increasing position, NaN counted as -inf,
    are committed.  Returns (new committed, fresh) as int32 arrays [B, L]."""
    conf = np.asarray(conf, np.float64)
    tokens = np.asarray(tokens)
    committed = np.array(committed, dtype=np.int32, copy=True)
    fresh = np.zeros_like(committed)
    B, L = committed.shape
    for b in range(B):
        if status is not None and status[b] != 0:
            continue
        masked = [i for i in range(L) if committed[b, i] == 0 and tokens[b, i] >= 0]
        n = len(masked)
        k = n if steps_left <= 1 else -(-n // steps_left)
        key = lambda i: (-(conf[b, i] if conf[b, i] == conf[b, i] else -np.inf), i)
        for i in sorted(masked, key=key)[:k]:
            committed[b, i] = 1
            fresh[b, i] = 1
    return committed, fresh
