"""GPU tests of the remasking step (fa_commit) and of a synthetic multi-step
generation: every step is checked against the fp64 oracle on the GPU's
current p, every commit against the selection's plain definition, and the
generated string must be accepted by the automaton."""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import configs
from tests import parity as PT
from tests.test_gpu_parity import CASES

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V", [1000, 999])
@pytest.mark.parametrize("steps_left", [3, 1])
@pytest.mark.parametrize("L", [300, 8192])
def test_commit_matches_definition(V, steps_left, L):
    """300: more positions than threads per workgroup, a ragged power of
    two for the sort; 8192: the longest row the selection takes."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    rng = np.random.default_rng(100 + V + steps_left + L)
    B = 3
    conf = np.round(rng.random((B, L)), 1).astype(np.float32)  # many ties
    conf[0, :5] = -np.inf
    conf[1, 7] = np.nan
    tokens = rng.integers(0, V, (B, L)).astype(np.int32)
    tokens[2, ::7] = -1
    committed = (rng.random((B, L)) < 0.3).astype(np.int32)
    status = np.array([0, 0, 0], np.int32)
    p = rng.random((B, L, V)).astype(np.float32)
    PT.log(f"[commit] V={V} steps_left={steps_left} L={L}")
    for flagged in (False, True):
        st = status.copy()
        if flagged:
            st[1] = 2
        dev = dict(conf=torch.from_numpy(conf).cuda(), tokens=torch.from_numpy(tokens).cuda(),
                   committed=torch.from_numpy(committed).cuda(), status=torch.from_numpy(st).cuda(),
                   p=torch.from_numpy(p).cuda())
        fresh = torch.full((B, L), 7, dtype=torch.int32, device="cuda")
        bufs = type("B", (), dict(conf=dev["conf"], tokens=dev["tokens"], status=dev["status"]))
        fa.commit(dev["p"], bufs, dev["committed"], fresh, steps_left,
                  torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want_c, want_f = oracle.commit_topk(conf, tokens, committed, st, steps_left)
        np.testing.assert_array_equal(dev["committed"].cpu().numpy(), want_c)
        np.testing.assert_array_equal(fresh.cpu().numpy(), want_f)
        pg = dev["p"].cpu().numpy()
        for b, i in zip(*np.nonzero(want_f)):
            row = np.zeros(V, np.float32)
            row[tokens[b, i]] = 1.0
            np.testing.assert_array_equal(pg[b, i], row)
        keep = want_f == 0
        np.testing.assert_array_equal(pg[keep], p[keep])


def _loop(w, T, conf_mode):
    """The generation written out step by step, each step checked."""
    import torch
    import constrained_decoding_diffusion_amd as fa
    tb = fa.Table.from_automaton(w.aut)
    p = torch.from_numpy(w.p.copy()).cuda()
    bufs = fa.StepBuffers(tb, w.B, w.L, want_q=True, device="cuda")
    committed = torch.zeros((w.B, w.L), dtype=torch.int32, device="cuda")
    fresh = torch.zeros_like(committed)
    stream = torch.cuda.current_stream().cuda_stream
    orc = oracle.Oracle(w.aut)
    for t in range(T):
        p_now = p.cpu().numpy()
        before = committed.cpu().numpy()
        fa.step(tb, p, w.seed + t, bufs, conf_mode=conf_mode)
        torch.cuda.synchronize()
        g = dict(table=tb, bufs=bufs, logZ=bufs.logZ.cpu().numpy(),
                 status=bufs.status.cpu().numpy(), states=bufs.states.cpu().numpy(),
                 tokens=bufs.tokens.cpu().numpy()[:, :w.L], conf=bufs.conf.cpu().numpy()[:, :w.L],
                 q=bufs.q.cpu().numpy())
        wt = dataclasses.replace(w, p=p_now, seed=w.seed + t)
        for b in range(w.B):
            PT.check_row(wt, g, b, orc, conf_mode=conf_mode)
        # committed positions keep their tokens
        assert (g["tokens"][before == 1] == np.argmax(p_now, -1)[before == 1]).all()
        fa.commit(p, bufs, committed, fresh, T - t, stream)
        torch.cuda.synchronize()
        want_c, want_f = oracle.commit_topk(g["conf"], g["tokens"], before, g["status"], T - t)
        np.testing.assert_array_equal(committed.cpu().numpy(), want_c)
        np.testing.assert_array_equal(fresh.cpu().numpy(), want_f)
    return tb, p, g["tokens"], committed.cpu().numpy()


@pytest.mark.parametrize("name,T,conf_mode", [("json-small", 6, 0), ("random-dfa", 8, 0),
                                               ("real-number", 3, 1), ("random-dfa", 8, 2),
                                               ("json-small", 4, 2)])
def test_generation_loop(name, T, conf_mode):
    import torch
    import constrained_decoding_diffusion_amd as fa
    w = CASES[name]()
    PT.log(f"[generate] {name} T={T} conf_mode={conf_mode}: {w.describe()}")
    tb, p, tokens, committed = _loop(w, T, conf_mode)
    assert (committed == 1).all()
    pg = p.cpu().numpy()
    assert (pg.max(-1) == 1.0).all() and (pg.sum(-1) == 1.0).all()
    np.testing.assert_array_equal(np.argmax(pg, -1), tokens)
    # the generated strings are accepted: the last step's replay above
    # checked them; check them once more through the automaton's edges
    aut = w.aut
    orc = oracle.Oracle(aut)
    for b in range(w.B):
        st = {aut.start: 1}
        for i in range(w.L):
            nxt = {}
            for a, c in st.items():
                for d in range(aut.S):
                    m = orc.edge_count(a, int(tokens[b, i]), d)
                    if m:
                        nxt[d] = nxt.get(d, 0) + c * m
            st = nxt
        assert any(s in st for s in aut.accept.tolist()), f"row {b} not accepted"
    # the driver gives the same generation
    p2 = torch.from_numpy(w.p.copy()).cuda()
    bufs2, committed2 = fa.generate(tb, p2, T, w.seed, conf_mode=conf_mode)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(committed2.cpu().numpy(), committed)
    np.testing.assert_array_equal(p2.cpu().numpy(), pg)
