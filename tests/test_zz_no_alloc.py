"""fa_span_tree_noalloc (its split-K partial tiles in the library's own
device array) against fa_span_tree (the caller's workspace), through the C
ABI: the same kernels, so the tree nodes, exponents, log Z and row status
must be bit-identical.  Two calls in a row, the second with a smaller input,
so the second call reads only what it wrote itself."""
import numpy as np
import pytest

from synth import automata as A
from synth import configs
from tests import parity as PT

pytestmark = pytest.mark.gpu


def _splits_k(Sp, B, Lpad):
    """Whether some tree level is split along K (the upper levels' few
    products): the case where the scratch array is used at all."""
    lvl, any_split = 1, False
    while (Lpad >> lvl) >= 1:
        nn = Lpad >> lvl
        big = B * nn * (Sp // 128) ** 2
        if not (Sp % 128 == 0 and big >= 256):
            small = B * nn * (Sp // 64) ** 2
            any_split |= (Sp // 64) % 2 == 0 and small * 2 <= 256 and Sp // 2 >= 256
        lvl += 1
    return any_split


def _compare(tb, w):
    import torch
    import constrained_decoding_diffusion_amd as fa
    dev = torch.device("cuda")
    if tb.buf is None:
        tb.upload(dev)
    p = torch.from_numpy(w.p).to(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ref = fa.StepBuffers(tb, w.B, w.L, want_q=False, device=dev)
    ref.status.zero_()
    fa.build_transitions(tb, p, ref, stream)
    # the leaves and the status after the emission reduce, for the second run
    leaves, meta0, st0 = ref.tree.clone(), ref.meta.clone(), ref.status.clone()
    fa.span_tree(tb, ref, stream)
    out = fa.StepBuffers(tb, w.B, w.L, want_q=False, device=dev)
    out.tree.copy_(leaves)
    out.meta.copy_(meta0)
    out.status.copy_(st0)
    out.logZ.fill_(7.0)
    fa.span_tree_noalloc(tb, out, stream)
    torch.cuda.synchronize()
    Lpad = 1 << max(0, (w.L - 1).bit_length())
    Sp = tb.info["Sp"]
    n = w.B * 2 * Lpad * Sp * Sp
    np.testing.assert_array_equal(out.tree[:n].cpu().numpy(), ref.tree[:n].cpu().numpy())
    m = w.B * 2 * Lpad * 3 * Sp
    np.testing.assert_array_equal(out.meta[:m].cpu().numpy(), ref.meta[:m].cpu().numpy())
    np.testing.assert_array_equal(out.logZ.cpu().numpy(), ref.logZ.cpu().numpy())
    np.testing.assert_array_equal(out.status.cpu().numpy(), ref.status.cpu().numpy())
    return ref.logZ.cpu().numpy()


def test_noalloc_span_tree_matches_workspace_form():
    import constrained_decoding_diffusion_amd as fa
    # Sp = 512 and one row: the top levels' few tiles split along K
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=480, V=20000, pool=256, string_size=13000),
                        7001, 37)
    tb = fa.Table.from_automaton(aut, first_level="dense")
    assert tb.info["first_sparse"] == 0 and tb.info["Sp"] == 512
    w1 = configs.from_automaton(aut, 1, 37, "normal4_zipf", 0, 7100, "json-like small")
    w2 = configs.from_automaton(aut, 1, 19, "normal4_zipf", 0, 7150, "json-like smaller")
    for w in (w1, w2):
        Lpad = 1 << (w.L - 1).bit_length()
        assert _splits_k(tb.info["Sp"], w.B, Lpad)
        PT.log(f"[noalloc] {w.describe()}")
        logZ = _compare(tb, w)
        assert np.isfinite(logZ).all()
    # and once more on the first, larger input after the smaller one
    _compare(tb, w1)


def test_noalloc_span_tree_other_tables():
    """A random DFA with one infeasible row (status and -inf log Z come out
    the same) and the real-number DFA at L = 1 (no product level at all)."""
    import constrained_decoding_diffusion_amd as fa
    w = configs.make(2, B=3, L=40)
    aut = w.aut
    first = set()
    for e in range(aut.E):
        if aut.src[e] == aut.start:
            first |= set(aut.edge_label(e).tolist())
    bad = next(v for v in range(aut.V) if v not in first)
    w.p[1, 0] = 0.0
    w.p[1, 0, bad] = 1.0
    tb = fa.Table.from_automaton(aut, first_level="dense")
    PT.log("[noalloc] random DFA with an infeasible row")
    logZ = _compare(tb, w)
    assert logZ[1] == -np.inf and np.isfinite(logZ[[0, 2]]).all()
    w1 = configs.make(1, L=1)
    PT.log("[noalloc] real-number DFA, L = 1")
    _compare(fa.Table.from_automaton(w1.aut, first_level="dense"), w1)
