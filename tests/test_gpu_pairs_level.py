"""GPU parity of the dense first span level whose operands are staged from
the pair values (FA_FIRST_LEVEL_PAIRS; such tables keep no dense leaves):
the whole step against the fp64 oracle with the level-1 nodes checked
against the oracle's two-leaf products, and the span tree against the same
table with dense leaves (FA_FIRST_LEVEL_DENSE), node for node and bit for
bit, since both stage the same folded operands into the same products.

Workloads: json-like tables at Sp = 256 (one tile per product) and Sp = 512
(four tiles per product, rows filtered per tile), an odd L (identity leaves
past the sequence end meet real ones in the first level), and a random DFA
whose K steps hold more entries than the threads keep in registers."""
import numpy as np
import pytest

import oracle
from tests import parity as PT
from synth import automata as A
from synth import configs

pytestmark = pytest.mark.gpu


def _json_256():
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=240, V=20000, pool=256, string_size=13000),
                        9501, 64)
    return configs.from_automaton(aut, 2, 64, "normal4_zipf", 8, 9600, "json-like Sp 256")


def _json_256_odd():
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=200, V=20000, pool=256, string_size=13000),
                        9701, 37)
    return configs.from_automaton(aut, 3, 37, "normal4_zipf", 0, 9800, "json-like Sp 256, L 37")


def _json_512():
    aut = configs._draw(lambda r: A.json_like_dfa(r, S=480, V=20000, pool=256, string_size=13000),
                        9901, 29)
    return configs.from_automaton(aut, 1, 29, "normal4_zipf", 0, 10000, "json-like Sp 512, L 29")


def _dense_columns():
    # about 17.6k pairs: a K step of 16 columns holds about 1100 entries,
    # more than the 1024 the threads hold in registers
    aut = configs._draw(lambda r: A.random_dfa(r, 256, 2048, 4, 80 / 2048), 9901, 16)
    return configs.from_automaton(aut, 2, 16, "gumbel3", 2, 10100, "random DFA 80 tokens per state")


CASES = {"json-256": _json_256, "json-256-odd": _json_256_odd, "json-512": _json_512,
         "dense-columns": _dense_columns}


def _table(fa, w, first_level):
    tb = fa.Table.from_automaton(w.aut, first_level=first_level)
    if first_level == "pairs":
        assert tb.info["first_pairs"] == 1 and tb.info["leafless"] == 1
    return tb


@pytest.mark.parametrize("name", list(CASES))
def test_pairs_first_level_parity(name):
    import constrained_decoding_diffusion_amd as fa
    w = CASES[name]()
    tb = _table(fa, w, "pairs")
    PT.log(f"[pairs-level] {name}: {w.describe()}, Sp {tb.info['Sp']}, pairs {tb.info['pairs']}")
    g = PT.run_gpu(w, table=tb)
    orc = oracle.Oracle(w.aut)
    near = draws = 0
    for b in range(w.B):
        rep = PT.check_row(w, g, b, orc)
        near += rep["near"] if rep else 0
        draws += rep["draws"] if rep else 0
    PT.check_span_nodes(w, g, 0, orc, level=1)
    if w.B > 1:
        PT.check_span_nodes(w, g, w.B - 1, orc, level=1)
    PT.log(f"[pairs-level] {name}: ok, near {near} of {draws}")
    assert near <= 0.01 * max(draws, 1)


def _tree(fa, torch, w, tb):
    p = torch.from_numpy(w.p).cuda()
    tb.upload(p.device)
    bufs = fa.StepBuffers(tb, w.B, w.L, want_q=False, device=p.device)
    stream = torch.cuda.current_stream().cuda_stream
    fa.build_transitions(tb, p, bufs, stream)
    fa.span_tree(tb, bufs, stream)
    torch.cuda.synchronize()
    Lpad = 1 << max(0, (w.L - 1).bit_length())
    Sp = tb.info["Sp"]
    tree = bufs.tree[: w.B * 2 * Lpad * Sp * Sp].view(w.B, 2 * Lpad, Sp, Sp)
    meta = bufs.meta[: w.B * 2 * Lpad * 3 * Sp].view(w.B, 2 * Lpad, 3, Sp)
    # internal nodes 1 .. Lpad-1 (the leaves differ: not written with pairs)
    return (tree[:, 1:Lpad].cpu().numpy(), meta[:, 1:Lpad].cpu().numpy(), bufs.logZ.cpu().numpy(),
            bufs.status.cpu().numpy())


@pytest.mark.parametrize("name", list(CASES))
def test_pairs_first_level_equals_dense_leaves(name):
    import torch
    import constrained_decoding_diffusion_amd as fa
    w = CASES[name]()
    tp = _tree(fa, torch, w, _table(fa, w, "pairs"))
    td = _tree(fa, torch, w, _table(fa, w, "dense"))
    for a, b, what in zip(tp, td, ("internal nodes", "exponents", "log Z", "status")):
        np.testing.assert_array_equal(a, b, err_msg=what)
    PT.log(f"[pairs-level] {name}: span tree equal to the dense-leaf one, bit for bit")
