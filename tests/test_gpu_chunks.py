"""Batches beyond one launch's grid (B * Lpad > 32767) run in row chunks,
each with its own workspace slot, the draws keyed by the batch row: every
row must match the oracle as if the batch had run in one launch."""
import numpy as np
import pytest

import oracle
from synth import configs
from tests import parity as PT

pytestmark = pytest.mark.gpu

B, L = 70, 1000   # Lpad 1024: 31 rows per chunk, three chunks (31, 31, 8)
ROWS = (0, 30, 31, 61, 62, 69)


def _workload():
    return configs.make(2, B=B, L=L)


def test_chunked_step_matches_oracle():
    w = _workload()
    PT.log(f"[chunks] {w.describe()}")
    g = PT.run_gpu(w)
    orc = oracle.Oracle(w.aut)
    for b in ROWS:
        PT.check_row(w, g, b, orc, q_positions=np.arange(0, L, 97))
    for b in range(B):
        lz = orc.forward_backward(orc.edge_weights(w.p[b]))["logZ"]
        assert abs(g["logZ"][b] - lz) <= PT.LOGZ_RTOL * max(1.0, abs(lz)), b
    PT.log("[chunks] step ok")


def test_chunked_chain_map_and_noalloc():
    import torch
    import constrained_decoding_diffusion_amd as fa
    from tests.test_gpu_chain import check_chain_row
    from tests.test_gpu_map import check_map_row
    w = _workload()
    tb = fa.Table.from_automaton(w.aut, first_level="dense")
    p = torch.from_numpy(w.p).cuda()
    orc = oracle.Oracle(w.aut)
    cb = fa.chain_step(tb, p, w.seed)
    torch.cuda.synchronize()
    gc = dict(logZ=cb.logZ.cpu().numpy(), status=cb.status.cpu().numpy(),
              states=cb.states.cpu().numpy(), tokens=cb.tokens.cpu().numpy()[:, :L])
    for b in ROWS:
        check_chain_row(w, gc, b, orc)
    del cb
    mb = fa.map_decode(tb, p)
    torch.cuda.synchronize()
    gm = dict(logmax=mb.logmax.cpu().numpy(), status=mb.status.cpu().numpy(),
              states=mb.states.cpu().numpy(), tokens=mb.tokens.cpu().numpy()[:, :L])
    for b in ROWS:
        check_map_row(w, gm, b, orc)
    del mb
    # the allocation-free span tree over the chunks gives the workspace form's log Z
    bufs = fa.StepBuffers(tb, B, L, want_q=False)
    stream = torch.cuda.current_stream().cuda_stream
    bufs.status.zero_()
    fa.build_transitions(tb, p, bufs, stream)
    leaves = bufs.tree.clone()
    fa.span_tree(tb, bufs, stream)
    ref = bufs.logZ.clone()
    bufs.tree.copy_(leaves)
    bufs.logZ.fill_(7.0)
    fa.span_tree_noalloc(tb, bufs, stream)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bufs.logZ.cpu().numpy(), ref.cpu().numpy())
    PT.log("[chunks] chain, MAP, no-alloc ok")
