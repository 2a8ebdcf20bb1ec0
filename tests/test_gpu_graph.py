"""The draft-tree cycle captured once in a HIP graph and replayed: every
replay reproduces the eager cycle's tree and verification outcome, with
other eager cycles (different target logits) run between the replays."""
import numpy as np
import pytest
import torch

from workloads import gen
from workloads.configs import BF16, C1_TINY, scaled, tiny_shape

from gpu_cases import GpuCycle, cycle_and_oracle, say

pytestmark = pytest.mark.gpu


def _outcome(gc):
    b = gc.buf
    t = gc.tree()
    return dict(t, accept=b.accept_len.cpu().numpy(), accepted=b.accepted.cpu().numpy(), bonus=b.bonus.cpu().numpy())


def _same(x, y):
    for k in x:
        np.testing.assert_array_equal(x[k], y[k], err_msg=k)


@pytest.mark.parametrize("mode", [0, 1])
def test_cycle_graph_replay_matches_eager(lib, mode):
    from eagle_draft_tree_amd.cycle import run_cycle
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=2048, dtype=BF16, theta=500000.0)
    w = scaled(C1_TINY, shape=shape, batch=2, depth=4, topk=3, keep=12, prefix=40, commit_rows=3,
               synthetic_prefix_kv=True, feat_scale=1.0)
    Wt, _, ci = cycle_and_oracle(w, seed=4)
    gc = GpuCycle(w, Wt, ci, keep_logits=False, pack=True)
    say("graph replay, mode", mode)
    L1 = torch.as_tensor(gen.target_logits(1, w.batch, w.keep + 1, shape.vocab, 2.0)).cuda()
    L2 = torch.as_tensor(gen.target_logits(2, w.batch, w.keep + 1, shape.vocab, 2.0)).cuda()
    ut, ur = [torch.as_tensor(u).cuda() for u in gen.uniforms(1, w.batch, w.keep + 1)]

    def cycle(L):
        run_cycle(gc.dr, gc.buf, gc.kv, gc.feats, gc.tokens, gc.pos, gc.ctx_after, gc.root_tok, gc.root_pos, L,
                  mode, 1.0, ut if mode == 1 else None, ur if mode == 1 else None)

    cycle(L1)
    torch.cuda.synchronize()
    ref1 = _outcome(gc)
    cycle(L2)
    torch.cuda.synchronize()
    ref2 = _outcome(gc)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cycle(L1)
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        _same(_outcome(gc), ref1)
        cycle(L2)  # eager work between replays
        torch.cuda.synchronize()
        _same(_outcome(gc), ref2)
