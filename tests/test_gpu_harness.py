"""GPU parity of the EAGLE-4 Harness path: eagle3_tree_confidence against
the oracle's DynamicTree (frontier and rerank-order scores, float32
bit for bit), and whole harness cycles (HarnessCycle: the library's host
rules on scores read back from the device) against the oracle's rules
applied to the same tree, decision by decision, with the verify tree bit
for bit; the fp32 drafter also against the oracle's independent
harness_cycle."""
import numpy as np
import pytest
import torch

from eagle_draft_tree_amd import binding as Bd
from eagle_draft_tree_amd.cycle import HarnessCycle, HarnessParams, KVCache
from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import BF16, C1_TINY, scaled, tiny_shape

from gpu_cases import GpuCycle, dev_i32, host_weights, say

pytestmark = pytest.mark.gpu


def _table():
    # a drafter round costs 0.2 ms + 0.05 ms per row per request; a verify
    # step 0.5 ms + 0.02 ms per row (batch and context independent)
    tok = [1, 2, 4, 8, 16, 32, 64]
    draft = [[[0.2 + 0.05 * n for n in tok]]]
    verify = [[[0.5 + 0.02 * n for n in tok]]]
    return Bd.HarnessTable([64], [1 << 20], tok, draft, verify)


def test_tree_confidence_matches_oracle_tree(lib):
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=2048, dtype=BF16, theta=500000.0)
    w = scaled(C1_TINY, shape=shape, batch=2, depth=4, topk=3, keep=12, prefix=30, commit_rows=2,
               synthetic_prefix_kv=True, feat_scale=1.0)
    Wt = gen.gen_weights(shape, seed=0)
    ci = gen.gen_cycle_inputs(w, seed=3)
    gc = GpuCycle(w, Wt, ci)
    gc.run()
    k, D, m = w.topk, w.depth, w.keep
    m_max = 30
    front = torch.empty(2 * k, dtype=torch.float32, device="cuda")
    pool = torch.empty(2 * m_max, dtype=torch.float32, device="cuda")
    Bd.eagle3_tree_confidence(2, k, D, m_max, gc.buf.tree_state, front, pool)
    torch.cuda.synchronize()
    front, pool = front.view(2, k).cpu().numpy(), pool.view(2, m_max).cpu().numpy()
    buf = gc.buf
    for b in range(2):
        tree = O.DynamicTree(k, D, int(ci.tokens[b, -1]), int(ci.ctx_len[b]) + w.commit_rows - 1)
        tree.init(buf.root_ids[b, 0].cpu().numpy(), buf.root_lp[b, 0].cpu().numpy())
        for r in range(D - 1):
            tree.step(buf.round_ids[r][b].cpu().numpy(), buf.round_lp[r][b].cpu().numpy())
        np.testing.assert_array_equal(front[b], np.array([tree.score[i] for i in tree.frontier], np.float32))
        sc = np.array(tree.sorted_scores(), np.float32)
        np.testing.assert_array_equal(pool[b, : len(sc)], sc[:m_max])


def _harness_setup(shape, batch, D_max, m_max, seed=3, prefix=30):
    w = scaled(C1_TINY, shape=shape, batch=batch, depth=D_max, topk=8, keep=m_max, prefix=prefix, commit_rows=2,
               synthetic_prefix_kv=True, feat_scale=1.0)
    Wt = gen.gen_weights(shape, seed=0, std=0.05)
    ci = gen.gen_cycle_inputs(w, seed=seed)
    return w, Wt, ci


def _device_inputs(w, ci, dr):
    s = w.shape
    tdt = dr.torch_dtype
    Bn, n = w.batch, w.commit_rows
    tk = torch.zeros(Bn, Bd.MAX_TREE_SLOTS, s.n_kv_heads, s.head_dim, dtype=tdt, device="cuda")
    kv = KVCache(ci.kv_k.torch("cuda"), ci.kv_v.torch("cuda"), tk, torch.zeros_like(tk), dev_i32(ci.ctx_len),
                 cap=ci.cap)
    pos = dev_i32(ci.ctx_len[:, None] + np.arange(n)[None, :])
    return dict(kv=kv, feats=ci.feats.torch("cuda"), tokens=dev_i32(ci.tokens), commit_pos=pos,
                ctx_after=dev_i32(ci.ctx_len + n), root_tok=dev_i32(ci.tokens[:, -1]),
                root_pos=dev_i32(ci.ctx_len + n - 1))


@pytest.mark.parametrize("params", [HarnessParams(0.0, 0.0, 0.0, 0.0), HarnessParams(1e9, 0.0, 1e9, 1e9),
                                    HarnessParams(0.3, 0.5, 2.0, 0.2), HarnessParams(1.0, 1.0, 8.0, 3.0),
                                    HarnessParams(0.05, 2.0, 0.5, 1.0)])
@pytest.mark.parametrize("batch", [1, 3])
def test_harness_cycle_decisions_match_oracle(lib, params, batch):
    from eagle_draft_tree_amd.cycle import Drafter
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=512, dtype=BF16, theta=500000.0)
    D_max, m_max = 4, 24
    w, Wt, ci = _harness_setup(shape, batch, D_max, m_max)
    dr = Drafter(shape, Wt)
    table = _table()
    hc = HarnessCycle(dr, batch, w.commit_rows, D_max, m_max, ci.cap, table, params)
    x = _device_inputs(w, ci, dr)
    ctx = int(ci.ctx_len.max()) + w.commit_rows
    dec = hc.run(x["kv"], x["feats"], x["tokens"], x["commit_pos"], x["ctx_after"], x["root_tok"], x["root_pos"], ctx)
    torch.cuda.synchronize()
    say("  decisions", dec, "params", params)
    td = table.as_dict()
    buf = hc.buf
    lp8 = buf.root_lp.view(batch, 8).cpu().numpy()
    ids8 = buf.root_ids.view(batch, 8).cpu().numpy()
    k = O.harness_branch_cap(td, batch, ctx, lp8, params.tau_branch)
    assert dec["k"] == k
    trees = []
    for b in range(batch):
        t = O.DynamicTree(k, D_max, int(ci.tokens[b, -1]), int(ci.ctx_len[b]) + w.commit_rows - 1)
        t.init(ids8[b, :k], lp8[b, :k])
        trees.append(t)
    rounds = 1
    for j in range(2, D_max + 1):
        front = np.array([[t.score[i] for i in t.frontier] for t in trees], np.float32)
        go, _ = O.harness_continue(td, batch, ctx, k, j - 1, front, params.tau_depth, params.alpha)
        if not go:
            break
        r = j - 2
        ids = buf.round_ids[r].view(-1)[: batch * k * k].view(batch, k, k).cpu().numpy()
        lps = buf.round_lp[r].view(-1)[: batch * k * k].view(batch, k, k).cpu().numpy()
        for b, t in enumerate(trees):
            t.step(ids[b], lps[b])
        rounds += 1
    assert dec["rounds"] == rounds
    pool_n = k + (rounds - 1) * k * k
    m_cap = min(m_max, pool_n)
    sc = np.array([t.sorted_scores()[:m_cap] for t in trees], np.float32)
    m = max(O.harness_verify_count(td, batch, ctx, sc, params.tau_verify), 1)
    assert dec["m"] == m
    gt = hc.tree(m)
    for b, t in enumerate(trees):
        vt = t.final(m)
        for name in ("tok", "parent", "depth", "pos"):
            np.testing.assert_array_equal(gt[name][b].cpu().numpy(), vt[name], err_msg=f"request {b}: {name}")
        np.testing.assert_array_equal(gt["anc"][b].cpu().numpy().view(np.uint64), vt["anc"])


def test_harness_cycle_fp32_equals_independent_oracle(lib):
    """fp32 tiny drafter: the GPU harness cycle equals the oracle's own
    harness_cycle run from the same inputs (decisions and tree)."""
    from eagle_draft_tree_amd.cycle import Drafter
    shape = tiny_shape(d=256, hq=4, hkv=4, hd=64, ffn=512, vocab=512, dtype="f32", theta=10000.0)
    table = _table()
    td = table.as_dict()
    seen = set()
    for params in (HarnessParams(0.3, 0.5, 2.0, 0.2), HarnessParams(0.02, 0.1, 0.3, 0.01),
                   HarnessParams(1.0, 1.0, 8.0, 3.0)):
        w, Wt, ci = _harness_setup(shape, 1, 4, 24, seed=5)
        dr = Drafter(shape, Wt)
        hc = HarnessCycle(dr, 1, w.commit_rows, 4, 24, ci.cap, table, params)
        x = _device_inputs(w, ci, dr)
        ctx = int(ci.ctx_len[0]) + w.commit_rows
        dec = hc.run(x["kv"], x["feats"], x["tokens"], x["commit_pos"], x["ctx_after"], x["root_tok"],
                     x["root_pos"], ctx)
        torch.cuda.synchronize()
        W = host_weights(Wt)
        vt, info = O.harness_cycle(shape, W, ci.feats.f32()[:2], ci.tokens[0], ci.kv_k.f32()[0].astype(np.float64),
                                   ci.kv_v.f32()[0].astype(np.float64), int(ci.ctx_len[0]), td, 24, 4,
                                   params.tau_depth, params.alpha, params.tau_verify, params.tau_branch, B=1)
        say("  gpu", dec, "oracle", info)
        assert dec == info
        gt = hc.tree(info["m"])
        for name in ("tok", "parent", "depth", "pos"):
            np.testing.assert_array_equal(gt[name][0].cpu().numpy(), vt[name])
        seen.add((info["k"], info["rounds"]))
    assert len(seen) >= 2, "thresholds should exercise more than one outcome"
