"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Discrete outputs (ids, tree, accepted nodes, bonus) are
bit-exact; floats within the stated tolerances."""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import BF16, C1_TINY, C3_8B_CHAIN, F32, scaled, tiny_shape

from gpu_cases import GpuCycle, compare_cycle, cycle_and_oracle, dev_i32, host_weights, oracle_cycle, say, topk_agrees

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4          # fp32 drafter vs fp64 oracle
TOL_BF16 = (2e-2, 1e-2)  # bf16 logits / fusion: atol, rtol


# ---------------------------------------------------------------- fusion
@pytest.mark.parametrize("n", [1, 10, 64, 130])
@pytest.mark.parametrize("pack", [False, True])
def test_fuse_bf16(lib, n, pack):
    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.cycle import Drafter
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=1024, dtype=BF16)
    Wt = gen.gen_weights(shape, seed=0)
    say("fuse bf16 n", n, "pack", pack)
    dr = Drafter(shape, Wt, pack=pack)
    feats = gen.draw(5, 1, (n, 3, 256), 1.0, BF16)
    g = torch.empty(n, 256, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(Bd.workspace_size(dr.dims, 1, n, 0), dtype=torch.uint8, device="cuda")
    Bd.eagle3_fuse(dr.dims, dr.weights, feats.torch("cuda"), n, g, ws)
    torch.cuda.synchronize()
    ref = O.fuse(shape, feats.f32(), Wt["fc"].f32())
    np.testing.assert_allclose(g.float().cpu().numpy(), ref, atol=TOL_BF16[0], rtol=TOL_BF16[1])


def test_fuse_fp32_tiny(lib):
    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.cycle import Drafter
    shape = C1_TINY.shape
    Wt = gen.gen_weights(shape, seed=0)
    dr = Drafter(shape, Wt)
    feats = gen.draw(1, 11, (64, 3, 256), 1 / 16, F32)
    g = torch.empty(64, 256, dtype=torch.float32, device="cuda")
    ws = torch.zeros(Bd.workspace_size(dr.dims, 1, 64, 0), dtype=torch.uint8, device="cuda")
    Bd.eagle3_fuse(dr.dims, dr.weights, feats.torch("cuda"), 64, g, ws)
    torch.cuda.synchronize()
    ref = O.fuse(shape, feats.f32(), Wt["fc"].f32())
    np.testing.assert_allclose(g.cpu().numpy(), ref, atol=TOL_F32, rtol=TOL_F32)


# ---------------------------------------------------------------- top-k
@pytest.mark.parametrize("V,k,rows", [(128256, 10, 10), (128256, 1, 3), (4096, 2, 5), (1000, 16, 4), (128256, 16, 2)])
def test_topk(lib, V, k, rows):
    from eagle_draft_tree_amd import binding as Bd
    say("topk", V, k, rows)
    g = np.random.default_rng(V + k)
    L = (g.standard_normal((rows, V)) * 2).astype(np.float32)
    L[:, 5] = L[:, 7] = L.max(axis=1) + 0.5        # exact tie at the top: lower id first
    L[0, V - 1] = L[0, 5]                          # three-way tie across partitions
    if rows > 1:
        L[1, :] = np.round(L[1, :], 1)             # many ties everywhere
    if rows > 2:
        L[2, :] = 0.25                             # all equal: ids 0..k-1
    if rows > 3:
        L[3, :] = np.minimum(L[3, :], 3.0)         # hundreds of equal values at the top of every partition
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    ids = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    lp = torch.empty(rows, k, dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    Bd.eagle3_topk(torch.as_tensor(L).cuda(), rows, V, k, ids, lp, lse, ws)
    torch.cuda.synchronize()
    for r in range(rows):
        o_ids, o_lp, o_lse = O.topk_logprobs(L[r], k)
        np.testing.assert_array_equal(ids[r].cpu().numpy(), o_ids)
        np.testing.assert_allclose(lp[r].cpu().numpy(), o_lp, atol=1e-4, rtol=0)
        assert abs(lse[r].item() - float(o_lse)) < 1e-4


# ---------------------------------------------------------------- tree expansion
@pytest.mark.parametrize("k,D,m,Bn,ties", [(10, 6, 60, 1, 0), (2, 3, 8, 3, 2), (4, 5, 30, 2, 2), (1, 3, 3, 4, 0),
                                           (16, 5, 63, 1, 3), (3, 4, 20, 2, 1)])
def test_tree_expand(lib, k, D, m, Bn, ties):
    from eagle_draft_tree_amd import binding as Bd
    say("tree", k, D, m, Bn, ties)
    V = 5000
    i32 = dict(dtype=torch.int32, device="cuda")
    state = torch.empty(Bd.tree_state_size(Bn, k, D), dtype=torch.uint8, device="cuda")
    root_tok = np.arange(Bn, dtype=np.int32) + 7
    root_pos = np.arange(Bn, dtype=np.int32) * 100 + 50
    trees = [O.DynamicTree(k, D, root_tok[b], root_pos[b]) for b in range(Bn)]
    ids0, lp0 = gen.random_topk_rows(k * 1000 + D, Bn, k, V, tie_every=ties)
    nt = torch.empty(Bn, k, **i32); npar = torch.empty(Bn, k, **i32)
    npos = torch.empty(Bn, k, **i32); nanc = torch.empty(Bn, k, dtype=torch.int64, device="cuda")
    Bd.eagle3_tree_expand(Bd.INIT, Bn, k, D, m, dev_i32(root_tok), dev_i32(root_pos), state,
                          dev_i32(ids0), torch.as_tensor(lp0).cuda(), nt, npar, npos, nanc)
    for b in range(Bn):
        trees[b].init(ids0[b], lp0[b])

    def check_rows():
        torch.cuda.synchronize()
        for b in range(Bn):
            rows = trees[b].next_rows()
            np.testing.assert_array_equal(nt[b].cpu().numpy(), [r[0] for r in rows])
            np.testing.assert_array_equal(npar[b].cpu().numpy(), [r[1] for r in rows])
            np.testing.assert_array_equal(npos[b].cpu().numpy(), [r[2] for r in rows])
            np.testing.assert_array_equal(nanc[b].cpu().numpy().view(np.uint64),
                                          np.array([r[3] for r in rows], dtype=np.uint64))
    if D > 1:
        check_rows()
    for j in range(2, D + 1):
        ids, lp = gen.random_topk_rows(k * 1000 + D * 10 + j, Bn * k, k, V, tie_every=ties)
        if ties:  # ties across rows as well: equal log-probs in different rows
            lp[1::2] = lp[0::2][: len(lp[1::2])]
        Bd.eagle3_tree_expand(Bd.STEP, Bn, k, D, m, None, None, state, dev_i32(ids),
                              torch.as_tensor(lp).cuda(), nt, npar, npos, nanc)
        for b in range(Bn):
            trees[b].step(ids[b * k:(b + 1) * k], lp[b * k:(b + 1) * k])
        if j < D:
            check_rows()
    vt = {n: torch.empty(Bn, m + 1, **i32) for n in ("tok", "parent", "depth", "pos")}
    vanc = torch.empty(Bn, m + 1, dtype=torch.int64, device="cuda")
    Bd.eagle3_tree_expand(Bd.FINAL, Bn, k, D, m, None, None, state, None, None, None, None, None, None,
                          vt["tok"], vt["parent"], vt["depth"], vt["pos"], vanc)
    torch.cuda.synchronize()
    for b in range(Bn):
        ref = trees[b].final(m)
        for n in ("tok", "parent", "depth", "pos"):
            np.testing.assert_array_equal(vt[n][b].cpu().numpy(), ref[n], err_msg=n)
        np.testing.assert_array_equal(vanc[b].cpu().numpy().view(np.uint64), ref["anc"])


# ---------------------------------------------------------------- verification
def _run_verify(Bn, m, V, tok, par, L, mode, T=1.0, ut=None, ur=None, Dmax=None):
    from eagle_draft_tree_amd import binding as Bd
    Dmax = Dmax or m + 1
    i32 = dict(dtype=torch.int32, device="cuda")
    al = torch.empty(Bn, **i32); acc = torch.empty(Bn, Dmax, **i32)
    bo = torch.empty(Bn, **i32); st = torch.empty(Bn, **i32)
    vws = torch.zeros(Bd.verify_workspace_size(Bn, m, V), dtype=torch.uint8, device="cuda")
    Bd.eagle3_verify(Bn, m, V, Dmax, dev_i32(tok), dev_i32(par), torch.as_tensor(L).cuda(), mode, T,
                     torch.as_tensor(ut).cuda() if ut is not None else None,
                     torch.as_tensor(ur).cuda() if ur is not None else None, al, acc, bo, st, vws)
    torch.cuda.synchronize()
    return al.cpu().numpy(), acc.cpu().numpy(), bo.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("V,m,depth,Bn,mode,T", [
    (128256, 60, 6, 2, "greedy", 1.0), (4096, 8, 3, 4, "greedy", 1.0), (4096, 8, 3, 4, "sample", 1.0),
    (128256, 60, 6, 2, "sample", 1.0), (50, 20, 4, 8, "sample", 0.7), (7, 5, 3, 16, "sample", 1.3),
    (128256, 3, 3, 64, "greedy", 1.0)])
def test_verify(lib, V, m, depth, Bn, mode, T):
    from eagle_draft_tree_amd import binding as Bd
    say("verify", V, m, depth, Bn, mode, T)
    toks, pars = [], []
    for b in range(Bn):
        t, p = gen.random_verify_tree(V * 7 + b, m, V, depth)
        toks.append(t); pars.append(p)
    toks, pars = np.array(toks), np.array(pars)
    L = gen.target_logits(V + m, Bn, m + 1, V, 3.0)
    gen.plant_agreement(L, toks, pars, np.full(Bn, 0.8), seed=V + m)
    ut, ur = gen.uniforms(V + m, Bn, m + 1)
    md = Bd.GREEDY if mode == "greedy" else Bd.SAMPLE
    al, acc, bo, st = _run_verify(Bn, m, V, toks, pars, L, md, T, ut, ur)
    for b in range(Bn):
        if mode == "greedy":
            ra, rb = O.verify_greedy(toks[b], pars[b], L[b])
        else:
            ra, rb = O.verify_sample(toks[b], pars[b], L[b], ut[b], ur[b], T)
        assert st[b] == 0
        assert al[b] == len(ra), (b, al[b], ra)
        assert list(acc[b][: al[b]]) == ra
        assert bo[b] == rb


def test_verify_reuses_its_workspace(lib):
    """One zero-filled verify workspace serves consecutive calls of different
    shapes (batch 8, then 3, then 8 again; greedy and sampling): the
    per-request arrival counters that hand the partials to the tree walk are
    left at zero by every call, so each call still matches the oracle."""
    from eagle_draft_tree_amd import binding as Bd
    V, m, depth = 5000, 12, 4
    i32 = dict(dtype=torch.int32, device="cuda")
    vws = torch.zeros(Bd.verify_workspace_size(8, m, V), dtype=torch.uint8, device="cuda")
    for call, (Bn, mode) in enumerate([(8, "greedy"), (3, "sample"), (8, "sample"), (8, "greedy")]):
        say("verify workspace reuse, call", call, Bn, mode)
        toks, pars = zip(*[gen.random_verify_tree(100 * call + b, m, V, depth) for b in range(Bn)])
        toks, pars = np.array(toks), np.array(pars)
        L = gen.target_logits(50 + call, Bn, m + 1, V, 3.0)
        gen.plant_agreement(L, toks, pars, np.full(Bn, 0.8), seed=50 + call)
        ut, ur = gen.uniforms(50 + call, Bn, m + 1)
        md = Bd.GREEDY if mode == "greedy" else Bd.SAMPLE
        al = torch.empty(Bn, **i32); acc = torch.empty(Bn, m + 1, **i32)
        bo = torch.empty(Bn, **i32); st = torch.empty(Bn, **i32)
        Bd.eagle3_verify(Bn, m, V, m + 1, dev_i32(toks), dev_i32(pars), torch.as_tensor(L).cuda(), md, 1.0,
                         torch.as_tensor(ut).cuda(), torch.as_tensor(ur).cuda(), al, acc, bo, st, vws)
        torch.cuda.synchronize()
        al, acc, bo, st = al.cpu().numpy(), acc.cpu().numpy(), bo.cpu().numpy(), st.cpu().numpy()
        for b in range(Bn):
            if mode == "greedy":
                ra, rb = O.verify_greedy(toks[b], pars[b], L[b])
            else:
                ra, rb = O.verify_sample(toks[b], pars[b], L[b], ut[b], ur[b], 1.0)
            assert st[b] == 0
            assert al[b] == len(ra) and list(acc[b][: al[b]]) == ra and bo[b] == rb, (call, b)


def test_verify_golden(lib):
    import json, os
    from eagle_draft_tree_amd import binding as Bd
    with open(os.path.join(os.path.dirname(__file__), "golden", "verify_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        L = np.array(c["logits"], np.float32)[None]
        tok = np.array(c["tok"])[None]; par = np.array(c["parent"])[None]
        m = len(c["tok"]) - 1
        if c["mode"] == "greedy":
            al, acc, bo, st = _run_verify(1, m, L.shape[2], tok, par, L, Bd.GREEDY)
        else:
            al, acc, bo, st = _run_verify(1, m, L.shape[2], tok, par, L, Bd.SAMPLE, c.get("T", 1.0),
                                          np.array(c["u_try"])[None], np.array(c["u_res"])[None])
        assert list(acc[0][: al[0]]) == c["expect_accepted"], c["name"]
        assert bo[0] == c["expect_bonus"], c["name"]


def test_verify_sampling_exact_breakpoints_large_vocab(lib):
    """Sampling decisions placed exactly on a breakpoint of the residual CDF,
    and one ulp below it, at a vocabulary that spans 33 partitions of the
    kernel.  All logits are 0, so every weight is exactly 1 and every sum on
    either side is an exact integer: the thresholds u * Rm land exactly on
    cumulative weights, including at partition boundaries and after
    rejected tokens, and the GPU must take the oracle's decision in each."""
    from eagle_draft_tree_amd import binding as Bd
    V = 131074
    tok = np.array([0, 100, 5000]); par = np.array([-1, 0, 0])   # both rejected: Rm = 2^17
    js = [1, 100, 4094, 4095, 4096 * 5 - 2, 4096 * 5 - 1, 4096 * 32 - 3, 131071]
    ur_vals = []
    for j in js:
        u = j / 131072.0
        ur_vals += [u, np.nextafter(u, 0.0)]
    Bn = len(ur_vals)
    L = np.zeros((Bn, 3, V), np.float32)
    ut = np.full((Bn, 3), 0.5)
    ur = np.zeros((Bn, 3)); ur[:, 0] = ur_vals
    toks, pars = np.stack([tok] * Bn), np.stack([par] * Bn)
    say("verify exact breakpoints, V", V, "requests", Bn)
    al, acc, bo, st = _run_verify(Bn, 2, V, toks, pars, L, Bd.SAMPLE, 1.0, ut, ur)
    for b in range(Bn):
        ra, rb = O.verify_sample(tok, par, L[b], ut[b], ur[b], 1.0)
        assert st[b] == 0 and al[b] == len(ra) == 0 and bo[b] == rb, (b, ur[b, 0], bo[b], rb)
    # the acceptance boundary: Rm = 2^17, u_try = 2^-17 rejects, one ulp below accepts
    V2 = 131072
    L2 = np.zeros((2, 2, V2), np.float32)
    tok2, par2 = np.array([0, 5]), np.array([-1, 0])
    ut2 = np.array([[0.0, 2.0 ** -17], [0.0, np.nextafter(2.0 ** -17, 0.0)]])
    ur2 = np.array([[0.25, 0.75], [0.25, 0.75]])
    al, acc, bo, st = _run_verify(2, 1, V2, np.stack([tok2] * 2), np.stack([par2] * 2), L2, Bd.SAMPLE, 1.0, ut2, ur2)
    for b in range(2):
        ra, rb = O.verify_sample(tok2, par2, L2[b], ut2[b], ur2[b], 1.0)
        assert al[b] == len(ra) and list(acc[b][: al[b]]) == ra and bo[b] == rb, (b, al[b], bo[b], ra, rb)
    assert al[0] == 0 and al[1] == 1


def test_verify_nan_and_neg_inf(lib):
    from eagle_draft_tree_amd import binding as Bd
    V = 300
    tok, par = gen.random_verify_tree(1, 6, V, 3)
    L = gen.target_logits(9, 2, 7, V, 2.0)
    L[0, 0, 17] = np.nan                 # request 0: NaN in the root row
    L[1, 0, :] = -np.inf                 # request 1: only token 3 possible at the root
    L[1, 0, 3] = 0.0
    toks = np.stack([tok, tok]); pars = np.stack([par, par])
    ut, ur = gen.uniforms(9, 2, 7)
    al, acc, bo, st = _run_verify(2, 6, V, toks, pars, L, Bd.SAMPLE, 1.0, ut, ur)
    assert st[0] == Bd.ENUMERIC and st[1] == 0
    ra, rb = O.verify_sample(tok, par, L[1], ut[1], ur[1])
    assert al[1] == len(ra) and bo[1] == rb


# ---------------------------------------------------------------- whole cycles
def test_c1_tiny_cycle_greedy_and_sample(lib):
    w = C1_TINY
    say("C1 cycle")
    Wt, W, ci = cycle_and_oracle(w)
    gc = GpuCycle(w, Wt, ci)
    L = gen.target_logits(1, 1, w.keep + 1, w.shape.vocab, w.target_sigma)
    ut, ur = gen.uniforms(1, 1, w.keep + 1)
    gc.run(L, 0)
    assert compare_cycle(gc, w, W, ci, (TOL_F32, TOL_F32)) == 0
    vt, _ = oracle_cycle(w, W, ci)
    ra, rb = O.verify_greedy(vt["tok"], vt["parent"], L[0])
    assert gc.buf.accept_len[0].item() == len(ra) and gc.buf.bonus[0].item() == rb
    # sampling verify on the same tree
    gc.run(L, 1, 1.0, ut, ur)
    ra, rb = O.verify_sample(vt["tok"], vt["parent"], L[0], ut[0], ur[0])
    assert gc.buf.accept_len[0].item() == len(ra) and gc.buf.bonus[0].item() == rb
    # planted agreement from the oracle's own tree exercises acceptance
    Lp = gen.plant_agreement(L.copy(), vt["tok"][None], vt["parent"][None], np.array([0.9]), seed=5)
    gc.run(Lp, 0)
    ra, rb = O.verify_greedy(vt["tok"], vt["parent"], Lp[0])
    assert len(ra) >= 1
    assert gc.buf.accept_len[0].item() == len(ra) and gc.buf.bonus[0].item() == rb
    acc = gc.buf.accepted[0].cpu().numpy()
    assert list(acc[: len(ra)]) == ra


def test_c1_cycle_is_deterministic(lib):
    w = C1_TINY
    Wt, W, ci = cycle_and_oracle(w, seed=2)
    gc = GpuCycle(w, Wt, ci)
    gc.run()
    a = [t.clone() for t in (gc.buf.h_tree, gc.buf.round_logits[0], gc.buf.v_tok)]
    gc.run()
    for x, y in zip(a, (gc.buf.h_tree, gc.buf.round_logits[0], gc.buf.v_tok)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("hkv,commit,ctx", [(2, 24, 0), (1, 5, 40), (4, 1, 100)])
@pytest.mark.parametrize("pack", [False, True])
def test_bf16_small_cycle(lib, hkv, commit, ctx, pack):
    """bf16 drafter (d=256) with synthetic prefix KV, multi-row commit and GQA,
    row-major and packed weight layouts."""
    say("bf16 small cycle", hkv, commit, ctx, pack)
    shape = tiny_shape(d=256, hq=4, hkv=hkv, hd=64, ffn=512, vocab=2048, dtype=BF16, theta=500000.0)
    w = scaled(C1_TINY, shape=shape, depth=4, topk=3, keep=12, prefix=ctx, commit_rows=commit,
               synthetic_prefix_kv=ctx > 0, feat_scale=1.0)
    Wt, W, ci = cycle_and_oracle(w, seed=3)
    gc = GpuCycle(w, Wt, ci, pack=pack)
    gc.run()
    exc = compare_cycle(gc, w, W, ci, TOL_BF16)
    assert exc <= 1


@pytest.mark.parametrize("commit,ctx", [(24, 70), (1, 300), (1, 1100)])
def test_bf16_small_cycle_hd128(lib, commit, ctx):
    """Head dim 128 (the 8B/70B drafters' head size) at a size the oracle runs
    whole: 4 query heads on one KV head, a 24-row commit (6 groups of 16 query
    vectors) or a long prefix with one root row; packed weights.  The
    1100-row prefix gives the attention 32 or more splits, where a
    workgroup merges its four waves' splits before the store."""
    say("bf16 small cycle hd128", commit, ctx)
    shape = tiny_shape(d=512, hq=4, hkv=1, hd=128, ffn=512, vocab=2048, dtype=BF16, theta=500000.0)
    w = scaled(C1_TINY, shape=shape, depth=4, topk=3, keep=12, prefix=ctx, commit_rows=commit,
               synthetic_prefix_kv=True, feat_scale=1.0)
    Wt, W, ci = cycle_and_oracle(w, seed=9)
    gc = GpuCycle(w, Wt, ci, pack=True)
    gc.run()
    exc = compare_cycle(gc, w, W, ci, TOL_BF16)
    assert exc <= 1


@pytest.mark.parametrize("bs", [4, 16])
def test_bf16_small_paged_cycle(lib, bs):
    """Paged KV (block tables, per-request prefix lengths) on a small bf16
    drafter, batch 6, tree 3 x 2."""
    say("bf16 small paged cycle, block size", bs)
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=2048, dtype=BF16, theta=500000.0)
    w = scaled(C3_8B_CHAIN, shape=shape, batch=6, depth=3, topk=2, keep=6, prefix=90, prefix_range=(10, 90),
               block_size=bs, feat_scale=1.0)
    Wt, W, ci = cycle_and_oracle(w, seed=5)
    gc = GpuCycle(w, Wt, ci, pack=True)
    gc.run()
    assert compare_cycle(gc, w, W, ci, TOL_BF16) <= 1


def test_bf16_paged_cycle_table_load_per_key(lib):
    """Paged KV with one token per block and prefixes of 18000-20000 tokens:
    a wave's run of keys spans more than 64 blocks, so the attention reads the
    block table once per key instead of from lanes.  Every stage against the
    oracle."""
    say("bf16 paged cycle, block size 1, 20k-token prefixes")
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=2048, dtype=BF16, theta=500000.0)
    w = scaled(C3_8B_CHAIN, shape=shape, batch=2, depth=3, topk=2, keep=4, prefix=20000,
               prefix_range=(18000, 20000), block_size=1, feat_scale=1.0)
    Wt, W, ci = cycle_and_oracle(w, seed=17)
    gc = GpuCycle(w, Wt, ci, pack=True)
    gc.run()
    assert compare_cycle(gc, w, W, ci, TOL_BF16) <= 1


def test_bf16_paged_cycle_more_than_64_rows(lib):
    """Tree rounds of 12 requests x 6 frontier rows = 72 query rows per draft
    step: the layer GEMMs run in 64-row chunks and the LM head keeps its
    logits for the partition top-k.  Every stage against the oracle (up to
    two requests excused by a near-tie in the oracle's own logits)."""
    say("bf16 paged cycle, 72 rows per tree round")
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=2048, dtype=BF16, theta=500000.0)
    w = scaled(C3_8B_CHAIN, shape=shape, batch=12, depth=3, topk=6, keep=12, prefix=90, prefix_range=(10, 90),
               block_size=16, feat_scale=1.0)
    Wt, W, ci = cycle_and_oracle(w, seed=13)
    gc = GpuCycle(w, Wt, ci, pack=True)
    gc.run()
    assert compare_cycle(gc, w, W, ci, TOL_BF16) <= 2


@pytest.mark.parametrize("batch,k,zero_lm,d", [(1, 6, False, 256), (1, 6, True, 256), (9, 2, False, 256),
                                               (9, 2, True, 256), (16, 4, False, 256), (21, 3, False, 256),
                                               (9, 2, False, 288)])
def test_tile_topk_matches_kept_logits(lib, batch, k, zero_lm, d):
    """Up to 64 rows per step: the LM head writes each 16-column tile's
    {max, sum exp} per row beside the logits, and the top-k reads those pairs
    and only the tiles that can hold one of the k best.  Its ids must be the
    k best of the kept logits (value desc, id asc) and its log-probabilities
    logit minus the logsumexp of the row.  Batch 1 (6 rows, 2 tiles per LM-head
    workgroup) and batch 9 x 2 (18 rows: the register-weight GEMM, 32 tiles
    per workgroup, the last one partly past the vocabulary); tree rounds of
    16 x 4 = 64 rows (the most one launch takes) and 21 x 3 = 63 rows.  Model
    width 288 (not a multiple of 64) takes the skinny GEMM at 18 rows.  With a zero LM head every logit is 0 and all 2049 tiles
    reach the threshold, more than the candidate-tile list holds: the k-round
    argmax path must give ids 0..k-1 and lp = -log V."""
    say("tile top-k, batch", batch, "k", k, "d", d, "zero LM head" if zero_lm else "random LM head")
    shape = tiny_shape(d=d, hq=4, hkv=2, hd=64, ffn=512, vocab=32784, dtype=BF16, theta=500000.0)
    w = scaled(C1_TINY, shape=shape, batch=batch, depth=3, topk=k, keep=2 * k, prefix=40, commit_rows=3,
               synthetic_prefix_kv=True, feat_scale=1.0)
    Wt = gen.gen_weights(shape, seed=11)
    if zero_lm:
        Wt["lm"] = gen.Tensor(np.zeros_like(Wt["lm"].raw), Wt["lm"].dtype)
    ci = gen.gen_cycle_inputs(w, seed=12)
    gc = GpuCycle(w, Wt, ci, keep_logits=True, pack=True)
    gc.run()
    b = gc.buf
    steps = [(b.root_ids, b.root_lp, b.commit_logits)]
    steps += [(b.round_ids[r], b.round_lp[r], b.round_logits[r]) for r in range(len(b.round_ids))]
    for ids, lp, lg in steps:
        lg = lg.cpu().numpy().astype(np.float64)
        lg = lg.reshape(-1, lg.shape[-1])
        ids = ids.cpu().numpy().reshape(lg.shape[0], -1)
        lp = lp.cpu().numpy().reshape(lg.shape[0], -1)
        k = ids.shape[1]
        for r in range(lg.shape[0]):
            row = lg[r]
            best = np.lexsort((np.arange(row.size), -row))[:k]
            np.testing.assert_array_equal(ids[r], best)
            m = row.max()
            lse = m + np.log(np.exp(row - m).sum())
            np.testing.assert_allclose(lp[r], row[best] - lse, atol=2e-5, rtol=0)
            if zero_lm:
                np.testing.assert_array_equal(ids[r], np.arange(k))


@pytest.mark.parametrize("d", [256, 288])
def test_top1_lm_head_without_logits_matches_logits_path(lib, d):
    """Top-1 drafting (k = 1) with more than 16 rows per step and no kept
    logits: the LM head reduces its columns to per-workgroup (max, sum exp,
    argmax) partials instead of writing logits.  The top-1 ids equal the
    kept-logits path bit for bit (same GEMM arithmetic) and are the argmax of
    those logits (lowest id on ties); log-probabilities agree to fp32
    rounding; the tree is identical.  Model width 256 takes the
    register-weight GEMM; 288 (not a multiple of 64) the skinny GEMM."""
    shape = tiny_shape(d=d, hq=4, hkv=2, hd=64, ffn=512, vocab=4112, dtype=BF16, theta=500000.0)
    w = scaled(C3_8B_CHAIN, shape=shape, batch=20, depth=3, topk=1, keep=2, prefix=90, prefix_range=(10, 90),
               block_size=16, feat_scale=1.0)
    say("top-1 LM head without logits, batch", w.batch)
    Wt = gen.gen_weights(shape, seed=7)
    ci = gen.gen_cycle_inputs(w, seed=8)
    a = GpuCycle(w, Wt, ci, keep_logits=True, pack=True)
    a.run()
    b = GpuCycle(w, Wt, ci, keep_logits=False, pack=True)
    b.run()
    pairs = [(a.buf.root_ids, b.buf.root_ids, a.buf.root_lp, b.buf.root_lp, a.buf.commit_logits)]
    pairs += [(a.buf.round_ids[r], b.buf.round_ids[r], a.buf.round_lp[r], b.buf.round_lp[r], a.buf.round_logits[r])
              for r in range(len(a.buf.round_ids))]
    for ia, ib, la, lb, lg in pairs:
        ia, ib = ia.cpu().numpy(), ib.cpu().numpy()
        np.testing.assert_array_equal(ia, ib)
        np.testing.assert_allclose(lb.cpu().numpy(), la.cpu().numpy(), atol=1e-5, rtol=1e-6)
        np.testing.assert_array_equal(ia[..., 0], np.argmax(lg.cpu().numpy(), axis=-1))
    ta, tb = a.tree(), b.tree()
    for n in ta:
        np.testing.assert_array_equal(ta[n], tb[n], err_msg=n)
