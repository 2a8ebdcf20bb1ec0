"""Shared set-up for the GPU parity tests: seeded inputs -> device tensors,
one GPU cycle through the C ABI, and the oracle's answer on the same inputs.
Nothing here feeds a GPU result into the oracle."""
from __future__ import annotations

import numpy as np
import torch

from eagle_draft_tree_amd import binding as Bd
from eagle_draft_tree_amd.cycle import CycleBuffers, CycleSpec, Drafter, KVCache, run_cycle
from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import BF16, F32


def host_weights(Wt):
    return {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}


def dev_i32(a):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def say(*a):
    print(*a, flush=True)


class GpuCycle:
    """Inputs of one cycle on the device plus the GPU run."""

    def __init__(self, w, Wt, ci, keep_logits=True, pack=False):
        s = w.shape
        self.w, self.s, self.ci = w, s, ci
        self.dr = Drafter(s, Wt, pack=pack)
        Bn, n = w.batch, w.commit_rows
        cap_rows = ci.cap
        self.spec = CycleSpec(Bn, n, w.topk, w.depth, w.keep, cap_rows)
        self.buf = CycleBuffers(self.dr, self.spec)
        if keep_logits:
            self.buf.keep_logits(s.vocab)
        tdt = self.dr.torch_dtype
        self.kv_k = ci.kv_k.torch("cuda")
        self.kv_v = ci.kv_v.torch("cuda")
        self.tk = torch.zeros(Bn, Bd.MAX_TREE_SLOTS, s.n_kv_heads, s.head_dim, dtype=tdt, device="cuda")
        self.tv = torch.zeros_like(self.tk)
        self.ctx = dev_i32(ci.ctx_len)
        self.ctx_after = dev_i32(ci.ctx_len + n)
        bt = dev_i32(ci.block_table) if ci.block_table is not None else None
        self.kv = KVCache(self.kv_k, self.kv_v, self.tk, self.tv, self.ctx,
                          cap=ci.cap if bt is None else 0, block_table=bt, block_size=w.block_size)
        self.feats = ci.feats.torch("cuda")
        self.tokens = dev_i32(ci.tokens)
        pos = ci.ctx_len[:, None] + np.arange(n)[None, :]
        self.pos = dev_i32(pos)
        self.root_tok = dev_i32(ci.tokens[:, -1])
        self.root_pos = dev_i32(ci.ctx_len + n - 1)

    def run(self, target_logits=None, mode=Bd.GREEDY, temperature=1.0, u_try=None, u_res=None):
        L = torch.as_tensor(target_logits).cuda() if target_logits is not None else None
        ut = torch.as_tensor(u_try).cuda() if u_try is not None else None
        ur = torch.as_tensor(u_res).cuda() if u_res is not None else None
        run_cycle(self.dr, self.buf, self.kv, self.feats, self.tokens, self.pos, self.ctx_after,
                  self.root_tok, self.root_pos, L, mode, temperature, ut, ur)
        torch.cuda.synchronize()

    def tree(self):
        b = self.buf
        return dict(tok=b.v_tok.cpu().numpy(), parent=b.v_parent.cpu().numpy(), depth=b.v_depth.cpu().numpy(),
                    pos=b.v_pos.cpu().numpy(), anc=b.v_anc.cpu().numpy().view(np.uint64))


def oracle_cycle(w, W, ci, b=0):
    """The oracle's cycle for request b (contiguous or gathered paged KV)."""
    s = w.shape
    n = w.commit_rows
    if ci.block_table is not None:
        L = int(ci.ctx_len[b])
        Kc = O.gather_paged(ci.kv_k.f32(), ci.block_table[b], L + n, w.block_size).astype(np.float64)
        Vc = O.gather_paged(ci.kv_v.f32(), ci.block_table[b], L + n, w.block_size).astype(np.float64)
    else:
        Kc = ci.kv_k.f32()[b].astype(np.float64)
        Vc = ci.kv_v.f32()[b].astype(np.float64)
    rec = {}
    feats = ci.feats.f32()[b * n:(b + 1) * n]
    vt = O.draft_cycle(s, W, feats, ci.tokens[b], Kc, Vc, int(ci.ctx_len[b]), w.topk, w.depth, w.keep,
                       record=rec)
    return vt, rec


def topk_agrees(gpu_ids, oracle_logits, k, tol):
    """GPU top-k ids vs the oracle's float32 logits: exact unless the oracle
    itself has a near-tie (gap <= tol) at a decision boundary, in which case
    every GPU id must still be a valid top-k member within tol.
    Returns (exact, excused)."""
    o_ids, _, _ = O.topk_logprobs(oracle_logits, k)
    if np.array_equal(np.asarray(gpu_ids), o_ids):
        return True, False
    l32 = np.asarray(oracle_logits, dtype=np.float64).astype(np.float32)
    srt = np.sort(l32)[::-1]
    kth = srt[k - 1]
    # valid: every chosen id within tol of the k-th value, and order consistent within tol
    ok = all(l32[i] >= kth - tol for i in gpu_ids)
    vals = l32[np.asarray(gpu_ids)]
    ok = ok and all(vals[j] >= vals[j + 1] - tol for j in range(len(vals) - 1))
    gaps = srt[:k] - srt[1:k + 1]
    near = np.min(gaps) <= tol
    return False, bool(ok and near)


def cycle_and_oracle(w, seed=1):
    Wt = gen.gen_weights(w.shape, seed=0)
    W = host_weights(Wt)
    ci = gen.gen_cycle_inputs(w, seed=seed)
    return Wt, W, ci


def compare_cycle(gc, w, W, ci, tol, reqs=None):
    """Compare every stage of the requests `reqs` (default: all); returns the
    number of requests excused by a near-tie in the oracle's logits."""
    excused = 0
    buf = gc.buf
    for b in (range(w.batch) if reqs is None else reqs):
        say("  oracle request", b)
        vt, rec = oracle_cycle(w, W, ci, b)
        atol, rtol = tol
        g_gpu = buf.g.float().cpu().numpy()[b * w.commit_rows:(b + 1) * w.commit_rows]
        np.testing.assert_allclose(g_gpu, rec["g"], atol=atol, rtol=rtol)
        cl = buf.commit_logits[b, 0].cpu().numpy()
        np.testing.assert_allclose(cl, rec["commit_logits"][-1], atol=atol, rtol=rtol)
        np.testing.assert_allclose(buf.h_tree[b, 0].cpu().numpy(), rec["commit_h2"][-1], atol=atol, rtol=rtol)
        exact, exc = topk_agrees(buf.root_ids[b, 0].cpu().numpy(), rec["commit_logits"][-1], w.topk, 2 * atol)
        if not exact:
            assert exc, "root top-k differs without a near-tie"
            excused += 1
            continue
        diverged = False
        for r, rd in enumerate(rec["rounds"]):
            gl = buf.round_logits[r][b].cpu().numpy()
            np.testing.assert_allclose(gl, rd["logits"], atol=atol, rtol=rtol)
            for row in range(w.topk):
                exact, exc = topk_agrees(buf.round_ids[r][b, row].cpu().numpy(), rd["logits"][row], w.topk,
                                         2 * atol)
                if not exact:
                    assert exc, f"round {r} row {row} top-k differs without a near-tie"
                    diverged = True
            if diverged:
                break
        if diverged:
            excused += 1
            continue
        t = gc.tree()
        for n in ("tok", "parent", "depth", "pos"):
            np.testing.assert_array_equal(t[n][b], vt[n], err_msg=n)
        np.testing.assert_array_equal(t["anc"][b], vt["anc"])
    return excused


# ---------------------------------------------------------------- full-size, stage by stage
def _request_kv(w, ci, b):
    n = w.commit_rows
    if ci.block_table is not None:
        L = int(ci.ctx_len[b])
        Kc = O.gather_paged(ci.kv_k.f32(), ci.block_table[b], L + n, w.block_size).astype(np.float64)
        Vc = O.gather_paged(ci.kv_v.f32(), ci.block_table[b], L + n, w.block_size).astype(np.float64)
    else:
        Kc = ci.kv_k.f32()[b].astype(np.float64)
        Vc = ci.kv_v.f32()[b].astype(np.float64)
    return Kc, Vc


def gpu_frontier(gc, b, r):
    """Rows the GPU drafted in tree round r (0-based) for request b, as the
    oracle's DynamicTree.next_rows() tuples (token, parent slot, position, ancestors)."""
    buf = gc.buf
    tok = buf.next_tok[r][b].cpu().numpy()
    par = buf.next_par[r][b].cpu().numpy()
    pos = buf.next_pos[r][b].cpu().numpy()
    anc = buf.next_anc[r][b].cpu().numpy().view(np.uint64)
    return [(int(tok[i]), int(par[i]), int(pos[i]), int(anc[i])) for i in range(len(tok))]


def oracle_on_gpu_rows(w, W, ci, b, gc, isolate=True):
    """The oracle's decoder on exactly the rows the GPU drafted for request b:
    the COMMIT rows, then round by round the GPU's frontier rows (token,
    parent state slot, position, ancestor slots).  Near-ties in the top-k
    cannot make the two sides decode different rows.

    isolate=True makes every stage start from the GPU's own inputs to that
    stage: the COMMIT rows take the GPU's g and each tree row its parent's
    GPU state (h_tree, fp32), while keys/values come from the oracle's own
    earlier rows.  In bf16 a single rounding flip upstream moves later fp32
    values by ~1e-4 relative and flips a few percent of the following bf16
    roundings, so an unisolated chain drifts by ~1e-3..1e-2 over the rounds
    at these sizes; isolation compares each stage on the same inputs."""
    s = w.shape
    n, k, D = w.commit_rows, w.topk, w.depth
    Kc, Vc = _request_kv(w, ci, b)
    cap = Kc.shape[0]
    N = cap + O.MAX_TREE_SLOTS
    K = np.zeros((N, s.n_kv_heads, s.head_dim))
    V = np.zeros((N, s.n_kv_heads, s.head_dim))
    K[:cap], V[:cap] = Kc, Vc
    g = O.fuse(s, ci.feats.f32()[b * n:(b + 1) * n], W["fc"], W.get("norm_fc"))
    g_in = gc.buf.g.float().cpu().numpy()[b * n:(b + 1) * n].astype(np.float64) if isolate else g
    L0 = int(ci.ctx_len[b])
    vis = np.zeros((n, N), bool)
    for r in range(n):
        vis[r, :L0 + r + 1] = True
    P = np.arange(L0, L0 + n)
    h2, logits = O.decoder_rows(s, W, g_in, ci.tokens[b], P, K, V, P, vis)
    h_tree = {0: h2[-1]}
    gpu_h = gc.buf.h_tree[b].cpu().numpy().astype(np.float64) if isolate else None
    out = dict(g=g, commit_logits=logits[-1], rounds=[])
    Lc = L0 + n
    for r in range(D - 1):
        rows = gpu_frontier(gc, b, r)
        base = r * k
        S = np.stack([gpu_h[p] if isolate else h_tree[p] for (_, p, _, _) in rows])
        T = np.array([t for (t, _, _, _) in rows])
        Pr = np.array([p for (_, _, p, _) in rows])
        vis = np.zeros((len(rows), N), bool)
        vis[:, :Lc] = True
        for i, (_, _, _, anc) in enumerate(rows):
            for sl in range(O.MAX_TREE_SLOTS):
                if (anc >> sl) & 1:
                    vis[i, cap + sl] = True
        h2, logits = O.decoder_rows(s, W, S, T, Pr, K, V, cap + base + np.arange(len(rows)), vis)
        for i in range(len(rows)):
            h_tree[1 + base + i] = h2[i]
        out["rounds"].append(logits)
    return out


def _same_rule(ids, lp, gpu_logits_row, k):
    """GPU top-k == the oracle's top-k rule on the GPU's own float32 logits."""
    o_ids, o_lp, _ = O.topk_logprobs(gpu_logits_row, k)
    np.testing.assert_array_equal(ids, o_ids)
    np.testing.assert_allclose(lp, o_lp, atol=1e-4, rtol=0)


def check_cycle_stagewise(gc, w, W, ci, reqs, tol, L=None, mode=None, u_try=None, u_res=None, keep=None):
    """Full-size parity of one GPU cycle, stage by stage, on the requests
    `reqs`: fusion, COMMIT and every tree round's logits against the oracle
    on the same rows and the same stage inputs (tolerance); each GPU top-k (ids exact, log-probs to
    1e-4) is the oracle's top-k rule applied to the GPU's own float32 logits,
    so both sides take the decision in the same precision on the same values;
    the tree built by the oracle's DynamicTree from the GPU's top-k equals
    the GPU tree bit for bit, frontier by frontier; the verification outcome
    equals the oracle's on that tree.  Returns the number of rows whose GPU
    top-k differs from the top-k of the oracle's own logits (each such row
    must be a near-tie there).  keep: an optional dict that receives the
    oracle's per-request results (request -> dict of logits)."""
    atol, rtol = tol
    buf = gc.buf
    k, D, m = w.topk, w.depth, w.keep
    excused = 0
    for b in reqs:
        say("  stage-wise oracle, request", b)
        o = oracle_on_gpu_rows(w, W, ci, b, gc)
        if keep is not None:
            keep[b] = o
        n = w.commit_rows
        np.testing.assert_allclose(buf.g.float().cpu().numpy()[b * n:(b + 1) * n], o["g"], atol=atol, rtol=rtol)
        np.testing.assert_allclose(buf.commit_logits[b, 0].cpu().numpy(), o["commit_logits"], atol=atol, rtol=rtol)
        root_ids = buf.root_ids[b, 0].cpu().numpy()
        _same_rule(root_ids, buf.root_lp[b, 0].cpu().numpy(), buf.commit_logits[b, 0].cpu().numpy(), k)
        exact, exc = topk_agrees(root_ids, o["commit_logits"], k, 2 * atol)
        assert exact or exc, f"request {b}: root top-k differs without a near-tie"
        excused += int(not exact)
        tree = O.DynamicTree(k, D, int(ci.tokens[b, -1]), int(ci.ctx_len[b]) + n - 1)
        tree.init(root_ids, buf.root_lp[b, 0].cpu().numpy())
        for r in range(D - 1):
            assert tree.next_rows() == gpu_frontier(gc, b, r), f"request {b}: frontier of round {r}"
            gl = buf.round_logits[r][b].cpu().numpy()
            np.testing.assert_allclose(gl, o["rounds"][r], atol=atol, rtol=rtol, err_msg=f"round {r}")
            ids = buf.round_ids[r][b].cpu().numpy()
            lps = buf.round_lp[r][b].cpu().numpy()
            for row in range(k):
                _same_rule(ids[row], lps[row], gl[row], k)
                exact, exc = topk_agrees(ids[row], o["rounds"][r][row], k, 2 * atol)
                assert exact or exc, f"request {b} round {r} row {row}: top-k differs without a near-tie"
                excused += int(not exact)
            tree.step(ids, buf.round_lp[r][b].cpu().numpy())
        vt = tree.final(m)
        t = gc.tree()
        for name in ("tok", "parent", "depth", "pos"):
            np.testing.assert_array_equal(t[name][b], vt[name], err_msg=f"request {b}: {name}")
        np.testing.assert_array_equal(t["anc"][b], vt["anc"])
        if L is not None:
            if mode == 1:
                ra, rb = O.verify_sample(vt["tok"], vt["parent"], L[b], u_try[b], u_res[b], w.temperature)
            else:
                ra, rb = O.verify_greedy(vt["tok"], vt["parent"], L[b])
            assert int(buf.accept_len[b].item()) == len(ra), f"request {b}: accept length"
            np.testing.assert_array_equal(buf.accepted[b, :len(ra)].cpu().numpy(), ra)
            assert int(buf.bonus[b].item()) == rb, f"request {b}: bonus"
    return excused


def snapshot_topk(gc, w, reqs):
    """The GPU's top-k ids, log-probs and (when kept) logits of requests
    `reqs`, per stage: request -> list of (name, ids, lp, logits or None)."""
    buf = gc.buf
    out = {}
    for b in reqs:
        cl = buf.commit_logits[b, 0].cpu().numpy() if buf.commit_logits is not None else None
        rows = [("root", buf.root_ids[b, 0].cpu().numpy(), buf.root_lp[b, 0].cpu().numpy(), cl)]
        for r in range(w.depth - 1):
            ids = buf.round_ids[r][b].cpu().numpy()
            lps = buf.round_lp[r][b].cpu().numpy()
            gl = buf.round_logits[r][b].cpu().numpy() if buf.round_logits is not None else None
            rows += [(f"round {r} row {i}", ids[i], lps[i], gl[i] if gl is not None else None)
                     for i in range(w.topk)]
        out[b] = rows
    return out


def check_logits_free_topk(gc, w, oracle_by_req, kept, tie_tol):
    """The cycle just run without kept logits (the configuration the
    benchmark times: for k = 1 at 17-64 rows the LM head keeps only
    per-block (max, sum exp, argmax) partials, never the logits) against

    * the kept-logits run on the GPU (same GEMM arithmetic): ids exact,
      log-probs equal up to float32 summation order (2e-5);
    * the oracle's own logits on the same rows: ids equal the oracle's
      top-k unless the oracle has a near-tie (gap <= tie_tol) there, and
      |lp - oracle lp| <= 2 max_y |GPU logit - oracle logit| + 2e-5 on that
      row (lp = logit - LSE, and the LSE moves by at most the largest logit
      difference), where the logits themselves pass the bf16 tolerance.

    Returns (near-tie rows, max |lp - oracle lp|, max |GPU logit - oracle
    logit| over the checked rows)."""
    excused, worst_lp, worst_l = 0, 0.0, 0.0
    free = snapshot_topk(gc, w, list(oracle_by_req))
    for b, o in oracle_by_req.items():
        orows = [o["commit_logits"]] + [o["rounds"][r][i] for r in range(w.depth - 1) for i in range(w.topk)]
        for (name, ids, lp, _), (_, kids, klp, kl), ol in zip(free[b], kept[b], orows):
            np.testing.assert_array_equal(ids, kids, err_msg=f"request {b} {name}: logits-free ids vs kept-logits ids")
            np.testing.assert_allclose(lp, klp, atol=2e-5, rtol=0, err_msg=f"request {b} {name}: lp vs kept-logits lp")
            o_ids, o_lp, _ = O.topk_logprobs(ol, w.topk)
            exact, exc = topk_agrees(ids, ol, w.topk, tie_tol)
            assert exact or exc, f"request {b} {name}: top-{w.topk} {ids} vs oracle {o_ids} without a near-tie"
            dl = float(np.max(np.abs(kl.astype(np.float64) - ol)))
            worst_l = max(worst_l, dl)
            if not exact:
                excused += 1
                continue
            d = float(np.max(np.abs(lp.astype(np.float64) - o_lp.astype(np.float64))))
            worst_lp = max(worst_lp, d)
            assert d <= 2 * dl + 2e-5, f"request {b} {name}: |lp - oracle lp| = {d} > 2 * {dl} + 2e-5"
    return excused, worst_lp, worst_l
