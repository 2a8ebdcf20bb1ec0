"""Host-side driver of one EAGLE-3 draft-tree cycle through the C ABI.

fuse -> draft_step(COMMIT) -> tree_expand(INIT) -> [draft_step(TREE) ->
tree_expand(STEP)] x (D-1) -> tree_expand(FINAL) -> verify.  Only ABI calls
are enqueued (on torch's current stream); every step runs in the library's
kernels.  Device buffers come from torch.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B


class Drafter:
    """Device-resident drafter weights plus their eagle3_dims/eagle3_weights.

    pack=True (bf16 only) converts the GEMM matrices once into the library's
    MFMA fragment order (eagle3_pack_weights) and drops the row-major copies."""

    def __init__(self, shape, weights: dict, device="cuda", pack=False):
        self.shape = shape
        self.tensors = {}
        for name, w in weights.items():
            if hasattr(w, "torch"):
                self.tensors[name] = w.torch(device)
            else:
                self.tensors[name] = torch.as_tensor(np.asarray(w, dtype=np.float32)).to(device)
        self.dims = B.dims_of(shape)
        self.weights = B.weights_of(self.tensors)
        self.torch_dtype = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        self.packed = None
        if pack and shape.dtype == "bf16":
            self.packed = torch.empty(B.packed_weights_size(self.dims), dtype=torch.uint8, device=device)
            self.weights = B.eagle3_pack_weights(self.dims, self.weights, self.packed)
            torch.cuda.synchronize()
            for n in ("fc", "qkv", "o", "gate_up", "down", "lm"):
                del self.tensors[n]
        self.head = None

    def set_lowrank_head(self, a, b, rank, candidates, device="cuda"):
        """Use the efficient LM head (EAGLE-4): low-rank factors a [V, rank]
        and b [rank, d] (generator Tensors or arrays), the `candidates` best
        low-rank scores per row re-scored exactly.  Packed like the drafter."""
        ta = a.torch(device) if hasattr(a, "torch") else torch.as_tensor(a).to(device)
        tb = b.torch(device) if hasattr(b, "torch") else torch.as_tensor(b).to(device)
        layout = B.LAYOUT_ROWMAJOR
        if self.packed is not None:
            pa, pb = torch.empty_like(ta), torch.empty_like(tb)
            B.eagle3_pack_matrix(ta, ta.shape[0], ta.shape[1], pa)
            B.eagle3_pack_matrix(tb, tb.shape[0], tb.shape[1], pb)
            torch.cuda.synchronize()
            ta, tb, layout = pa, pb, B.LAYOUT_PACKED
        self.head_tensors = (ta, tb)
        self.head = B.LowrankHead(ta.data_ptr(), tb.data_ptr(), rank, candidates, layout)


@dataclass
class CycleSpec:
    batch: int
    commit_rows: int
    k: int
    depth: int
    keep: int
    cap_rows: int      # KV rows per request (contiguous cap, or max_blocks*block_size)


class CycleBuffers:
    """Every device buffer one cycle needs (allocated once, reused)."""

    def __init__(self, drafter: Drafter, spec: CycleSpec, device="cuda"):
        s, dv = drafter.shape, device
        Bn, n, k, D, m = spec.batch, spec.commit_rows, spec.k, spec.depth, spec.keep
        i32 = dict(dtype=torch.int32, device=dv)
        self.spec = spec
        self.g = torch.empty(Bn * n, s.d, dtype=drafter.torch_dtype, device=dv)
        self.h_tree = torch.zeros(Bn, B.MAX_TREE_SLOTS + 1, s.d, dtype=torch.float32, device=dv)
        max_rows = max(n, k)
        self.ws = torch.zeros(B.workspace_size(drafter.dims, Bn, max_rows, spec.cap_rows), dtype=torch.uint8,
                              device=dv)
        self.root_ids = torch.empty(Bn, 1, k, **i32)
        self.root_lp = torch.empty(Bn, 1, k, dtype=torch.float32, device=dv)
        self.round_ids = [torch.empty(Bn, k, k, **i32) for _ in range(max(D - 1, 0))]
        self.round_lp = [torch.empty(Bn, k, k, dtype=torch.float32, device=dv) for _ in range(max(D - 1, 0))]
        self.next_tok = [torch.empty(Bn, k, **i32) for _ in range(max(D - 1, 0))]
        self.next_par = [torch.empty(Bn, k, **i32) for _ in range(max(D - 1, 0))]
        self.next_pos = [torch.empty(Bn, k, **i32) for _ in range(max(D - 1, 0))]
        self.next_anc = [torch.empty(Bn, k, dtype=torch.int64, device=dv) for _ in range(max(D - 1, 0))]
        self.tree_state = torch.empty(B.tree_state_size(Bn, k, D), dtype=torch.uint8, device=dv)
        self.v_tok = torch.empty(Bn, m + 1, **i32)
        self.v_parent = torch.empty(Bn, m + 1, **i32)
        self.v_depth = torch.empty(Bn, m + 1, **i32)
        self.v_pos = torch.empty(Bn, m + 1, **i32)
        self.v_anc = torch.empty(Bn, m + 1, dtype=torch.int64, device=dv)
        self.accept_len = torch.empty(Bn, **i32)
        self.accepted = torch.empty(Bn, D, **i32)
        self.bonus = torch.empty(Bn, **i32)
        self.status = torch.empty(Bn, **i32)
        # zero-filled once: per-request arrival counters the library keeps at zero
        self.vws = torch.zeros(B.verify_workspace_size(Bn, m, s.vocab), dtype=torch.uint8, device=dv)
        self.commit_logits = None
        self.round_logits = None
        self.commit_cand = self.round_cand = None  # efficient head: candidate ids and exact logits (tests)

    def keep_candidates(self, c, device="cuda"):
        """Also write the efficient head's candidates and their exact logits (tests)."""
        Bn, k, D = self.spec.batch, self.spec.k, self.spec.depth
        mk = lambda rows: (torch.empty(Bn, rows, c, dtype=torch.int32, device=device),
                           torch.empty(Bn, rows, c, dtype=torch.float32, device=device))
        self.commit_cand = mk(1)
        self.round_cand = [mk(k) for _ in range(max(D - 1, 0))]

    def keep_logits(self, vocab, device="cuda"):
        """Also write LM-head logits (for parity checks; not on the hot path)."""
        Bn, k, D = self.spec.batch, self.spec.k, self.spec.depth
        self.commit_logits = torch.empty(Bn, 1, vocab, dtype=torch.float32, device=device)
        self.round_logits = [torch.empty(Bn, k, vocab, dtype=torch.float32, device=device)
                             for _ in range(max(D - 1, 0))]


def draft_step(dr: Drafter, buf: CycleBuffers, kv, mode, Bn, rows, state, parent, tokens, pos, anc, slot_base, k,
               topk_rows, ids, lp, logits, cand=None):
    """One eagle3_draft_step, through the efficient head when the drafter has one."""
    if dr.head is None:
        B.eagle3_draft_step(dr.dims, dr.weights, kv, mode, Bn, rows, state, parent, tokens, pos, anc, slot_base, k,
                            topk_rows, buf.h_tree, ids, lp, logits, buf.ws)
    else:
        B.eagle3_draft_step_lowrank(dr.dims, dr.weights, kv, mode, Bn, rows, state, parent, tokens, pos, anc,
                                    slot_base, k, topk_rows, buf.h_tree, ids, lp, logits, dr.head,
                                    cand[0] if cand is not None else None, cand[1] if cand is not None else None,
                                    buf.ws)


class KVCache:
    """Committed KV (contiguous or paged) + tree slots, as an eagle3_kv."""

    def __init__(self, k, v, tk, tv, ctx_len, cap=0, block_table=None, block_size=16):
        self.k, self.v, self.tk, self.tv = k, v, tk, tv
        self.ctx_len = ctx_len
        self.block_table = block_table
        self.cap = cap
        self.block_size = block_size

    def struct(self, ctx_len=None):
        cl = self.ctx_len if ctx_len is None else ctx_len
        bt = self.block_table
        return B.KV(self.k.data_ptr(), self.v.data_ptr(), self.cap,
                    bt.data_ptr() if bt is not None else None,
                    bt.shape[1] if bt is not None else 0, self.block_size if bt is not None else 0,
                    cl.data_ptr(), self.tk.data_ptr(), self.tv.data_ptr())


def run_draft_steps(dr: Drafter, buf: CycleBuffers, kv: KVCache, tokens, commit_pos, ctx_after):
    """Enqueue only the cycle's draft steps (COMMIT, then the D-1 TREE rounds)
    on the inputs a previous run_cycle left in `buf` (fused rows, frontier
    rows): the same calls as run_cycle, without fusion, tree expansion or
    verification."""
    sp = buf.spec
    Bn, n, k, D = sp.batch, sp.commit_rows, sp.k, sp.depth
    kv_commit = kv.struct()
    kv_tree = kv.struct(ctx_after)
    draft_step(dr, buf, kv_commit, B.COMMIT, Bn, n, buf.g, None, tokens, commit_pos, None, 0, k, B.TOPK_LAST,
               buf.root_ids, buf.root_lp, buf.commit_logits, buf.commit_cand)
    for j in range(2, D + 1):
        r = j - 2
        draft_step(dr, buf, kv_tree, B.TREE, Bn, k, None, buf.next_par[r], buf.next_tok[r], buf.next_pos[r],
                   buf.next_anc[r], r * k, k, B.TOPK_ALL, buf.round_ids[r], buf.round_lp[r],
                   buf.round_logits[r] if buf.round_logits is not None else None,
                   buf.round_cand[r] if buf.round_cand is not None else None)


def run_cycle(dr: Drafter, buf: CycleBuffers, kv: KVCache, feats, tokens, commit_pos, ctx_after,
              root_tok, root_pos, target_logits=None, mode=B.GREEDY, temperature=1.0, u_try=None,
              u_res=None, verify=True):
    """Enqueue one cycle.  feats [B*n,3,d], tokens/commit_pos [B,n] int32,
    ctx_after [B] (committed rows incl. the new ones), root_tok/root_pos [B]."""
    sp = buf.spec
    Bn, n, k, D, m = sp.batch, sp.commit_rows, sp.k, sp.depth, sp.keep
    B.eagle3_fuse(dr.dims, dr.weights, feats, Bn * n, buf.g, buf.ws)
    kv_commit = kv.struct()
    kv_tree = kv.struct(ctx_after)
    draft_step(dr, buf, kv_commit, B.COMMIT, Bn, n, buf.g, None, tokens, commit_pos, None, 0, k, B.TOPK_LAST,
               buf.root_ids, buf.root_lp, buf.commit_logits, buf.commit_cand)
    B.eagle3_tree_expand(B.INIT, Bn, k, D, m, root_tok, root_pos, buf.tree_state, buf.root_ids, buf.root_lp,
                         buf.next_tok[0] if D > 1 else buf.v_tok, buf.next_par[0] if D > 1 else buf.v_tok,
                         buf.next_pos[0] if D > 1 else buf.v_tok, buf.next_anc[0] if D > 1 else buf.v_anc)
    for j in range(2, D + 1):
        r = j - 2
        draft_step(dr, buf, kv_tree, B.TREE, Bn, k, None, buf.next_par[r], buf.next_tok[r], buf.next_pos[r],
                   buf.next_anc[r], r * k, k, B.TOPK_ALL, buf.round_ids[r], buf.round_lp[r],
                   buf.round_logits[r] if buf.round_logits is not None else None,
                   buf.round_cand[r] if buf.round_cand is not None else None)
        nr = r + 1 if j < D else r  # the last STEP emits no rows (buffers unused)
        B.eagle3_tree_expand(B.STEP, Bn, k, D, m, None, None, buf.tree_state, buf.round_ids[r],
                             buf.round_lp[r], buf.next_tok[nr], buf.next_par[nr], buf.next_pos[nr],
                             buf.next_anc[nr])
    B.eagle3_tree_expand(B.FINAL, Bn, k, D, m, None, None, buf.tree_state, None, None, None, None, None, None,
                         buf.v_tok, buf.v_parent, buf.v_depth, buf.v_pos, buf.v_anc)
    if verify and target_logits is not None:
        B.eagle3_verify(Bn, m, dr.shape.vocab, D, buf.v_tok, buf.v_parent, target_logits, mode, temperature,
                        u_try, u_res, buf.accept_len, buf.accepted, buf.bonus, buf.status, buf.vws)


@dataclass
class HarnessParams:
    """Thresholds of the EAGLE-4 Harness rules (eagle3_harness_*)."""
    tau_depth: float = 0.5     # depth rule: tau0 of tau0 * (1 + alpha * depth)
    alpha: float = 0.25
    tau_verify: float = 0.5    # expected accepted tokens per extra verify millisecond
    tau_branch: float = 0.5    # ... per extra drafting millisecond of 8 branches over 4


class HarnessCycle:
    """A draft cycle under the EAGLE-4 Harness: the COMMIT round's top-8
    decides the branch cap k (8 or 4); before every further round the depth
    rule decides whether to draft another layer (at most D_max rounds); the
    verify-count rule picks m <= m_max from the pool.  Each decision reads a
    few scores back to the host (eagle3_tree_confidence) and runs the
    library's host-side rules on the warm-up table.

    Buffers are sized for k = 8, D_max and m_max; a call with k = 4 or a
    smaller m uses their leading elements (the library reads and writes
    them as packed [B][rows][k] / [B][m+1] arrays)."""

    def __init__(self, drafter: Drafter, batch, commit_rows, D_max, m_max, cap_rows, table, params: HarnessParams,
                 device="cuda"):
        self.dr, self.table, self.p = drafter, table, params
        self.Bn, self.n, self.D, self.m_max = batch, commit_rows, D_max, m_max
        self.buf = CycleBuffers(drafter, CycleSpec(batch, commit_rows, 8, D_max, m_max, cap_rows), device)
        i32 = dict(dtype=torch.int32, device=device)
        self.root_ids4 = torch.empty(batch, 1, 4, **i32)
        self.root_lp4 = torch.empty(batch, 1, 4, dtype=torch.float32, device=device)
        self.front = torch.empty(batch * 8, dtype=torch.float32, device=device)
        self.pool = torch.empty(batch * m_max, dtype=torch.float32, device=device)
        self.decisions = None

    def tree(self, m):
        b = self.buf
        M1 = m + 1
        flat = lambda t: t.view(-1)[: self.Bn * M1].view(self.Bn, M1)
        return dict(tok=flat(b.v_tok), parent=flat(b.v_parent), depth=flat(b.v_depth), pos=flat(b.v_pos),
                    anc=flat(b.v_anc))

    def run(self, kv: KVCache, feats, tokens, commit_pos, ctx_after, root_tok, root_pos, ctx_for_cost):
        """Enqueue and decide one cycle; returns dict(k=, rounds=, m=) and
        leaves the verify tree in tree(m)."""
        dr, buf, Bn, n, D = self.dr, self.buf, self.Bn, self.n, self.D
        B.eagle3_fuse(dr.dims, dr.weights, feats, Bn * n, buf.g, buf.ws)
        kv_commit = kv.struct()
        kv_tree = kv.struct(ctx_after)
        draft_step(dr, buf, kv_commit, B.COMMIT, Bn, n, buf.g, None, tokens, commit_pos, None, 0, 8, B.TOPK_LAST,
                   buf.root_ids, buf.root_lp, buf.commit_logits, buf.commit_cand)
        lp8 = buf.root_lp.view(Bn, 8).cpu().numpy()
        k = B.harness_branch_cap(self.table, Bn, ctx_for_cost, lp8, self.p.tau_branch)
        ids, lp = buf.root_ids, buf.root_lp
        if k == 4:
            self.root_ids4.copy_(buf.root_ids[:, :, :4])
            self.root_lp4.copy_(buf.root_lp[:, :, :4])
            ids, lp = self.root_ids4, self.root_lp4
        B.eagle3_tree_expand(B.INIT, Bn, k, D, self.m_max, root_tok, root_pos, buf.tree_state, ids, lp,
                             buf.next_tok[0] if D > 1 else buf.v_tok, buf.next_par[0] if D > 1 else buf.v_tok,
                             buf.next_pos[0] if D > 1 else buf.v_tok, buf.next_anc[0] if D > 1 else buf.v_anc)
        rounds = 1
        for j in range(2, D + 1):
            B.eagle3_tree_confidence(Bn, k, D, 0, buf.tree_state, self.front, None)
            front = self.front[: Bn * k].view(Bn, k).cpu().numpy()
            if not B.harness_continue(self.table, Bn, ctx_for_cost, k, j - 1, front, self.p.tau_depth, self.p.alpha):
                break
            r = j - 2
            draft_step(dr, buf, kv_tree, B.TREE, Bn, k, None, buf.next_par[r], buf.next_tok[r], buf.next_pos[r],
                       buf.next_anc[r], r * k, k, B.TOPK_ALL, buf.round_ids[r], buf.round_lp[r],
                       buf.round_logits[r] if buf.round_logits is not None else None, None)
            nr = r + 1 if j < D else r
            B.eagle3_tree_expand(B.STEP, Bn, k, D, self.m_max, None, None, buf.tree_state, buf.round_ids[r],
                                 buf.round_lp[r], buf.next_tok[nr], buf.next_par[nr], buf.next_pos[nr],
                                 buf.next_anc[nr])
            rounds += 1
        pool_n = k + (rounds - 1) * k * k
        m_cap = min(self.m_max, pool_n)
        B.eagle3_tree_confidence(Bn, k, D, m_cap, buf.tree_state, None, self.pool)
        pool = self.pool[: Bn * m_cap].view(Bn, m_cap).cpu().numpy()
        m = max(B.harness_verify_count(self.table, Bn, ctx_for_cost, pool, self.p.tau_verify), 1)
        B.eagle3_tree_expand(B.FINAL, Bn, k, D, m, None, None, buf.tree_state, None, None, None, None, None, None,
                             buf.v_tok, buf.v_parent, buf.v_depth, buf.v_pos, buf.v_anc)
        self.decisions = dict(k=k, rounds=rounds, m=m)
        return self.decisions
