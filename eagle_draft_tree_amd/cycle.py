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
