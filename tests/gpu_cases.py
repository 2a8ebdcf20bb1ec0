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
