"""How far the oracle moves from itself when its arithmetic is float32
instead of fp64: the bf16 rounding cascade at a benchmark shape.

The GPU accumulates every GEMM in float32 and carries the residual stream
(s, h1, h2) in float32; the oracle does both in fp64.  Both round the GEMM
inputs to bf16 at the same points, so a float32 accumulation error (about
sqrt(K) * 2^-24 relative, K up to 28672) can flip a bf16 rounding, and each
flip moves everything downstream by up to one bf16 ulp times a weight.
This script decodes the same rows with the oracle three ways -- fp64, fp64
with the states rounded to float32 after every round, and with every GEMM
accumulated in float32 (numpy sgemm) plus float32 states -- each variant
from its own upstream values (not stage-isolated), and reports how far the
logits of each round move from the fp64 run.  It is run by hand (python
tests/rounding_cascade.py c4), not collected by pytest: at the 70B shape it
takes a few minutes on the CPU.  Nothing here calls the GPU library.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import eagle3_oracle as O  # noqa: E402
from workloads import gen  # noqa: E402
from workloads.configs import C2_8B_TREE, C4_70B_TREE  # noqa: E402


def _matmul_wt_f32(x, W):
    """x @ W.T with float32 inputs and float32 accumulation (BLAS sgemm)."""
    x32 = np.asarray(x, dtype=np.float32)
    out = np.empty((x32.shape[0], W.shape[0]), dtype=np.float64)
    for s0 in range(0, W.shape[0], 8192):
        out[:, s0:s0 + 8192] = x32 @ np.asarray(W[s0:s0 + 8192], dtype=np.float32).T
    return out


def run(w, rounds=2):
    s = w.shape
    t0 = time.time()
    Wt = gen.gen_weights(s, seed=0)
    W = {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}
    del Wt
    ci = gen.gen_cycle_inputs(w, seed=1)
    print(f"{w.name}: inputs in {time.time() - t0:.0f} s", flush=True)
    Kc = ci.kv_k.f32()[0].astype(np.float64)
    Vc = ci.kv_v.f32()[0].astype(np.float64)
    cap = Kc.shape[0]
    N = cap + O.MAX_TREE_SLOTS
    L0 = int(ci.ctx_len[0])
    out = {}
    exact_mm = O.matmul_wt
    for variant in ("fp64", "fp32", "f32gemm"):
        O.matmul_wt = _matmul_wt_f32 if variant == "f32gemm" else exact_mm
        g = O.fuse(s, ci.feats.f32()[:1], W["fc"])
        K = np.zeros((N, s.n_kv_heads, s.head_dim)); V = np.zeros_like(K)
        K[:cap], V[:cap] = Kc, Vc
        vis = np.zeros((1, N), bool); vis[0, :L0 + 1] = True
        h2, logits = O.decoder_rows(s, W, g, ci.tokens[0], [L0], K, V, [L0], vis)
        ids, lp, _ = O.topk_logprobs(logits[0], w.topk)
        root = h2[0] if variant == "fp64" else h2[0].astype(np.float32).astype(np.float64)
        rec = [("commit", logits[0])]
        if variant == "fp64":
            tree = O.DynamicTree(w.topk, w.depth, int(ci.tokens[0, -1]), L0)
            tree.init(ids, lp)
            rows_by_round = []
        h_tree = {0: root}
        for r in range(rounds):
            rows = tree.next_rows() if variant == "fp64" else out["rows"][r]
            if variant == "fp64":
                rows_by_round.append(rows)
            base = r * w.topk
            S = np.stack([h_tree[p] if variant == "fp64" else h_tree[p] for (_, p, _, _) in rows])
            T = np.array([t for (t, _, _, _) in rows]); P = np.array([p for (_, _, p, _) in rows])
            vis = np.zeros((len(rows), N), bool); vis[:, :L0 + 1] = True
            for i, (_, _, _, anc) in enumerate(rows):
                for sl in range(O.MAX_TREE_SLOTS):
                    if (anc >> sl) & 1:
                        vis[i, cap + sl] = True
            h2r, lg = O.decoder_rows(s, W, S, T, P, K, V, cap + base + np.arange(len(rows)), vis)
            for i in range(len(rows)):
                h_tree[1 + base + i] = h2r[i] if variant == "fp64" else h2r[i].astype(np.float32).astype(np.float64)
            rec.append((f"tree round {r}", lg))
            if variant == "fp64":
                tid, tlp = zip(*[O.topk_logprobs(lg[i], w.topk)[:2] for i in range(len(rows))])
                tree.step(np.array(tid), np.array(tlp))
        out[variant] = rec
        if variant == "fp64":
            out["rows"] = rows_by_round
        print(f"  {variant} pass done at {time.time() - t0:.0f} s", flush=True)
    O.matmul_wt = exact_mm
    for v in ("fp32", "f32gemm"):
        for (name, a), (_, b) in zip(out["fp64"], out[v]):
            d = np.abs(np.asarray(a) - np.asarray(b))
            bound = 2e-2 + 1e-2 * np.abs(np.asarray(a))
            print(f"  {v} vs fp64, {name}: max |logit diff| = {d.max():.4g}, mean {d.mean():.3g}, "
                  f"{int((d > bound).sum())} of {d.size} beyond 2e-2 + 1e-2|l|", flush=True)


if __name__ == "__main__":
    which = sys.argv[1] if len(sys.argv) > 1 else "c4"
    run(C4_70B_TREE if which == "c4" else C2_8B_TREE)
