#!/usr/bin/env python3
"""Benchmark: EAGLE-3 draft-tree cycles on one MI355X.

One step = one full draft-tree cycle of the Llama-3.1-8B-shaped drafter at
batch 1 (d=4096, 32/8 heads x 128, SwiGLU 14336, vocab 128256, bf16 weights,
fp32 accumulation; prefix KV 2048): fusion of the root's 3-layer features,
the COMMIT round, 5 tree rounds (top-10 each), dynamic-tree expansion and
top-60 rerank, and greedy verification against synthetic target logits
(N(0,3), planted argmax agreement 0.8).  Inputs sit in HBM before timing.

Prints one JSON line: draft-tree steps/s (value), verified tokens/s, the LM
head's HBM roofline (the dominant kernel; bytes/launch / HIP-event-measured
launch time), the whole cycle's algorithmic-bytes roofline, a per-kernel-class
breakdown, and the CPU oracle timed on the host (cpu_baseline).  Under
"workloads" the same line carries the other shapes: the 8B drafter at batch
64 (paged chain of 3), the 70B drafter (tree 6/10/60, sampling verify) and
the training-time-test forward (8 x 2048 tokens, 5 steps; MFMA roofline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KC = dict(fuse=0, rowops=1, qkv=2, attn=3, o=4, gate_up=5, down=6, lm_head=7, topk=8, tree=9, verify=10)
KC_TTT = dict(rowops=1, ttt_gemm=11, ttt_attn=12, ttt_ce=13)


def kernel_source_hash():
    """Hash of the sources that build the LM-head kernel (for the traffic record)."""
    h = hashlib.sha256()
    for f in ("gemm_rows.hpp", "draft.hip", "common.hpp"):
        with open(os.path.join(ROOT, "eagle_draft_tree_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, src_hash):
    """Counter-measured HBM bytes per LM-head launch, if recorded for these sources."""
    path = os.path.join(ROOT, "profiles", "lm_head_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(workload)
    if not r or r.get("source_hash") != src_hash:
        return None
    return r.get("bytes_per_launch")


def cpu_baseline(w, Wt, ci, seconds_cap=60.0):
    """The oracle as it stands: one full cycle of request 0 on the host cores."""
    import numpy as np

    from oracle import eagle3_oracle as O
    W = {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}
    np.dot(np.ones((64, 64)), np.ones((64, 64)))  # loads the BLAS, so that its thread pool can be read
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max(int(i.get("num_threads", 1)) for i in pools) if pools else 1
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)" for i in pools)
    except Exception:
        threads, blas = os.cpu_count() or 1, "unknown"
    n = w.commit_rows
    Kc = ci.kv_k.f32()[0].astype(np.float64)
    Vc = ci.kv_v.f32()[0].astype(np.float64)
    t0 = time.time()
    O.draft_cycle(w.shape, W, ci.feats.f32()[:n], ci.tokens[0], Kc, Vc, int(ci.ctx_len[0]), w.topk, w.depth,
                  w.keep)
    dt = time.time() - t0
    try:
        model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")][0]
    except Exception:
        model = "unknown"
    return {"value": 1.0 / dt, "unit": "draft-tree steps/s", "cores": threads, "kind": "oracle",
            "sample": f"one full cycle (fuse + commit + {w.depth - 1} tree rounds + rerank) of request 0, "
                      f"fp64 NumPy, {dt:.1f} s; cpu_count={os.cpu_count()}, "
                      f"affinity={len(os.sched_getaffinity(0))}, {model}; BLAS: {blas or 'none detected'}"}


def cycle_bench(w, dr, steps, warmup, n_plant=8, graph=True):
    """Time `steps` cycles of workload w; returns the measurement dict and the
    cycle inputs.  Target logits: n_plant seeded sets, each planted (when the
    workload plants agreement) on the tree the drafter builds; the timed loop
    cycles through them, and tokens/cycle is their mean accept length + 1.

    Two timed passes: eager launches with per-kernel-class HIP-event timing
    (the breakdown and the LM-head roofline), then, with graph=True, the same
    cycles replayed from one captured HIP graph per target-logit set (the
    step rate).  Every replay's verification outcome is checked against the
    eager one."""
    import numpy as np
    import torch

    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.cycle import CycleBuffers, CycleSpec, KVCache, run_cycle, run_draft_steps
    from workloads import gen

    s = w.shape
    ci = gen.gen_cycle_inputs(w, seed=1)
    Bn, n, k, D, m = w.batch, w.commit_rows, w.topk, w.depth, w.keep
    spec = CycleSpec(Bn, n, k, D, m, ci.cap)
    buf = CycleBuffers(dr, spec)
    i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    tk = torch.zeros(Bn, Bd.MAX_TREE_SLOTS, s.n_kv_heads, s.head_dim, dtype=dr.torch_dtype, device="cuda")
    bt = i32(ci.block_table) if ci.block_table is not None else None
    kv = KVCache(ci.kv_k.torch("cuda"), ci.kv_v.torch("cuda"), tk, torch.zeros_like(tk), i32(ci.ctx_len),
                 cap=ci.cap if bt is None else 0, block_table=bt, block_size=w.block_size)
    ctx_after = i32(ci.ctx_len + n)
    feats = ci.feats.torch("cuda")
    tokens = i32(ci.tokens)
    pos = i32(ci.ctx_len[:, None] + np.arange(n)[None, :])
    root_tok = i32(ci.tokens[:, -1])
    root_pos = i32(ci.ctx_len + n - 1)
    mode = Bd.SAMPLE if w.verify_modes[0] == "sample" else Bd.GREEDY
    ut, ur = gen.uniforms(1, Bn, m + 1)
    ut_d, ur_d = torch.as_tensor(ut).cuda(), torch.as_tensor(ur).cuda()

    def cycle(L):
        run_cycle(dr, buf, kv, feats, tokens, pos, ctx_after, root_tok, root_pos, L, mode, w.temperature,
                  ut_d if mode == Bd.SAMPLE else None, ur_d if mode == Bd.SAMPLE else None)

    cycle(None)  # the tree the drafter builds for these inputs (deterministic)
    torch.cuda.synchronize()
    v_tok, v_par = buf.v_tok.cpu().numpy(), buf.v_parent.cpu().numpy()
    Ls, accepted = [], []
    for p in range(n_plant):
        L = gen.target_logits(1 + p, Bn, m + 1, s.vocab, w.target_sigma)
        if ci.accept_prob is not None:
            gen.plant_agreement(L, v_tok, v_par, ci.accept_prob, seed=1 + p)
        Ls.append(torch.as_tensor(L).cuda())
        cycle(Ls[-1])
        torch.cuda.synchronize()
        assert int(buf.status.cpu().numpy().max()) == 0
        accepted.append(buf.accept_len.cpu().numpy().astype(np.float64))
    tokens_per_cycle = float(np.mean(np.stack(accepted) + 1.0)) * Bn
    for i in range(max(warmup - n_plant, 0)):
        cycle(Ls[i % n_plant])
    torch.cuda.synchronize()

    for c in KC.values():
        Bd.timing_enable(c, (D + 2) * (steps + 1))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        cycle(Ls[i % n_plant])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per_class = {}
    for name, c in KC.items():
        per_class[name] = Bd.timing_read(c)
        Bd.timing_enable(c, 0)
    ms_eager = total_ms / steps
    ms = ms_eager
    if graph:
        graphs = []
        for L in Ls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cycle(L)
            graphs.append(g)
        for p in range(n_plant):  # every graph reproduces the eager outcome
            graphs[p].replay()
            torch.cuda.synchronize()
            assert np.array_equal(buf.accept_len.cpu().numpy().astype(np.float64), accepted[p]), "graph replay differs"
        for i in range(warmup):
            graphs[i % n_plant].replay()
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            graphs[i % n_plant].replay()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        graphs[(steps - 1) % n_plant].replay()
        torch.cuda.synchronize()
        assert np.array_equal(buf.accept_len.cpu().numpy().astype(np.float64), accepted[(steps - 1) % n_plant])
        # per-cycle spread, in a pass of its own (one event between replays),
        # so that the rate above stays an uninterrupted loop
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record()
        for i in range(steps):
            graphs[i % n_plant].replay()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per_cycle = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
        cycle_pct = {"p10": round(float(np.percentile(per_cycle, 10)), 4),
                     "median": round(float(np.median(per_cycle)), 4),
                     "p90": round(float(np.percentile(per_cycle, 90)), 4)}
        del graphs
        # the cycle's D draft steps alone (COMMIT + D-1 TREE rounds), replayed on
        # the inputs the last cycle left in place
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            run_draft_steps(dr, buf, kv, tokens, pos, ctx_after)
        for i in range(warmup):
            gs.replay()
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            gs.replay()
        end.record()
        torch.cuda.synchronize()
        ms_steps = start.elapsed_time(end) / steps
        del gs

    # algorithmic bytes: bf16 weights read once per round, every request's KV once per round
    es = 2
    d, F, V, hq, hkv, hd = s.d, s.ffn, s.vocab, s.n_q_heads, s.n_kv_heads, s.head_dim
    w_fc = d * 3 * d * es
    w_layer = ((hq + 2 * hkv) * hd * 2 * d + d * hq * hd + 2 * F * d + d * F) * es
    w_lm = V * d * es
    kv_round = int(np.sum(ci.ctx_len + n)) * hkv * hd * 2 * es
    bytes_cycle = w_fc + D * (w_layer + w_lm + kv_round)
    # LM head launches: COMMIT (top-k of the last row of each request) then D-1 tree rounds (k rows each)
    rows = [Bn] + [Bn * k] * (D - 1)

    def lm_out_bytes(r):
        # tiles per LM-head workgroup: 2 up to 16 rows (rows GEMM), 32 for 17..64
        # rows (register-weight GEMM, model width a multiple of 64)
        nt16 = V // 16
        tpw = 2 if r <= 16 else 32
        # top-1 on 17..64 rows without kept logits: the LM head writes per-workgroup
        # (max, sum exp, argmax) partials (16 B per row) instead of fp32 logits
        if k == 1 and 16 < r <= 64:
            return r * -(-nt16 // tpw) * 16
        out = r * V * 4
        if r <= 64:
            # plus each 16-column tile's (max, sum exp) per row, 8 B, in slots grouped by XCD
            out += r * 8 * tpw * -(-(-(-nt16 // tpw)) // 8) * 8
        return out

    lm_bytes = [w_lm + r * d * es + lm_out_bytes(r) for r in rows]
    bytes_steps = D * (w_layer + kv_round) + sum(lm_bytes)  # the D draft steps
    lm_flops = [2.0 * r * V * d for r in rows]
    lm_ms, lm_cnt = per_class["lm_head"]
    reps = lm_cnt // len(rows) if lm_cnt else 0
    lm_gbs = sum(lm_bytes) * reps / (lm_ms * 1e-3) / 1e9 if lm_ms > 0 else None
    lm_tflops = sum(lm_flops) * reps / (lm_ms * 1e-3) / 1e12 if lm_ms > 0 else None
    res = {
        "workload": w.name,
        "steps": steps,
        "ms_per_step": round(ms, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "graph": graph,
        "draft_tree_steps_per_s": round(1000.0 / ms, 2),
        "verified_tokens_per_s": round(1000.0 / ms * tokens_per_cycle, 1),
        "tokens_per_cycle": round(tokens_per_cycle, 3),
        "verify": w.verify_modes[0],
        "lm_head": {"GBs": round(lm_gbs, 1) if lm_gbs else None,
                    "hbm_frac": round(lm_gbs / HBM_PEAK_GBS, 4) if lm_gbs else None,
                    "TFLOPs": round(lm_tflops, 2) if lm_tflops else None,
                    "mfma_frac": round(lm_tflops / MFMA_BF16_PEAK_TFLOPS, 4) if lm_tflops else None,
                    "bytes_per_launch": round(sum(lm_bytes) / len(lm_bytes)),
                    "avg_launch_us": round(lm_ms / lm_cnt * 1e3, 2) if lm_cnt else None},
        "cycle_roofline": {"bytes": bytes_cycle, "achieved_GBs": round(bytes_cycle / (ms * 1e-3) / 1e9, 1),
                           "frac": round(bytes_cycle / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernel_ms_per_cycle": {kk: round(v[0] / steps, 4) for kk, v in per_class.items()},
    }
    if graph:
        res["cycle_ms_percentiles"] = cycle_pct
        gbs = bytes_steps / (ms_steps * 1e-3) / 1e9
        res["draft_step_roofline"] = {"steps": D, "bytes_per_step": round(bytes_steps / D),
                                      "us_per_step": round(ms_steps * 1e3 / D, 2), "achieved_GBs": round(gbs, 1),
                                      "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return res, ci


def ttt_bench(w, dr, steps, warmup):
    """Time the training-time-test forward (B x S tokens, R rollout steps)."""
    import numpy as np
    import torch

    from eagle_draft_tree_amd import binding as Bd
    from workloads import gen

    s = w.shape
    B, S, R = w.batch, w.ttt_seq, w.ttt_steps
    ti = gen.gen_ttt_inputs(s, B, S, R, seed=1)
    feats = ti.feats.torch("cuda")
    tokens = torch.as_tensor(ti.tokens).cuda()
    pred = torch.empty(B, R, S, dtype=torch.int32, device="cuda")
    ce = torch.empty(B, R, S, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(Bd.ttt_workspace_size(dr.dims, B, S, R), dtype=torch.uint8, device="cuda")

    def run():
        Bd.eagle3_ttt_forward(dr.dims, dr.weights, feats, tokens, B, S, R, None, pred, ce, loss, ws)

    for _ in range(max(warmup, 1)):
        run()
    torch.cuda.synchronize()
    for c in KC_TTT.values():
        Bd.timing_enable(c, 64 * (steps + 1))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    per_class = {}
    for name, c in KC_TTT.items():
        per_class[name] = Bd.timing_read(c)
        Bd.timing_enable(c, 0)
    M = B * S
    d, F, V, hq, hkv, hd = s.d, s.ffn, s.vocab, s.n_q_heads, s.n_kv_heads, s.head_dim
    qd, kvd = hq * hd, hkv * hd
    f_gemm = 2.0 * M * d * 3 * d + R * (2.0 * M * 2 * d * (qd + 2 * kvd) + 2.0 * M * qd * d
                                        + 2.0 * M * d * 2 * F + 2.0 * M * F * d)
    f_lm = R * 2.0 * M * d * V
    keys = B * S * (S + 1) / 2.0
    f_attn = sum(4.0 * (keys + M * (j - 1)) * hq * hd for j in range(1, R + 1))
    tf = lambda f, name: f / (per_class[name][0] / steps * 1e-3) / 1e12 if per_class[name][0] > 0 else None
    lm_tf = tf(f_lm, "ttt_ce")
    lm_launch_us = per_class["ttt_ce"][0] / per_class["ttt_ce"][1] * 1e3 if per_class["ttt_ce"][1] else None
    return {
        "workload": w.name,
        "steps": steps,
        "ms_per_step": round(ms, 3),
        "rows_per_s": round(M * R / (ms * 1e-3), 1),
        "tokens_per_s": round(M / (ms * 1e-3), 1),
        "loss": round(float(loss.item()), 4),
        "TFLOPs": round((f_gemm + f_lm + f_attn) / (ms * 1e-3) / 1e12, 1),
        "mfma_frac": round((f_gemm + f_lm + f_attn) / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(lm_tf, 1) if lm_tf else None,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(lm_tf / MFMA_BF16_PEAK_TFLOPS, 4) if lm_tf else None, "traffic": None,
                     "kernel": "LM-head GEMM with CE epilogue", "flops_per_launch": f_lm / R,
                     "avg_launch_us": round(lm_launch_us, 1) if lm_launch_us else None},
        "class_TFLOPs": {"projection_gemms": round(tf(f_gemm, "ttt_gemm"), 1),
                         "lm_head_ce": round(lm_tf, 1), "attention": round(tf(f_attn, "ttt_attn"), 1)},
        "kernel_ms_per_step": {kk: round(v[0] / steps, 3) for kk, v in per_class.items()},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["c2", "c3", "c4", "ttt"], default=None,
                    help="run one workload only (profiling); the main line is then that workload's")
    ap.add_argument("--main-only", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}))
        return

    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.cycle import Drafter
    from workloads import gen
    from workloads.configs import C2_8B_TREE, C3_8B_CHAIN, C4_70B_TREE, C5_8B_TTT

    Bd.load()
    t0 = time.time()
    s8 = C2_8B_TREE.shape
    Wt8 = gen.gen_weights(s8, seed=0) if args.only != "c4" else None
    dr8 = Drafter(s8, Wt8, pack=True) if Wt8 is not None else None
    setup_s = time.time() - t0

    if args.only == "ttt":
        r = ttt_bench(C5_8B_TTT, dr8, max(1, min(args.steps, 10)), 1)
        print(json.dumps(r), flush=True)
        return
    if args.only == "c2":
        args.main_only = True
    if args.only in ("c3", "c4"):
        w = C3_8B_CHAIN if args.only == "c3" else C4_70B_TREE
        dr = dr8 if args.only == "c3" else Drafter(w.shape, gen.gen_weights(w.shape, seed=0), pack=True)
        r, _ = cycle_bench(w, dr, args.steps, args.warmup, graph=not args.no_graph)
        print(json.dumps(r), flush=True)
        return

    w = C2_8B_TREE
    r, ci = cycle_bench(w, dr8, args.steps, args.warmup, graph=not args.no_graph)
    lm = r["lm_head"]
    src_hash = kernel_source_hash()
    traffic = load_traffic("llama3.1-8b-b1-tree", src_hash)
    out = {
        "metric": "draft-tree steps/s + verified tokens/s at 1 GPU; % peak HBM GB/s / MFMA",
        "value": r["draft_tree_steps_per_s"],
        "unit": "draft-tree steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "ms_per_step_eager": r["ms_per_step_eager"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) features/KV, N(0,3) target logits planted 0.8)",
        "config": {"workload": w.name, "batch": w.batch, "prefix": int(ci.ctx_len[0]), "depth": w.depth,
                   "topk": w.topk, "keep": w.keep, "verify": "greedy", "graph": r["graph"], "weights": "packed"},
        "verified_tokens_per_s": r["verified_tokens_per_s"],
        "tokens_per_cycle": r["tokens_per_cycle"],
        "roofline": {"bound": "hbm", "achieved": lm["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": lm["hbm_frac"], "traffic": traffic, "kernel": "lm_head rows GEMM",
                     "bytes_per_launch": lm["bytes_per_launch"], "avg_launch_us": lm["avg_launch_us"]},
        "cycle_ms_percentiles": r.get("cycle_ms_percentiles"),
        "cycle_roofline": r["cycle_roofline"],
        "draft_step_roofline": r.get("draft_step_roofline"),
        "kernel_ms_per_cycle": r["kernel_ms_per_cycle"],
        "setup_s": round(setup_s, 1),
    }
    if not args.main_only:
        wl = {}
        r3, _ = cycle_bench(C3_8B_CHAIN, dr8, max(args.steps // 2, 1), args.warmup, graph=not args.no_graph)
        wl[C3_8B_CHAIN.name] = r3
        r5 = ttt_bench(C5_8B_TTT, dr8, 5, 1)
        wl[C5_8B_TTT.name] = r5
        del dr8
        torch.cuda.empty_cache()
        dr70 = Drafter(C4_70B_TREE.shape, gen.gen_weights(C4_70B_TREE.shape, seed=0), pack=True)
        r4, _ = cycle_bench(C4_70B_TREE, dr70, max(args.steps // 3, 1), args.warmup, graph=not args.no_graph)
        wl[C4_70B_TREE.name] = r4
        del dr70
        out["workloads"] = wl
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, Wt8, ci)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
