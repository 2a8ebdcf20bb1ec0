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
KC = dict(fuse=0, rowops=1, qkv=2, attn=3, o=4, gate_up=5, down=6, lm_head=7, topk=8, tree=9, verify=10,
          lr_scores=14)
KC_TTT = dict(rowops=1, ttt_gemm=11, ttt_attn=12, ttt_ce=13)
KC_TTT_TRAIN = dict(KC_TTT, ttt_bwd_gemm=18, ttt_bwd_attn=19, ttt_wgrad=20, ttt_bwd_rows=21)


# sources that build each workload's dominant kernel (a traffic record is
# used only while their hash is unchanged)
KERNEL_SOURCES = {
    "rows_gemm": ("gemm_rows.hpp", "layer_ops.hpp", "draft.hip", "common.hpp"),
    "rows_rx": ("rows_rx.hpp", "rows_dma.hpp", "layer_ops.hpp", "draft.hip", "common.hpp"),
    "lr_scores": ("lowrank.hip", "draft.hip", "common.hpp"),
    "ttt_ce": ("bigemm.hpp", "ttt.hip", "ttt_common.hpp", "common.hpp"),
    "ttt_dy": ("bigemm.hpp", "ttt.hip", "ttt_common.hpp", "common.hpp"),
    "target_gate_up": ("gemm_rows.hpp", "rows_dma.hpp", "rows_rx.hpp", "layer_ops.hpp", "target.hip", "common.hpp"),
}


def kernel_source_hash(kind="rows_gemm"):
    """Hash of the sources that build a kernel (for the traffic record)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "eagle_draft_tree_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kind):
    """Counter-measured HBM bytes per launch of a workload's dominant kernel,
    if recorded (profiles/traffic.json) for the current sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(workload)
    if not r or r.get("source_hash") != kernel_source_hash(kind):
        return None
    return r.get("bytes_per_launch")


def _host_info():
    """Threads the oracle's BLAS uses, a description of it, and the CPU model."""
    import numpy as np
    np.dot(np.ones((64, 64)), np.ones((64, 64)))  # loads the BLAS, so that its thread pool can be read
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max(int(i.get("num_threads", 1)) for i in pools) if pools else 1
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)" for i in pools)
    except Exception:
        threads, blas = os.cpu_count() or 1, "unknown"
    try:
        model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")][0]
    except Exception:
        model = "unknown"
    desc = (f"cpu_count={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}, {model}; "
            f"BLAS: {blas or 'none detected'}")
    return threads, desc


def _oracle_request_kv(w, ci, b):
    import numpy as np

    from oracle import eagle3_oracle as O
    n = w.commit_rows
    if ci.block_table is not None:
        L = int(ci.ctx_len[b])
        return (O.gather_paged(ci.kv_k.f32(), ci.block_table[b], L + n, w.block_size).astype(np.float64),
                O.gather_paged(ci.kv_v.f32(), ci.block_table[b], L + n, w.block_size).astype(np.float64))
    return ci.kv_k.f32()[b].astype(np.float64), ci.kv_v.f32()[b].astype(np.float64)


def cpu_baseline(w, Wt, ci, vin, reqs=None, head=None):
    """The oracle as it stands, on the host cores: full cycles (fusion,
    commit, D-1 tree rounds, rerank and verification) of the requests
    `reqs` (default: all), scaled to whole-batch cycles per second.  vin =
    (target logits [B, m+1, V], mode, temperature, u_try, u_res) of the
    GPU's timed loop; the oracle verifies its own tree on them."""
    from oracle import eagle3_oracle as O
    W = {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}
    threads, desc = _host_info()
    L, mode, T, ut, ur = vin
    if head is not None:
        head = dict(A=head["A"].f32(), B=head["B"].f32(), c=head["c"])
    reqs = list(range(w.batch)) if reqs is None else list(reqs)
    n = w.commit_rows
    t0 = time.time()
    for b in reqs:
        Kc, Vc = _oracle_request_kv(w, ci, b)
        vt = O.draft_cycle(w.shape, W, ci.feats.f32()[b * n:(b + 1) * n], ci.tokens[b], Kc, Vc, int(ci.ctx_len[b]),
                           w.topk, w.depth, w.keep, head=head)
        if mode == "sample":
            O.verify_sample(vt["tok"], vt["parent"], L[b], ut[b], ur[b], T)
        else:
            O.verify_greedy(vt["tok"], vt["parent"], L[b])
    dt = time.time() - t0
    per_cycle = dt * w.batch / len(reqs)
    what = ("request 0" if w.batch == 1 else
            f"requests {reqs} of {w.batch}, scaled by {w.batch}/{len(reqs)} (extrapolated)")
    hd = " through the efficient LM head" if head is not None else ""
    return {"value": 1.0 / per_cycle, "unit": "draft-tree steps/s", "cores": threads, "kind": "oracle",
            "sample": f"full cycle(s) (fuse + commit + {w.depth - 1} tree rounds{hd} + rerank + {mode} verify) of "
                      f"{what}, fp64 NumPy, {dt:.1f} s; {desc}"}


def cpu_baseline_ttt(w, Wt, ti, positions=(700, 2047)):
    """The oracle's TTT forward on a bounded slice: sequence 0, the rollout
    rows (j, i) of a few positions i (all R steps each; the step-1 keys of
    every earlier position are computed too), timed on the host cores and
    scaled to rows per second and to one whole forward (extrapolated)."""
    from oracle import eagle3_oracle as O
    W = {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}
    threads, desc = _host_info()
    R, B, S = w.ttt_steps, w.batch, w.ttt_seq
    t0 = time.time()
    O.ttt_forward(w.shape, W, ti.feats.f32()[0], ti.tokens[0], R, positions=list(positions))
    dt = time.time() - t0
    rows = len(positions) * R
    rate = rows / dt
    return {"value": rate, "unit": "TTT rollout rows/s", "cores": threads, "kind": "oracle",
            "extrapolated_ms_per_forward": round(B * S * R / rate * 1e3, 1),
            "sample": f"sequence 0, positions {list(positions)} x {R} steps = {rows} rollout rows (plus the step-1 "
                      f"keys of positions <= {max(positions)}), fp64 NumPy, {dt:.1f} s; the per-forward time scales "
                      f"this to {B} x {S} x {R} rows (extrapolated); {desc}"}


def reporting_fields(w, ci=None):
    """Quantities the pages ask a drafter evaluation to report: target-feature
    bytes read per cycle (or per TTT forward) and the drafter's device
    memory (weights, KV)."""
    s = w.shape
    es = 2 if s.dtype == "bf16" else 4
    d, F, V = s.d, s.ffn, s.vocab
    weights = (d * 3 * d + V * d + (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim * 2 * d
               + d * s.n_q_heads * s.head_dim + 2 * F * d + d * F + V * d) * es
    if w.ttt_seq:
        return {"target_feature_bytes_per_forward": w.batch * w.ttt_seq * 3 * d * es, "draft_weight_bytes": weights}
    kv_rows = int(ci.kv_k.raw.size // (s.n_kv_heads * s.head_dim)) if ci is not None else 0
    return {"target_feature_bytes_per_cycle": w.batch * w.commit_rows * 3 * d * es,
            "draft_weight_bytes": weights,
            "draft_kv_bytes": 2 * kv_rows * s.n_kv_heads * s.head_dim * es
                              + 2 * w.batch * 64 * s.n_kv_heads * s.head_dim * es}


def make_drafter(w, Wt=None):
    """Packed device drafter of workload w; with an efficient head the LM head
    is drawn with its low-rank part (gen_lowrank_head) and the factors are
    attached.  Returns (drafter, host weights, row-major LM head on the device
    or None)."""
    import torch

    from eagle_draft_tree_amd.cycle import Drafter
    from workloads import gen
    Wt = dict(Wt) if Wt is not None else gen.gen_weights(w.shape, seed=0)
    lm_rows = head = None
    if w.lowrank_rank:
        head = gen.gen_lowrank_head(w.shape, w.lowrank_rank, energy=w.lowrank_energy, seed=0)
        Wt["lm"] = head["lm"]
        lm_rows = head["lm"].torch("cuda")   # for the recall measurement only
    dr = Drafter(w.shape, Wt, pack=True)
    if w.lowrank_rank:
        dr.set_lowrank_head(head["a"], head["b"], w.lowrank_rank, w.lowrank_candidates)
        head = dict(A=head["a"], B=head["b"], c=w.lowrank_candidates)
    torch.cuda.synchronize()
    return dr, Wt, lm_rows, head


def lowrank_recall(w, dr, buf, lm_rows):
    """Recall of the efficient head on the cycle just run: for every drafted
    LM-head row, the share of the full head's exact top-k (float32 logits of
    torch's matmul on y = bf16(rms(h2) * gain), ties by lowest id) found
    among the GPU's candidates."""
    import torch
    s, k = w.shape, w.topk
    D = w.depth
    h = [buf.h_tree[:, 0]] + [buf.h_tree[:, 1 + r * k:1 + (r + 1) * k].reshape(-1, s.d) for r in range(D - 1)]
    cands = [buf.commit_cand[0][:, 0]] + [buf.round_cand[r][0].reshape(-1, w.lowrank_candidates)
                                         for r in range(D - 1)]
    hits = total = 0
    gain = dr.tensors["norm_out"]
    for hh, cc in zip(h, cands):
        y = torch.nn.functional.rms_norm(hh.float(), (s.d,), gain, eps=s.rms_eps).to(torch.bfloat16).float()
        logits = y @ lm_rows.float().t()
        top = torch.topk(logits, k, dim=1, sorted=True).indices
        for i in range(top.shape[0]):
            hits += len(set(top[i].tolist()) & set(cc[i].tolist()))
            total += k
    return hits / max(total, 1)


def cycle_bench(w, dr, steps, warmup, n_plant=8, graph=True, lm_rows=None):
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
    vin = (Ls[0].cpu().numpy(), w.verify_modes[0], w.temperature, ut, ur)
    for i in range(max(warmup - n_plant, 0)):
        cycle(Ls[i % n_plant])
    torch.cuda.synchronize()

    for c in KC.values():
        Bd.timing_enable(c, (D + 2) * (steps + 1))
    # the roofline kernels record their own start and end (the dispatch
    # timestamps a profiler reads); every other class is timed by events
    # around its launches
    Bd.timing_mode(KC["lm_head"], 0 if w.lowrank_rank else 1)
    Bd.timing_mode(KC["lr_scores"], 1)
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

    recall = None
    if w.lowrank_rank and lm_rows is not None:
        buf.keep_candidates(w.lowrank_candidates)
        cycle(Ls[0])
        torch.cuda.synchronize()
        recall = lowrank_recall(w, dr, buf, lm_rows)
        buf.commit_cand = buf.round_cand = None
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
    if w.lowrank_rank:
        # efficient head, stage 1 (the LM-head class): both low-rank factors, y,
        # z written and read, the scores and their tile pairs; stage 2 (the top-k
        # class) reads c rows of the full LM head per row
        rr, cc = w.lowrank_rank, w.lowrank_candidates
        lm_bytes = [V * rr * es + rr * d * es + r * d * es + 2 * r * rr * es + r * V * 4 + r * (V // 16) * 8
                    for r in rows]
        w_lm = V * rr * es + rr * d * es
        bytes_cycle = w_fc + D * (w_layer + kv_round) + sum(lm_bytes) + sum(rows) * cc * d * es
    bytes_steps = D * (w_layer + kv_round) + sum(lm_bytes)  # the D draft steps
    if w.lowrank_rank:
        bytes_steps += sum(rows) * w.lowrank_candidates * d * es
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
    # the dominant kernel (the LM head): bytes per launch over its HIP-event launch time
    kind = "rows_rx" if k == 1 and 16 < Bn <= 64 else "rows_gemm"
    res["roofline"] = {"bound": "hbm", "achieved": res["lm_head"]["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": res["lm_head"]["hbm_frac"], "traffic": load_traffic(w.name, kind),
                       "kernel": "LM head (" + ("register-weight GEMM, top-1 partials" if kind == "rows_rx"
                                                else "rows GEMM with tile statistics") + ")",
                       "scope": "dominant kernel only; the whole draft step is draft_step_roofline",
                       "bytes_per_launch": res["lm_head"]["bytes_per_launch"],
                       "avg_launch_us": res["lm_head"]["avg_launch_us"]}
    res["reporting"] = reporting_fields(w, ci)
    if w.lowrank_rank:
        res["efficient_head"] = {"rank": w.lowrank_rank, "candidates": w.lowrank_candidates,
                                 "lm_head_energy_in_rank": w.lowrank_energy,
                                 "recall_at_k": round(recall, 4) if recall is not None else None,
                                 "note": "LM-head class = both low-rank GEMMs + candidate selection; the exact "
                                         "candidate logits and their top-k are in the top-k class"}
        # the efficient head's own kernel: the low-rank scores (the factor A, y's
        # projection z and the scores with their tile maxima) per launch
        sc_ms, sc_cnt = per_class["lr_scores"]
        nt16 = V // 16
        sc_bytes = [V * rr * es + r * rr * es + r * V * 4 + r * (nt16 + 16) * 8 for r in rows]
        sc_gbs = sum(sc_bytes) * (sc_cnt // len(rows)) / (sc_ms * 1e-3) / 1e9 if sc_ms > 0 else None
        res["roofline"] = {"bound": "hbm", "achieved": round(sc_gbs, 1) if sc_gbs else None, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(sc_gbs / HBM_PEAK_GBS, 4) if sc_gbs else None,
                           "traffic": load_traffic(w.name, "lr_scores"),
                           "kernel": "efficient LM head, low-rank scores (stage 1)",
                           "scope": "the efficient head's streaming kernel; the whole draft step is draft_step_roofline",
                           "bytes_per_launch": round(sum(sc_bytes) / len(sc_bytes)),
                           "avg_launch_us": round(sc_ms / sc_cnt * 1e3, 2) if sc_cnt else None}
    if graph:
        res["cycle_ms_percentiles"] = cycle_pct
        gbs = bytes_steps / (ms_steps * 1e-3) / 1e9
        res["draft_step_roofline"] = {"steps": D, "bytes_per_step": round(bytes_steps / D),
                                      "us_per_step": round(ms_steps * 1e3 / D, 2), "achieved_GBs": round(gbs, 1),
                                      "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return res, ci, vin


def device_info():
    """The GPU the numbers were taken on: name, architecture, compute units."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count}


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
    Bd.timing_mode(KC_TTT["ttt_ce"], 1)  # the CE GEMM's own start and end
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
                     "frac": round(lm_tf / MFMA_BF16_PEAK_TFLOPS, 4) if lm_tf else None,
                     "traffic": load_traffic(w.name, "ttt_ce"),
                     "kernel": "LM-head GEMM with CE epilogue", "flops_per_launch": f_lm / R,
                     "avg_launch_us": round(lm_launch_us, 1) if lm_launch_us else None},
        "flops_per_forward": f_gemm + f_lm + f_attn,
        "reporting": reporting_fields(w),
        "class_TFLOPs": {"projection_gemms": round(tf(f_gemm, "ttt_gemm"), 1),
                         "lm_head_ce": round(lm_tf, 1), "attention": round(tf(f_attn, "ttt_attn"), 1)},
        "kernel_ms_per_step": {kk: round(v[0] / steps, 3) for kk, v in per_class.items()},
    }, ti


def ttt_flops(w):
    """Algorithmic flops of one TTT forward: (projection GEMMs, LM head, attention)."""
    s = w.shape
    B, S, R = w.batch, w.ttt_seq, w.ttt_steps
    M = B * S
    d, F, V, hq, hkv, hd = s.d, s.ffn, s.vocab, s.n_q_heads, s.n_kv_heads, s.head_dim
    qd, kvd = hq * hd, hkv * hd
    f_fc = 2.0 * M * d * 3 * d
    f_layer = R * (2.0 * M * 2 * d * (qd + 2 * kvd) + 2.0 * M * qd * d + 2.0 * M * d * 2 * F + 2.0 * M * F * d)
    f_lm = R * 2.0 * M * d * V
    keys = B * S * (S + 1) / 2.0
    f_attn = sum(4.0 * (keys + M * (j - 1)) * hq * hd for j in range(1, R + 1))
    return f_fc, f_layer, f_lm, f_attn


def ttt_train_bench(w, dr, steps, warmup):
    """Time one TTT training step: the forward keeping every step's
    activations plus the backward to every trained parameter's gradient
    (eagle3_ttt_train), B x S tokens, R rollout steps."""
    import torch

    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.train import TTTTrain
    from workloads import gen

    s = w.shape
    B, S, R = w.batch, w.ttt_seq, w.ttt_steps
    ti = gen.gen_ttt_inputs(s, B, S, R, seed=1)
    feats = ti.feats.torch("cuda")
    tokens = torch.as_tensor(ti.tokens).cuda()
    tr = TTTTrain(dr, B, S, R)

    def run():
        tr.run(feats, tokens)

    for _ in range(max(warmup, 1)):
        run()
    torch.cuda.synchronize()
    for c in KC_TTT_TRAIN.values():
        Bd.timing_enable(c, 256 * (steps + 1))
    # principal kernels: the dy GEMM (dlogits . W_lm) and the weight-gradient GEMMs
    Bd.timing_mode(KC_TTT_TRAIN["ttt_bwd_gemm"], 1)
    Bd.timing_mode(KC_TTT_TRAIN["ttt_wgrad"], 1)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    per_class = {}
    for name, c in KC_TTT_TRAIN.items():
        per_class[name] = Bd.timing_read(c)
        Bd.timing_enable(c, 0)
        Bd.timing_mode(c, 0)
    M = B * S
    f_fc, f_layer, f_lm, f_attn = ttt_flops(w)
    f_fwd = f_fc + f_layer + f_lm + f_attn
    # backward: dy (LM head, no weight gradient), the layer GEMMs' data and
    # weight gradients (2 x forward), dW_fc, attention (dP, dQ, dK, dV: 2 x forward)
    f_bwd = f_lm + 2 * f_layer + f_fc + 2 * f_attn
    dy_launches = per_class["ttt_bwd_gemm"][1]
    dy_ms = per_class["ttt_bwd_gemm"][0] / steps
    dy_tf = f_lm / (dy_ms * 1e-3) / 1e12 if dy_ms > 0 else None
    wg_ms = per_class["ttt_wgrad"][0] / steps
    f_wgrad = f_layer + f_fc
    return {
        "workload": w.name + "-train",
        "steps": steps,
        "ms_per_step": round(ms, 3),
        "tokens_per_s": round(M / (ms * 1e-3), 1),
        "rows_per_s": round(M * R / (ms * 1e-3), 1),
        "loss": round(float(tr.loss.item()), 4),
        "TFLOPs": round((f_fwd + f_bwd) / (ms * 1e-3) / 1e12, 1),
        "mfma_frac": round((f_fwd + f_bwd) / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(dy_tf, 1) if dy_tf else None,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dy_tf / MFMA_BF16_PEAK_TFLOPS, 4) if dy_tf else None,
                     "traffic": load_traffic(w.name + "-train", "ttt_dy"),
                     "kernel": "dy GEMM (dlogits . W_lm, the LM head's backward)",
                     "flops_per_launch": f_lm / R,
                     "avg_launch_us": round(per_class["ttt_bwd_gemm"][0] / dy_launches * 1e3, 1)
                     if dy_launches else None},
        "wgrad_TFLOPs": round(f_wgrad / (wg_ms * 1e-3) / 1e12, 1) if wg_ms > 0 else None,
        "flops_per_step": {"forward": f_fwd, "backward": f_bwd},
        "workspace_GB": round(tr.ws.numel() / 1e9, 2),
        "kernel_ms_per_step": {kk: round(v[0] / steps, 3) for kk, v in per_class.items()},
        "timing_note": "kernel_ms_per_step: ttt_bwd_gemm and ttt_wgrad are their principal kernels' own "
                       "durations (dy GEMM; the five weight-gradient GEMMs), the other classes event pairs "
                       "around their launch scopes",
    }, ti


def cpu_baseline_ttt_train(w, Wt, ti, S_sample=128):
    """The gradient oracle (fp64 autograd over the TTT forward) on a bounded
    slice: the first S_sample tokens of sequence 0, all R steps, forward and
    backward, timed on the host cores and scaled to rows per second and to
    one whole training step (extrapolated)."""
    import torch

    from oracle import ttt_grad as G
    W = {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}
    threads, desc = _host_info()
    R, B, S = w.ttt_steps, w.batch, w.ttt_seq
    feats = ti.feats.f32()[:1, :S_sample]
    toks = ti.tokens[:1, :S_sample]
    t0 = time.time()
    G.ttt_loss_and_grads(w.shape, W, feats, toks, R)
    dt = time.time() - t0
    rows = S_sample * R
    rate = rows / dt
    return {"value": rate, "unit": "TTT rollout rows/s (forward + backward)", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "extrapolated_ms_per_step": round(B * S * R / rate * 1e3, 1),
            "sample": f"sequence 0, tokens 0..{S_sample - 1} x {R} steps = {rows} rollout rows, loss and the "
                      f"gradients of every trained parameter, fp64 PyTorch autograd, {dt:.1f} s (includes the "
                      f"weights' fp64 copies); the per-step time scales this to {B} x {S} x {R} rows "
                      f"(extrapolated; attention grows with S, so this understates the oracle's cost); {desc}"}


def target_bench(w, Wt, steps, warmup):
    """Time the target's verification step of workload w: the forward of
    all target layers over the B x (m+1) verify rows (root + kept nodes)
    with float32 logits and the three features, then verification of those
    logits (w.verify_modes[0]) and the KV commit of the accepted rows
    (lengths left unchanged, so every step sees the same inputs).  Target
    layers and prefix keys/values are drawn on the GPU (torch's seeded
    generator); embedding and LM head are the drafter's (Wt).  Returns the
    measurement dict and what the CPU baseline needs."""
    import numpy as np
    import torch

    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.target import TargetCache, TargetWeights, VerifyForward
    from workloads import gen

    s, tm = w.shape, w.target
    L, Bn, m = tm.n_layers, w.batch, w.keep
    rows = m + 1
    ti = gen.gen_target_inputs(w, L, layers=[], seed=1)
    t0 = time.time()
    layers = gen.target_weights_cuda(s, L, seed=0)
    tw = TargetWeights(s, layers, Wt["emb"], Wt["lm"], np.ones(s.d, np.float32), tm.feat_layers, pack=True)
    del layers
    i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    if w.paged:
        k, v = gen.target_kv_cuda(s, L, (ti.n_blocks, w.block_size), seed=0)
        cache = TargetCache(s, L, Bn, 0, torch.bfloat16, paged=True, block_size=w.block_size,
                            block_table=torch.as_tensor(ti.block_table), k=k, v=v)
    else:
        k, v = gen.target_kv_cuda(s, L, (Bn, ti.cap), seed=0)
        cache = TargetCache(s, L, Bn, ti.cap, torch.bfloat16, k=k, v=v)
    cache.ctx_len.copy_(torch.as_tensor(ti.ctx_len))
    vf = VerifyForward(tw, cache, rows)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    tokens, pos = i32(ti.v_tok), i32(ti.v_pos)
    anc = torch.as_tensor(ti.v_anc.view(np.int64)).cuda()
    v_par = i32(ti.v_parent)
    mode = Bd.SAMPLE if w.verify_modes[0] == "sample" else Bd.GREEDY
    ut, ur = gen.uniforms(1, Bn, rows)
    ut_d, ur_d = torch.as_tensor(ut).cuda(), torch.as_tensor(ur).cuda()
    Dmax = m
    acc_len = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    accepted = torch.zeros(Bn, Dmax, dtype=torch.int32, device="cuda")
    bonus = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    status = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    vws = torch.zeros(Bd.verify_workspace_size(Bn, m, s.vocab), dtype=torch.uint8, device="cuda")
    feats_next = torch.empty(Bn, Dmax + 1, 3, s.d, dtype=torch.bfloat16, device="cuda")

    def step():
        vf.run(tokens, pos, anc)
        Bd.eagle3_verify(Bn, m, s.vocab, Dmax, tokens, v_par, vf.logits, mode, w.temperature,
                         ut_d if mode == Bd.SAMPLE else None, ur_d if mode == Bd.SAMPLE else None, acc_len, accepted,
                         bonus, status, vws)
        vf.commit(acc_len, accepted, Dmax, feats_next=feats_next)

    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()
    assert int(status.max()) == 0
    kc_t = {"target": 15, "tgt_gate_up": 16, "tgt_lm_head": 17}
    for c in kc_t.values():
        Bd.timing_enable(c, L * (steps + 1))
    Bd.timing_mode(kc_t["tgt_gate_up"], 1)
    Bd.timing_mode(kc_t["tgt_lm_head"], 1)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    per = {name: Bd.timing_read(c) for name, c in kc_t.items()}
    for c in kc_t.values():
        Bd.timing_enable(c, 0)
    acc_mean = float(acc_len.float().mean())
    # algorithmic bytes (bf16 weights and activations, fp32 logits)
    es = 2
    d, F, V, hq, hkv, hd = s.d, s.ffn, s.vocab, s.n_q_heads, s.n_kv_heads, s.head_dim
    R = Bn * rows
    w_layer = ((hq + 2 * hkv) * hd * d + d * hq * hd + 2 * F * d + d * F) * es
    kv_read = int(np.sum(ti.ctx_len)) * hkv * hd * 2 * es
    fwd_bytes = L * (w_layer + kv_read + R * hkv * hd * 2 * es) + V * d * es + R * V * 4 + R * 3 * d * es
    gu_ms, gu_cnt = per["tgt_gate_up"]
    lm_ms, lm_cnt = per["tgt_lm_head"]
    fw_ms, fw_cnt = per["target"]
    chunks = -(-R // 64)
    # launches per layer (gate/up) and per forward (LM head): one over all row
    # chunks when the library launches them together, else one per chunk; a
    # launch streams the whole matrix and its own rows
    gu_lpl = max(1, round(gu_cnt / (fw_cnt * L))) if gu_cnt and fw_cnt else 1
    lm_lpf = max(1, round(lm_cnt / fw_cnt)) if lm_cnt and fw_cnt else 1
    gu_launch_bytes = 2 * F * d * es + (R * d * es + R * F * es) / gu_lpl
    lm_launch_bytes = V * d * es + (R * d * es + R * V * 4) / lm_lpf
    gu_us = gu_ms / gu_cnt * 1e3 if gu_cnt else None
    gu_gbs = gu_launch_bytes / (gu_us * 1e-6) / 1e9 if gu_us else None
    lm_gbs = lm_launch_bytes / (lm_ms / lm_cnt * 1e-3) / 1e9 if lm_cnt else None
    fw_ms_each = fw_ms / fw_cnt if fw_cnt else None
    res = {
        "workload": w.name,
        "target": {"n_layers": L, "feat_layers": list(tm.feat_layers), "weight_bytes": L * w_layer + 2 * V * d * es},
        "steps": steps,
        "ms_per_step": round(ms, 4),
        "verification_steps_per_s": round(1000.0 / ms, 2),
        "verify_rows_per_s": round(R * 1000.0 / ms, 1),
        "forward_ms": round(fw_ms_each, 4) if fw_ms_each else None,
        "accepted_mean": round(acc_mean, 3),
        "verify": w.verify_modes[0],
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 1) if gu_gbs else None, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4) if gu_gbs else None,
                     "traffic": load_traffic(w.name, "target_gate_up"),
                     "kernel": "target gate/up GEMM with the SwiGLU epilogue ("
                               + (f"{gu_lpl} launches per layer, one per 64-row chunk)" if gu_lpl > 1 else
                                  f"one launch per layer over {chunks} row chunks)" if chunks > 1 else
                                  "one launch per layer)"),
                     "scope": "dominant kernel only; the whole forward is forward_roofline",
                     "bytes_per_launch": round(gu_launch_bytes), "avg_launch_us": round(gu_us, 2) if gu_us else None},
        "forward_roofline": {"bytes": fwd_bytes,
                             "achieved_GBs": round(fwd_bytes / (fw_ms_each * 1e-3) / 1e9, 1) if fw_ms_each else None,
                             "frac": round(fwd_bytes / (fw_ms_each * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                             if fw_ms_each else None},
        "lm_head": {"GBs": round(lm_gbs, 1) if lm_gbs else None,
                    "frac": round(lm_gbs / HBM_PEAK_GBS, 4) if lm_gbs else None,
                    "avg_launch_us": round(lm_ms / lm_cnt * 1e3, 2) if lm_cnt else None},
        "note": "random target weights: the kept nodes are random tokens, so acceptance is ~0 and the verify and "
                "commit do minimal work; the forward's cost does not depend on the weights' values",
        "setup_s": round(setup_s, 1),
    }
    del vf, cache, tw
    torch.cuda.empty_cache()
    return res, ti


def harness_bench(w, Wt, cycles, warmup, params=None):
    """The 8B tree under the EAGLE-4 Harness.  Warm-up (the rules' cost
    table): one TREE draft round of the drafter at 1..16 rows per request,
    and one verification step of the 8B target (32 layers, forward +
    greedy verify) at 2..64 rows, each timed with HIP events.  Then harness
    cycles (HarnessCycle: branch cap from the root's top-8, the depth rule
    before each round, the verify count from the pool), timed on the host
    clock around each cycle (the decisions read scores back, so a cycle is
    synchronous), next to plain cycles (k 10, 6 rounds, 60 nodes) on the
    same drafter.  Returns the measurement dict and the table."""
    import numpy as np
    import torch

    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.cycle import (CycleBuffers, CycleSpec, Drafter, HarnessCycle, HarnessParams, KVCache,
                                            run_cycle)
    from eagle_draft_tree_amd.target import TargetCache, TargetWeights, VerifyForward
    from workloads import gen

    s = w.shape
    params = params or HarnessParams(tau_depth=1.0, alpha=0.25, tau_verify=4.0, tau_branch=2.0)
    Wh = dict(Wt)
    Wh["norm_out"] = np.full(s.d, 5.0, np.float32)
    dr = Drafter(s, Wh, pack=True)
    ci = gen.gen_cycle_inputs(w, seed=1)
    i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    ctx = int(ci.ctx_len[0]) + 1
    # ---- warm-up: drafter rounds
    buf = CycleBuffers(dr, CycleSpec(1, 64, 16, 2, 16, ci.cap))
    tk = torch.zeros(1, Bd.MAX_TREE_SLOTS, s.n_kv_heads, s.head_dim, dtype=dr.torch_dtype, device="cuda")
    kv = KVCache(ci.kv_k.torch("cuda"), ci.kv_v.torch("cuda"), tk, torch.zeros_like(tk), i32(ci.ctx_len), cap=ci.cap)
    kvs = kv.struct(i32(ci.ctx_len + 1))
    toks = [1, 2, 4, 8, 16, 32, 64]   # rows per request, one grid for both tables
    # the rows' parent state (the root slot): N(0,1), so the timed rounds see
    # ordinary logits (an all-zero state would tie every logit)
    buf.h_tree.normal_(0.0, 1.0, generator=torch.Generator(device="cuda").manual_seed(11))
    draft_ms = []
    for n in toks:
        par = torch.zeros(1, n, dtype=torch.int32, device="cuda")
        tok = i32(np.arange(n)[None] + 100)
        pos = i32(np.full((1, n), ctx))
        anc = torch.as_tensor((np.uint64(1) << np.arange(n, dtype=np.uint64)).view(np.int64)[None]).cuda()
        ids = torch.empty(1, n, min(n, 16), dtype=torch.int32, device="cuda")
        lps = torch.empty(1, n, min(n, 16), dtype=torch.float32, device="cuda")
        call = lambda: Bd.eagle3_draft_step(dr.dims, dr.weights, kvs, Bd.TREE, 1, n, None, par, tok, pos, anc, 0,
                                            min(n, 16), Bd.TOPK_ALL, buf.h_tree, ids, lps, None, buf.ws)
        for _ in range(3):
            call()
        a, b = ev(), ev()
        a.record()
        for _ in range(20):
            call()
        b.record()
        torch.cuda.synchronize()
        draft_ms.append(a.elapsed_time(b) / 20)
    # ---- warm-up: target verification steps
    tm = w.target
    L = tm.n_layers
    layers = gen.target_weights_cuda(s, L, seed=0)
    tw = TargetWeights(s, layers, Wt["emb"], Wt["lm"], np.ones(s.d, np.float32), tm.feat_layers, pack=True)
    del layers
    cap = ctx + 64
    k_, v_ = gen.target_kv_cuda(s, L, (1, cap), seed=0)
    cache = TargetCache(s, L, 1, cap, torch.bfloat16, k=k_, v=v_)
    cache.ctx_len.fill_(ctx - 1)
    verify_ms = []
    for n in toks:
        vf = VerifyForward(tw, cache, n)
        par = np.arange(-1, n - 1, dtype=np.int32)[None]
        tok, pos = i32(np.arange(n)[None] + 7), i32(ctx - 1 + np.arange(n)[None])
        anc = torch.as_tensor(gen.ancestor_bits(par[0]).view(np.int64)[None]).cuda()
        vpar = i32(par)
        al, acc = torch.zeros(1, dtype=torch.int32, device="cuda"), torch.zeros(1, n, dtype=torch.int32, device="cuda")
        bo, stt = torch.zeros(1, dtype=torch.int32, device="cuda"), torch.zeros(1, dtype=torch.int32, device="cuda")
        vws = torch.zeros(Bd.verify_workspace_size(1, n - 1, s.vocab), dtype=torch.uint8, device="cuda")

        def vstep():
            vf.run(tok, pos, anc)
            Bd.eagle3_verify(1, n - 1, s.vocab, n, tok, vpar, vf.logits, Bd.GREEDY, 1.0, None, None, al, acc, bo, stt,
                             vws)
        for _ in range(2):
            vstep()
        a, b = ev(), ev()
        a.record()
        for _ in range(5):
            vstep()
        b.record()
        torch.cuda.synchronize()
        verify_ms.append(a.elapsed_time(b) / 5)
        del vf
    del tw, cache
    torch.cuda.empty_cache()
    table = Bd.HarnessTable([1], [ctx], toks, [[draft_ms]], [[verify_ms]])
    # ---- harness cycles and plain cycles on the same drafter and inputs
    hc = HarnessCycle(dr, 1, 1, w.depth, w.keep, ci.cap, table, params)
    x = dict(kv=kv, feats=ci.feats.torch("cuda"), tokens=i32(ci.tokens), commit_pos=i32(ci.ctx_len[:, None]),
             ctx_after=i32(ci.ctx_len + 1), root_tok=i32(ci.tokens[:, -1]), root_pos=i32(ci.ctx_len))
    for _ in range(warmup):
        hc.run(x["kv"], x["feats"], x["tokens"], x["commit_pos"], x["ctx_after"], x["root_tok"], x["root_pos"], ctx)
    torch.cuda.synchronize()
    t_h, decs = [], []
    for _ in range(cycles):
        t0 = time.perf_counter()
        decs.append(dict(hc.run(x["kv"], x["feats"], x["tokens"], x["commit_pos"], x["ctx_after"], x["root_tok"],
                                x["root_pos"], ctx)))
        torch.cuda.synchronize()
        t_h.append((time.perf_counter() - t0) * 1e3)
    d0 = decs[-1]
    pool = hc.pool[: min(w.keep, d0["k"] + (d0["rounds"] - 1) * d0["k"] ** 2)].cpu().numpy()
    exp_tokens = float(np.exp(pool[: d0["m"]].astype(np.float64)).sum())
    pbuf = CycleBuffers(dr, CycleSpec(1, 1, w.topk, w.depth, w.keep, ci.cap))
    for _ in range(warmup):
        run_cycle(dr, pbuf, kv, x["feats"], x["tokens"], x["commit_pos"], x["ctx_after"], x["root_tok"],
                  x["root_pos"], verify=False)
    torch.cuda.synchronize()
    t_p = []
    for _ in range(cycles):
        t0 = time.perf_counter()
        run_cycle(dr, pbuf, kv, x["feats"], x["tokens"], x["commit_pos"], x["ctx_after"], x["root_tok"],
                  x["root_pos"], verify=False)
        torch.cuda.synchronize()
        t_p.append((time.perf_counter() - t0) * 1e3)
    vt = lambda m: Bd.harness_cost(table, Bd.COST_VERIFY, 1, ctx, m + 1)
    med = lambda a: float(np.median(a))
    res = {
        "workload": w.name,
        "params": dict(tau_depth=params.tau_depth, alpha=params.alpha, tau_verify=params.tau_verify,
                       tau_branch=params.tau_branch),
        "warmup_table": {"rows_per_request": toks, "draft_round_ms": [round(v, 4) for v in draft_ms],
                         "verification_step_ms": [round(v, 4) for v in verify_ms]},
        "decisions": d0,
        "decisions_constant": all(dd == d0 for dd in decs),
        "harness_cycle_ms_median": round(med(t_h), 4),
        "plain_cycle_ms_median": round(med(t_p), 4),
        "verify_ms_at_m_from_table": round(vt(d0["m"]), 4),
        "plain_verify_ms_from_table": round(vt(w.keep), 4),
        "expected_accepted_tokens_verified": round(exp_tokens, 3),
        "note": "host-clock time per cycle including the decisions' read-backs (harness) / eager launches (plain), "
                "drafting only; verification times are the warm-up table's at the verified row counts",
    }
    return res, table


def cpu_baseline_harness(w, Wt, table, params, ci=None):
    """The oracle's harness_cycle (the same rules and table, fp64 NumPy
    decoder) for request 0, timed on the host cores."""
    import numpy as np

    from oracle import eagle3_oracle as O
    from workloads import gen
    threads, desc = _host_info()
    W = {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}
    W["norm_out"] = np.full(w.shape.d, 5.0)
    ci = ci or gen.gen_cycle_inputs(w, seed=1)
    t0 = time.time()
    _, info = O.harness_cycle(w.shape, W, ci.feats.f32()[:1], ci.tokens[0], ci.kv_k.f32()[0].astype(np.float64),
                              ci.kv_v.f32()[0].astype(np.float64), int(ci.ctx_len[0]), table.as_dict(), w.keep,
                              w.depth, params["tau_depth"], params["alpha"], params["tau_verify"],
                              params["tau_branch"])
    dt = time.time() - t0
    return {"value": 1.0 / dt, "unit": "harness cycles/s", "cores": threads, "kind": "oracle",
            "decisions": info,
            "sample": f"one harness cycle of request 0 (fuse + commit + {info['rounds'] - 1} tree rounds + rules + "
                      f"rerank), fp64 NumPy, {dt:.1f} s; {desc}"}


def cpu_baseline_target(w, Wt, ti):
    """The oracle's verification forward on a bounded sample: request 0's
    m+1 verify rows through one target layer (host-drawn weights of the
    same shapes) plus the final norm and LM head, timed on the host cores;
    the forward time scales the layer time by the layer count
    (extrapolated)."""
    import numpy as np

    from oracle import eagle3_oracle as O
    from workloads import gen
    s, tm = w.shape, w.target
    threads, desc = _host_info()
    T1 = gen.gen_target_weights(s, 2, seed=0, layers=[0])
    T1["layers"] = [{k: (v.f32() if hasattr(v, "f32") else v) for k, v in T1["layers"][0].items()}] * 2
    T1["emb"], T1["lm"] = Wt["emb"].f32(), Wt["lm"].f32()
    rows = w.keep + 1
    cap = int(ti.ctx_len[0]) + rows
    rng = np.random.default_rng(0)
    Ks = [rng.standard_normal((cap + O.MAX_TREE_SLOTS, s.n_kv_heads, s.head_dim))] * 2
    Vs = [rng.standard_normal((cap + O.MAX_TREE_SLOTS, s.n_kv_heads, s.head_dim))] * 2
    t0 = time.time()
    h, _, _ = O.target_verify_forward(s, T1, ti.v_tok[0], ti.v_pos[0], ti.v_anc[0], Ks, Vs, int(ti.ctx_len[0]),
                                      (1, 1, 1), 0, 1)
    t_layer = time.time() - t0
    t0 = time.time()
    O.matmul_wt(O._rnd(s, O.rmsnorm(h, T1["norm_out"], s.rms_eps)), T1["lm"])
    t_lm = time.time() - t0
    per_fwd = (t_layer * tm.n_layers + t_lm) * w.batch
    return {"value": 1.0 / per_fwd, "unit": "verification forwards/s", "cores": threads, "kind": "oracle",
            "extrapolated_ms_per_forward": round(per_fwd * 1e3, 1),
            "sample": f"request 0's {rows} verify rows through 1 target layer ({t_layer:.1f} s) and the final norm + "
                      f"LM head ({t_lm:.1f} s), fp64 NumPy; one forward = {tm.n_layers} layers + LM head"
                      + (f", x {w.batch} requests" if w.batch > 1 else "") + f" (extrapolated); {desc}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["c2", "c3", "c4", "ttt", "tttb", "c2e", "c4e", "c2v", "c3v", "c4v", "c2n",
                                       "c2h"],
                    default=None,
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
    from workloads.configs import (C2_8B_TREE, C2E_8B_TREE_LOWRANK, C2H_8B_TREE_HARNESS, C2N_8B_TREE_NORMS,
                                   C2V_8B_TARGET_TREE, C3_8B_CHAIN, C3V_8B_TARGET_CHAIN, C4_70B_TREE,
                                   C4E_70B_TREE_LOWRANK, C4V_70B_TARGET_TREE, C5_8B_TTT)

    if args.only == "c2h":
        w = C2H_8B_TREE_HARNESS
        Wt = gen.gen_weights(w.shape, seed=0)
        r, table = harness_bench(w, Wt, max(3, min(args.steps, 30)), min(args.warmup, 3))
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline_harness(w, Wt, table, r["params"])
        print(json.dumps(r), flush=True)
        return
    if args.only == "c2n":
        w = C2N_8B_TREE_NORMS
        Wt = gen.gen_weights(w.shape, seed=0)
        Wt.update(gen.gen_norm_variant_gains(w.shape, True, True, seed=1))
        dr = Drafter(w.shape, Wt, pack=True)
        r, ci, vin = cycle_bench(w, dr, args.steps, args.warmup, graph=not args.no_graph)
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline(w, Wt, ci, vin)
        print(json.dumps(r), flush=True)
        return

    if args.only in ("c2v", "c3v", "c4v"):
        w = {"c2v": C2V_8B_TARGET_TREE, "c3v": C3V_8B_TARGET_CHAIN, "c4v": C4V_70B_TARGET_TREE}[args.only]
        Wt = gen.gen_weights(w.shape, seed=0, only=("emb", "lm"))
        r, ti = target_bench(w, Wt, max(1, min(args.steps, 20)), min(args.warmup, 3))
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline_target(w, Wt, ti)
        print(json.dumps(r), flush=True)
        return

    Bd.load()
    t0 = time.time()
    s8 = C2_8B_TREE.shape
    Wt8 = gen.gen_weights(s8, seed=0) if args.only not in ("c4", "c4e") else None
    dr8 = Drafter(s8, Wt8, pack=True) if Wt8 is not None and args.only not in ("c2e",) else None
    setup_s = time.time() - t0
    if args.only in ("c2e", "c4e"):
        w = C2E_8B_TREE_LOWRANK if args.only == "c2e" else C4E_70B_TREE_LOWRANK
        dr, Wt, lm_rows, head = make_drafter(w, Wt8)
        r, ci, vin = cycle_bench(w, dr, args.steps, args.warmup, graph=not args.no_graph, lm_rows=lm_rows)
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline(w, Wt, ci, vin, None, head)
        print(json.dumps(r), flush=True)
        return

    # sampled requests of the batch-64 chain for its CPU baseline (the oracle
    # drafts one request at a time)
    c3_reqs = (0, 21, 42, 63)
    if args.only == "ttt":
        r, ti = ttt_bench(C5_8B_TTT, dr8, max(1, min(args.steps, 10)), 1)
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline_ttt(C5_8B_TTT, Wt8, ti)
        r["device"] = device_info()
        print(json.dumps(r), flush=True)
        return
    if args.only == "tttb":
        r, ti = ttt_train_bench(C5_8B_TTT, dr8, max(1, min(args.steps, 5)), 1)
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline_ttt_train(C5_8B_TTT, Wt8, ti)
        print(json.dumps(r), flush=True)
        return
    if args.only == "c2":
        args.main_only = True
    if args.only in ("c3", "c4"):
        w = C3_8B_CHAIN if args.only == "c3" else C4_70B_TREE
        Wt = Wt8 if args.only == "c3" else gen.gen_weights(w.shape, seed=0)
        dr = dr8 if args.only == "c3" else Drafter(w.shape, Wt, pack=True)
        r, ci, vin = cycle_bench(w, dr, args.steps, args.warmup, graph=not args.no_graph)
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline(w, Wt, ci, vin, c3_reqs if args.only == "c3" else None)
        print(json.dumps(r), flush=True)
        return

    w = C2_8B_TREE
    r, ci, vin = cycle_bench(w, dr8, args.steps, args.warmup, graph=not args.no_graph)
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
        "roofline": r["roofline"],
        "cycle_ms_percentiles": r.get("cycle_ms_percentiles"),
        "cycle_roofline": r["cycle_roofline"],
        "draft_step_roofline": r.get("draft_step_roofline"),
        "kernel_ms_per_cycle": r["kernel_ms_per_cycle"],
        "reporting": r["reporting"],
        "setup_s": round(setup_s, 1),
        "device": device_info(),
    }
    # the GPU legs first, then every CPU baseline (host work only)
    cpu_jobs = [("main", w, Wt8, ci, vin, None, None)]
    if not args.main_only:
        wl = {}
        r3, ci3, vin3 = cycle_bench(C3_8B_CHAIN, dr8, max(args.steps // 2, 1), args.warmup, graph=not args.no_graph)
        wl[C3_8B_CHAIN.name] = r3
        cpu_jobs.append((C3_8B_CHAIN.name, C3_8B_CHAIN, Wt8, ci3, vin3, c3_reqs, None))
        r5, ti = ttt_bench(C5_8B_TTT, dr8, 5, 1)
        wl[C5_8B_TTT.name] = r5
        cpu_jobs.append((C5_8B_TTT.name, C5_8B_TTT, Wt8, ti, None, None, None))
        r5t, ti5t = ttt_train_bench(C5_8B_TTT, dr8, 3, 1)
        wl[r5t["workload"]] = r5t
        cpu_jobs.append((r5t["workload"], C5_8B_TTT, Wt8, ti5t, None, "train", None))
        torch.cuda.empty_cache()
        del dr8
        torch.cuda.empty_cache()
        # the 8B tree through the efficient LM head (same drafter, structured LM head)
        w2e = C2E_8B_TREE_LOWRANK
        dr2e, Wt2e, lm_rows, head2e = make_drafter(w2e, Wt8)
        r2e, ci2e, vin2e = cycle_bench(w2e, dr2e, args.steps, args.warmup, graph=not args.no_graph, lm_rows=lm_rows)
        wl[w2e.name] = r2e
        cpu_jobs.append((w2e.name, w2e, Wt2e, ci2e, vin2e, None, head2e))
        del dr2e, lm_rows
        torch.cuda.empty_cache()
        Wt70 = gen.gen_weights(C4_70B_TREE.shape, seed=0)
        dr70 = Drafter(C4_70B_TREE.shape, Wt70, pack=True)
        r4, ci4, vin4 = cycle_bench(C4_70B_TREE, dr70, max(args.steps // 3, 1), args.warmup, graph=not args.no_graph)
        wl[C4_70B_TREE.name] = r4
        cpu_jobs.append((C4_70B_TREE.name, C4_70B_TREE, Wt70, ci4, vin4, None, None))
        del dr70
        torch.cuda.empty_cache()
        w4e = C4E_70B_TREE_LOWRANK
        dr4e, Wt4e, lm_rows, head4e = make_drafter(w4e, Wt70)
        r4e, ci4e, vin4e = cycle_bench(w4e, dr4e, max(args.steps // 3, 1), args.warmup, graph=not args.no_graph,
                                       lm_rows=lm_rows)
        wl[w4e.name] = r4e
        cpu_jobs.append((w4e.name, w4e, Wt4e, ci4e, vin4e, None, head4e))
        del dr4e, lm_rows
        torch.cuda.empty_cache()
        # the target's verification step (forward over the verify rows + verify + KV commit)
        for wv, Wt in ((C2V_8B_TARGET_TREE, Wt8), (C3V_8B_TARGET_CHAIN, Wt8), (C4V_70B_TARGET_TREE, Wt70)):
            rv, tiv = target_bench(wv, Wt, max(args.steps // 5, 2), min(args.warmup, 3))
            wl[wv.name] = rv
            cpu_jobs.append((wv.name, wv, Wt, tiv, None, None, None))
        del Wt70
        # the EAGLE-3.1 norm variants on the 8B tree
        wn = C2N_8B_TREE_NORMS
        WtN = dict(Wt8)
        WtN.update(gen.gen_norm_variant_gains(wn.shape, True, True, seed=1))
        drn = Drafter(wn.shape, WtN, pack=True)
        rn, cin, vinn = cycle_bench(wn, drn, args.steps, args.warmup, graph=not args.no_graph)
        wl[wn.name] = rn
        cpu_jobs.append((wn.name, wn, WtN, cin, vinn, None, None))
        del drn
        torch.cuda.empty_cache()
        # the EAGLE-4 Harness on the 8B tree (warm-up table, then harness cycles)
        wh = C2H_8B_TREE_HARNESS
        rh, table_h = harness_bench(wh, Wt8, max(args.steps // 5, 3), min(args.warmup, 3))
        wl[wh.name] = rh
        cpu_jobs.append((wh.name, wh, Wt8, table_h, rh["params"], "harness", None))
        torch.cuda.empty_cache()
        out["workloads"] = wl
    if not args.no_cpu_baseline:
        for name, wk, Wt, inp, vi, reqs, hd in cpu_jobs:
            print(f"cpu baseline: {wk.name}", file=sys.stderr, flush=True)
            if reqs == "harness":
                cb = cpu_baseline_harness(wk, Wt, inp, vi)
            elif reqs == "train":
                cb = cpu_baseline_ttt_train(wk, Wt, inp)
            elif wk.target is not None:
                cb = cpu_baseline_target(wk, Wt, inp)
            elif wk.ttt_seq:
                cb = cpu_baseline_ttt(wk, Wt, inp)
            else:
                cb = cpu_baseline(wk, Wt, inp, vi, reqs, hd)
            if name == "main":
                out["cpu_baseline"] = cb
            else:
                out["workloads"][name]["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
