"""Seeded synthetic inputs for the EAGLE-3 draft-and-verify path.

This module only draws data: weights, target features, tokens, KV prefixes,
target logits and uniforms.  It holds none of the method's arithmetic; both
the CPU oracle and the GPU path consume what it returns.

RNG: every tensor comes from numpy's PCG64 seeded with
``SeedSequence([seed, tensor_id, chunk])``.  Large tensors are drawn in
2**24-element chunks (each with its own stream) so that generation can run on
several threads and still be reproducible bit for bit.  Normal draws are made
in float32, scaled by the standard deviation in float32, and for bf16
workloads rounded once (round-to-nearest-even) to bfloat16; the same bits go
to both sides.

Seed streams: weights 0; inputs 1..10; target logits 100+s; planting 200+s;
uniforms 300+s.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .configs import BF16, F32, DrafterShape, Workload

CHUNK = 1 << 24
_THREADS = max(1, min(16, os.cpu_count() or 1))

# tensor ids inside the weight stream
TID = dict(fc=1, emb=2, qkv=3, o=4, gate_up=5, down=6, lm=7)


def _rng(seed, tid, chunk=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def normal_f32(seed: int, tid: int, shape, std: float) -> np.ndarray:
    """N(0, std) float32 array, chunked and multi-threaded, reproducible."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nch = (n + CHUNK - 1) // CHUNK

    def fill(c):
        s = c * CHUNK
        e = min(n, s + CHUNK)
        _rng(seed, tid, c).standard_normal(e - s, dtype=np.float32, out=out[s:e])
        out[s:e] *= np.float32(std)

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nch)))
    return out.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    n = flat_u.size

    def conv(c):
        s = c * CHUNK
        e = min(n, s + CHUNK)
        x = flat_u[s:e]
        lsb = (x >> np.uint32(16)) & np.uint32(1)
        r = (x + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        flat_o[s:e] = r.astype(np.uint16)

    nch = (n + CHUNK - 1) // CHUNK
    if nch <= 1:
        if n:
            conv(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(conv, range(nch)))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A generated tensor: ``raw`` is what the GPU receives (float32 or bf16
    bits as uint16); ``f32`` gives the exact values as float32."""
    raw: np.ndarray
    dtype: str

    @property
    def shape(self):
        return self.raw.shape

    def f32(self) -> np.ndarray:
        if self.dtype == BF16:
            return bf16_bits_to_f32(self.raw)
        return self.raw

    def torch(self, device="cpu"):
        import torch
        if self.dtype == BF16:
            t = torch.from_numpy(self.raw.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(self.raw)
        return t.to(device)


def draw(seed, tid, shape, std, dtype) -> Tensor:
    x = normal_f32(seed, tid, shape, std)
    if dtype == BF16:
        return Tensor(f32_to_bf16_bits(x), BF16)
    return Tensor(x, F32)


def gen_weights(shape: DrafterShape, seed: int = 0, std: float = 0.02, only=None) -> dict:
    """All drafter matrices N(0, std) (layout [out, in]); RMSNorm gains are 1.

    fc [d,3d]; emb [V,d]; qkv [(Hq+2Hkv)hd, 2d]; o [d, Hq hd];
    gate_up [2F, d] (gate rows then up rows); down [d, F]; lm [V, d].
    """
    d, V, F = shape.d, shape.vocab, shape.ffn
    shapes = dict(fc=(d, 3 * d), emb=(V, d), qkv=(shape.qkv_rows, 2 * d),
                  o=(d, shape.n_q_heads * shape.head_dim), gate_up=(2 * F, d),
                  down=(d, F), lm=(V, d))
    W = {}
    for name, shp in shapes.items():
        if only is not None and name not in only:
            continue
        W[name] = draw(seed, TID[name], shp, std, shape.dtype)
    for g in ("norm_e", "norm_s", "norm_ffn", "norm_out"):
        W[g] = np.ones(d, dtype=np.float32)
    return W


def gen_target_weights(shape: DrafterShape, n_layers: int, seed: int = 0, std: float = 0.02,
                       layers=None, gains: str = "ones") -> dict:
    """A target model of `n_layers` decoder layers of the drafter's layer
    shape with a d-wide attention input: per layer qkv [(Hq+2Hkv)hd, d],
    o [d, Hq hd], gate_up [2F, d], down [d, F], N(0, std); emb and lm are the
    drafter's (same stream ids, so gen_weights(shape, seed) gives the same
    matrices).  `layers` limits which layers are drawn (others are None);
    gains "ones" or "random" (1 + 0.5 N(0,1), a distinct vector per norm)."""
    d, F = shape.d, shape.ffn
    shapes = dict(qkv=(shape.qkv_rows, d), o=(d, shape.n_q_heads * shape.head_dim), gate_up=(2 * F, d),
                  down=(d, F))
    g = _rng(seed, 49)
    gain = (lambda: np.ones(d, dtype=np.float32)) if gains == "ones" else \
        (lambda: (1.0 + 0.5 * g.standard_normal(d)).astype(np.float32))
    out = dict(layers=[])
    for l in range(n_layers):
        Lw = dict(norm_attn=gain(), norm_ffn=gain())
        if layers is None or l in layers:
            for j, (name, shp) in enumerate(shapes.items()):
                Lw[name] = draw(seed, 1000 + 8 * l + j, shp, std, shape.dtype)
        out["layers"].append(Lw)
    out["norm_out"] = gain()
    shared = gen_weights(shape, seed, std, only=("emb", "lm"))
    out["emb"], out["lm"] = shared["emb"], shared["lm"]
    return out


def target_weights_cuda(shape: DrafterShape, n_layers: int, seed: int = 0, std: float = 0.02):
    """Device-resident target layer matrices for throughput runs, drawn on
    the GPU with torch's seeded generator (the host generator would take
    minutes at 70B scale).  Same shapes and N(0, std) as gen_target_weights,
    bf16; not the same values.  Returns a list of per-layer dicts of torch
    tensors, gains on the device as float32 ones."""
    import torch
    d, F = shape.d, shape.ffn
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7919 * (seed + 1))
    shapes = dict(qkv=(shape.qkv_rows, d), o=(d, shape.n_q_heads * shape.head_dim), gate_up=(2 * F, d),
                  down=(d, F))
    layers = []
    for _ in range(n_layers):
        Lw = {}
        for name, shp in shapes.items():
            t = torch.empty(shp, dtype=torch.bfloat16, device="cuda")
            t.normal_(0.0, std, generator=gen)
            Lw[name] = t
        Lw["norm_attn"] = torch.ones(d, dtype=torch.float32, device="cuda")
        Lw["norm_ffn"] = torch.ones(d, dtype=torch.float32, device="cuda")
        layers.append(Lw)
    return layers


def target_kv_cuda(shape: DrafterShape, n_layers: int, rows_per_layer_shape, seed: int = 0):
    """Device-resident N(0,1) bf16 keys and values [n_layers, *rows_per_layer_shape,
    Hkv, hd] for throughput runs (torch's seeded generator)."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(104729 * (seed + 1))
    shp = (n_layers,) + tuple(rows_per_layer_shape) + (shape.n_kv_heads, shape.head_dim)
    k = torch.empty(shp, dtype=torch.bfloat16, device="cuda").normal_(0.0, 1.0, generator=gen)
    v = torch.empty(shp, dtype=torch.bfloat16, device="cuda").normal_(0.0, 1.0, generator=gen)
    return k, v


def gen_norm_variant_gains(shape: DrafterShape, fc_norm: bool, post_norm: bool, seed: int = 0) -> dict:
    """Gains of the EAGLE-3.1 norm variants, 1 + 0.5 N(0,1) each (a distinct
    vector per norm): norm_fc for the FC norm, norm_post_attn and
    norm_post_ffn for the post-norm."""
    g = _rng(seed, 48)
    out = {}
    for name, on in (("norm_fc", fc_norm), ("norm_post_attn", post_norm), ("norm_post_ffn", post_norm)):
        v = (1.0 + 0.5 * g.standard_normal(shape.d)).astype(np.float32)
        if on:
            out[name] = v
    return out


def gen_drafter_gains(shape: DrafterShape, seed: int = 0) -> dict:
    """Non-unit RMSNorm gains of the drafter, 1 + 0.5 N(0,1) each (a distinct
    vector per norm): norm_e, norm_s, norm_ffn, norm_out."""
    g = _rng(seed, 47)
    return {name: (1.0 + 0.5 * g.standard_normal(shape.d)).astype(np.float32)
            for name in ("norm_e", "norm_s", "norm_ffn", "norm_out")}


def gen_lowrank_head(shape: DrafterShape, rank: int, energy: float = 0.9, seed: int = 0,
                     std: float = 0.02) -> dict:
    """A synthetic LM head with a low-rank part, and that part's factors.

    W_lm = a (P Q) + b E with P [V, rank] ~ N(0,1), Q [rank, d] ~ N(0,1)/sqrt(rank)
    and E [V, d] ~ N(0,1), so every entry of P Q has unit variance; a^2 =
    energy * std^2 and b^2 = (1 - energy) * std^2 keep the entries' standard
    deviation at std while `energy` of it lies in the rank-`rank` part.  The
    low-rank head is A = a P [V, rank] and B = Q [rank, d].  Returns dict(lm=,
    a=, b=) as Tensors of the shape's dtype (each rounded once)."""
    V, d = shape.vocab, shape.d
    a = np.float32(std * math.sqrt(energy))
    b = np.float32(std * math.sqrt(1.0 - energy))
    P = normal_f32(seed, 41, (V, rank), 1.0)
    Q = normal_f32(seed, 42, (rank, d), 1.0 / math.sqrt(rank))
    lm = normal_f32(seed, 43, (V, d), 1.0)
    lm *= b
    step = 16384
    for s0 in range(0, V, step):      # lm += a * P Q, row block by row block (float32)
        lm[s0:s0 + step] += a * (P[s0:s0 + step] @ Q)
    P *= a
    if shape.dtype == BF16:
        return dict(lm=Tensor(f32_to_bf16_bits(lm), BF16), a=Tensor(f32_to_bf16_bits(P), BF16),
                    b=Tensor(f32_to_bf16_bits(Q), BF16))
    return dict(lm=Tensor(lm, F32), a=Tensor(P, F32), b=Tensor(Q, F32))


@dataclass
class CycleInputs:
    """Inputs of one draft-tree cycle (batch B)."""
    feats: Tensor                 # [B*commit_rows, 3, d]
    tokens: np.ndarray            # [B, commit_rows] int32 (the last is the root token)
    ctx_len: np.ndarray           # [B] committed rows before the COMMIT step
    kv_k: Tensor = None           # contiguous [B, cap, Hkv, hd] or paged pool [nb, bs, Hkv, hd]
    kv_v: Tensor = None
    cap: int = 0
    block_table: np.ndarray = None  # [B, max_blocks] int32 (paged only)
    accept_prob: np.ndarray = None  # [B] planted agreement per request


def gen_cycle_inputs(w: Workload, seed: int = 1) -> CycleInputs:
    s = w.shape
    B, n = w.batch, w.commit_rows
    hkv, hd = s.n_kv_heads, s.head_dim
    feats = draw(seed, 11, (B * n, 3, s.d), w.feat_scale, s.dtype)
    tokens = _rng(seed, 12).integers(0, s.vocab, size=(B, n)).astype(np.int32)
    if w.prefix_range is not None:
        lo, hi = w.prefix_range
        ctx = _rng(seed, 13).integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        ctx = np.full(B, w.prefix if w.synthetic_prefix_kv else 0, dtype=np.int32)
    ci = CycleInputs(feats=feats, tokens=tokens, ctx_len=ctx)
    if w.planted_accept_range is not None:
        lo, hi = w.planted_accept_range
        ci.accept_prob = _rng(seed, 14).uniform(lo, hi, size=B)
    elif w.planted_accept is not None:
        ci.accept_prob = np.full(B, w.planted_accept)
    if w.paged:
        bs = w.block_size
        need = [(int(L) + n + bs - 1) // bs for L in ctx]
        nb = int(sum(need))
        perm = _rng(seed, 15).permutation(nb).astype(np.int32)
        maxb = max(need)
        table = np.full((B, maxb), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            table[b, :need[b]] = perm[off:off + need[b]]
            off += need[b]
        ci.kv_k = draw(seed, 16, (nb, bs, hkv, hd), 1.0, s.dtype)
        ci.kv_v = draw(seed, 17, (nb, bs, hkv, hd), 1.0, s.dtype)
        ci.block_table = table
        ci.cap = maxb * bs
    else:
        cap = int(ctx.max()) + n
        ci.cap = cap
        if w.synthetic_prefix_kv:
            ci.kv_k = draw(seed, 16, (B, cap, hkv, hd), 1.0, s.dtype)
            ci.kv_v = draw(seed, 17, (B, cap, hkv, hd), 1.0, s.dtype)
        else:
            dt = np.float32 if s.dtype == F32 else np.uint16
            ci.kv_k = Tensor(np.zeros((B, cap, hkv, hd), dtype=dt), s.dtype)
            ci.kv_v = Tensor(np.zeros((B, cap, hkv, hd), dtype=dt), s.dtype)
    return ci


def target_logits(seed: int, B: int, rows: int, V: int, sigma: float) -> np.ndarray:
    """Synthetic target logits [B, rows, V] float32, N(0, sigma)."""
    return normal_f32(100 + seed, 1, (B, rows, V), sigma)


def plant_agreement(logits: np.ndarray, v_tok: np.ndarray, v_parent: np.ndarray,
                    accept_prob: np.ndarray, seed: int) -> np.ndarray:
    """Plant argmax agreement into target logits (in place; returns logits).

    For every verify-tree row that has at least one kept child: with
    probability a, the first child's token becomes the row's strict argmax
    (rowmax + 1); otherwise, if that token already is the argmax, it is
    pushed to rowmin - 1.  One uniform per row is drawn, in row order.
    """
    B, R, _ = logits.shape
    u = _rng(200 + seed, 1).random((B, R))
    for b in range(B):
        first_child = {}
        for c in range(1, R):
            p = int(v_parent[b, c])
            if p >= 0 and p not in first_child:
                first_child[p] = c
        for r in range(R):
            if r not in first_child:
                continue
            tok = int(v_tok[b, first_child[r]])
            row = logits[b, r]
            if u[b, r] < accept_prob[b]:
                row[tok] = row.max() + np.float32(1.0)
            elif int(np.argmax(row)) == tok:
                row[tok] = row.min() - np.float32(1.0)
    return logits


def uniforms(seed: int, B: int, rows: int):
    """Verification uniforms: (u_try, u_res), each [B, rows] float64 in [0, 1)."""
    g = _rng(300 + seed, 1)
    return g.random((B, rows)), g.random((B, rows))


# --------------------------------------------------------------------------- TTT
@dataclass
class TTTInputs:
    feats: Tensor        # [B, S, 3, d]
    tokens: np.ndarray   # [B, S] int32
    forced: np.ndarray   # [B, R-1, S] int32 (tokens fed at steps 2..R in forced mode)


def gen_ttt_inputs(shape: DrafterShape, B: int, S: int, R: int, seed: int = 1,
                   feat_std: float = 1.0) -> TTTInputs:
    feats = draw(seed, 21, (B, S, 3, shape.d), feat_std, shape.dtype)
    tokens = _rng(seed, 22).integers(0, shape.vocab, size=(B, S)).astype(np.int32)
    forced = _rng(seed, 23).integers(0, shape.vocab, size=(B, max(R - 1, 0), S)).astype(np.int32)
    return TTTInputs(feats, tokens, forced)


# ------------------------------------------------------------ tree-stage inputs
def random_topk_rows(seed: int, rows: int, k: int, V: int, tie_every: int = 0):
    """Synthetic per-row top-k (ids distinct within a row, log-probs <= 0 and
    non-increasing), for exercising tree expansion in isolation.  With
    ``tie_every`` > 0, some log-probs are duplicated to create exact ties."""
    g = _rng(seed, 31)
    ids = np.empty((rows, k), dtype=np.int32)
    lp = np.empty((rows, k), dtype=np.float32)
    for r in range(rows):
        ids[r] = g.choice(V, size=k, replace=False)
        v = np.sort(-g.exponential(1.5, size=k).astype(np.float32))[::-1].copy()
        if tie_every:
            for i in range(1, k):
                if g.integers(tie_every) == 0:
                    v[i] = v[i - 1]
        lp[r] = v
    return ids, lp


def random_verify_tree(seed: int, m: int, V: int, depth: int, root_tok: int = 0):
    """A random valid verify tree in canonical order: root 0, nodes sorted by
    (depth, parent index), children of a node contiguous, sibling tokens
    distinct.  Returns (v_tok [m+1], v_parent [m+1])."""
    g = _rng(seed, 32)
    parents = [-1]
    depths = [0]
    while len(parents) < m + 1:
        cand = [i for i in range(len(parents)) if depths[i] < depth]
        p = int(g.choice(cand))
        parents.append(p)
        depths.append(depths[p] + 1)
    # canonicalise: BFS by depth, children grouped by parent's new index
    new_index = {0: 0}
    out_par = [-1]
    out_dep = [0]
    level = [0]
    while level:
        nxt = []
        for p in level:
            kids = [i for i in range(1, m + 1) if parents[i] == p]
            for c in kids:
                new_index[c] = len(out_par)
                out_par.append(new_index[p])
                out_dep.append(depths[c])
                nxt.append(c)
        level = nxt
    v_parent = np.array(out_par, dtype=np.int32)
    v_tok = np.empty(m + 1, dtype=np.int32)
    v_tok[0] = root_tok
    for p in range(m + 1):
        kids = np.nonzero(v_parent == p)[0]
        if len(kids):
            v_tok[kids] = g.choice(V, size=len(kids), replace=False)
    return v_tok, v_parent


def ancestor_bits(v_parent) -> np.ndarray:
    """uint64 ancestor-or-self bitsets of a tree whose parents precede
    their children (bit i of node i set, plus every bit of its parent)."""
    n = len(v_parent)
    out = np.zeros(n, dtype=np.uint64)
    for i in range(n):
        p = int(v_parent[i])
        out[i] = np.uint64(1 << i) | (out[p] if p >= 0 else np.uint64(0))
    return out


@dataclass
class TargetInputs:
    """Inputs of one verification forward of B requests (m+1 rows each)."""
    kv_k: list                    # per layer: [B, cap, Hkv, hd] or paged pool [nb, bs, Hkv, hd] (None: not drawn)
    kv_v: list
    cap: int                      # contiguous capacity, or max_blocks * block_size
    block_table: np.ndarray       # [B, max_blocks] int32 (paged) or None
    n_blocks: int
    ctx_len: np.ndarray           # [B] committed rows
    v_tok: np.ndarray             # [B, m+1] int32, row 0 = root
    v_parent: np.ndarray          # [B, m+1] int32
    v_pos: np.ndarray             # [B, m+1] int32 = ctx_len + depth
    v_anc: np.ndarray             # [B, m+1] uint64


def gen_target_inputs(w: Workload, n_layers: int, layers=None, seed: int = 1) -> TargetInputs:
    """Synthetic verification-forward inputs: committed prefixes of w.prefix
    rows (or U[w.prefix_range] per request) with N(0,1) keys/values in every
    layer (`layers` limits which layers are drawn), room for the m+1 rows a
    commit may append, and one random verify tree per request (depth <=
    w.depth, m = w.keep kept nodes; a chain when w.topk == 1)."""
    s = w.shape
    Bn, m = w.batch, w.keep
    rows = m + 1
    hkv, hd = s.n_kv_heads, s.head_dim
    if w.prefix_range is not None:
        lo, hi = w.prefix_range
        ctx = _rng(seed, 51).integers(lo, hi + 1, size=Bn).astype(np.int32)
    else:
        ctx = np.full(Bn, w.prefix, dtype=np.int32)
    v_tok = np.empty((Bn, rows), np.int32)
    v_par = np.empty((Bn, rows), np.int32)
    roots = _rng(seed, 52).integers(0, s.vocab, size=Bn)
    g = _rng(seed, 53)
    for b in range(Bn):
        if w.topk == 1:
            v_par[b] = np.arange(-1, m, dtype=np.int32)
            v_tok[b] = g.integers(0, s.vocab, size=rows)
            v_tok[b, 0] = roots[b]
        else:
            v_tok[b], v_par[b] = random_verify_tree(seed * 1000 + b, m, s.vocab, w.depth, root_tok=int(roots[b]))
    depth = np.zeros((Bn, rows), np.int32)
    v_anc = np.zeros((Bn, rows), np.uint64)
    for b in range(Bn):
        for i in range(1, rows):
            depth[b, i] = depth[b, v_par[b, i]] + 1
        v_anc[b] = ancestor_bits(v_par[b])
    v_pos = (ctx[:, None] + depth).astype(np.int32)
    want = range(n_layers) if layers is None else layers
    kv_k, kv_v = [None] * n_layers, [None] * n_layers
    table, nb = None, 0
    if w.paged:
        bs = w.block_size
        need = [(int(c) + rows + bs - 1) // bs for c in ctx]
        nb = int(sum(need))
        perm = _rng(seed, 54).permutation(nb).astype(np.int32)
        maxb = max(need)
        table = np.full((Bn, maxb), -1, dtype=np.int32)
        off = 0
        for b in range(Bn):
            table[b, :need[b]] = perm[off:off + need[b]]
            off += need[b]
        cap = maxb * bs
        shp = (nb, bs, hkv, hd)
    else:
        cap = int(ctx.max()) + rows
        shp = (Bn, cap, hkv, hd)
    for l in want:
        kv_k[l] = draw(seed, 2000 + 2 * l, shp, 1.0, s.dtype)
        kv_v[l] = draw(seed, 2001 + 2 * l, shp, 1.0, s.dtype)
    return TargetInputs(kv_k, kv_v, cap, table, nb, ctx, v_tok, v_par, v_pos, v_anc)
