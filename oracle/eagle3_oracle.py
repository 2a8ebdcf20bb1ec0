"""CPU oracle for the EAGLE-3 draft-and-verify hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

Plain, slow NumPy written to be checked by eye against the pages:

* "EAGLE-3 精读" (edgeai1 speculative-decoding knowledge base), §1 为什么推翻
  feature regression: low/mid/high target features are concatenated to 3d and
  projected to d ("g"); a one-layer draft decoder combines g (or its own
  state) with the token embedding; target model and LM head are frozen.
* same page, §2 Training-Time Test: about 5 self-fed rollout steps built in
  one graph under a special attention mask, CE at the rollout positions;
  inference uses EAGLE-2's confidence-value dynamic tree and strict target
  verification.
* same page, §5 正确性、复现与风险: the drafter is only a proposal; the standard
  verifier keeps greedy sequence / sampling distribution when the residual
  correction is kept; rollout nodes must not peek at future ground truth.
* EAGLE-4 blog (10100.com), 几条技术路线正在收敛: confidence = product of draft
  probabilities; "EAGLE-3" quote page (scholarfeed): each extra tree depth is
  one more sequential drafter round.

Precision: fp64 throughout.  For bf16 workloads the values are rounded to
bfloat16 (round to nearest even) at the same points as the GPU path: weights
and embeddings (already bf16 on input), g, every GEMM input operand (x, the
attention output, u, silu(gate)*up, rms(h2)) and q/k/v after RoPE (the KV
cache).  The residual stream s, h1, h2 is not rounded.  Decisions that turn
floats into integers are taken in the precision the GPU path uses: top-k and
argmax on float32 logits, tree scores as float32 sums of float32 log-probs,
sampling verification in fp64.

Where the pages are silent the oracle follows one explicit reading; each is
named where it is used (R1..R41).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp

F32 = "f32"
BF16 = "bf16"
MAX_TREE_SLOTS = 64

# --------------------------------------------------------------------------
# numeric helpers


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even, directly from fp64.

    bfloat16 keeps 8 significant bits: write x = m * 2**e with 0.5 <= |m| < 1,
    round m * 2**8 to the nearest integer (numpy's rint is ties-to-even) and
    scale back.  Values are assumed to be inside bf16's normal range.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _rnd(cfg, x):
    return bf16_round(x) if cfg.dtype == BF16 else np.asarray(x, dtype=np.float64)


def matmul_wt(x, W):
    """x @ W.T in fp64 (W is [out, in]); W is up-cast in row blocks to bound memory."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty((x.shape[0], W.shape[0]), dtype=np.float64)
    step = 8192
    for s in range(0, W.shape[0], step):
        out[:, s:s + step] = x @ np.asarray(W[s:s + step], dtype=np.float64).T
    return out


def rmsnorm(v, gain, eps):
    """v / sqrt(mean(v^2) + eps) * gain  (pre-norm RMSNorm; reading R2)."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * np.asarray(gain, np.float64)


def rope(x, pos, theta):
    """Rotate-half rotary embedding (reading R6).

    x: [..., H, hd]; pos: [...] integer positions.  Pair (i, i + hd/2) is
    rotated by angle pos * theta**(-2i/hd).
    """
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------
# step 1: multi-layer feature fusion  ("EAGLE-3 精读" §1)


def fuse(cfg, feats, W_fc, norm_fc=None):
    """g = [f_low ; f_mid ; f_high] . W_fc^T.

    feats [n, 3, d] -> g [n, d].  No bias and no norm after the projection
    (reading R2: the FC norm first appears in EAGLE-3.1 per the EAGLE-4 blog).
    With norm_fc (EAGLE-3.1's FC Norm, which EAGLE-4 keeps -- EAGLE-4 blog,
    the paragraph on what EAGLE-4 keeps of EAGLE-3.1; reading R37) the
    projection is RMS-normalised: g = rms(FC x) * norm_fc.  bf16 workloads
    round g to bfloat16 (once, after the norm).
    """
    n = feats.shape[0]
    cat = np.asarray(feats, dtype=np.float64).reshape(n, -1)
    y = matmul_wt(cat, W_fc)
    if norm_fc is not None:
        y = rmsnorm(y, norm_fc, cfg.rms_eps)
    return _rnd(cfg, y)


# --------------------------------------------------------------------------
# step 2: the one-layer draft decoder ("EAGLE-3 精读" §1; readings R1-R8)


def _self_attention(cfg, W_qkv, x, P, Kc, Vc, write_idx, visible):
    """The attention block shared by the drafter and the target layers.

    x [R, K]: the rows' (already rounded) attention input.  q, k, v =
    split(W_qkv x); RoPE on q and k at positions P; bf16 workloads round
    q/k/v; row r stores its k, v at cache index write_idx[r] (in place), then
    attends over the keys visible[r] marks:
      a_h = softmax(q_h . K_g(h)^T / sqrt(hd)) V_g(h),  g(h) = floor(h Hkv / Hq)  (R7)
    Returns a [R, Hq*hd], rounded like every GEMM input."""
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    R = x.shape[0]
    qkv = matmul_wt(x, W_qkv)
    q = qkv[:, : Hq * hd].reshape(R, Hq, hd)
    k = qkv[:, Hq * hd: (Hq + Hkv) * hd].reshape(R, Hkv, hd)
    v = qkv[:, (Hq + Hkv) * hd:].reshape(R, Hkv, hd)
    q = _rnd(cfg, rope(q, P, cfg.rope_theta))
    k = _rnd(cfg, rope(k, P, cfg.rope_theta))
    v = _rnd(cfg, v)
    for r in range(R):
        Kc[write_idx[r]] = k[r]
        Vc[write_idx[r]] = v[r]
    a = np.empty((R, Hq, hd), dtype=np.float64)
    scale = 1.0 / math.sqrt(hd)
    for r in range(R):
        idx = np.nonzero(visible[r])[0]
        Kr = np.asarray(Kc[idx], dtype=np.float64)
        Vr = np.asarray(Vc[idx], dtype=np.float64)
        for h in range(Hq):
            g = (h * Hkv) // Hq
            sc = Kr[:, g, :] @ q[r, h] * scale
            p = np.exp(sc - sc.max())
            p /= p.sum()
            a[r, h] = p @ Vr[:, g, :]
    return _rnd(cfg, a.reshape(R, Hq * hd))


def _ffn_residual(cfg, gain, W_gate_up, W_down, h1):
    """h2 = h1 + W_down (silu(W_gate u) * W_up u),  u = rms(h1) * gain; bf16
    workloads round u and the SwiGLU product (GEMM inputs)."""
    F = cfg.ffn
    u = _rnd(cfg, rmsnorm(h1, gain, cfg.rms_eps))
    gu = matmul_wt(u, W_gate_up)
    z = _rnd(cfg, silu(gu[:, :F]) * gu[:, F:])
    return h1 + matmul_wt(z, W_down)


def decoder_rows(cfg, W, S, T, P, Kc, Vc, write_idx, visible, want_logits=True):
    """Run the drafter layer on R query rows.

    S [R, d]: state of each row (g for committed rows, the parent's h_out
    for tree rows); T [R]: token ids; P [R]: positions.
    Kc, Vc [N, Hkv, hd]: the key/value cache the rows can see (modified in
    place: row r writes its k, v at index write_idx[r] before attention).
    visible [R, N] bool: the keys row r attends to.

    Returns (h2 [R, d], logits [R, V] or None).

    Per row (R1: combine = concatenate the two normed halves; R3: residual on
    the state stream; R4: children receive h2; R8: frozen target embedding):
      x  = [rms(Emb[t]) ; rms(s)]                      (2d)
      q, k, v = split(W_qkv x); RoPE(q, k) at position p
      a_h = softmax(q_h . K_g(h)^T / sqrt(hd)) V_g(h),  g(h) = floor(h Hkv / Hq)  (R7)
      h1 = s + W_o a
      h2 = h1 + W_down (silu(W_gate u) * W_up u),  u = rms(h1)
      logits = W_lm rms(h2)
    With W["norm_post_attn"] and W["norm_post_ffn"] (the post-norm variant,
    R38) instead:
      h1 = rms(s + W_o a) * norm_post_attn
      h2 = rms(h1 + W_down (silu(W_gate h1) * W_up h1)) * norm_post_ffn
    """
    eps = cfg.rms_eps
    S = np.asarray(S, dtype=np.float64)
    e = np.asarray(W["emb"][np.asarray(T)], dtype=np.float64)
    x = np.concatenate([rmsnorm(e, W["norm_e"], eps), rmsnorm(S, W["norm_s"], eps)], axis=1)
    a = _self_attention(cfg, W["qkv"], _rnd(cfg, x), P, Kc, Vc, write_idx, visible)
    if W.get("norm_post_attn") is not None:
        # EAGLE-3.1's Post-norm (EAGLE-4 blog; reading R38): every residual
        # sum is RMS-normalised, and the FFN reads the normalised h1 directly
        h1 = rmsnorm(S + matmul_wt(a, W["o"]), W["norm_post_attn"], eps)
        F = cfg.ffn
        gu = matmul_wt(_rnd(cfg, h1), W["gate_up"])
        z = _rnd(cfg, silu(gu[:, :F]) * gu[:, F:])
        h2 = rmsnorm(h1 + matmul_wt(z, W["down"]), W["norm_post_ffn"], eps)
    else:
        h1 = S + matmul_wt(a, W["o"])
        h2 = _ffn_residual(cfg, W["norm_ffn"], W["gate_up"], W["down"], h1)
    logits = None
    if want_logits:
        logits = matmul_wt(lm_input(cfg, W, h2), W["lm"])
    return h2, logits


def lm_input(cfg, W, h2):
    """The LM head's input y = rms(h2) * gamma_out, rounded to bfloat16 for
    bf16 workloads (R4: the final norm acts on h2)."""
    return _rnd(cfg, rmsnorm(h2, W["norm_out"], cfg.rms_eps))


# --------------------------------------------------------------------------
# step 3a: LM head log-probs and per-row top-k


def topk_logprobs(logits_row, k):
    """Top-k of one row of logits and their log-probabilities.

    The decision is taken on float32 logits, ordered by (value desc, id asc)
    (ties go to the lowest id).  LSE = logsumexp of the float32 logits,
    rounded to float32; lp = logit - LSE in float32.
    Returns (ids [k] int32, lp [k] float32, lse float32).
    """
    l32 = np.asarray(logits_row, dtype=np.float64).astype(np.float32)
    order = np.argsort(-l32, kind="stable")[:k].astype(np.int32)
    lse = np.float32(logsumexp(l32.astype(np.float64)))
    lp = (l32[order] - lse).astype(np.float32)
    return order, lp, lse


# --------------------------------------------------------------------------
# step 3a': the efficient draft LM head (EAGLE-4 blog, the paragraph "EAGLE
# Efficient LM Head" and the section 关于 Efficient LM Head: a low-rank head
# first scores the whole vocabulary and keeps its top candidates; the full LM
# head then computes exact logits for those candidates only; readings
# R31-R32)


def efficient_head_topk(cfg, W, y_row, A, Bm, c, k):
    """Two-stage draft LM head for one row.

    Stage 1 (recall): z = Bm . y, rounded to bfloat16 for bf16 workloads
    like every GEMM input; scores s = A . z over the whole vocabulary.  The c
    best float32 scores (value desc, id asc) are the candidates.
    Stage 2 (exact): the full LM head's logits of the candidates only,
    l_i = W_lm[cand_i] . y.
    The top-k are the k best candidates by (float32 logit desc, id asc).
    Log-probabilities are normalised over the candidate set (R31): lp = l -
    logsumexp of the c candidate logits, in float32.

    y_row [d]; A [V, r]; Bm [r, d].  Returns (ids [k] int32, lp [k] float32,
    cand [c] int32 in score order, cand_logits [c] fp64).
    """
    y = np.asarray(y_row, dtype=np.float64)[None]
    z = _rnd(cfg, matmul_wt(y, Bm))
    s32 = matmul_wt(z, A)[0].astype(np.float32)
    cand = np.argsort(-s32, kind="stable")[:c].astype(np.int32)
    cl = (y @ np.asarray(W["lm"][cand], dtype=np.float64).T)[0]
    l32 = cl.astype(np.float32)
    order = np.array(sorted(range(c), key=lambda i: (-float(l32[i]), int(cand[i]))), dtype=np.int64)[:k]
    lse = np.float32(logsumexp(l32.astype(np.float64)))
    lp = (l32[order] - lse).astype(np.float32)
    return cand[order].astype(np.int32), lp, cand, cl


# --------------------------------------------------------------------------
# step 3b: EAGLE-2 confidence-value dynamic tree ("EAGLE-3 精读" §2; EAGLE-4
# blog 几条技术路线正在收敛: confidence is the product of draft probabilities;
# readings R9-R13)


class DynamicTree:
    """Candidate pool of one request.

    Confidence is kept as a float32 sum of float32 log-probs (R12: the
    logarithm of the product of draft probabilities).  Beam width = k: each
    round expands the k best candidates of the previous depth (R9).
    """

    def __init__(self, k, D, root_tok, root_pos):
        self.k, self.D = k, D
        self.root_tok, self.root_pos = int(root_tok), int(root_pos)
        # pool node fields
        self.tok, self.parent, self.depth = [], [], []
        self.score, self.flat, self.rank, self.slot, self.anc = [], [], [], [], []
        self.frontier = []   # pool indices, in frontier-rank order
        self.round = 1       # depth of the nodes most recently added

    def _add(self, tok, parent, depth, score, flat, rank):
        self.tok.append(int(tok))
        self.parent.append(int(parent))
        self.depth.append(int(depth))
        self.score.append(np.float32(score))
        self.flat.append(int(flat))
        self.rank.append(int(rank))
        self.slot.append(-1)
        self.anc.append(0)
        return len(self.tok) - 1

    def _assign_slots(self):
        """Frontier nodes of depth j get tree slots (j-1)k + rank; their
        bitset is the parent's bitset plus the own slot."""
        j = self.round
        for rho, n in enumerate(self.frontier):
            s = (j - 1) * self.k + rho
            assert s < MAX_TREE_SLOTS
            self.slot[n] = s
            p = self.parent[n]
            self.anc[n] = (self.anc[p] if p >= 0 else 0) | (1 << s)

    def next_rows(self):
        """Draft rows for the frontier: (token, h-state index of the parent
        (0 = root, 1 + slot otherwise), position, ancestor bitset)."""
        out = []
        for n in self.frontier:
            p = self.parent[n]
            out.append((self.tok[n], 0 if p < 0 else 1 + self.slot[p],
                        self.root_pos + self.depth[n], self.anc[n]))
        return out

    def init(self, ids, lp):
        """The root's top-k become the depth-1 nodes; frontier = all of them."""
        for i in range(self.k):
            self._add(ids[i], -1, 1, lp[i], i, i)
        self.frontier = list(range(self.k))
        self.round = 1
        if self.D > 1:
            self._assign_slots()

    def step(self, ids, lp):
        """One expansion round: ids/lp [k, k] are the top-k of each frontier
        row (row rho = frontier rank rho).  score = score(parent) + lp as one
        float32 add; all k^2 candidates join the pool; the new frontier is
        the first k by (score desc, flat asc) with flat = rho*k + i (R13)."""
        j = self.round + 1
        cands = []
        for rho, par in enumerate(self.frontier):
            for i in range(self.k):
                sc = np.float32(self.score[par] + np.float32(lp[rho][i]))
                cands.append(self._add(ids[rho][i], par, j, sc, rho * self.k + i, i))
        cands.sort(key=lambda n: (-float(self.score[n]), self.flat[n]))
        self.frontier = cands[: self.k]
        self.round = j
        if j < self.D:
            self._assign_slots()

    def sorted_scores(self):
        """Pool scores in rerank order (score desc, depth asc, flat asc): the
        confidences the harness's verify-count rule reads (R40)."""
        order = sorted(range(len(self.tok)), key=lambda n: (-float(self.score[n]), self.depth[n], self.flat[n]))
        return [self.score[n] for n in order]

    def final(self, m):
        """Keep the top-m of the pool by (score desc, depth asc, flat asc) and
        lay them out in canonical verify order: root 0, then by (depth asc,
        parent's verify index asc, child rank asc).  Returns dict of arrays
        (tok, parent, depth, pos, anc) of length m+1."""
        n_pool = len(self.tok)
        order = sorted(range(n_pool), key=lambda n: (-float(self.score[n]), self.depth[n], self.flat[n]))
        kept = set(order[:m])
        for n in kept:  # ancestor closure (child score <= parent score, ties prefer shallow)
            p = self.parent[n]
            assert p < 0 or p in kept, "kept set not closed under ancestors"
        vidx = {-1: 0}
        vt, vp, vd, vpos = [self.root_tok], [-1], [0], [self.root_pos]
        for depth in range(1, self.D + 1):
            nodes = [n for n in kept if self.depth[n] == depth]
            nodes.sort(key=lambda n: (vidx[self.parent[n]], self.rank[n]))
            for n in nodes:
                vidx[n] = len(vt)
                vt.append(self.tok[n])
                vp.append(vidx[self.parent[n]])
                vd.append(depth)
                vpos.append(self.root_pos + depth)
        M = len(vt)
        anc = [0] * M
        for i in range(M):
            a = 1 << i
            p = vp[i]
            if p >= 0:
                a |= anc[p]
            anc[i] = a
        return dict(tok=np.array(vt, np.int32), parent=np.array(vp, np.int32),
                    depth=np.array(vd, np.int32), pos=np.array(vpos, np.int32),
                    anc=np.array(anc, dtype=np.uint64))


# --------------------------------------------------------------------------
# step 4: verification ("EAGLE-3 精读" §5; readings R14-R17)


def children_of(v_parent):
    kids = {}
    for c in range(1, len(v_parent)):
        kids.setdefault(int(v_parent[c]), []).append(c)
    return kids


def verify_greedy(v_tok, v_parent, L):
    """Longest accepted path under greedy decoding of the target.

    At the current node take t* = argmax of its target logits (float32,
    lowest id on ties); move to the kept child whose token is t*, else stop
    and emit t* as the bonus token.  Returns (accepted node list, bonus).
    """
    kids = children_of(v_parent)
    node, acc = 0, []
    while True:
        row = np.asarray(L[node], dtype=np.float32)
        t = int(np.argmax(row))   # numpy returns the first maximum
        nxt = [c for c in kids.get(node, []) if int(v_tok[c]) == t]
        if not nxt:
            return acc, t
        node = nxt[0]
        acc.append(node)


def verify_sample(v_tok, v_parent, L, u_try, u_res, temperature=1.0):
    """Rejection sampling with residual correction, deterministic candidates.

    The tree's children are top-k picks, so the proposal for each candidate
    is a point mass (R14).  At a node with unnormalised target weights
    w(y) = exp((L[y] - max L) / T) (fp64) and remaining mass Rm = sum w:
    try the kept children in sibling order; child c is accepted when
    u_try[c] * Rm < w(tok c); a rejected child's token leaves the support
    (Rm -= w(tok c)).  When every child is rejected, or the node is a leaf,
    the bonus is the smallest y outside the rejected set with cumulative
    weight (id order, rejected tokens skipped) > u_res[node] * Rm.
    If rounding leaves no such y, the last y with w(y) > 0 outside the
    rejected set is taken.  Returns (accepted node list, bonus).
    """
    kids = children_of(v_parent)
    node, acc = 0, []
    while True:
        l = np.asarray(L[node], dtype=np.float32).astype(np.float64)
        w = np.exp((l - l.max()) / float(temperature))
        Rm = float(np.sum(w))
        rejected = set()
        moved = False
        for c in kids.get(node, []):
            t = int(v_tok[c])
            if u_try[c] * Rm < w[t]:
                acc.append(c)
                node = c
                moved = True
                break
            rejected.add(t)
            Rm = Rm - w[t]
        if moved:
            continue
        thr = u_res[node] * Rm
        wm = w.copy()
        for t in rejected:
            wm[t] = 0.0
        cs = np.cumsum(wm)
        hit = np.nonzero(cs > thr)[0]
        if len(hit):
            return acc, int(hit[0])
        return acc, int(np.nonzero(wm > 0)[0][-1])


# --------------------------------------------------------------------------
# the draft-tree cycle (fuse + commit + D-1 tree rounds + rerank), per request


def _row_topk(cfg, W, h2_row, logits_row, k, head):
    """Top-k of one drafted row: from the full logits, or through the
    efficient head (head = dict(A=, B=, c=))."""
    if head is None:
        return topk_logprobs(logits_row, k)[:2]
    ids, lp, _, _ = efficient_head_topk(cfg, W, lm_input(cfg, W, h2_row[None])[0], head["A"], head["B"],
                                        head["c"], k)
    return ids, lp


def draft_cycle(cfg, W, feats, tokens, Kc, Vc, ctx_len, k, D, m, record=None, head=None):
    """One EAGLE-3 draft cycle of one request, before verification.

    feats [n, 3, d] and tokens [n]: the n rows to commit (the last one is
    the root).  Kc, Vc [cap, Hkv, hd]: committed cache holding ctx_len rows
    (copied, not modified).  head: None for the full LM head, or dict(A=,
    B=, c=) for the efficient head (efficient_head_topk).  Returns the
    verify tree (dict) and, if ``record`` is a dict, per-round intermediate
    values.
    """
    n = len(tokens)
    Hkv, hd = cfg.n_kv_heads, cfg.head_dim
    g = fuse(cfg, feats, W["fc"], W.get("norm_fc"))
    cap = Kc.shape[0]
    N = cap + MAX_TREE_SLOTS
    K = np.zeros((N, Hkv, hd))
    V = np.zeros((N, Hkv, hd))
    K[:cap] = Kc
    V[:cap] = Vc
    L0 = int(ctx_len)
    # COMMIT: rows at positions L0..L0+n-1, causal over the committed prefix
    vis = np.zeros((n, N), dtype=bool)
    for r in range(n):
        vis[r, : L0 + r + 1] = True
    P = np.arange(L0, L0 + n)
    h2, logits = decoder_rows(cfg, W, g, tokens, P, K, V, P, vis)
    root_pos = L0 + n - 1
    h_tree = {0: h2[-1]}
    ids, lp = _row_topk(cfg, W, h2[-1], logits[-1], k, head)
    tree = DynamicTree(k, D, tokens[-1], root_pos)
    tree.init(ids, lp)
    if record is not None:
        record.update(g=g, commit_h2=h2, commit_logits=logits, rounds=[])
    Lc = L0 + n
    for j in range(2, D + 1):
        rows = tree.next_rows()
        slot_base = (j - 2) * k
        S = np.stack([h_tree[pidx] for (_, pidx, _, _) in rows])
        T = np.array([t for (t, _, _, _) in rows])
        Pr = np.array([p for (_, _, p, _) in rows])
        vis = np.zeros((len(rows), N), dtype=bool)
        vis[:, :Lc] = True
        for r, (_, _, _, anc) in enumerate(rows):
            for s in range(MAX_TREE_SLOTS):
                if (anc >> s) & 1:
                    vis[r, cap + s] = True
        widx = cap + slot_base + np.arange(len(rows))
        h2, logits = decoder_rows(cfg, W, S, T, Pr, K, V, widx, vis)
        ids = np.zeros((len(rows), k), np.int32)
        lps = np.zeros((len(rows), k), np.float32)
        for r in range(len(rows)):
            h_tree[1 + slot_base + r] = h2[r]
            ids[r], lps[r] = _row_topk(cfg, W, h2[r], logits[r], k, head)
        if record is not None:
            record["rounds"].append(dict(rows=rows, h2=h2, logits=logits, ids=ids, lp=lps))
        tree.step(ids, lps)
    vt = tree.final(m)
    if record is not None:
        record.update(tree=tree, root_ids=ids if D == 1 else None)
    return vt


# --------------------------------------------------------------------------
# step 5: training-time test forward ("EAGLE-3 精读" §2 and §5; R18-R22)


def ttt_forward(cfg, W, feats, tokens, R, forced=None, positions=None):
    """TTT forward of one sequence.

    feats [S, 3, d]; tokens x [S].  Rows (j, i), j = 1..R, i = 0..S-1.
    Step 1 feeds (s, t) = (g_i, x_i) at position i.  Step j >= 2 feeds the
    previous step's h2 and its argmax token (or forced[j-2, i]) at position
    i + j - 1.  Query (j, i) sees step-1 keys at i' <= i and its own chain
    keys (j', i) for 2 <= j' <= j: a rollout position never sees ground
    truth beyond x_i.  Label of (j, i) is x_{i+j}, valid when i + j <= S-1.

    positions: optional subset of i to evaluate for steps (all keys of step
    1 up to max(positions) are still computed).  Returns dict of arrays
    [R, len(positions)]: ce (0 where invalid), valid, pred, plus logits of
    every evaluated row when ``positions`` is small.
    """
    S = len(tokens)
    Hkv, hd = cfg.n_kv_heads, cfg.head_dim
    pos_list = np.arange(S) if positions is None else np.asarray(sorted(positions))
    imax = int(pos_list.max())
    g = fuse(cfg, feats[: imax + 1], W["fc"])
    # step-1 keys/values for i' <= imax come from the teacher-forced rows
    n1 = imax + 1
    N = n1 + R
    K1 = np.zeros((n1, Hkv, hd))
    V1 = np.zeros((n1, Hkv, hd))
    # keys of step 1 depend only on (g_i, x_i, i): compute them for all i' <= imax
    kv_only = _kv_rows(cfg, W, g, tokens[: imax + 1], np.arange(n1))
    K1[:], V1[:] = kv_only
    out = dict(ce=np.zeros((R, len(pos_list))), valid=np.zeros((R, len(pos_list)), bool),
               pred=np.zeros((R, len(pos_list)), np.int32), logits=[])
    for col, i in enumerate(pos_list):
        K = np.zeros((N, Hkv, hd))
        V = np.zeros((N, Hkv, hd))
        K[:n1], V[:n1] = K1, V1
        s = g[i][None]
        t = np.array([tokens[i]])
        for j in range(1, R + 1):
            p = i + j - 1
            vis = np.zeros((1, N), bool)
            vis[0, : i + 1] = True
            if j >= 2:
                vis[0, n1: n1 + j - 1] = True   # chain keys (2..j, i)
                widx = [n1 + j - 2]
            else:
                widx = [i]                      # recomputes step-1 key i (same value)
            h2, logits = decoder_rows(cfg, W, s, t, [p], K, V, widx, vis)
            l32 = logits[0].astype(np.float32)
            pred = int(np.argmax(l32))
            out["pred"][j - 1, col] = pred
            if positions is not None and len(pos_list) <= 64:
                out["logits"].append(logits[0])
            if i + j <= S - 1:
                lab = int(tokens[i + j])
                out["ce"][j - 1, col] = logsumexp(l32.astype(np.float64)) - float(l32[lab])
                out["valid"][j - 1, col] = True
            s = h2
            t = np.array([pred if forced is None else int(forced[j - 1, i])]) if j < R else t
    return out


def _kv_rows(cfg, W, S, T, P):
    """Keys/values (after RoPE and rounding) of teacher-forced rows; the same
    projections as decoder_rows, stopped after the KV write."""
    d, Hq, Hkv, hd, eps = cfg.d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    R = len(T)
    e = np.asarray(W["emb"][np.asarray(T)], dtype=np.float64)
    x = _rnd(cfg, np.concatenate([rmsnorm(e, W["norm_e"], eps),
                                  rmsnorm(np.asarray(S, np.float64), W["norm_s"], eps)], axis=1))
    Wkv = W["qkv"][Hq * hd:]
    kv = matmul_wt(x, Wkv)
    k = kv[:, : Hkv * hd].reshape(R, Hkv, hd)
    v = kv[:, Hkv * hd:].reshape(R, Hkv, hd)
    return _rnd(cfg, rope(k, P, cfg.rope_theta)), _rnd(cfg, v)


def ttt_forward_full(cfg, W, feats, tokens, R, forced=None):
    """TTT forward over every position, step by step (all rows of a step at
    once), for small sequences.  Same semantics as ``ttt_forward``.
    Returns ce [R, S], valid [R, S], pred [R, S], logits [R, S, V]."""
    S = len(tokens)
    Hkv, hd = cfg.n_kv_heads, cfg.head_dim
    g = fuse(cfg, feats, W["fc"])
    N = S * R
    K = np.zeros((N, Hkv, hd))
    V = np.zeros((N, Hkv, hd))
    ce = np.zeros((R, S))
    valid = np.zeros((R, S), bool)
    pred = np.zeros((R, S), np.int32)
    all_logits = np.zeros((R, S, cfg.vocab))
    s = g
    t = np.asarray(tokens)
    for j in range(1, R + 1):
        P = np.arange(S) + j - 1
        widx = (j - 1) * S + np.arange(S)          # key (j, i) lives at (j-1)*S + i
        vis = np.zeros((S, N), bool)
        for i in range(S):
            vis[i, : i + 1] = True                 # step-1 keys i' <= i
            for jj in range(2, j + 1):
                vis[i, (jj - 1) * S + i] = True    # own chain keys
        h2, logits = decoder_rows(cfg, W, s, t, P, K, V, widx, vis)
        l32 = logits.astype(np.float32)
        all_logits[j - 1] = logits
        pred[j - 1] = np.argmax(l32, axis=1)
        for i in range(S):
            if i + j <= S - 1:
                lab = int(tokens[i + j])
                ce[j - 1, i] = logsumexp(l32[i].astype(np.float64)) - float(l32[i, lab])
                valid[j - 1, i] = True
        s = h2
        if j < R:
            t = pred[j - 1].copy() if forced is None else np.asarray(forced[j - 1])
    return dict(ce=ce, valid=valid, pred=pred, logits=all_logits,
                loss=float(ce[valid].mean()) if valid.any() else 0.0)


def gather_paged(pool, table, n_rows, block_size):
    """Rows 0..n_rows-1 of one request from a paged pool [n_blocks, bs, ...]:
    logical row p lives in block table[p // bs] at offset p % bs."""
    out = np.empty((n_rows,) + pool.shape[2:], dtype=pool.dtype)
    for p in range(n_rows):
        out[p] = pool[table[p // block_size], p % block_size]
    return out


# --------------------------------------------------------------------------
# the target's tree-verification forward ("EAGLE-3 精读" §2: inference keeps
# strict target verification; §5: the target's standard verifier; §1: the
# target exposes low/mid/high hidden states; the "EAGLE-3" quote page
# (scholarfeed): verification is the larger part of the computation).
# Readings R33-R36.


def target_layer(cfg, Lw, h, P, Kc, Vc, write_idx, visible):
    """One target decoder layer on rows h [R, d] (R33: pre-norm, the
    drafter's layer shape with a d-wide attention input):
      x  = rms(h) * norm_attn                       (rounded for bf16)
      a  = attention of x as in the drafter (q/k/v, RoPE, GQA, visible keys)
      h1 = h + W_o a
      h2 = h1 + W_down (silu(W_gate u) * W_up u),  u = rms(h1) * norm_ffn
    Kc, Vc [N, Hkv, hd] are this layer's keys/values (row r writes index
    write_idx[r]).  Returns h2 [R, d] (fp64, not rounded)."""
    h = np.asarray(h, dtype=np.float64)
    x = _rnd(cfg, rmsnorm(h, Lw["norm_attn"], cfg.rms_eps))
    a = _self_attention(cfg, Lw["qkv"], x, P, Kc, Vc, write_idx, visible)
    h1 = h + matmul_wt(a, Lw["o"])
    return _ffn_residual(cfg, Lw["norm_ffn"], Lw["gate_up"], Lw["down"], h1)


def target_forward(cfg, Tw, tokens, P, Ks, Vs, write_idx, visible, feat_layers, begin=0, end=None, h=None):
    """Target layers begin..end-1 on R rows (R33, R34).

    Tw: dict(emb, lm, norm_out, layers=[dict(qkv, o, gate_up, down, norm_attn,
    norm_ffn)]); Ks[l], Vs[l] [N, Hkv, hd]: layer l's keys/values (written in
    place); visible [R, N] as in decoder_rows.  begin == 0 starts the residual
    stream at the token embedding emb[tokens]; otherwise h [R, d] is the state
    after `begin` layers.  feat_layers (l_low, l_mid, l_high), counted from 1:
    feature j is the state after layer feat_layers[j], rounded to bf16 for bf16
    workloads (the fusion input's dtype); features of layers outside the range
    stay NaN.  With end == n_layers the logits W_lm (rms(h) * norm_out) are
    returned too.  Returns (h [R, d], feats [R, 3, d], logits or None)."""
    n_layers = len(Tw["layers"])
    end = n_layers if end is None else end
    R = len(tokens)
    if begin == 0:
        h = np.asarray(Tw["emb"][np.asarray(tokens)], dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    feats = np.full((R, 3, cfg.d), np.nan)
    for l in range(begin, end):
        h = target_layer(cfg, Tw["layers"][l], h, P, Ks[l], Vs[l], write_idx, visible)
        for j, fl in enumerate(feat_layers):
            if fl == l + 1:
                feats[:, j] = _rnd(cfg, h)
    logits = None
    if end == n_layers:
        logits = matmul_wt(_rnd(cfg, rmsnorm(h, Tw["norm_out"], cfg.rms_eps)), Tw["lm"])
    return h, feats, logits


def target_tree_visibility(v_anc, ctx_len, cap):
    """Keys seen by the verify rows (R35): the key space is `cap` committed
    rows followed by MAX_TREE_SLOTS tree slots; row i sees committed rows
    0..ctx_len-1 and every slot j with bit j of v_anc[i] set (its ancestors
    and itself; row i's own k/v go to slot i)."""
    n = len(v_anc)
    vis = np.zeros((n, cap + MAX_TREE_SLOTS), dtype=bool)
    vis[:, :ctx_len] = True
    for i in range(n):
        bits = int(v_anc[i])
        for j in range(MAX_TREE_SLOTS):
            if (bits >> j) & 1:
                vis[i, cap + j] = True
    return vis


def target_verify_forward(cfg, Tw, v_tok, v_pos, v_anc, Ks, Vs, ctx_len, feat_layers, begin=0, end=None, h=None):
    """The verification forward of one request (R35): the m+1 verify rows
    (root first) through target layers begin..end-1.  Ks[l], Vs[l] [cap + 64,
    Hkv, hd]: committed rows then the tree slots (row i writes slot i).
    Returns target_forward's (h, feats, logits); logits row i are the target
    logits after node i, the input of verify_greedy / verify_sample."""
    cap = Ks[begin].shape[0] - MAX_TREE_SLOTS
    vis = target_tree_visibility(v_anc, ctx_len, cap)
    widx = cap + np.arange(len(v_tok))
    return target_forward(cfg, Tw, v_tok, v_pos, Ks, Vs, widx, vis, feat_layers, begin, end, h)


def commit_rows(accept_len, accepted):
    """Verify rows whose keys/values and features are committed after
    verification (R36): the root, then the accepted nodes in path order."""
    return [0] + [int(a) for a in accepted[:accept_len]]


def kv_commit(Ks, Vs, ctx_len, accept_len, accepted):
    """Move the committed rows' keys/values from the tree slots to committed
    rows ctx_len, ctx_len+1, ... of every layer (R36), in place.  Returns the
    new committed length ctx_len + accept_len + 1."""
    rows = commit_rows(accept_len, accepted)
    for K, V in zip(Ks, Vs):
        cap = K.shape[0] - MAX_TREE_SLOTS
        for j, i in enumerate(rows):
            K[ctx_len + j] = K[cap + i]
            V[ctx_len + j] = V[cap + i]
    return ctx_len + len(rows)


# --------------------------------------------------------------------------
# EAGLE-4 Harness: cost-aware control of the tree (EAGLE-4 blog, the
# EAGLE-Harness paragraph: a warm-up measures draft and verify times over
# batch sizes, context lengths and token counts into a lookup table; every
# round asks, in three places, whether the expected extra accepted tokens
# divided by the extra time exceed a threshold -- one more draft layer, how
# many tokens to verify, and the branch cap per node, 8 at light load and 4
# at heavy load; the section on converging trends: the confidence is the
# product of draft probabilities, with a threshold that rises with depth).
# Readings R39-R41.

DRAFT, VERIFY = 0, 1


def harness_cost(table, kind, B, ctx, n):
    """Time (ms) of one drafter round (kind DRAFT, n rows per request) or
    one verification step (kind VERIFY, n verify rows per request) from the
    warm-up table (R39): table = dict(batch=[...], ctx=[...], tok=[...]
    ascending, draft=[nb][nc][nt], verify=[nb][nc][nt]).  B and ctx take the
    smallest measured value at or above them (the largest if none is); n is
    interpolated linearly between the measured token counts and clamped to
    their range."""
    def snap(vals, x):
        for i, v in enumerate(vals):
            if v >= x:
                return i
        return len(vals) - 1
    ib, ic = snap(table["batch"], B), snap(table["ctx"], ctx)
    row = np.asarray(table["draft" if kind == DRAFT else "verify"], dtype=np.float64)[ib, ic]
    tok = np.asarray(table["tok"], dtype=np.float64)
    return float(np.interp(float(n), tok, row))


def harness_continue(table, B, ctx, k, depth, frontier_logconf, tau0, alpha):
    """One more draft layer?  (R40) Each frontier node j of request b
    reaches its children with probability c = exp(log-confidence), so one
    more layer can add at most sum_j c_bj expected accepted tokens to request
    b; the layer costs one drafter round of k rows per request.  The rounds
    are shared by the batch, so the batch drafts on while

        sum_b sum_j c_bj / T_draft(B, ctx, k)  >  tau0 * (1 + alpha * depth)

    (the threshold rising with depth).  Returns (decision, per-request
    gains)."""
    c = np.exp(np.asarray(frontier_logconf, dtype=np.float64))
    gains = c.sum(axis=1)
    t = harness_cost(table, DRAFT, B, ctx, k)
    tau = tau0 * (1.0 + alpha * depth)
    return bool(gains.sum() / t > tau) if t > 0 else True, gains


def harness_verify_count(table, B, ctx, logconf_sorted, tau):
    """How many drafted tokens to verify (R40): rank i (0-based) of every
    request's rerank order (confidences descending) adds sum_b c_b,i
    expected accepted tokens and raises the verify rows per request from
    i+1 to i+2 (the root is row 0).  Ranks are taken in order while

        sum_b c_b,i / (T_verify(B, ctx, i+2) - T_verify(B, ctx, i+1))  >  tau

    (a rank whose extra time is not positive is always taken).  Returns the
    number of ranks kept, 0..m_max."""
    c = np.exp(np.asarray(logconf_sorted, dtype=np.float64))
    m_max = c.shape[1]
    n = 0
    while n < m_max:
        gain = c[:, n].sum()
        dt = harness_cost(table, VERIFY, B, ctx, n + 2) - harness_cost(table, VERIFY, B, ctx, n + 1)
        if dt > 0 and not gain / dt > tau:
            break
        n += 1
    return n


def harness_branch_cap(table, B, ctx, root_lp, tau):
    """Branches per node, 8 or 4 (R41): the root's children of ranks 5..8
    add sum_b sum_{i=4..7} p_b,i expected accepted tokens (p = the root's
    draft probabilities, exp of its top-8 log-probs) for the extra time of
    drafting 8 instead of 4 rows per request in a round; 8 while

        gain / (T_draft(B, ctx, 8) - T_draft(B, ctx, 4))  >  tau

    (or when the extra time is not positive), else 4.  Light load (small B)
    makes the extra time small and keeps 8; heavy load makes it large and
    drops to 4."""
    p = np.exp(np.asarray(root_lp, dtype=np.float64))
    gain = p[:, 4:8].sum()
    dt = harness_cost(table, DRAFT, B, ctx, 8) - harness_cost(table, DRAFT, B, ctx, 4)
    return 8 if dt <= 0 or gain / dt > tau else 4


def harness_cycle(cfg, W, feats, tokens, Kc, Vc, ctx_len, table, m_max, D_max, tau_depth0, tau_alpha, tau_verify,
                  tau_branch, B=1):
    """A draft cycle of one request under the harness: the root's top-8
    decides the branch cap k (R41); after every round the depth rule decides
    whether to draft another layer (R40, at most D_max rounds); the verify
    count rule picks m <= m_max from the pool's confidences.  B is the batch
    size the cost table is read at (the request's share of a batch).
    Returns (verify tree, dict(k=, rounds=, m=))."""
    n = len(tokens)
    Hkv, hd = cfg.n_kv_heads, cfg.head_dim
    g = fuse(cfg, feats, W["fc"], W.get("norm_fc"))
    cap = Kc.shape[0]
    N = cap + MAX_TREE_SLOTS
    K = np.zeros((N, Hkv, hd))
    V = np.zeros((N, Hkv, hd))
    K[:cap], V[:cap] = Kc, Vc
    L0 = int(ctx_len)
    vis = np.zeros((n, N), dtype=bool)
    for r in range(n):
        vis[r, : L0 + r + 1] = True
    P = np.arange(L0, L0 + n)
    h2, logits = decoder_rows(cfg, W, g, tokens, P, K, V, P, vis)
    ids8, lp8, _ = topk_logprobs(logits[-1], 8)
    k = harness_branch_cap(table, B, L0 + n, lp8[None], tau_branch)
    tree = DynamicTree(k, D_max, tokens[-1], L0 + n - 1)
    tree.init(ids8[:k], lp8[:k])
    h_tree = {0: h2[-1]}
    Lc = L0 + n
    rounds = 1
    for j in range(2, D_max + 1):
        front = np.array([[tree.score[i] for i in tree.frontier]], dtype=np.float32)
        go, _ = harness_continue(table, B, Lc, k, j - 1, front, tau_depth0, tau_alpha)
        if not go:
            break
        rows = tree.next_rows()
        slot_base = (j - 2) * k
        S = np.stack([h_tree[pidx] for (_, pidx, _, _) in rows])
        T = np.array([t for (t, _, _, _) in rows])
        Pr = np.array([p for (_, _, p, _) in rows])
        vis = np.zeros((len(rows), N), dtype=bool)
        vis[:, :Lc] = True
        for r, (_, _, _, anc) in enumerate(rows):
            for s_ in range(MAX_TREE_SLOTS):
                if (anc >> s_) & 1:
                    vis[r, cap + s_] = True
        widx = cap + slot_base + np.arange(len(rows))
        h2, logits = decoder_rows(cfg, W, S, T, Pr, K, V, widx, vis)
        ids = np.zeros((len(rows), k), np.int32)
        lps = np.zeros((len(rows), k), np.float32)
        for r in range(len(rows)):
            h_tree[1 + slot_base + r] = h2[r]
            ids[r], lps[r], _ = topk_logprobs(logits[r], k)
        tree.step(ids, lps)
        rounds += 1
    sc = tree.sorted_scores()
    m_cap = min(m_max, len(sc))
    m = harness_verify_count(table, B, Lc, np.asarray(sc[:m_cap], np.float32)[None], tau_verify)
    m = max(m, 1)
    return tree.final(m), dict(k=k, rounds=rounds, m=m)
