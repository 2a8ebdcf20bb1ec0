"""Pins of the oracle's target verification forward (target_layer,
target_forward, target_verify_forward, kv_commit) against things other than
itself:

* a causal language model written with torch's own operators (rms_norm,
  linear, scaled_dot_product_attention with is_causal, silu) and RoPE as a
  complex rotation: the oracle run as a chain over a prompt gives the same
  hidden states after every layer and the same logits, with a different
  random gain in every norm;
* the tree mask against sequential decoding: every verify row's logits and
  features equal those of decoding its root path one token at a time with a
  growing cache;
* greedy verification on the target's own logits, followed by the KV
  commit, reproduces the target's greedy continuation token for token over
  several cycles, and the committed keys/values equal a fresh prefill of the
  committed sequence.
"""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import BF16, F32, tiny_shape


def _target(cfg, n_layers, seed=0, std=0.2, gains="random"):
    Tw = gen.gen_target_weights(cfg, n_layers, seed=seed, std=std, gains=gains)
    f = lambda t: t.f32().astype(np.float64) if hasattr(t, "f32") else np.asarray(t, np.float64)
    out = dict(emb=f(Tw["emb"]), lm=f(Tw["lm"]), norm_out=f(Tw["norm_out"]), layers=[])
    for Lw in Tw["layers"]:
        out["layers"].append({k: f(v) for k, v in Lw.items()})
    return out


def _torch_causal_lm(cfg, Tw, tokens, bf16=False):
    """Prefill of `tokens` (positions 0..n-1) with torch's operators.
    Returns (hidden state after every layer [L][n, d], logits [n, V])."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    rnd = (lambda z: z.to(torch.bfloat16).to(torch.float64)) if bf16 else (lambda z: z)
    d, Hq, Hkv, hd, F, eps = cfg.d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.rms_eps
    n = len(tokens)
    pos = torch.arange(n, dtype=torch.float64)
    rms = torch.nn.functional.rms_norm
    lin = torch.nn.functional.linear

    def rot(z):
        zc = torch.complex(z[..., : hd // 2], z[..., hd // 2:])
        ang = pos[:, None, None] * cfg.rope_theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
        w = zc * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([w.real, w.imag], -1)

    h = t(Tw["emb"])[torch.as_tensor(np.asarray(tokens, dtype=np.int64))]
    states = []
    for Lw in Tw["layers"]:
        x = rnd(rms(h, (d,), t(Lw["norm_attn"]), eps=eps))
        qkv = lin(x, t(Lw["qkv"]))
        q = rnd(rot(qkv[:, : Hq * hd].reshape(n, Hq, hd))).transpose(0, 1)
        k = rnd(rot(qkv[:, Hq * hd:(Hq + Hkv) * hd].reshape(n, Hkv, hd))).transpose(0, 1)
        v = rnd(qkv[:, (Hq + Hkv) * hd:].reshape(n, Hkv, hd)).transpose(0, 1)
        rep = Hq // Hkv
        a = torch.nn.functional.scaled_dot_product_attention(q, k.repeat_interleave(rep, 0),
                                                             v.repeat_interleave(rep, 0), is_causal=True)
        a = rnd(a.transpose(0, 1).reshape(n, Hq * hd))
        h1 = h + lin(a, t(Lw["o"]))
        u = rnd(rms(h1, (d,), t(Lw["norm_ffn"]), eps=eps))
        gu = lin(u, t(Lw["gate_up"]))
        h = h1 + lin(rnd(torch.nn.functional.silu(gu[:, :F]) * gu[:, F:]), t(Lw["down"]))
        states.append(h.numpy().copy())
    logits = lin(rnd(rms(h, (d,), t(Tw["norm_out"]), eps=eps)), t(Tw["lm"]))
    return states, logits.numpy()


def _empty_kv(cfg, n_layers, cap):
    N = cap + O.MAX_TREE_SLOTS
    Ks = [np.zeros((N, cfg.n_kv_heads, cfg.head_dim)) for _ in range(n_layers)]
    Vs = [np.zeros((N, cfg.n_kv_heads, cfg.head_dim)) for _ in range(n_layers)]
    return Ks, Vs


def _chain_anc(n):
    return [(1 << (i + 1)) - 1 for i in range(n)]


@pytest.mark.parametrize("dtype,hkv", [(F32, 2), (F32, 4), (BF16, 1)])
def test_target_chain_forward_matches_torch_causal_lm(dtype, hkv):
    """A prompt run as one chain of verify rows from an empty cache is a
    causal prefill: hidden states after every layer, the three features and
    the logits equal torch's causal LM (distinct gains in every norm)."""
    cfg = tiny_shape(d=32, hq=4, hkv=hkv, hd=8, ffn=48, vocab=50, dtype=dtype)
    L = 3
    Tw = _target(cfg, L)
    if dtype == BF16:
        for key in ("emb", "lm"):
            Tw[key] = O.bf16_round(Tw[key])
        for Lw in Tw["layers"]:
            for key in ("qkv", "o", "gate_up", "down"):
                Lw[key] = O.bf16_round(Lw[key])
    tokens = np.array([5, 17, 3, 44, 0, 9, 9, 31])
    n = len(tokens)
    Ks, Vs = _empty_kv(cfg, L, 16)
    h, feats, logits = O.target_verify_forward(cfg, Tw, tokens, np.arange(n), _chain_anc(n), Ks, Vs, 0, (1, 2, 3))
    states, lg_t = _torch_causal_lm(cfg, Tw, tokens, bf16=(dtype == BF16))
    tol = 1e-10 if dtype == F32 else 1e-9
    for l in range(L):
        want = O.bf16_round(states[l]) if dtype == BF16 else states[l]
        np.testing.assert_allclose(feats[:, l], want, rtol=tol, atol=tol, err_msg=f"feature after layer {l + 1}")
    np.testing.assert_allclose(h, states[-1], rtol=tol, atol=tol)
    np.testing.assert_allclose(logits, lg_t, rtol=tol, atol=tol)
    # the final norm's gain matters at this size
    Tw1 = dict(Tw, norm_out=np.ones(32))
    _, _, l1 = O.target_verify_forward(cfg, Tw1, tokens, np.arange(n), _chain_anc(n), *_empty_kv(cfg, L, 16), 0,
                                       (1, 2, 3))
    assert np.max(np.abs(l1 - logits)) > 1e-3


def _sequential(cfg, Tw, prompt, path):
    """Decode prompt + path one token per call with a growing cache; returns
    the (features, logits) of the last call."""
    L = len(Tw["layers"])
    cap = len(prompt) + len(path) + 1
    Ks, Vs = _empty_kv(cfg, L, cap)
    seq = list(prompt) + list(path)
    out = None
    for i, tok in enumerate(seq):
        vis = np.zeros((1, cap + O.MAX_TREE_SLOTS), bool)
        vis[0, : i + 1] = True
        _, f, lg = O.target_forward(cfg, Tw, np.array([tok]), np.array([i]), Ks, Vs, np.array([i]), vis, (1, 2, 3))
        out = (f[0], lg[0])
    return out


def _prefill(cfg, Tw, prompt, cap):
    L = len(Tw["layers"])
    Ks, Vs = _empty_kv(cfg, L, cap)
    n = len(prompt)
    vis = np.tril(np.ones((n, cap + O.MAX_TREE_SLOTS), bool), 0)
    vis[:, n:] = False
    O.target_forward(cfg, Tw, np.array(prompt), np.arange(n), Ks, Vs, np.arange(n), vis, (1, 2, 3))
    return Ks, Vs


@pytest.mark.parametrize("m,depth,seed", [(6, 3, 0), (12, 4, 1), (9, 9, 2)])
def test_target_tree_rows_equal_sequential_decode(m, depth, seed):
    """Verify row i's logits and features equal a sequential decode of the
    committed prompt followed by node i's root path."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=40)
    Tw = _target(cfg, 3, seed=seed)
    prompt = [3, 1, 4, 1, 5]
    v_tok, v_par = gen.random_verify_tree(seed, m, 40, depth, root_tok=9)
    depth_of = [0] * (m + 1)
    anc = [1] + [0] * m
    for i in range(1, m + 1):
        depth_of[i] = depth_of[v_par[i]] + 1
        anc[i] = anc[v_par[i]] | (1 << i)
    ctx = len(prompt)
    Ks, Vs = _prefill(cfg, Tw, prompt, ctx + 4)
    _, feats, logits = O.target_verify_forward(cfg, Tw, v_tok, ctx + np.array(depth_of), anc, Ks, Vs, ctx, (1, 2, 3))
    for i in range(m + 1):
        path, n = [], i
        while n >= 0:
            path.append(int(v_tok[n]))
            n = int(v_par[n])
        f_seq, l_seq = _sequential(cfg, Tw, prompt, list(reversed(path)))
        np.testing.assert_allclose(logits[i], l_seq, rtol=1e-10, atol=1e-10, err_msg=f"row {i}")
        np.testing.assert_allclose(feats[i], f_seq, rtol=1e-10, atol=1e-10, err_msg=f"row {i}")


def test_target_layer_ranges_compose():
    """Layers 0..a then a..L from the carried state equal 0..L in one call."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=40, dtype=BF16)
    Tw = _target(cfg, 4, seed=3)
    v_tok, v_par = gen.random_verify_tree(5, 7, 40, 3, root_tok=2)
    anc = [1] + [0] * 7
    dep = [0] * 8
    for i in range(1, 8):
        anc[i] = anc[v_par[i]] | (1 << i)
        dep[i] = dep[v_par[i]] + 1
    pos = 6 + np.array(dep)
    Ks, Vs = _prefill(cfg, Tw, [1, 2, 3, 4, 5, 6], 8)
    h, f, lg = O.target_verify_forward(cfg, Tw, v_tok, pos, anc, [k.copy() for k in Ks], [v.copy() for v in Vs], 6,
                                       (1, 3, 4))
    K2, V2 = [k.copy() for k in Ks], [v.copy() for v in Vs]
    ha, fa, la = O.target_verify_forward(cfg, Tw, v_tok, pos, anc, K2, V2, 6, (1, 3, 4), 0, 2)
    assert la is None and np.isnan(fa[:, 1:]).all()
    hb, fb, lb = O.target_verify_forward(cfg, Tw, v_tok, pos, anc, K2, V2, 6, (1, 3, 4), 2, 4, h=ha)
    np.testing.assert_array_equal(hb, h)
    np.testing.assert_array_equal(lb, lg)
    np.testing.assert_array_equal(fa[:, 0], f[:, 0])
    np.testing.assert_array_equal(fb[:, 1:], f[:, 1:])


def _greedy_tree(cfg, Tw, seq, rng, m, depth, V):
    """A verify tree whose first branch follows the target's greedy
    continuation for a random number of steps; other nodes are random."""
    cont = []
    s = list(seq)
    n_true = int(rng.integers(0, depth + 1))
    for _ in range(n_true):
        _, lg = _sequential(cfg, Tw, s[:-1], [s[-1]])
        t = int(np.argmax(lg.astype(np.float32)))
        cont.append(t)
        s.append(t)
    v_tok, v_par = [int(seq[-1])], [-1]
    for j, t in enumerate(cont):          # the greedy spine: node j+1 is the child of node j
        v_tok.append(t)
        v_par.append(j)
    while len(v_tok) < m + 1:              # distractors under random nodes
        p = int(rng.integers(0, len(v_tok)))
        d = 0
        n = p
        while n > 0:
            d += 1
            n = v_par[n]
        if d >= depth:
            continue
        sib = {v_tok[c] for c in range(1, len(v_tok)) if v_par[c] == p}
        t = int(rng.integers(0, V))
        if t in sib:
            continue
        v_tok.append(t)
        v_par.append(p)
    # canonical order is not needed by the oracle's verify: parents come first
    return np.array(v_tok), np.array(v_par)


def test_greedy_verification_on_the_target_reproduces_target_greedy():
    """Cycles of (tree forward, greedy verify, KV commit) emit exactly the
    target's greedy continuation; the committed cache equals a fresh prefill
    of the committed sequence."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=12)
    Tw = _target(cfg, 2, seed=4, std=0.4)
    V = 12
    prompt = [1, 7, 3]
    n_new = 10
    ref = list(prompt)
    while len(ref) < len(prompt) + n_new + 1:
        _, lg = _sequential(cfg, Tw, ref[:-1], [ref[-1]])
        ref.append(int(np.argmax(lg.astype(np.float32))))
    cap = 40
    seq = list(prompt)
    Ks, Vs = _prefill(cfg, Tw, seq[:-1], cap)   # the last prompt token is the first root
    ctx = len(seq) - 1
    rng = np.random.default_rng(11)
    accepted_total = 0
    while len(seq) < len(prompt) + n_new:
        v_tok, v_par = _greedy_tree(cfg, Tw, seq, rng, m=7, depth=3, V=V)
        n = len(v_tok)
        anc, dep = [1] + [0] * (n - 1), [0] * n
        for i in range(1, n):
            anc[i] = anc[v_par[i]] | (1 << i)
            dep[i] = dep[v_par[i]] + 1
        _, feats, logits = O.target_verify_forward(cfg, Tw, v_tok, ctx + np.array(dep), anc, Ks, Vs, ctx, (1, 1, 2))
        acc, bonus = O.verify_greedy(v_tok, v_par, logits)
        accepted_total += len(acc)
        ctx = O.kv_commit(Ks, Vs, ctx, len(acc), acc)
        seq += [int(v_tok[a]) for a in acc] + [bonus]
        assert ctx == len(seq) - 1
    assert seq == ref[: len(seq)]
    assert accepted_total > 0            # the planted spines were taken
    K_ref, V_ref = _prefill(cfg, Tw, seq[:-1], cap)
    for l in range(2):
        np.testing.assert_allclose(Ks[l][:ctx], K_ref[l][:ctx], rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(Vs[l][:ctx], V_ref[l][:ctx], rtol=1e-10, atol=1e-10)
