"""Pins of the CPU oracle: each test ties an oracle function to something
other than itself (a library routine, a closed form, an invariant of the
method, or brute force on tiny inputs)."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import BF16, F32, tiny_shape


def weights_f(shape, seed=0, std=0.02):
    Wt = gen.gen_weights(shape, seed=seed, std=std)
    return {k: (v.f32() if hasattr(v, "f32") else v) for k, v in Wt.items()}


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_matches_torch_conversion():
    """torch's float32 -> bfloat16 cast rounds to nearest even."""
    g = np.random.default_rng(5)
    x = (g.standard_normal(200000) * np.exp(g.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7 -> even mantissa (1.0)
    assert O.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is the midpoint of 1+2^-7 and 1+2^-6 -> even mantissa (1+2^-6)
    assert O.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.bf16_round(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    # just above the midpoint rounds up
    assert O.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7


def test_generator_bf16_bits_match_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 3
    bits = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


# ---------------------------------------------------------------- fusion
def test_fuse_is_block_sum_of_three_layers():
    """g = W_low f_low + W_mid f_mid + W_high f_high, W_fc = [W_low|W_mid|W_high]:
    pins the concat order of the three features against the fused matrix."""
    cfg = tiny_shape(d=24)
    g = np.random.default_rng(2)
    W = g.standard_normal((24, 72))
    f = g.standard_normal((5, 3, 24))
    ref = sum(f[:, i, :] @ W[:, 24 * i: 24 * (i + 1)].T for i in range(3))
    np.testing.assert_allclose(O.fuse(cfg, f, W), ref, rtol=1e-13, atol=1e-13)
    lin = torch.nn.functional.linear(torch.from_numpy(f.reshape(5, 72)), torch.from_numpy(W)).numpy()
    np.testing.assert_allclose(O.fuse(cfg, f, W), lin, rtol=1e-13, atol=1e-13)


def test_fuse_bf16_output_is_rounded():
    cfg = tiny_shape(d=16, dtype=BF16)
    g = np.random.default_rng(3)
    W = g.standard_normal((16, 48))
    f = g.standard_normal((4, 3, 16))
    out = O.fuse(cfg, f, W)
    exact = f.reshape(4, 48) @ W.T
    ref = torch.from_numpy(exact.astype(np.float64)).to(torch.bfloat16).double().numpy()
    # direct fp64 -> bf16 rounding equals torch's unless fp64->fp32 double-rounding bites
    assert np.mean(out == ref) > 0.999
    assert np.max(np.abs(out - exact) / np.abs(exact)) <= 2.0 ** -8


# ---------------------------------------------------------------- norms, RoPE
def test_rmsnorm_matches_torch():
    v = np.random.default_rng(4).standard_normal((7, 33))
    gain = np.random.default_rng(5).standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (33,), torch.from_numpy(gain), eps=1e-5).numpy()
    np.testing.assert_allclose(O.rmsnorm(v, gain, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_rope_identity_at_zero_and_norm_preserving():
    x = np.random.default_rng(6).standard_normal((3, 4, 16))
    np.testing.assert_allclose(O.rope(x, np.zeros(3), 10000.0), x, atol=0)
    y = O.rope(x, np.array([5, 77, 4096]), 500000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    g = np.random.default_rng(7)
    q = g.standard_normal((1, 1, 32))
    k = g.standard_normal((1, 1, 32))
    for theta in (10000.0, 500000.0):
        base = (O.rope(q, [9], theta) * O.rope(k, [4], theta)).sum()
        for shift in (1, 100, 3000):
            s = (O.rope(q, [9 + shift], theta) * O.rope(k, [4 + shift], theta)).sum()
            assert abs(s - base) < 1e-9


def test_rope_equals_complex_rotation_of_half_pairs():
    """Rotate-half RoPE: (a_i + i b_i) * exp(i p theta^(-2i/hd))."""
    g = np.random.default_rng(8)
    x = g.standard_normal((1, 2, 16))
    p = 37
    z = x[..., :8] + 1j * x[..., 8:]
    w = z * np.exp(1j * p * 500000.0 ** (-np.arange(0, 16, 2) / 16.0))
    ref = np.concatenate([w.real, w.imag], axis=-1)
    np.testing.assert_allclose(O.rope(x, [p], 500000.0), ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- attention / decoder
def _layer_setup(cfg, seed=0, std=0.2):
    return weights_f(cfg, seed=seed, std=std)


def test_decoder_attention_matches_torch_sdpa_with_gqa():
    """The attention inside decoder_rows equals torch's SDPA (fp64) on the same
    q/k/v with each KV head repeated Hq/Hkv times (GQA == MHA with repeats)."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=16)
    W = _layer_setup(cfg)
    g = np.random.default_rng(9)
    R, N = 3, 10
    K = g.standard_normal((N, 2, 8))
    V = g.standard_normal((N, 2, 8))
    S = g.standard_normal((R, 32))
    T = np.array([1, 5, 7])
    P = np.array([7, 8, 9])
    vis = g.random((R, N)) < 0.6
    widx = np.array([7, 8, 9])
    vis[np.arange(R), widx] = True
    Kc, Vc = K.copy(), V.copy()
    h2, _ = O.decoder_rows(cfg, W, S, T, P, Kc, Vc, widx, vis)
    # recompute q by hand-free route: project, rope; run SDPA; push through the rest
    eps = cfg.rms_eps
    x = np.concatenate([O.rmsnorm(W["emb"][T], 1, eps), O.rmsnorm(S, 1, eps)], axis=1)
    q = O.rope((x @ W["qkv"].T)[:, :32].reshape(R, 4, 8), P, cfg.rope_theta)
    kr = np.repeat(Kc, 2, axis=1)   # head h uses kv head h // 2
    vr = np.repeat(Vc, 2, axis=1)
    out = np.empty((R, 4, 8))
    for r in range(R):
        qq = torch.from_numpy(q[r][:, None, :])               # [H, 1, hd]
        kk = torch.from_numpy(kr.transpose(1, 0, 2).copy())     # [H, N, hd]
        vv = torch.from_numpy(vr.transpose(1, 0, 2).copy())
        m = torch.from_numpy(vis[r][None, None, :].repeat(4, 0))
        out[r] = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m)[:, 0].numpy()
    h1 = S + out.reshape(R, 32) @ W["o"].T
    u = O.rmsnorm(h1, 1, eps)
    gu = u @ W["gate_up"].T
    h2_ref = h1 + (torch.nn.functional.silu(torch.from_numpy(gu[:, :48])).numpy() * gu[:, 48:]) @ W["down"].T
    np.testing.assert_allclose(h2, h2_ref, rtol=1e-10, atol=1e-10)


def _torch_decoder_row_block(cfg, W, S, T, P, K, V, widx, vis, gains, bf16=False):
    """The drafter layer written with torch's own operators, independent of
    the oracle: rms_norm with each gain where it belongs, linear, RoPE as a
    complex rotation of the half pairs, scaled_dot_product_attention with a
    boolean mask and the KV heads repeated, silu.  With bf16=True the values
    are cast to bfloat16 at the rounding points (x, q/k/v, a, u, the SwiGLU
    output, the normalised final state)."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    rnd = (lambda z: z.to(torch.bfloat16).to(torch.float64)) if bf16 else (lambda z: z)
    d, Hq, Hkv, hd, F, eps = cfg.d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.rms_eps
    R = len(T)
    s = t(S)
    e = t(W["emb"])[torch.as_tensor(np.asarray(T, dtype=np.int64))]
    rms = torch.nn.functional.rms_norm
    x = rnd(torch.cat([rms(e, (d,), t(gains["norm_e"]), eps=eps), rms(s, (d,), t(gains["norm_s"]), eps=eps)], 1))
    qkv = torch.nn.functional.linear(x, t(W["qkv"]))

    def rot(z, pos):
        zc = torch.complex(z[..., : hd // 2], z[..., hd // 2:])
        ang = t(pos)[:, None, None] * cfg.rope_theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
        w = zc * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([w.real, w.imag], -1)
    q = rnd(rot(qkv[:, : Hq * hd].reshape(R, Hq, hd), P))
    k = rnd(rot(qkv[:, Hq * hd:(Hq + Hkv) * hd].reshape(R, Hkv, hd), P))
    v = rnd(qkv[:, (Hq + Hkv) * hd:].reshape(R, Hkv, hd))
    Kt, Vt = t(K).clone(), t(V).clone()
    Kt[torch.as_tensor(widx)] = k
    Vt[torch.as_tensor(widx)] = v
    rep = Hq // Hkv
    kk = Kt.repeat_interleave(rep, dim=1).transpose(0, 1)   # [Hq, N, hd]
    vv = Vt.repeat_interleave(rep, dim=1).transpose(0, 1)
    a = torch.empty(R, Hq, hd, dtype=torch.float64)
    for r in range(R):
        m = torch.as_tensor(vis[r])[None, None, :].expand(Hq, 1, -1)
        a[r] = torch.nn.functional.scaled_dot_product_attention(q[r][:, None, :], kk, vv, attn_mask=m)[:, 0]
    a = rnd(a.reshape(R, Hq * hd))
    h1 = s + torch.nn.functional.linear(a, t(W["o"]))
    u = rnd(rms(h1, (d,), t(gains["norm_ffn"]), eps=eps))
    gu = torch.nn.functional.linear(u, t(W["gate_up"]))
    z = rnd(torch.nn.functional.silu(gu[:, :F]) * gu[:, F:])
    h2 = h1 + torch.nn.functional.linear(z, t(W["down"]))
    y = rnd(rms(h2, (d,), t(gains["norm_out"]), eps=eps))
    logits = torch.nn.functional.linear(y, t(W["lm"]))
    return h2.numpy(), logits.numpy(), Kt.numpy(), Vt.numpy()


@pytest.mark.parametrize("dtype,hkv", [(F32, 2), (F32, 4), (BF16, 1)])
def test_decoder_layer_and_lm_head_match_torch_with_distinct_gains(dtype, hkv):
    """decoder_rows (state h2, the K/V it writes and the LM-head logits)
    equals the same layer written with torch's operators.  Every RMSNorm gain
    is a different random vector, so feeding the LM head the wrong state
    (h1 for h2), a gain to the wrong norm or a missing final norm fails."""
    cfg = tiny_shape(d=32, hq=4, hkv=hkv, hd=8, ffn=48, vocab=40, dtype=dtype)
    W = _layer_setup(cfg)
    g = np.random.default_rng(31)
    for name in ("norm_e", "norm_s", "norm_ffn", "norm_out"):
        W[name] = 1.0 + 0.5 * g.standard_normal(32)
    if dtype == BF16:
        W = {kk: (O.bf16_round(vv) if not kk.startswith("norm") else vv) for kk, vv in W.items()}
    R, N = 4, 12
    K = g.standard_normal((N, hkv, 8))
    V = g.standard_normal((N, hkv, 8))
    if dtype == BF16:
        K, V = O.bf16_round(K), O.bf16_round(V)
    S = g.standard_normal((R, 32))
    T = np.array([3, 17, 0, 39])
    P = np.array([5, 9, 10, 11])
    widx = np.array([5, 9, 10, 11])
    vis = g.random((R, N)) < 0.5
    vis[np.arange(R), widx] = True
    Kc, Vc = K.copy(), V.copy()
    h2, logits = O.decoder_rows(cfg, W, S, T, P, Kc, Vc, widx, vis)
    h2_t, lg_t, K_t, V_t = _torch_decoder_row_block(cfg, W, S, T, P, K, V, widx, vis, W, bf16=(dtype == BF16))
    tol = 1e-10 if dtype == F32 else 1e-9
    np.testing.assert_allclose(Kc, K_t, rtol=tol, atol=tol)
    np.testing.assert_allclose(Vc, V_t, rtol=tol, atol=tol)
    np.testing.assert_allclose(h2, h2_t, rtol=tol, atol=tol)
    np.testing.assert_allclose(logits, lg_t, rtol=tol, atol=tol)
    # the gains matter at this size: unit gains give other logits
    W1 = dict(W, norm_out=np.ones(32))
    _, l1 = O.decoder_rows(cfg, W1, S, T, P, K.copy(), V.copy(), widx, vis)
    assert np.max(np.abs(l1 - logits)) > 1e-3


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_gather_paged_equals_contiguous(bs):
    """A request's rows scattered block by block into shuffled physical
    blocks of a shared pool come back in logical order, and attention over
    the gathered rows equals attention over the contiguous rows."""
    g = np.random.default_rng(40 + bs)
    Hkv, hd, L = 2, 8, 53
    nb_req = -(-L // bs)
    n_blocks = 3 * nb_req + 5
    contig_k = g.standard_normal((L, Hkv, hd))
    contig_v = g.standard_normal((L, Hkv, hd))
    pool_k = g.standard_normal((n_blocks, bs, Hkv, hd))   # other requests' data everywhere else
    pool_v = g.standard_normal((n_blocks, bs, Hkv, hd))
    table = g.permutation(n_blocks)[:nb_req].astype(np.int32)
    for j in range(nb_req):   # logical block j -> physical block table[j]
        rows = contig_k[j * bs:(j + 1) * bs]
        pool_k[table[j], : len(rows)] = rows
        pool_v[table[j], : len(rows)] = contig_v[j * bs:(j + 1) * bs]
    gk = O.gather_paged(pool_k, table, L, bs)
    gv = O.gather_paged(pool_v, table, L, bs)
    np.testing.assert_array_equal(gk, contig_k)
    np.testing.assert_array_equal(gv, contig_v)
    cfg = tiny_shape(d=32, hq=4, hkv=Hkv, hd=hd, ffn=48, vocab=16)
    W = _layer_setup(cfg)
    S = g.standard_normal((2, 32))
    vis = np.zeros((2, L + 2), bool)
    vis[0, : L + 1] = True
    vis[1, : L + 2] = True
    outs = []
    for K0, V0 in ((contig_k, contig_v), (gk, gv)):
        K = np.zeros((L + 2, Hkv, hd)); V = np.zeros((L + 2, Hkv, hd))
        K[:L], V[:L] = K0, V0
        outs.append(O.decoder_rows(cfg, W, S, [1, 2], [L, L + 1], K, V, [L, L + 1], vis))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_commit_in_two_batches_equals_one_batch():
    """Causal commit is incremental: rows [0,a) then [a,n) == rows [0,n) at once."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=16)
    W = _layer_setup(cfg)
    g = np.random.default_rng(10)
    n, a = 9, 4
    S = g.standard_normal((n, 32))
    T = g.integers(0, 16, n)
    P = np.arange(n)
    K1 = np.zeros((n, 2, 8)); V1 = np.zeros((n, 2, 8))
    vis = np.tril(np.ones((n, n), bool))
    h_all, l_all = O.decoder_rows(cfg, W, S, T, P, K1, V1, P, vis)
    K2 = np.zeros((n, 2, 8)); V2 = np.zeros((n, 2, 8))
    h_a, l_a = O.decoder_rows(cfg, W, S[:a], T[:a], P[:a], K2, V2, P[:a], vis[:a])
    h_b, l_b = O.decoder_rows(cfg, W, S[a:], T[a:], P[a:], K2, V2, P[a:], vis[a:])
    np.testing.assert_allclose(np.vstack([h_a, h_b]), h_all, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.vstack([l_a, l_b]), l_all, rtol=1e-12, atol=1e-12)


def test_decoder_invariant_to_global_position_shift():
    """All keys produced by the model at shifted positions: RoPE makes the
    output depend only on relative positions."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=16)
    W = _layer_setup(cfg)
    g = np.random.default_rng(11)
    n = 6
    S = g.standard_normal((n, 32)); T = g.integers(0, 16, n)
    vis = np.tril(np.ones((n, n), bool))
    outs = []
    for shift in (0, 1000):
        K = np.zeros((n, 2, 8)); V = np.zeros((n, 2, 8))
        P = np.arange(n) + shift
        outs.append(O.decoder_rows(cfg, W, S, T, P, K, V, np.arange(n), vis))
    np.testing.assert_allclose(outs[0][0], outs[1][0], rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------- top-k
def test_topk_matches_bruteforce_and_scipy():
    g = np.random.default_rng(12)
    for trial in range(50):
        V = int(g.integers(5, 300))
        l = np.round(g.standard_normal(V) * 2, 1)   # many exact ties
        k = int(g.integers(1, min(V, 16) + 1))
        ids, lp, lse = O.topk_logprobs(l, k)
        brute = sorted(range(V), key=lambda y: (-np.float32(l[y]), y))[:k]
        assert list(ids) == brute
        assert abs(float(lse) - logsumexp(l.astype(np.float32).astype(np.float64))) < 1e-5
        assert np.all(lp <= 0)
        np.testing.assert_allclose(np.exp(lp.astype(np.float64)),
                                   softmax(l.astype(np.float32).astype(np.float64))[ids], rtol=1e-5)


# ---------------------------------------------------------------- dynamic tree
def _table_drafter(V, seed, sigma=1.5):
    """A drafter stand-in: log-probs as a deterministic function of the path."""
    cache = {}

    def lp_of(path):
        key = tuple(path)
        if key not in cache:
            h = abs(hash((seed,) + key)) % (2 ** 32)
            l = np.random.default_rng(h).standard_normal(V) * sigma
            cache[key] = l
        return cache[key]
    return lp_of


def _build_tree_with_table(V, k, D, m, seed):
    lp_of = _table_drafter(V, seed)
    root = (0,)
    tree = O.DynamicTree(k, D, 0, 100)
    ids, lp, _ = O.topk_logprobs(lp_of(root), k)
    tree.init(ids, lp)
    paths = {}
    for j in range(2, D + 1):
        rows_ids, rows_lp = [], []
        for n in tree.frontier:
            path = _path(tree, n)
            i2, l2, _ = O.topk_logprobs(lp_of(root + path), k)
            rows_ids.append(i2); rows_lp.append(l2)
        tree.step(np.array(rows_ids), np.array(rows_lp))
    return tree, tree.final(m), lp_of


def _path(tree, n):
    out = []
    while n >= 0:
        out.append(tree.tok[n])
        n = tree.parent[n]
    return tuple(reversed(out))


@pytest.mark.parametrize("V,k,D,m,seed", [(6, 2, 3, 5, 0), (5, 3, 3, 9, 1), (7, 3, 4, 12, 2), (4, 4, 3, 20, 3)])
def test_tree_equals_literal_beam_enumeration(V, k, D, m, seed):
    """Brute force: enumerate the beam by hand over explicit paths with fp64
    cumulative log-probs and compare pool, frontiers and the kept set."""
    tree, vt, lp_of = _build_tree_with_table(V, k, D, m, seed)
    root = (0,)

    def lps(path):
        l = lp_of(root + path).astype(np.float32).astype(np.float64)
        return l - logsumexp(l)

    # literal beam: level 1 = the k best tokens; then each level's k best of k*k children
    level = sorted(range(V), key=lambda y: (-np.float32(lp_of(root)[y]), y))[:k]
    level = [((y,), lps(())[y]) for y in level]
    pool = list(level)
    for j in range(2, D + 1):
        cands = []
        for rho, (path, sc) in enumerate(level):
            l = lp_of(root + path)
            kids = sorted(range(V), key=lambda y: (-np.float32(l[y]), y))[:k]
            for i, y in enumerate(kids):
                cands.append((path + (y,), sc + lps(path)[y], rho * k + i))
        pool += [(p, s) for p, s, _ in cands]
        cands.sort(key=lambda c: (-c[1], c[2]))
        level = [(p, s) for p, s, _ in cands[:k]]
    got_pool = {_path(tree, n): float(tree.score[n]) for n in range(len(tree.tok))}
    assert len(got_pool) == len(pool) == k + (D - 1) * k * k
    for p, s in pool:
        assert abs(got_pool[p] - s) < 1e-4
    # kept set = the m best of the pool (fp64 scores; ties cannot occur with continuous draws)
    best = sorted(pool, key=lambda t: (-t[1], len(t[0])))[:m]
    kept_paths = set()
    for i in range(1, m + 1):
        path = []
        n = i
        while n > 0:
            path.append(int(vt["tok"][n])); n = int(vt["parent"][n])
        kept_paths.add(tuple(reversed(path)))
    assert kept_paths == {p for p, _ in best}


def test_tree_final_canonical_order_and_bitsets():
    tree, vt, _ = _build_tree_with_table(9, 3, 4, 15, 7)
    par, dep, anc, pos = vt["parent"], vt["depth"], vt["anc"], vt["pos"]
    assert par[0] == -1 and dep[0] == 0
    for i in range(1, len(par)):
        assert par[i] < i and dep[i] == dep[par[i]] + 1 and pos[i] == 100 + dep[i]
        assert int(anc[i]) == (int(anc[par[i]]) | (1 << i))
        if i > 1:
            assert (dep[i - 1], par[i - 1]) <= (dep[i], par[i])
    # siblings have distinct tokens
    for p in set(par[1:].tolist()):
        toks = vt["tok"][par == p]
        assert len(set(toks.tolist())) == len(toks)


def test_tree_ties_prefer_shallow_and_low_flat():
    """Exact ties: child score == parent score (lp = 0) keeps the parent first;
    equal-score siblings keep the lower flat index."""
    k, D = 2, 3
    tree = O.DynamicTree(k, D, 0, 0)
    tree.init(np.array([3, 4]), np.array([-1.0, -1.0], np.float32))
    tree.step(np.array([[5, 6], [7, 8]]), np.array([[0.0, -2.0], [0.0, -2.0]], np.float32))
    assert tree.frontier == [2, 4]          # flat 0 and 2 (tied scores, lower flat first)
    tree.step(np.array([[9, 10], [11, 12]]), np.array([[-0.5, -0.5], [-0.5, -0.5]], np.float32))
    vt = tree.final(3)
    # best: depth-1 {3,4} (score -1) tie with depth-2 {5,7} (-1) -> shallow first
    assert sorted(vt["tok"][1:].tolist()) == [3, 4, 5]


def test_k1_tree_is_greedy_chain():
    """k = 1: every kept node is the argmax of its parent's distribution."""
    V = 11
    tree, vt, lp_of = _build_tree_with_table(V, 1, 5, 4, 9)
    path = ()
    for i in range(1, 5):
        y = int(np.argmax(lp_of((0,) + path).astype(np.float32)))
        assert int(vt["tok"][i]) == y and int(vt["parent"][i]) == i - 1
        path += (y,)


# ---------------------------------------------------------------- verification
def _hash_target(V, seed, sigma=2.0):
    cache = {}

    def logits(seq):
        key = tuple(int(t) for t in seq)
        if key not in cache:
            h = abs(hash((seed, 1) + key)) % (2 ** 32)
            cache[key] = (np.random.default_rng(h).standard_normal(V) * sigma).astype(np.float32)
        return cache[key]
    return logits


def _feats_for(seq, d, seed):
    h = abs(hash((seed, 2) + tuple(int(t) for t in seq))) % (2 ** 32)
    return np.random.default_rng(h).standard_normal((3, d)) * 0.5


@pytest.mark.parametrize("k,D,m", [(2, 3, 5), (3, 2, 6), (1, 4, 3)])
def test_greedy_speculative_decoding_reproduces_target_greedy(k, D, m):
    """Multi-cycle draft + greedy verify against a deterministic hash target
    emits exactly the target's own greedy sequence, whatever the drafter."""
    cfg = tiny_shape(d=16, hq=2, hkv=1, hd=8, ffn=32, vocab=8)
    W = weights_f(cfg, std=0.3)
    tgt = _hash_target(8, seed=k * 10 + D)
    prompt = [1, 4, 2]
    n_new = 14
    ref = list(prompt)
    while len(ref) < len(prompt) + n_new:
        ref.append(int(np.argmax(tgt(ref))))
    seq = list(prompt)
    accepted_total = 0
    while len(seq) < len(prompt) + n_new:
        feats = np.stack([_feats_for(seq[: i + 1], 16, 0) for i in range(len(seq))])
        Kc = np.zeros((len(seq), 1, 8)); Vc = np.zeros((len(seq), 1, 8))
        vt = O.draft_cycle(cfg, W, feats, np.array(seq), Kc, Vc, 0, k, D, m)
        L = []
        for i in range(len(vt["tok"])):
            path = []
            n = i
            while n > 0:
                path.append(int(vt["tok"][n])); n = int(vt["parent"][n])
            L.append(tgt(seq + list(reversed(path))))
        acc, bonus = O.verify_greedy(vt["tok"], vt["parent"], np.array(L))
        accepted_total += len(acc)
        seq += [int(vt["tok"][a]) for a in acc] + [bonus]
    assert seq[: len(ref)] == ref


def test_sampling_accept_threshold_is_target_probability():
    """With one candidate x, the acceptance boundary in u_try is p(x) (found
    by bisection on the oracle's decision)."""
    g = np.random.default_rng(13)
    for trial in range(20):
        V = 6
        L = (g.standard_normal((2, V)) * 2).astype(np.float32)
        x = int(g.integers(V))
        T = float(g.choice([0.7, 1.0, 1.6]))
        v_tok = np.array([0, x]); v_par = np.array([-1, 0])
        lo, hi = 0.0, 1.0
        for _ in range(60):
            mid = (lo + hi) / 2
            acc, _ = O.verify_sample(v_tok, v_par, L, [0.0, mid], [0.5, 0.5], T)
            lo, hi = (mid, hi) if acc else (lo, mid)
        p = softmax(L[0].astype(np.float64) / T)[x]
        assert abs(lo - p) < 1e-12


def test_sampling_residual_cdf_breakpoints():
    """After rejecting x, the bonus as a function of u_res switches at the
    cumulative residual distribution p(y)/(1-p(x)) over y != x, in id order."""
    g = np.random.default_rng(14)
    V = 5
    L = (g.standard_normal((2, V)) * 1.5).astype(np.float32)
    x = 2
    v_tok = np.array([0, x]); v_par = np.array([-1, 0])
    p = softmax(L[0].astype(np.float64))
    res = p.copy(); res[x] = 0; res /= res.sum()
    cdf = np.cumsum(res)
    for y in range(V):
        if y == x:
            continue
        below = cdf[y] - res[y]
        # just inside the y interval
        for u in (below + 1e-9, cdf[y] - 1e-9):
            _, b = O.verify_sample(v_tok, v_par, L, [0.0, 0.999999999], [u, 0.5])
            assert b == y


def _enumerate_target_dist(tgt, prefix, n, V, T):
    """Target's own distribution over the next n tokens (library softmax)."""
    out = {}

    def rec(seq, prob, left):
        if left == 0:
            out[tuple(seq[len(prefix):])] = prob
            return
        p = softmax(tgt(seq).astype(np.float64) / T)
        for y in range(V):
            rec(seq + [y], prob * p[y], left - 1)
    rec(list(prefix), 1.0, n)
    return out


def test_sampling_verify_preserves_target_distribution_montecarlo():
    """The first emitted token follows p exactly; the first two emitted
    tokens follow the target's joint distribution (chi-square over 2e5
    seeded runs on V=4 and a depth-2 tree)."""
    V, T = 4, 1.0
    tgt = _hash_target(V, seed=77, sigma=1.2)
    prefix = [0]
    # a fixed depth-2 tree: root -> {1, 3}; node(1) -> {2}; node(3) -> {0, 1}
    v_tok = np.array([0, 1, 3, 2, 0, 1]); v_par = np.array([-1, 0, 0, 1, 2, 2])
    L = []
    for i in range(len(v_tok)):
        path, n = [], i
        while n > 0:
            path.append(int(v_tok[n])); n = int(v_par[n])
        L.append(tgt(prefix + list(reversed(path))))
    L = np.array(L)
    target = _enumerate_target_dist(tgt, prefix, 2, V, T)
    g = np.random.default_rng(15)
    N = 200000
    counts = {}
    for _ in range(N):
        acc, bonus = O.verify_sample(v_tok, v_par, L, g.random(6), g.random(6), T)
        toks = [int(v_tok[a]) for a in acc] + [bonus]
        if len(toks) < 2:
            # extend with the target's own sampler at the bonus position
            p = softmax(tgt(prefix + toks).astype(np.float64) / T)
            toks.append(int(g.choice(V, p=p)))
        key = tuple(toks[:2])
        counts[key] = counts.get(key, 0) + 1
    chi2 = 0.0
    for key, pr in target.items():
        e = N * pr
        chi2 += (counts.get(key, 0) - e) ** 2 / e
    # 15 degrees of freedom: the 1e-4 upper quantile is about 44
    assert chi2 < 44.0, chi2


def _bisect(pred, lo=0.0, hi=1.0):
    """sup{u in [lo, hi] : pred(u)} for a predicate true below a threshold."""
    if not pred(lo):
        return lo
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if mid in (lo, hi):
            break
        lo, hi = (mid, hi) if pred(mid) else (lo, mid)
    return lo


def _enumerate_verify_outcomes(run, v_tok, v_par, V):
    """Exact distribution of (accepted nodes, bonus) of a verifier `run(u_try,
    u_res) -> (accepted, bonus)` over independent U(0,1) uniforms.

    Along any walk each uniform is consulted at most once: u_try[c] when
    child c is tried (accepted below a threshold), u_res[n] at the node
    where the walk stops (the bonus is non-decreasing in it).  Each
    threshold is found by bisection on `run` itself, with the uniforms
    already decided held inside their intervals, so the probability of an
    outcome is the product of its interval lengths."""
    M = len(v_tok)
    kids = {}
    for c in range(1, M):
        kids.setdefault(int(v_par[c]), []).append(c)
    out = {}

    def visit(node, acc, ut, ur, prob):
        ut = ut.copy()
        for c in kids.get(node, []):
            def accepts(u, c=c):
                t = ut.copy(); t[c] = u
                a, _ = run(t, ur)
                return len(a) > len(acc) and a[len(acc)] == c
            th = _bisect(accepts)
            if th > 0.0:
                t = ut.copy(); t[c] = 0.5 * th
                visit(c, acc + [c], t, ur, prob * th)
            prob *= (1.0 - th)
            ut[c] = 0.5 * (1.0 + th)
            if prob == 0.0:
                return
        lo = 0.0
        for y in range(V):
            def at_most(u, y=y):
                r = ur.copy(); r[node] = u
                a, b = run(ut, r)
                assert a == acc
                return b <= y
            hi = 1.0 if y == V - 1 else _bisect(at_most)
            if hi > lo:
                key = (tuple(acc), y)
                out[key] = out.get(key, 0.0) + prob * (hi - lo)
                lo = hi
    visit(0, [], np.full(M, 0.5), np.full(M, 0.5), 1.0)
    return out


def _first_tokens_distribution(outcomes, v_tok, p_next, n):
    """Distribution of the first n emitted tokens when every cycle after this
    one samples from the target (p_next(seq) = target probabilities after
    the sequence): an outcome emitting fewer than n tokens is continued by
    the target."""
    dist = {}

    def extend(seq, pr):
        if len(seq) >= n:
            key = tuple(seq[:n])
            dist[key] = dist.get(key, 0.0) + pr
            return
        p = p_next(seq)
        for y in range(len(p)):
            if p[y] > 0:
                extend(seq + [y], pr * p[y])
    for (acc, bonus), pr in outcomes.items():
        extend([int(v_tok[a]) for a in acc] + [bonus], pr)
    return dist


@pytest.mark.parametrize("T,tree", [
    (1.0, ([0, 1, 3, 2, 0, 1], [-1, 0, 0, 1, 2, 2])),    # depth 2, siblings of 2 and 1 children
    (0.7, ([0, 4, 2, 0, 3, 1], [-1, 0, 0, 0, 1, 1])),     # three root children
    (1.6, ([0, 2, 2, 1], [-1, 0, 1, 1])),                 # a chain node with two children
    (1.0, ([0, 3], [-1, 0])),                             # one candidate
])
def test_sampling_verify_exact_enumeration_preserves_target(T, tree):
    """Exact enumeration on V = 5, depth <= 2: the probability of every
    sequence of emitted tokens equals the target's autoregressive
    probability to 1e-12.  A target logit of -inf (probability 0) is part of
    the vocabulary.  The same enumeration of a verifier that draws the bonus
    from p instead of the residual (a plausible mistake) is off by far more."""
    V = 5
    v_tok, v_par = np.array(tree[0]), np.array(tree[1])
    tgt = _hash_target(V, seed=int(T * 10) + len(v_tok), sigma=1.3)

    def logits_after(seq):
        l = tgt(seq).copy()
        if len(seq) == 2:
            l[4] = -np.inf     # one token impossible after some prefixes
        return l

    def p_next(seq):
        return softmax(logits_after([0] + list(seq)).astype(np.float64) / T)
    L = []
    for i in range(len(v_tok)):
        path, nd = [], i
        while nd > 0:
            path.append(int(v_tok[nd])); nd = int(v_par[nd])
        L.append(logits_after([0] + list(reversed(path))))
    L = np.array(L)
    run = lambda ut, ur: O.verify_sample(v_tok, v_par, L, ut, ur, T)
    outcomes = _enumerate_verify_outcomes(run, v_tok, v_par, V)
    assert abs(sum(outcomes.values()) - 1.0) < 1e-12
    depth = int(max(len(a) for a, _ in outcomes)) + 1
    got = _first_tokens_distribution(outcomes, v_tok, p_next, depth)
    for seq in set(got) | set(_first_tokens_distribution({((), y): p_next([])[y] for y in range(V)},
                                                          v_tok, p_next, depth)):
        ref = 1.0
        for i in range(len(seq)):
            ref *= p_next(list(seq[:i]))[seq[i]]
        assert abs(got.get(seq, 0.0) - ref) <= 1e-12, (seq, got.get(seq, 0.0), ref)

    def no_residual(ut, ur):
        """Mistaken verifier: after rejections the bonus is drawn from p itself."""
        acc, b = O.verify_sample(v_tok, v_par, L, ut, ur, T)
        node = acc[-1] if acc else 0
        leaf_tok, leaf_par = np.array([v_tok[node]]), np.array([-1])
        _, b2 = O.verify_sample(leaf_tok, leaf_par, L[node:node + 1], ut[:1], ur[node:node + 1], T)
        return acc, b2
    bad = _first_tokens_distribution(_enumerate_verify_outcomes(no_residual, v_tok, v_par, V), v_tok, p_next,
                                     depth)
    err = 0.0
    for seq, pr in bad.items():
        ref = 1.0
        for i in range(len(seq)):
            ref *= p_next(list(seq[:i]))[seq[i]]
        err = max(err, abs(pr - ref))
    assert err > 1e-3


def test_sampling_wrong_rule_is_detected():
    """A plausible mistake (dropping the residual correction: bonus drawn from
    p instead of p with rejected tokens removed) fails the same test."""
    V, T = 3, 1.0
    L = np.array([[1.5, 0.1, -0.4], [0.0, 0.0, 0.0]], np.float32)
    v_tok = np.array([0, 0]); v_par = np.array([-1, 0])
    p = softmax(L[0].astype(np.float64))
    g = np.random.default_rng(16)
    N = 100000
    c_good = np.zeros(V)
    c_bad = np.zeros(V)
    for _ in range(N):
        ut, ur = g.random(2), g.random(2)
        acc, b = O.verify_sample(v_tok, v_par, L, ut, ur, T)
        c_good[0 if acc else b] += 1
        # mistaken variant: on rejection sample the bonus from p itself
        if ut[1] < p[0]:
            c_bad[0] += 1
        else:
            c_bad[int(np.searchsorted(np.cumsum(p), ur[0], side="right"))] += 1
    e = N * p
    assert ((c_good - e) ** 2 / e).sum() < 25
    assert ((c_bad - e) ** 2 / e).sum() > 100


# ---------------------------------------------------------------- golden fixtures
def test_golden_verify_fixtures():
    import json, os
    path = os.path.join(os.path.dirname(__file__), "golden", "verify_small.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        L = np.array(c["logits"], np.float32)
        if c["mode"] == "greedy":
            acc, b = O.verify_greedy(np.array(c["tok"]), np.array(c["parent"]), L)
        else:
            acc, b = O.verify_sample(np.array(c["tok"]), np.array(c["parent"]), L,
                                     c["u_try"], c["u_res"], c.get("T", 1.0))
        assert acc == c["expect_accepted"] and b == c["expect_bonus"], c["name"]


# ---------------------------------------------------------------- TTT
def _ttt_setup(S=10, V=12, R=4, seed=0, dtype=F32):
    cfg = tiny_shape(d=16, hq=2, hkv=1, hd=8, ffn=24, vocab=V, dtype=dtype)
    W = weights_f(cfg, std=0.3)
    g = np.random.default_rng(seed)
    feats = g.standard_normal((S, 3, 16))
    toks = g.integers(0, V, S)
    return cfg, W, feats, toks


def test_ttt_no_peek_at_future_ground_truth():
    """Changing x_{i'} and F_{i'} for i' > i leaves every prediction at (j, i)
    unchanged; only CE moves (through its label)."""
    cfg, W, feats, toks = _ttt_setup()
    R, S, i = 4, 10, 4
    a = O.ttt_forward_full(cfg, W, feats, toks, R)
    feats2 = feats.copy(); toks2 = toks.copy()
    feats2[i + 1:] += 1.7
    toks2[i + 1:] = (toks2[i + 1:] + 3) % 12
    b = O.ttt_forward_full(cfg, W, feats2, toks2, R)
    np.testing.assert_array_equal(a["logits"][:, : i + 1], b["logits"][:, : i + 1])
    np.testing.assert_array_equal(a["pred"][:, : i + 1], b["pred"][:, : i + 1])
    assert not np.array_equal(a["logits"][:, i + 1:], b["logits"][:, i + 1:])


def test_ttt_step_j_equals_greedy_chain_round_j():
    """logits(j, i) == round j of a k = 1 greedy chain rooted at commit row i."""
    cfg, W, feats, toks = _ttt_setup(S=8, V=12, R=4)
    R = 4
    full = O.ttt_forward_full(cfg, W, feats, toks, R)
    for i in (0, 3, 7):
        rec = {}
        n = i + 1
        Kc = np.zeros((n, 1, 8)); Vc = np.zeros((n, 1, 8))
        O.draft_cycle(cfg, W, feats[:n], toks[:n], Kc, Vc, 0, 1, R, R - 1, record=rec)
        np.testing.assert_allclose(rec["commit_logits"][-1], full["logits"][0, i], rtol=1e-10, atol=1e-10)
        for j in range(2, R + 1):
            np.testing.assert_allclose(rec["rounds"][j - 2]["logits"][0], full["logits"][j - 1, i],
                                       rtol=1e-10, atol=1e-10)


def test_ttt_sampled_positions_equal_full():
    cfg, W, feats, toks = _ttt_setup(S=9, V=12, R=4, dtype=BF16)
    full = O.ttt_forward_full(cfg, W, feats, toks, 4)
    part = O.ttt_forward(cfg, W, feats, toks, 4, positions=[2, 6, 8])
    for col, i in enumerate([2, 6, 8]):
        np.testing.assert_array_equal(part["pred"][:, col], full["pred"][:, i])
        np.testing.assert_allclose(part["ce"][:, col], full["ce"][:, i], rtol=1e-12, atol=1e-12)


def test_ttt_forced_tokens_and_ce_matches_torch():
    cfg, W, feats, toks = _ttt_setup(S=8, V=12, R=3)
    forced = np.random.default_rng(3).integers(0, 12, (2, 8))
    out = O.ttt_forward_full(cfg, W, feats, toks, 3, forced=forced)
    for j in range(3):
        for i in range(8):
            if i + j + 1 <= 7:
                l = torch.from_numpy(out["logits"][j, i].astype(np.float32).astype(np.float64))[None]
                ce = torch.nn.functional.cross_entropy(l, torch.tensor([int(toks[i + j + 1])])).item()
                assert abs(out["ce"][j, i] - ce) < 1e-9
    # forced tokens really are fed: step-2 equals a chain whose depth-1 token is forced
    sampled = O.ttt_forward(cfg, W, feats, toks, 3, forced=forced, positions=[5])
    np.testing.assert_array_equal(sampled["pred"][:, 0], out["pred"][:, 5])
    assert out["valid"].sum() == sum(max(0, 8 - j) for j in range(1, 4))


# ---------------------------------------------------------------- tree == sequential decode
@pytest.mark.parametrize("dtype,k,D,m,hkv", [(F32, 2, 3, 8, 4), (F32, 3, 4, 14, 2), (BF16, 2, 4, 9, 1)])
def test_tree_nodes_equal_sequential_decode_along_root_path(dtype, k, D, m, hkv):
    """Each drafted tree node's h2 and logits equal a plain sequential decode
    of its root path: one row per step, causal cache, position root_pos + s.
    Pins the ancestor-bitset tree mask, the slot layout and the state hand-off."""
    cfg = tiny_shape(d=32, hq=4, hkv=hkv, hd=8, ffn=48, vocab=24, dtype=dtype)
    W = weights_f(cfg, std=0.25)
    g = np.random.default_rng(21)
    n = 6
    feats = g.standard_normal((n, 3, 32)) * 0.5
    toks = g.integers(0, 24, n)
    cap = n
    Kc = np.zeros((cap, hkv, 8)); Vc = np.zeros((cap, hkv, 8))
    rec = {}
    O.draft_cycle(cfg, W, feats, toks, Kc, Vc, 0, k, D, m, record=rec)
    tree = rec["tree"]
    g_fused = O.fuse(cfg, feats, W["fc"])
    checked = 0
    for node in range(len(tree.tok)):
        if tree.slot[node] < 0:
            continue
        path = []
        p = node
        while p >= 0:
            path.append(p); p = tree.parent[p]
        path.reverse()
        # plain causal decode: commit rows, then one row per path node
        N = n + len(path)
        K = np.zeros((N, hkv, 8)); V = np.zeros((N, hkv, 8))
        vis = np.tril(np.ones((n, N), bool))
        h, _ = O.decoder_rows(cfg, W, g_fused, toks, np.arange(n), K, V, np.arange(n), vis)
        s = h[-1:]
        for step, pn in enumerate(path, start=1):
            row = n + step - 1
            vis1 = np.zeros((1, N), bool); vis1[0, : row + 1] = True
            s, lg = O.decoder_rows(cfg, W, s, [tree.tok[pn]], [n - 1 + step], K, V, [row], vis1)
        j = tree.depth[node]
        rho = tree.slot[node] - (j - 1) * k
        rd = rec["rounds"][j - 1]
        tol = 1e-10
        np.testing.assert_allclose(rd["h2"][rho], s[0], rtol=tol, atol=tol)
        np.testing.assert_allclose(rd["logits"][rho], lg[0], rtol=tol, atol=tol)
        checked += 1
    assert checked == (D - 1) * k


# ---------------------------------------------------------------- efficient LM head (EAGLE-4)
def _bf16_setup(V=300, d=32, seed=50):
    cfg = tiny_shape(d=d, hq=4, hkv=2, hd=8, ffn=48, vocab=V, dtype=BF16)
    W = weights_f(cfg, std=0.3)
    g = np.random.default_rng(seed)
    y = O.bf16_round(g.standard_normal(d))
    return cfg, W, g, y


@pytest.mark.parametrize("c", [300, 40, 7])
def test_efficient_head_with_exact_factors_is_the_full_head(c):
    """Special case: B = I (rank d) and A = W_lm make the stage-1 scores the
    exact logits (z = y is already bf16), so the candidates are the exact
    top-c (brute force) and the top-k is the full head's top-k; the
    log-probs differ from the full head's by the log of the candidates'
    share of the softmax mass (scipy logsumexp), and equal them at c = V."""
    cfg, W, g, y = _bf16_setup()
    k = 5
    ids, lp, cand, cl = O.efficient_head_topk(cfg, W, y, W["lm"], np.eye(32), c, k)
    lm = np.asarray(W["lm"], np.float64)
    exact = torch.nn.functional.linear(torch.from_numpy(y[None]), torch.from_numpy(lm)).numpy()[0]
    e32 = exact.astype(np.float32)
    brute = sorted(range(300), key=lambda t: (-e32[t], t))
    assert list(cand) == brute[:c]
    assert list(ids) == brute[:k]
    np.testing.assert_allclose(cl, exact[cand], rtol=1e-12, atol=1e-12)
    full_ids, full_lp, _ = O.topk_logprobs(exact, k)
    assert list(full_ids) == list(ids)
    shift = logsumexp(e32.astype(np.float64)) - logsumexp(e32[np.array(brute[:c])].astype(np.float64))
    np.testing.assert_allclose(lp.astype(np.float64), full_lp.astype(np.float64) + shift, atol=2e-6)
    if c == 300:
        np.testing.assert_array_equal(lp, full_lp)


def test_efficient_head_stages_match_torch_and_brute_force():
    """Random low-rank factors: the candidates are the brute-force top-c of
    the low-rank scores computed with torch (z cast to bf16 between the two
    products), the candidate logits equal torch's linear on the gathered LM
    rows, and the top-k is the brute-force order of those logits."""
    cfg, W, g, y = _bf16_setup(seed=51)
    r, c, k = 8, 24, 6
    A = O.bf16_round(g.standard_normal((300, r)))
    Bm = O.bf16_round(g.standard_normal((r, 32)) * 0.3)
    ids, lp, cand, cl = O.efficient_head_topk(cfg, W, y, A, Bm, c, k)
    yt = torch.from_numpy(y[None])
    z = torch.nn.functional.linear(yt, torch.from_numpy(Bm)).to(torch.bfloat16).double()
    sc = torch.nn.functional.linear(z, torch.from_numpy(A)).numpy()[0].astype(np.float32)
    brute = sorted(range(300), key=lambda t: (-sc[t], t))[:c]
    assert list(cand) == brute
    exact_c = torch.nn.functional.linear(yt, torch.from_numpy(np.asarray(W["lm"][np.array(brute)], np.float64))).numpy()[0]
    np.testing.assert_allclose(cl, exact_c, rtol=1e-12, atol=1e-12)
    e32 = exact_c.astype(np.float32)
    order = sorted(range(c), key=lambda i: (-e32[i], brute[i]))[:k]
    assert list(ids) == [brute[i] for i in order]
    np.testing.assert_allclose(np.exp(lp.astype(np.float64)), softmax(e32.astype(np.float64))[order], rtol=1e-5)


def test_efficient_head_ties_take_lowest_ids():
    """An all-zero low-rank head scores every token equal: the candidates
    are the c lowest ids, in id order."""
    cfg, W, g, y = _bf16_setup(seed=52)
    ids, lp, cand, cl = O.efficient_head_topk(cfg, W, y, np.zeros((300, 8)), np.zeros((8, 32)), 20, 4)
    assert list(cand) == list(range(20))
    assert set(ids.tolist()) <= set(range(20))


def test_draft_cycle_with_exact_factor_head_equals_full_head():
    """A whole draft cycle through the efficient head with B = I, A = W_lm
    and c = V builds the same tree as the full head."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=40, dtype=BF16)
    W = {kk: (O.bf16_round(vv) if not kk.startswith("norm") else vv) for kk, vv in weights_f(cfg, std=0.25).items()}
    g = np.random.default_rng(53)
    n = 5
    feats = O.bf16_round(g.standard_normal((n, 3, 32)) * 0.5)
    toks = g.integers(0, 40, n)
    Kc = np.zeros((n, 2, 8)); Vc = np.zeros((n, 2, 8))
    a = O.draft_cycle(cfg, W, feats, toks, Kc, Vc, 0, 3, 3, 7)
    b = O.draft_cycle(cfg, W, feats, toks, Kc, Vc, 0, 3, 3, 7, head=dict(A=W["lm"], B=np.eye(32), c=40))
    for name in ("tok", "parent", "depth", "pos", "anc"):
        np.testing.assert_array_equal(a[name], b[name])
