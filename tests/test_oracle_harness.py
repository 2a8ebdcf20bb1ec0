"""Pins of the oracle's EAGLE-3.1 variants (FC norm, post-norm) and of the
EAGLE-4 Harness rules (harness_cost, harness_continue,
harness_verify_count, harness_branch_cap, harness_cycle) against things
other than themselves: torch's operators for the norms, closed forms of the
rules on linear and constant cost tables, and the plain draft cycle at the
thresholds that make every rule pass or fail."""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from workloads.configs import BF16, F32, tiny_shape

from test_oracle_pins import _torch_decoder_row_block, weights_f


def _gains(W, d, names, seed):
    g = np.random.default_rng(seed)
    for name in names:
        W[name] = 1.0 + 0.5 * g.standard_normal(d)
    return W


# ---------------------------------------------------------------- FC norm
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_fc_norm_matches_torch(dtype):
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=40, dtype=dtype)
    W = weights_f(cfg, std=0.2)
    gain = 1.0 + 0.5 * np.random.default_rng(3).standard_normal(32)
    feats = np.random.default_rng(4).standard_normal((5, 3, 32))
    if dtype == BF16:
        W["fc"] = O.bf16_round(W["fc"])
        feats = O.bf16_round(feats)
    g = O.fuse(cfg, feats, W["fc"], gain)
    t = torch.nn.functional.rms_norm(torch.nn.functional.linear(torch.as_tensor(feats.reshape(5, -1), dtype=torch.float64),
                                                                torch.as_tensor(W["fc"], dtype=torch.float64)),
                                     (32,), torch.as_tensor(gain), eps=cfg.rms_eps)
    if dtype == BF16:
        t = t.to(torch.bfloat16).to(torch.float64)
    np.testing.assert_allclose(g, t.numpy(), rtol=1e-12, atol=1e-12)
    # with unit gain the fused rows have unit RMS (up to eps) -- the norm is really applied
    cfg32 = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=40)
    g1 = O.fuse(cfg32, feats, W["fc"], np.ones(32))
    np.testing.assert_allclose(np.sqrt(np.mean(g1 ** 2, axis=1)), 1.0, rtol=1e-4)


# ---------------------------------------------------------------- post-norm
def _torch_post_norm_block(cfg, W, S, T, P, K, V, widx, vis, bf16=False):
    """The post-norm drafter layer with torch's operators: the pre-norm
    block's attention, then h1 = rms_norm(s + o a), FFN on h1 itself,
    h2 = rms_norm(h1 + ffn)."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    rnd = (lambda z: z.to(torch.bfloat16).to(torch.float64)) if bf16 else (lambda z: z)
    d, Hq, Hkv, hd, F, eps = cfg.d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.rms_eps
    R = len(T)
    rms = torch.nn.functional.rms_norm
    s = t(S)
    e = t(W["emb"])[torch.as_tensor(np.asarray(T, dtype=np.int64))]
    x = rnd(torch.cat([rms(e, (d,), t(W["norm_e"]), eps=eps), rms(s, (d,), t(W["norm_s"]), eps=eps)], 1))
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
    kk = Kt.repeat_interleave(rep, dim=1).transpose(0, 1)
    vv = Vt.repeat_interleave(rep, dim=1).transpose(0, 1)
    a = torch.empty(R, Hq, hd, dtype=torch.float64)
    for r in range(R):
        m = torch.as_tensor(vis[r])[None, None, :].expand(Hq, 1, -1)
        a[r] = torch.nn.functional.scaled_dot_product_attention(q[r][:, None, :], kk, vv, attn_mask=m)[:, 0]
    a = rnd(a.reshape(R, Hq * hd))
    h1 = rms(s + torch.nn.functional.linear(a, t(W["o"])), (d,), t(W["norm_post_attn"]), eps=eps)
    gu = torch.nn.functional.linear(rnd(h1), t(W["gate_up"]))
    z = rnd(torch.nn.functional.silu(gu[:, :F]) * gu[:, F:])
    h2 = rms(h1 + torch.nn.functional.linear(z, t(W["down"])), (d,), t(W["norm_post_ffn"]), eps=eps)
    y = rnd(rms(h2, (d,), t(W["norm_out"]), eps=eps))
    return h2.numpy(), torch.nn.functional.linear(y, t(W["lm"])).numpy()


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_post_norm_layer_matches_torch(dtype):
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=40, dtype=dtype)
    W = _gains(weights_f(cfg, std=0.2), 32, ("norm_e", "norm_s", "norm_ffn", "norm_out", "norm_post_attn",
                                             "norm_post_ffn"), 31)
    if dtype == BF16:
        W = {kk: (O.bf16_round(vv) if not kk.startswith("norm") else vv) for kk, vv in W.items()}
    g = np.random.default_rng(5)
    R, N = 4, 12
    K = g.standard_normal((N, 2, 8))
    V = g.standard_normal((N, 2, 8))
    if dtype == BF16:
        K, V = O.bf16_round(K), O.bf16_round(V)
    S = g.standard_normal((R, 32))
    T = np.array([3, 17, 0, 39])
    P = np.array([5, 9, 10, 11])
    widx = P.copy()
    vis = g.random((R, N)) < 0.5
    vis[np.arange(R), widx] = True
    h2, lg = O.decoder_rows(cfg, W, S, T, P, K.copy(), V.copy(), widx, vis)
    h2_t, lg_t = _torch_post_norm_block(cfg, W, S, T, P, K, V, widx, vis, bf16=(dtype == BF16))
    tol = 1e-10 if dtype == F32 else 1e-9
    np.testing.assert_allclose(h2, h2_t, rtol=tol, atol=tol)
    np.testing.assert_allclose(lg, lg_t, rtol=tol, atol=tol)
    # the state children receive has the post-norm's RMS: rms(h2 / gain) = 1
    np.testing.assert_allclose(np.sqrt(np.mean((h2 / W["norm_post_ffn"]) ** 2, axis=1)), 1.0, rtol=1e-4)
    # and differs from the pre-norm layer on the same inputs
    Wp = {kk: vv for kk, vv in W.items() if kk not in ("norm_post_attn", "norm_post_ffn")}
    h2p, _ = O.decoder_rows(cfg, Wp, S, T, P, K.copy(), V.copy(), widx, vis)
    h2pt, _, _, _ = _torch_decoder_row_block(cfg, Wp, S, T, P, K, V, widx, vis, Wp, bf16=(dtype == BF16))
    np.testing.assert_allclose(h2p, h2pt, rtol=tol, atol=tol)
    assert np.max(np.abs(h2p - h2)) > 1e-2


# ---------------------------------------------------------------- harness rules
def _table(draft_fn, verify_fn, batch=(1, 8, 64), ctx=(512, 2048, 8192), tok=(1, 2, 4, 8, 16, 32, 64)):
    return dict(batch=list(batch), ctx=list(ctx), tok=list(tok),
                draft=[[[draft_fn(b, c, n) for n in tok] for c in ctx] for b in batch],
                verify=[[[verify_fn(b, c, n) for n in tok] for c in ctx] for b in batch])


def test_cost_lookup_snaps_and_interpolates():
    tb = _table(lambda b, c, n: 1.0 + 0.01 * b + 1e-4 * c + 0.05 * n, lambda b, c, n: 2.0 + 0.1 * n * b)
    # measured points are returned exactly; tokens in between interpolate linearly (exact for a linear row)
    assert O.harness_cost(tb, O.DRAFT, 8, 2048, 4) == pytest.approx(1.0 + 0.08 + 0.2048 + 0.2)
    assert O.harness_cost(tb, O.DRAFT, 8, 2048, 6) == pytest.approx(1.0 + 0.08 + 0.2048 + 0.3)
    # batch 5 and context 1000 take the next measured values up (8, 2048)
    assert O.harness_cost(tb, O.DRAFT, 5, 1000, 6) == pytest.approx(1.0 + 0.08 + 0.2048 + 0.3)
    # beyond the table: the largest bucket; tokens clamp to the measured range
    assert O.harness_cost(tb, O.VERIFY, 100, 9000, 200) == pytest.approx(2.0 + 0.1 * 64 * 64)
    assert O.harness_cost(tb, O.VERIFY, 1, 1, 0) == pytest.approx(2.0 + 0.1)


@pytest.mark.parametrize("tau,slope", [(0.5, 0.2), (3.0, 0.05), (0.0, 0.1), (1e9, 0.1)])
def test_verify_count_closed_form_on_linear_cost(tau, slope):
    """With T_verify linear in the rows (slope per row), every extra rank
    costs `slope`, so the count is the length of the leading run of ranks
    whose summed confidence exceeds tau * slope."""
    tb = _table(lambda b, c, n: 1.0, lambda b, c, n: 0.7 + slope * n)
    rng = np.random.default_rng(7)
    for B in (1, 3):
        lc = np.sort(np.log(rng.uniform(0.01, 1.0, size=(B, 40))), axis=1)[:, ::-1].astype(np.float32)
        sums = np.exp(lc.astype(np.float64)).sum(axis=0)
        ok = sums > tau * slope
        want = int(np.argmin(ok)) if not ok.all() else len(ok)
        assert O.harness_verify_count(tb, B, 1000, lc, tau) == want


def test_continue_and_branch_cap_closed_forms():
    tb = _table(lambda b, c, n: 0.5 * n, lambda b, c, n: 1.0)
    front = np.log(np.array([[0.5, 0.25, 0.125, 0.0625]], np.float32))
    gain = 0.9375
    # draft time of a round of k = 4 rows: 2.0 ms; threshold tau0 (1 + alpha depth)
    for depth in (1, 3, 5):
        for tau0, alpha in ((0.1, 0.5), (0.2, 1.0), (0.05, 2.0)):
            go, gains = O.harness_continue(tb, 1, 100, 4, depth, front, tau0, alpha)
            assert go == (gain / 2.0 > tau0 * (1 + alpha * depth))
            np.testing.assert_allclose(gains, [gain], rtol=1e-6)
    # branch cap: ranks 5..8 of the root (probabilities 0.04 each) vs the extra 2 ms of 8 rows instead of 4
    lp = np.log(np.array([[0.3, 0.2, 0.1, 0.1, 0.04, 0.04, 0.04, 0.04]], np.float32))
    assert O.harness_branch_cap(tb, 1, 100, lp, 0.079) == 8
    assert O.harness_branch_cap(tb, 1, 100, lp, 0.081) == 4
    # a heavier load (cost per extra row grows with the batch) drops to 4 at the same threshold
    tb2 = _table(lambda b, c, n: 0.5 * n * (1 if b < 8 else 4), lambda b, c, n: 1.0)
    lp8 = np.repeat(lp, 8, axis=0)
    assert O.harness_branch_cap(tb2, 1, 100, lp, 0.05) == 8
    assert O.harness_branch_cap(tb2, 8, 100, lp8, 0.2) == 4


def test_harness_cycle_at_extreme_thresholds_is_the_plain_cycle():
    """Thresholds every rule passes give the plain cycle with k = 8, D = D_max
    and m = m_max; thresholds every rule fails give k = 4, one round and the
    single best node."""
    cfg = tiny_shape(d=32, hq=4, hkv=2, hd=8, ffn=48, vocab=64)
    W = weights_f(cfg, std=0.3)
    tb = _table(lambda b, c, n: 0.1 * n, lambda b, c, n: 0.2 * n)
    rng = np.random.default_rng(2)
    feats = rng.standard_normal((3, 3, 32)) * 0.3
    tokens = np.array([5, 9, 11])
    Kc = np.zeros((3, 2, 8)); Vc = np.zeros((3, 2, 8))
    vt, info = O.harness_cycle(cfg, W, feats, tokens, Kc, Vc, 0, tb, m_max=20, D_max=3, tau_depth0=0.0,
                               tau_alpha=0.0, tau_verify=0.0, tau_branch=0.0)
    assert info == dict(k=8, rounds=3, m=20)
    ref = O.draft_cycle(cfg, W, feats, tokens, Kc, Vc, 0, 8, 3, 20)
    for key in ("tok", "parent", "depth", "pos", "anc"):
        np.testing.assert_array_equal(vt[key], ref[key])
    vt, info = O.harness_cycle(cfg, W, feats, tokens, Kc, Vc, 0, tb, m_max=20, D_max=3, tau_depth0=1e9,
                               tau_alpha=0.0, tau_verify=1e9, tau_branch=1e9)
    assert info == dict(k=4, rounds=1, m=1)
    ref = O.draft_cycle(cfg, W, feats, tokens, Kc, Vc, 0, 4, 1, 1)
    for key in ("tok", "parent", "depth", "pos", "anc"):
        np.testing.assert_array_equal(vt[key], ref[key])
