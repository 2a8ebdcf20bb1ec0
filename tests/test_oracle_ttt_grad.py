"""Pins of the TTT gradient oracle (oracle/ttt_grad.py) against what the
mathematics fixes, independently of the oracle's own autograd graph:

* its forward (loss, CE, predictions, float32 logits) equals the NumPy TTT
  forward ``eagle3_oracle.ttt_forward_full``, which has its own pins;
* every trained parameter's gradient equals central finite differences of
  that NumPy forward's loss (fp32 drafter, so the loss is smooth), with
  forced and with self-fed (argmax) tokens -- the argmax choices are checked
  not to move under the perturbation;
* the bf16 straight-through gradient (R43) stays within bf16 rounding scale
  of the same finite differences;
* the batch loss's gradient is the mean of the per-sequence ones (equal
  valid counts), and a batch without labels trains nothing.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import eagle3_oracle as O
from oracle import ttt_grad as G
from workloads import gen
from workloads.configs import BF16, F32, tiny_shape


def _setup(dtype=F32, B=2, S=10, R=4, V=12, seed=0):
    cfg = tiny_shape(d=16, hq=4, hkv=2, hd=8, ffn=24, vocab=V, dtype=dtype)
    Wt = gen.gen_weights(cfg, seed=seed, std=0.3)
    W = {k: (v.f32() if hasattr(v, "f32") else v).astype(np.float64) for k, v in Wt.items()}
    W.update({k: v.astype(np.float64) for k, v in gen.gen_drafter_gains(cfg, seed + 1).items()})
    g = np.random.default_rng(seed + 2)
    feats = g.standard_normal((B, S, 3, cfg.d))
    if dtype == BF16:
        feats = O.bf16_round(feats)
    toks = g.integers(0, V, (B, S))
    forced = g.integers(0, V, (B, R - 1, S))
    return cfg, W, feats, toks, forced


def _numpy_loss(cfg, W, feats, toks, R, forced):
    """Mean valid CE of the NumPy forward, taken on its fp64 logits (its own
    CE reads float32 logits, whose rounding would swamp a finite difference)."""
    tot, cnt, preds = 0.0, 0, []
    S = toks.shape[1]
    for b in range(len(toks)):
        o = O.ttt_forward_full(cfg, W, feats[b], toks[b], R, forced=None if forced is None else forced[b])
        n = 0
        for j in range(R):
            for i in range(S - j - 1):
                row = o["logits"][j, i]
                tot += logsumexp(row) - row[toks[b, i + j + 1]]
                n += 1
        assert n == int(o["valid"].sum())
        cnt += n
        preds.append(o["pred"])
    return tot / cnt, np.array(preds)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("use_forced", [False, True])
def test_forward_equals_numpy_forward(dtype, use_forced):
    cfg, W, feats, toks, forced = _setup(dtype)
    R = 4
    fz = forced if use_forced else None
    out = G.ttt_loss_and_grads(cfg, W, feats, toks, R, forced=fz, want_grads=False)
    for b in range(len(toks)):
        o = O.ttt_forward_full(cfg, W, feats[b], toks[b], R, forced=None if fz is None else fz[b])
        np.testing.assert_array_equal(out["pred"][b], o["pred"])
        np.testing.assert_allclose(out["ce"][b], o["ce"], rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.array(out["logits"][b]), o["logits"].astype(np.float32).astype(np.float64))
    ref = np.mean([O.ttt_forward_full(cfg, W, feats[b], toks[b], R, forced=None if fz is None else fz[b])["ce"]
                   [:, :].sum() for b in range(len(toks))])
    cnt = sum(max(toks.shape[1] - j, 0) for j in range(1, R + 1))
    assert abs(out["loss"] - ref / cnt) < 1e-12


def _fd_check(cfg, W, feats, toks, R, forced, grads, rtol, atol, n_per=10, seed=7, h=1e-5):
    g = np.random.default_rng(seed)
    _, pred0 = _numpy_loss(cfg, W, feats, toks, R, forced)
    worst = 0.0
    for name in G.TRAINED:
        flat = W[name].reshape(-1)
        idx = g.choice(flat.size, size=min(n_per, flat.size), replace=False)
        for e in idx:
            old = flat[e]
            flat[e] = old + h
            lp, pp = _numpy_loss(cfg, W, feats, toks, R, forced)
            flat[e] = old - h
            lm, pm = _numpy_loss(cfg, W, feats, toks, R, forced)
            flat[e] = old
            if forced is None:   # the self-fed tokens must not move under the perturbation
                np.testing.assert_array_equal(pp, pred0)
                np.testing.assert_array_equal(pm, pred0)
            fd = (lp - lm) / (2 * h)
            an = grads[name].reshape(-1)[e]
            assert abs(an - fd) <= atol + rtol * abs(fd), f"{name}[{e}]: autograd {an} fd {fd}"
            worst = max(worst, abs(an - fd))
    return worst


@pytest.mark.parametrize("use_forced", [True, False])
def test_fp32_gradients_equal_finite_differences(use_forced):
    cfg, W, feats, toks, forced = _setup(F32)
    R = 4
    fz = forced if use_forced else None
    out = G.ttt_loss_and_grads(cfg, W, feats, toks, R, forced=fz)
    _fd_check(cfg, W, feats, toks, R, fz, out["grads"], rtol=1e-6, atol=1e-9)


def test_single_step_gradients_equal_finite_differences():
    """R = 1: plain teacher-forced CE of one decoder layer."""
    cfg, W, feats, toks, _ = _setup(F32, B=1, S=9)
    out = G.ttt_loss_and_grads(cfg, W, feats, toks, 1)
    _fd_check(cfg, W, feats, toks, 1, None, out["grads"], rtol=1e-6, atol=1e-9, n_per=6)


def test_bf16_straight_through_gradients_are_near_the_exact_ones():
    """R43: the bf16 forward's straight-through gradient is the derivative of
    the unrounded layer at rounded values, so it lies within bf16 rounding
    scale of the exact gradient of the same (bf16-valued) weights."""
    cfg32, W, feats, toks, forced = _setup(F32)
    cfg16 = tiny_shape(d=16, hq=4, hkv=2, hd=8, ffn=24, vocab=12, dtype=BF16)
    feats = O.bf16_round(feats)
    ex = G.ttt_loss_and_grads(cfg32, W, feats, toks, 4, forced=forced)["grads"]
    st = G.ttt_loss_and_grads(cfg16, W, feats, toks, 4, forced=forced)["grads"]
    for name in G.TRAINED:
        rel = np.linalg.norm(st[name] - ex[name]) / np.linalg.norm(ex[name])
        assert 0 < rel < 3e-2, (name, rel)


def test_batch_gradient_is_mean_of_sequence_gradients():
    cfg, W, feats, toks, forced = _setup(F32, B=3)
    R = 3
    full = G.ttt_loss_and_grads(cfg, W, feats, toks, R, forced=forced[:, : R - 1])["grads"]
    parts = [G.ttt_loss_and_grads(cfg, W, feats[b:b + 1], toks[b:b + 1], R, forced=forced[b:b + 1, : R - 1])["grads"]
             for b in range(3)]
    for name in G.TRAINED:
        np.testing.assert_allclose(full[name], sum(p[name] for p in parts) / 3, rtol=1e-12, atol=1e-15)


def test_no_valid_label_gives_zero_gradient():
    """S = 1: no row has a label, the loss is 0 and nothing is trained."""
    cfg, W, feats, toks, _ = _setup(F32, B=1, S=1)
    out = G.ttt_loss_and_grads(cfg, W, feats, toks, 2)
    assert out["loss"] == 0.0
    for name in G.TRAINED:
        assert not np.any(out["grads"][name])


def test_precision_variants_stay_near_the_exact_gradient():
    """The bf16-gradient and fp32-product variants (tolerance calibration
    only) move the bf16 drafter's gradients by rounding-sized amounts."""
    cfg, W, feats, toks, forced = _setup(BF16)
    ex = G.ttt_loss_and_grads(cfg, W, feats, toks, 4, forced=forced)
    for kw in (dict(grad_bf16=True), dict(gemm_f32=True), dict(grad_bf16=True, gemm_f32=True)):
        va = G.ttt_loss_and_grads(cfg, W, feats, toks, 4, forced=forced, **kw)
        assert abs(va["loss"] - ex["loss"]) < 1e-3
        for name in G.TRAINED:
            rel = np.linalg.norm(va["grads"][name] - ex["grads"][name]) / np.linalg.norm(ex["grads"][name])
            assert 0 < rel < 2e-2, (kw, name, rel)
