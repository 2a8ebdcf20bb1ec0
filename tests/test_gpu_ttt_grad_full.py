"""The training-time-test backward at the benchmark's sizes.

* At the 8B drafter's full shape (d 4096, 32/8 heads, ffn 14336, vocab
  128256) on a slice the oracle can afford (one sequence of 64 tokens, five
  forced steps): every gradient against the fp64 autograd oracle, within
  twice the distance of the oracle's fp32-product, bf16-gradient variant from
  it, in relative Frobenius norm (at least the tolerance of
  test_gpu_ttt_grad) and in the largest entry.
* At the benchmark's full size (8 x 2048 tokens, five self-fed steps, packed
  weights: the launch configuration bench.py times), properties that hold at
  any size:
  - the forward outputs equal eagle3_ttt_forward's bit for bit;
  - batch additivity: the batch's gradients are the mean of the eight
    single-sequence runs' (the loss's divisor is 8x, the dlogits scale by an
    exact power of two, each row's arithmetic is independent of the batch,
    so only fp32 summation order differs);
  - first-order Taylor agreement (forced tokens, so no argmax choice jumps):
    for a random direction in the fp32 gains and in W_o, the central
    difference of the forward's loss equals the gradient's inner product with
    the perturbation.
"""
import numpy as np
import pytest
import torch

from oracle import ttt_grad as G
from workloads import gen
from workloads.configs import C5_8B_TTT

from gpu_cases import dev_i32, host_weights, say
from test_gpu_ttt_grad import compare_grads

pytestmark = pytest.mark.gpu


def _train(dr, B, S, R, feats, tokens, forced=None):
    from eagle_draft_tree_amd.train import TTTTrain
    tr = TTTTrain(dr, B, S, R)
    tr.run(feats, tokens, forced)
    torch.cuda.synchronize()
    out = (tr.pred.cpu().numpy(), tr.ce.cpu().numpy(), float(tr.loss.item()),
           {n: g.cpu().numpy() for n, g in tr.grads.items()})
    del tr
    torch.cuda.empty_cache()
    return out


def _forward_loss(dr, B, S, R, feats, tokens, forced=None):
    from eagle_draft_tree_amd import binding as Bd
    pred = torch.empty(B, R, S, dtype=torch.int32, device="cuda")
    ce = torch.empty(B, R, S, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(Bd.ttt_workspace_size(dr.dims, B, S, R), dtype=torch.uint8, device="cuda")
    Bd.eagle3_ttt_forward(dr.dims, dr.weights, feats, tokens, B, S, R, forced, pred, ce, loss, ws)
    torch.cuda.synchronize()
    return pred.cpu().numpy(), ce.cpu().numpy(), float(loss.item())


@pytest.mark.timeout(900)
def test_c5_train_full_model_shape_vs_oracle(lib):
    from eagle_draft_tree_amd.cycle import Drafter
    s = C5_8B_TTT.shape
    B, S, R = 1, 64, C5_8B_TTT.ttt_steps
    say("TTT train at the 8B shape: weights")
    Wt = gen.gen_weights(s, seed=0)
    Wt.update(gen.gen_drafter_gains(s, seed=1))
    ti = gen.gen_ttt_inputs(s, B, S, R, seed=2)
    dr = Drafter(s, Wt, pack=True)
    say("GPU train B", B, "S", S, "R", R, "forced")
    gp, gce, gloss, gg = _train(dr, B, S, R, ti.feats.torch("cuda"), dev_i32(ti.tokens), dev_i32(ti.forced))
    del dr
    torch.cuda.empty_cache()
    say("oracle (fp64 autograd), and its fp32-product, bf16-gradient variant")
    W = host_weights(Wt)
    ref = G.ttt_loss_and_grads(s, W, ti.feats.f32(), ti.tokens, R, forced=ti.forced)
    var = G.ttt_loss_and_grads(s, W, ti.feats.f32(), ti.tokens, R, forced=ti.forced, grad_bf16=True, gemm_f32=True)
    # At d = 4096 the forward's own bf16 roundings (fp32 products rounding
    # now and then to the other neighbour) move every gradient by several
    # 1e-3; the variant shows how far: the GPU may lie twice as far.
    bounds = {n: 2 * np.linalg.norm(var["grads"][n] - ref["grads"][n]) / np.linalg.norm(ref["grads"][n])
              for n in G.TRAINED}
    abs_bounds = {n: 2 * np.abs(var["grads"][n] - ref["grads"][n]).max() for n in G.TRAINED}
    np.testing.assert_allclose(gloss, ref["loss"], rtol=1e-2, atol=2e-2)
    compare_grads({n: g.astype(np.float64) for n, g in gg.items()}, ref["grads"], "8B-shape", bounds, abs_bounds)


@pytest.mark.timeout(900)
def test_c5_train_full_size_properties(lib):
    from eagle_draft_tree_amd.cycle import Drafter
    w = C5_8B_TTT
    s = w.shape
    B, S, R = w.batch, w.ttt_seq, w.ttt_steps
    say("full-size TTT train: weights")
    Wt = gen.gen_weights(s, seed=0)
    Wt.update(gen.gen_drafter_gains(s, seed=1))
    ti = gen.gen_ttt_inputs(s, B, S, R, seed=1)
    feats = ti.feats.torch("cuda")
    tokens = dev_i32(ti.tokens)
    dr = Drafter(s, Wt, pack=True)
    say("GPU train B", B, "S", S, "R", R, "self-fed")
    gp, gce, gloss, gg = _train(dr, B, S, R, feats, tokens)
    for n, g in gg.items():
        assert np.all(np.isfinite(g)), n
        assert np.any(g != 0), n
    fp, fce, floss = _forward_loss(dr, B, S, R, feats, tokens)
    np.testing.assert_array_equal(gp, fp)
    np.testing.assert_array_equal(gce, fce)
    assert gloss == floss

    say("batch additivity: eight single-sequence runs")
    acc = {n: np.zeros(g.shape, np.float64) for n, g in gg.items()}
    for b in range(B):
        pb, ceb, lb, gb = _train(dr, 1, S, R, feats[b:b + 1].contiguous(), tokens[b:b + 1].contiguous())
        np.testing.assert_array_equal(pb[0], gp[b])
        np.testing.assert_array_equal(ceb[0], gce[b])
        for n in acc:
            acc[n] += gb[n]
    for n in acc:
        mean = acc[n] / B
        rel = np.linalg.norm(gg[n] - mean) / np.linalg.norm(mean)
        say(f"  {n}: rel {rel:.2e}")
        assert rel < 1e-4, (n, rel)

    say("first-order Taylor checks on the forward's loss (forced tokens: no argmax jumps)")
    g = torch.Generator().manual_seed(11)
    del dr
    torch.cuda.empty_cache()
    dr = Drafter(s, Wt, pack=False)   # row-major: perturb weights in place
    forced = dev_i32(ti.forced)
    gg = _train(dr, B, S, R, feats, tokens, forced)[3]
    # The step follows the gradient's signs, so the loss moves by ~1e-2, far
    # above the bf16 forward's rounding noise (~1e-4 on the loss); a gradient
    # entry of the wrong size or sign shows as a mismatch.  Gains (fp32) move
    # by 1e-2; bf16 matrices move by 2^-5 of each entry (8 bf16 steps) on a
    # random 2 % of the entries.
    bad = []
    for name in G.TRAINED:
        base = dr.tensors[name].clone()
        b64 = base.to("cpu", torch.float64)
        sg = torch.sign(torch.from_numpy(gg[name]).to(torch.float64))
        if name.startswith("norm_"):
            step = 1e-2 * sg
        else:
            mask = (torch.rand(b64.shape, generator=g, dtype=torch.float64) < 0.02).to(torch.float64)
            step = 2.0 ** -5 * b64.abs() * sg * mask
        plus = (b64 + step).to(base.dtype)
        minus = (b64 - step).to(base.dtype)
        dr.tensors[name].copy_(plus.to("cuda"))
        lp = _forward_loss(dr, B, S, R, feats, tokens, forced)[2]
        dr.tensors[name].copy_(minus.to("cuda"))
        lm = _forward_loss(dr, B, S, R, feats, tokens, forced)[2]
        dr.tensors[name].copy_(base)
        actual = plus.to(torch.float64) - minus.to(torch.float64)
        pred_change = float((torch.from_numpy(gg[name]).to(torch.float64) * actual).sum())
        say(f"  {name}: loss change {lp - lm:.6e} predicted {pred_change:.6e}")
        if not abs((lp - lm) - pred_change) <= 0.03 * abs(pred_change) + 5e-5:
            bad.append(name)
    assert not bad, bad
