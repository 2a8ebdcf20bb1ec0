"""GPU parity of the training-time-test backward (eagle3_ttt_train) against
the gradient oracle (oracle/ttt_grad.py, fp64 autograd with straight-through
bf16 roundings) on the same seeded inputs and weights, with non-unit gains.

Tolerance (per gradient tensor): the GPU rounds every gradient tensor that
feeds a GEMM to bf16 (dlogits, dh2, d(gate, up), dh1, dO, dqkv, d g), one
relative error of up to 2^-9 per element per rounding, and sums up to R*B*S
rows in fp32.  Each rounding perturbs a gradient by about 2^-9 / sqrt(n)
relative over n independent terms; with the seven roundings chained over R
steps the relative Frobenius error stays well under 1e-2, the bound tested
(REL).  Elementwise, entries must agree to ABS_FRAC of the tensor's largest
entry plus REL of their own size.  Forward outputs (loss, predictions, CE)
are those of eagle3_ttt_forward and are checked to match it bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import ttt_grad as G
from workloads import gen
from workloads.configs import BF16, tiny_shape

from gpu_cases import dev_i32, host_weights, say

pytestmark = pytest.mark.gpu

REL = 1e-2        # relative Frobenius error per gradient tensor
ABS_FRAC = 5e-3   # elementwise: |gpu - ref| <= ABS_FRAC * max|ref| + 4 * REL * |ref|


def _weights(shape, seed):
    Wt = gen.gen_weights(shape, seed=seed)
    Wt.update(gen.gen_drafter_gains(shape, seed=seed + 1))
    return Wt


def run_gpu_train(shape, Wt, ti, B, S, R, forced, pack):
    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.cycle import Drafter
    from eagle_draft_tree_amd.train import TTTTrain
    dr = Drafter(shape, Wt, pack=pack)
    tr = TTTTrain(dr, B, S, R)
    tr.run(ti.feats.torch("cuda"), dev_i32(ti.tokens), dev_i32(ti.forced) if forced else None)
    torch.cuda.synchronize()
    # the plain forward on the same inputs
    pred = torch.empty(B, R, S, dtype=torch.int32, device="cuda")
    ce = torch.empty(B, R, S, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(Bd.ttt_workspace_size(dr.dims, B, S, R), dtype=torch.uint8, device="cuda")
    Bd.eagle3_ttt_forward(dr.dims, dr.weights, ti.feats.torch("cuda"), dev_i32(ti.tokens), B, S, R,
                          dev_i32(ti.forced) if forced else None, pred, ce, loss, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(tr.pred.cpu().numpy(), pred.cpu().numpy())
    np.testing.assert_array_equal(tr.ce.cpu().numpy(), ce.cpu().numpy())
    assert float(tr.loss.item()) == float(loss.item())
    return tr.pred.cpu().numpy(), float(tr.loss.item()), {n: g.cpu().numpy().astype(np.float64)
                                                         for n, g in tr.grads.items()}


def compare_grads(gpu, ref, label, rel_bounds=None, abs_bounds=None):
    """Every gradient within REL (or rel_bounds[name] when given) in relative
    Frobenius norm, and elementwise within ABS_FRAC * max|ref| + 4 REL |ref|
    (or abs_bounds[name] when given)."""
    for n in G.TRAINED:
        a, r = gpu[n], ref[n]
        assert a.shape == r.shape, (n, a.shape, r.shape)
        assert np.all(np.isfinite(a)), f"{label} {n}: non-finite"
        rb = max(REL, rel_bounds[n]) if rel_bounds else REL
        rel = np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-30)
        bound = abs_bounds[n] if abs_bounds else ABS_FRAC * np.abs(r).max() + 4 * REL * np.abs(r)
        worst = float(np.max(np.abs(a - r) - bound))
        say(f"  {label} {n}: rel {rel:.2e} (bound {rb:.2e}) worst-excess {worst:.2e}")
        assert rel <= rb, f"{label} {n}: relative error {rel}"
        assert worst <= 0, f"{label} {n}: an entry exceeds the elementwise bound by {worst}"


CASES = [
    # (name, shape kwargs, B, S, R, forced, pack)
    ("hd64-gqa2-forced", dict(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=4112), 2, 128, 3, True, False),
    ("hd64-gqa2-forced-packed-s192", dict(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=4112), 1, 192, 3, True, True),
    ("hd128-gqa4-forced", dict(d=512, hq=4, hkv=1, hd=128, ffn=512, vocab=2048), 1, 128, 4, True, True),
    ("hd128-gqa1-r1", dict(d=256, hq=2, hkv=2, hd=128, ffn=512, vocab=1040), 2, 64, 1, False, True),
    ("hd64-gqa8-forced-r5", dict(d=512, hq=8, hkv=1, hd=64, ffn=512, vocab=1024), 1, 128, 5, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ttt_gradients_match_oracle(lib, case):
    name, kw, B, S, R, forced, pack = case
    shape = tiny_shape(dtype=BF16, theta=10000.0, **kw)
    Wt = _weights(shape, 3)
    ti = gen.gen_ttt_inputs(shape, B, S, R, seed=4)
    say("ttt-grad", name, "B", B, "S", S, "R", R, "forced", forced, "pack", pack)
    gp, gloss, gg = run_gpu_train(shape, Wt, ti, B, S, R, forced, pack)
    ref = G.ttt_loss_and_grads(shape, host_weights(Wt), ti.feats.f32(), ti.tokens, R,
                               forced=ti.forced if forced else None)
    if not forced:
        np.testing.assert_array_equal(gp, ref["pred"])   # the same self-fed chain
    np.testing.assert_allclose(gloss, ref["loss"], rtol=1e-2, atol=2e-2)
    compare_grads(gg, ref["grads"], name)


def test_ttt_self_fed_gradients_match_oracle(lib):
    """Self-fed steps: the GPU's argmax chain must be the oracle's, then the
    gradients are compared as above.  The seeds are ones whose oracle chain
    has no near-tie (every top-2 gap of the float32 logits >= MIN_GAP, checked
    here on the oracle alone), so a bf16-level logit difference cannot flip
    a fed token."""
    MIN_GAP = 4e-3
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=512, dtype=BF16, theta=10000.0)
    Wt = gen.gen_weights(shape, seed=8, std=0.05)
    Wt.update(gen.gen_drafter_gains(shape, seed=9))
    ti = gen.gen_ttt_inputs(shape, 1, 64, 3, seed=8)
    ref = G.ttt_loss_and_grads(shape, host_weights(Wt), ti.feats.f32(), ti.tokens, 3)
    for lj in ref["logits"][0]:
        top2 = np.sort(np.asarray(lj, np.float32), axis=1)[:, -2:]
        assert (top2[:, 1] - top2[:, 0]).min() >= MIN_GAP
    say("ttt-grad self-fed")
    gp, gloss, gg = run_gpu_train(shape, Wt, ti, 1, 64, 3, False, True)
    np.testing.assert_array_equal(gp, ref["pred"])
    np.testing.assert_allclose(gloss, ref["loss"], rtol=1e-2, atol=2e-2)
    compare_grads(gg, ref["grads"], "self-fed")


def test_ttt_train_is_deterministic_and_layout_independent(lib):
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=4112, dtype=BF16, theta=10000.0)
    Wt = _weights(shape, 7)
    ti = gen.gen_ttt_inputs(shape, 2, 128, 3, seed=8)
    say("ttt-grad determinism")
    a = run_gpu_train(shape, Wt, ti, 2, 128, 3, True, True)
    b = run_gpu_train(shape, Wt, ti, 2, 128, 3, True, True)
    c = run_gpu_train(shape, Wt, ti, 2, 128, 3, True, False)
    for x in (b, c):
        for n in G.TRAINED:
            np.testing.assert_array_equal(a[2][n], x[2][n], err_msg=n)
