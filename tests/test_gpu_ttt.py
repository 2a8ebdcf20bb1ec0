"""GPU parity of the training-time-test forward (eagle3_ttt_forward) against
the oracle's step-by-step TTT forward on the same seeded inputs.

Predictions (argmax of float32 logits) are exact unless the oracle's own
logits have a near-tie at the top; a prediction feeds the next step's input
token, so once a position's prediction is excused as a near-tie the later
steps of that position are not compared in unforced mode (they follow a
different, equally valid chain).  CE values are within the bf16 tolerance."""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import BF16, tiny_shape

from gpu_cases import dev_i32, host_weights, say

pytestmark = pytest.mark.gpu

CE_TOL = (2e-2, 1e-2)   # bf16 CE: atol, rtol
TIE = 2e-3              # top-2 gap of the oracle's float32 logits treated as a near-tie


def run_gpu_ttt(shape, Wt, ti, B, S, R, forced, pack):
    from eagle_draft_tree_amd import binding as Bd
    from eagle_draft_tree_amd.cycle import Drafter
    dr = Drafter(shape, Wt, pack=pack)
    feats = ti.feats.torch("cuda")
    tokens = dev_i32(ti.tokens)
    fz = dev_i32(ti.forced) if forced else None
    pred = torch.empty(B, R, S, dtype=torch.int32, device="cuda")
    ce = torch.empty(B, R, S, dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(Bd.ttt_workspace_size(dr.dims, B, S, R), dtype=torch.uint8, device="cuda")
    Bd.eagle3_ttt_forward(dr.dims, dr.weights, feats, tokens, B, S, R, fz, pred, ce, loss, ws)
    torch.cuda.synchronize()
    return pred.cpu().numpy(), ce.cpu().numpy(), float(loss.item())


def compare(shape, W, ti, B, S, R, forced, gp, gce, gloss, tie=TIE):
    tot, cnt, excused, compared = 0.0, 0, 0, 0
    for b in range(B):
        say("  oracle sequence", b)
        o = O.ttt_forward_full(shape, W, ti.feats.f32()[b], ti.tokens[b], R,
                               forced=ti.forced[b] if forced else None)
        tot += float(o["ce"][o["valid"]].sum())
        cnt += int(o["valid"].sum())
        live = np.ones(S, bool)  # positions whose chain still matches the oracle's
        for j in range(R):
            l32 = o["logits"][j].astype(np.float32)
            for i in np.nonzero(live)[0]:
                compared += 1
                if o["valid"][j, i]:
                    np.testing.assert_allclose(gce[b, j, i], o["ce"][j, i], atol=CE_TOL[0], rtol=CE_TOL[1],
                                               err_msg=f"ce b={b} step={j + 1} i={i}")
                else:
                    assert gce[b, j, i] == 0.0
                if gp[b, j, i] != o["pred"][j, i]:
                    srt = np.sort(l32[i])[::-1]
                    gap = float(srt[0] - srt[1])
                    ok = gap <= tie and l32[i, gp[b, j, i]] >= srt[0] - tie
                    assert ok, f"pred b={b} step={j + 1} i={i}: gpu {gp[b, j, i]} oracle {o['pred'][j, i]} gap {gap}"
                    excused += 1
                    if not forced:
                        live[i] = False
    say("  compared", compared, "excused near-ties", excused)
    assert excused <= max(2, compared // 50)
    ref_loss = tot / cnt if cnt else 0.0
    if forced or excused == 0:
        np.testing.assert_allclose(gloss, ref_loss, atol=CE_TOL[0], rtol=CE_TOL[1])


CASES = [
    # (name, shape kwargs, B, S, R, forced, pack)
    ("hd64-gqa2-forced", dict(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=4112), 2, 192, 3, True, False),
    ("hd64-gqa2-self", dict(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=4112), 2, 192, 3, False, True),
    ("hd128-gqa4-self", dict(d=512, hq=4, hkv=1, hd=128, ffn=512, vocab=2048), 1, 128, 4, False, True),
    ("r1", dict(d=256, hq=2, hkv=2, hd=64, ffn=512, vocab=1040), 1, 64, 1, False, True),
    # query-head groups of 3 take the attention kernel without LDS staging
    ("hd64-gqa3-self", dict(d=384, hq=6, hkv=2, hd=64, ffn=512, vocab=2064), 1, 128, 2, False, True),
    # widths 1024 and 2048: the one-pass prologue and RMSNorm with two and four 512-column chunks per row
    ("d1024-forced", dict(d=1024, hq=8, hkv=2, hd=128, ffn=1024, vocab=1040), 1, 64, 2, True, True),
    ("d2048-forced", dict(d=2048, hq=16, hkv=4, hd=128, ffn=1024, vocab=1024), 1, 64, 2, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ttt_matches_oracle(lib, case):
    name, kw, B, S, R, forced, pack = case
    shape = tiny_shape(dtype=BF16, theta=10000.0, **kw)
    Wt = gen.gen_weights(shape, seed=3)
    ti = gen.gen_ttt_inputs(shape, B, S, R, seed=4)
    say("ttt", name, "B", B, "S", S, "R", R, "forced", forced, "pack", pack)
    gp, gce, gloss = run_gpu_ttt(shape, Wt, ti, B, S, R, forced, pack)
    compare(shape, host_weights(Wt), ti, B, S, R, forced, gp, gce, gloss)


def test_ttt_is_deterministic_and_layout_independent(lib):
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=4112, dtype=BF16)
    Wt = gen.gen_weights(shape, seed=5)
    ti = gen.gen_ttt_inputs(shape, 2, 128, 3, seed=6)
    say("ttt determinism")
    a = run_gpu_ttt(shape, Wt, ti, 2, 128, 3, False, True)
    b = run_gpu_ttt(shape, Wt, ti, 2, 128, 3, False, True)
    c = run_gpu_ttt(shape, Wt, ti, 2, 128, 3, False, False)
    for x, y in ((a, b), (a, c)):
        np.testing.assert_array_equal(x[0], y[0])
        np.testing.assert_array_equal(x[1], y[1])
        assert x[2] == y[2]


def test_ttt_large_scores_move_the_softmax_maximum(lib):
    """q and k rows of W_qkv scaled by 16 (exact in bf16): attention scores
    spread by about 50 instead of 0.2, so in later key blocks a row's running
    maximum of the online softmax jumps by more than its lazy-rescale
    threshold, on some lanes of a wave and not others, and the rescale of
    the partial output runs there too (with small scores it runs only at a
    row's first block).  Attention this close to one-hot passes rounding-level
    score differences on to the logits: the CE differs from the oracle's by up
    to about 1e-2 here (with the running maximum moved at every block as much
    as with the lazy one), so predictions are excused up to that top-2 gap."""
    shape = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=768, vocab=4112, dtype=BF16, theta=10000.0)
    Wt = gen.gen_weights(shape, seed=3)
    f = Wt["qkv"].f32().copy()
    f[: (shape.n_q_heads + shape.n_kv_heads) * shape.head_dim] *= 16.0
    Wt["qkv"] = gen.Tensor(gen.f32_to_bf16_bits(f), BF16)
    ti = gen.gen_ttt_inputs(shape, 2, 192, 3, seed=4)
    say("ttt large scores")
    gp, gce, gloss = run_gpu_ttt(shape, Wt, ti, 2, 192, 3, True, True)
    compare(shape, host_weights(Wt), ti, 2, 192, 3, True, gp, gce, gloss, tie=1e-2)
