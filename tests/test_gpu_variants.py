"""GPU parity of the EAGLE-3.1 norm variants that EAGLE-4 keeps (the FC
norm after the fusion projection; post-norm in the drafter layer) against
the oracle (fuse with norm_fc; decoder_rows with norm_post_attn /
norm_post_ffn), through the C ABI: the fusion output, and whole cycles
stage by stage (fusion, COMMIT and every tree round's logits, every top-k
decision on the GPU's own logits, the tree bit for bit, the verification
outcome)."""
import numpy as np
import pytest
import torch

from eagle_draft_tree_amd import binding as Bd
from eagle_draft_tree_amd.cycle import Drafter
from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import BF16, C1_TINY, C2_8B_TREE, scaled, tiny_shape

from gpu_cases import GpuCycle, check_cycle_stagewise, host_weights, say

pytestmark = pytest.mark.gpu

TOL = (2e-2, 1e-2)
SHAPE = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=2048, dtype=BF16, theta=500000.0, name="variants")


@pytest.mark.parametrize("n", [5, 40, 130])
@pytest.mark.parametrize("pack", [False, True])
def test_fuse_fc_norm(lib, n, pack):
    """n = 5 and 40 take the split / unsplit fusion GEMM of up to 64 rows,
    130 the 64-row chunks with a float32 projection in the workspace."""
    Wt = gen.gen_weights(SHAPE, seed=0)
    Wt.update(gen.gen_norm_variant_gains(SHAPE, True, False, seed=1))
    dr = Drafter(SHAPE, Wt, pack=pack)
    feats = gen.draw(5, 1, (n, 3, SHAPE.d), 1.0, BF16)
    g = torch.empty(n, SHAPE.d, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(Bd.workspace_size(dr.dims, 1, n, 0), dtype=torch.uint8, device="cuda")
    Bd.eagle3_fuse(dr.dims, dr.weights, feats.torch("cuda"), n, g, ws)
    torch.cuda.synchronize()
    ref = O.fuse(SHAPE, feats.f32(), Wt["fc"].f32(), Wt["norm_fc"])
    np.testing.assert_allclose(g.float().cpu().numpy(), ref, atol=TOL[0], rtol=TOL[1])
    # the norm is applied: unit RMS after dividing by the gain
    rms = np.sqrt(np.mean((g.float().cpu().numpy() / Wt["norm_fc"]) ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=2e-2)


def _variant_cycle(w, fc, post, pack, seed=3):
    Wt = gen.gen_weights(w.shape, seed=0)
    Wt.update(gen.gen_norm_variant_gains(w.shape, fc, post, seed=1))
    ci = gen.gen_cycle_inputs(w, seed=seed)
    gc = GpuCycle(w, Wt, ci, pack=pack)
    return Wt, host_weights(Wt), ci, gc


@pytest.mark.parametrize("fc,post,pack,batch", [(True, False, True, 1), (False, True, True, 2), (True, True, False, 3),
                                                (True, True, True, 20)])
def test_variant_small_cycle(lib, fc, post, pack, batch):
    """bf16 drafter (d=256), multi-row commit, GQA; batch 20 takes the
    split-K row kernels (more than 16 rows per round)."""
    w = scaled(C1_TINY, shape=SHAPE, batch=batch, depth=4, topk=3, keep=12, prefix=40, commit_rows=5,
               synthetic_prefix_kv=True, feat_scale=1.0)
    say("variant cycle fc", fc, "post", post, "pack", pack, "batch", batch)
    Wt, W, ci, gc = _variant_cycle(w, fc, post, pack)
    L = gen.target_logits(2, batch, w.keep + 1, SHAPE.vocab, 2.0)
    gc.run(L, 0)
    exc = check_cycle_stagewise(gc, w, W, ci, range(batch), TOL, L=L, mode=0)
    say("  near-tie decisions:", exc)
    if post:
        # children receive the post-norm state: unit RMS after dividing by its gain
        h = gc.buf.h_tree[0, :1 + (w.depth - 1) * w.topk].cpu().numpy()
        np.testing.assert_allclose(np.sqrt(np.mean((h / Wt["norm_post_ffn"]) ** 2, axis=1)), 1.0, rtol=1e-3)


@pytest.mark.timeout(600)
def test_variant_8b_full_size(lib):
    """The 8B tree (prefix 2048, tree 6 x 10, keep 60) with both variants on."""
    w = C2_8B_TREE
    say("variants, 8B full size")
    Wt, W, ci, gc = _variant_cycle(w, True, True, True, seed=1)
    L = gen.target_logits(1, 1, w.keep + 1, w.shape.vocab, w.target_sigma)
    gc.run(L, 0)
    exc = check_cycle_stagewise(gc, w, W, ci, [0], TOL, L=L, mode=0)
    say("  near-tie decisions:", exc)
