"""The allocation-free verify entry point (static per-device scratch)
returns exactly what eagle3_verify returns with a caller workspace, on two
calls in a row (the second smaller, so it finds the first call's partials
in the shared array), in both modes, and rejects a shape beyond its static
scratch before launching anything."""
import numpy as np
import pytest
import torch

from workloads import gen

from gpu_cases import dev_i32, say

pytestmark = pytest.mark.gpu


def _inputs(Bn, m, V, depth, seed):
    toks, pars = [], []
    for b in range(Bn):
        t, p = gen.random_verify_tree(seed * 100 + b, m, V, depth)
        toks.append(t); pars.append(p)
    L = gen.target_logits(seed, Bn, m + 1, V, 2.0)
    ut, ur = gen.uniforms(seed, Bn, m + 1)
    return np.array(toks), np.array(pars), L, ut, ur


def _call(Bd, noalloc, Bn, m, V, Dmax, toks, pars, L, mode, ut, ur):
    i32 = dict(dtype=torch.int32, device="cuda")
    al = torch.full((Bn,), -7, **i32); acc = torch.full((Bn, Dmax), -7, **i32)
    bo = torch.full((Bn,), -7, **i32); st = torch.full((Bn,), -7, **i32)
    args = (Bn, m, V, Dmax, dev_i32(toks), dev_i32(pars), torch.as_tensor(L).cuda(), mode, 1.0,
            torch.as_tensor(ut).cuda(), torch.as_tensor(ur).cuda(), al, acc, bo, st)
    if noalloc:
        Bd.eagle3_verify_noalloc(*args)
    else:
        vws = torch.zeros(Bd.verify_workspace_size(Bn, m, V), dtype=torch.uint8, device="cuda")
        Bd.eagle3_verify(*args, vws)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (al, acc, bo, st)]


@pytest.mark.parametrize("mode", [0, 1])
def test_verify_noalloc_matches_verify(lib, mode):
    from eagle_draft_tree_amd import binding as Bd
    for (Bn, m, V, depth, seed) in ((8, 60, 128256, 6, 3), (3, 12, 50000, 4, 4)):
        say("verify_noalloc mode", mode, "B", Bn, "m", m, "V", V)
        toks, pars, L, ut, ur = _inputs(Bn, m, V, depth, seed)
        # plant agreement so that walks go deep
        gen.plant_agreement(L, toks, pars, np.full(Bn, 0.9), seed=seed)
        ref = _call(Bd, False, Bn, m, V, depth, toks, pars, L, mode, ut, ur)
        got = _call(Bd, True, Bn, m, V, depth, toks, pars, L, mode, ut, ur)
        for a, b in zip(ref, got):
            np.testing.assert_array_equal(a, b)
        assert np.all(got[3] == 0)


def test_verify_noalloc_rejects_beyond_static_scratch(lib):
    from eagle_draft_tree_amd import binding as Bd
    Bn, m, V = 256, 63, 262144        # 256 * 64 * 64 partial rows: far beyond 8 MiB
    with pytest.raises(Bd.Eagle3Error) as e:
        Bd.eagle3_verify_noalloc(Bn, m, V, 6, *([None] * 3), 0, 1.0, None, None, *([None] * 4))
    assert e.value.code == Bd.EINVAL       # NULL pointers are caught first
    x = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(Bd.Eagle3Error) as e:
        Bd.eagle3_verify_noalloc(Bn, m, V, 6, x, x, torch.zeros(1, device="cuda"), 0, 1.0, None, None, x, x, x, x)
    assert e.value.code == Bd.ECAPACITY
