"""GPU parity of the target's verification forward (eagle3_target_forward)
and the KV commit (eagle3_kv_commit) against the oracle's
target_verify_forward / target_layer / kv_commit, through the C ABI.

Layer by layer (stage-isolated): the GPU runs one layer per call; the oracle
applies the same layer to the GPU's own input state, so every layer is
checked against the oracle without the bf16 rounding cascade of the layers
before it.  The tree-slot keys/values each layer writes, the features (bit
for bit the bf16 rounding of the GPU's own state) and the logits (the
oracle's final norm + LM head on the GPU's last state) are checked too; the
one-call forward equals the layer-by-layer run bit for bit.  Small shapes
also compare the GPU's one-call forward with the oracle's independent run.

Full-size layers take the bf16 tolerance plus the arithmetic's own
sensitivity: inside one layer, float32 accumulation (K up to 28672) flips a
fraction of the bf16 roundings of u and silu(gate)*up, and with the random
N(0, 0.02) weights the layer output is large (|h| up to ~40 at the 70B
shape), so even the oracle moves by up to ~0.1 when its GEMMs accumulate in
float32 instead of fp64.  The test runs that float32-accumulating variant of
the oracle on the same inputs and bounds the GPU by it: per element
|gpu - o64| <= atol + rtol |o64| + 2 max|o32 - o64|, and no more elements
beyond atol + rtol |o64| than twice the variant's count (plus 0.1 %).
"""
import contextlib
import numpy as np
import pytest
import torch

from eagle_draft_tree_amd import binding as Bd
from eagle_draft_tree_amd.target import TargetCache, TargetWeights, VerifyForward
from oracle import eagle3_oracle as O
from workloads import gen
from workloads.configs import (BF16, C2V_8B_TARGET_TREE, C3V_8B_TARGET_CHAIN, C4V_70B_TARGET_TREE, F32, Workload,
                               tiny_shape)

from gpu_cases import dev_i32, say

pytestmark = pytest.mark.gpu

TOL_BF16 = (2e-2, 1e-2)
TOL_F32 = (1e-4, 1e-4)


def _f64(t):
    """Host values for the oracle: the exact float32 values of generator
    tensors (the oracle up-casts blocks to fp64 itself), fp64 otherwise."""
    return t.f32() if hasattr(t, "f32") else np.asarray(t, np.float64)


class Case:
    """A target, its inputs on the device and the oracle's view of them."""

    def __init__(self, w, n_layers, feat_layers, pack=True, gains="random", seed=1):
        s = w.shape
        self.w, self.s, self.L, self.fl = w, s, n_layers, feat_layers
        self.Tw = gen.gen_target_weights(s, n_layers, seed=0, gains=gains)
        self.ti = gen.gen_target_inputs(w, n_layers, seed=seed)
        ti = self.ti
        self.rows = w.keep + 1
        self.tw = TargetWeights(s, list(self.Tw["layers"]), self.Tw["emb"], self.Tw["lm"], self.Tw["norm_out"],
                                feat_layers, pack=pack)
        k = torch.stack([t.torch("cuda") for t in ti.kv_k])
        v = torch.stack([t.torch("cuda") for t in ti.kv_v])
        dt = torch.bfloat16 if s.dtype == BF16 else torch.float32
        if w.paged:
            self.cache = TargetCache(s, n_layers, w.batch, 0, dt, paged=True, block_size=w.block_size,
                                     block_table=torch.as_tensor(ti.block_table), k=k, v=v)
        else:
            self.cache = TargetCache(s, n_layers, w.batch, ti.cap, dt, k=k, v=v)
        self.cache.ctx_len.copy_(torch.as_tensor(ti.ctx_len))
        self.vf = VerifyForward(self.tw, self.cache, self.rows)
        self.tokens = dev_i32(ti.v_tok)
        self.pos = dev_i32(ti.v_pos)
        self.anc = torch.as_tensor(ti.v_anc.view(np.int64)).cuda()
        self.TwO = dict(emb=_f64(self.Tw["emb"]), lm=_f64(self.Tw["lm"]), norm_out=_f64(self.Tw["norm_out"]),
                        layers=[{kk: _f64(vv) for kk, vv in Lw.items()} for Lw in self.Tw["layers"]])

    def oracle_kv(self, b, l):
        """Layer l's keys/values of request b as the oracle sees them:
        committed rows then 64 empty tree slots."""
        ti, w = self.ti, self.w
        if w.paged:
            n = self.ti.cap
            K = O.gather_paged(ti.kv_k[l].f32(), ti.block_table[b], n, w.block_size)
            V = O.gather_paged(ti.kv_v[l].f32(), ti.block_table[b], n, w.block_size)
        else:
            K, V = ti.kv_k[l].f32()[b], ti.kv_v[l].f32()[b]
        z = np.zeros((O.MAX_TREE_SLOTS,) + K.shape[1:])
        return np.concatenate([K, z]).astype(np.float64), np.concatenate([V, z]).astype(np.float64)

    def run(self, begin=0, end=None, logits=True):
        self.vf.run(self.tokens, self.pos, self.anc, begin, end, logits)
        torch.cuda.synchronize()


def _matmul_wt_f32(x, W):
    """x @ W.T with float32 operands and float32 accumulation (BLAS sgemm)."""
    x32 = np.asarray(x, dtype=np.float32)
    out = np.empty((x32.shape[0], W.shape[0]), dtype=np.float64)
    for s0 in range(0, W.shape[0], 8192):
        out[:, s0:s0 + 8192] = x32 @ np.asarray(W[s0:s0 + 8192], dtype=np.float32).T
    return out


@contextlib.contextmanager
def _f32_accumulation():
    exact = O.matmul_wt
    O.matmul_wt = _matmul_wt_f32
    try:
        yield
    finally:
        O.matmul_wt = exact


def assert_within_cascade(gpu, o64, o32, tol, what):
    """gpu vs the fp64 oracle, allowing the drift a float32-accumulating
    implementation shows on the same inputs (o32: the oracle with float32
    GEMM accumulation)."""
    base = tol[0] + tol[1] * np.abs(o64)
    drift = np.abs(o32 - o64)
    err = np.abs(gpu - o64)
    assert np.all(err <= base + 2 * drift.max()), \
        f"{what}: max error {err.max():.4g} > bound (variant's max drift {drift.max():.4g})"
    n_gpu, n_var = int((err > base).sum()), int((drift > base).sum())
    assert n_gpu <= 2 * n_var + 1e-3 * err.size, f"{what}: {n_gpu} elements beyond tolerance (variant: {n_var})"
    return err.max(), drift.max(), n_gpu, n_var


def check_layerwise(case, reqs, tol, cascade=False):
    """Stage-isolated parity of every layer for requests `reqs`; returns the
    GPU's (hidden, feats, logits) of the layer-by-layer run.  cascade=True
    bounds h by the float32-accumulation drift (full-size layers)."""
    s, L, rows = case.s, case.L, case.rows
    ti = case.ti
    h_prev = None
    for l in range(L):
        case.run(l, l + 1, logits=(l == L - 1))
        h_gpu = case.vf.hidden.cpu().numpy()
        for b in reqs:
            Ks, Vs = [None] * L, [None] * L
            Ks[l], Vs[l] = case.oracle_kv(b, l)
            cap = Ks[l].shape[0] - O.MAX_TREE_SLOTS
            vis = O.target_tree_visibility(ti.v_anc[b], int(ti.ctx_len[b]), cap)
            widx = cap + np.arange(rows)
            h_in = None if l == 0 else h_prev[b].astype(np.float64)
            h_o, _, _ = O.target_forward(s, case.TwO, ti.v_tok[b], ti.v_pos[b], Ks, Vs, widx, vis, case.fl, l, l + 1,
                                         h_in)
            if cascade:
                K32, V32 = [None] * L, [None] * L
                K32[l], V32[l] = case.oracle_kv(b, l)
                with _f32_accumulation():
                    h_32, _, _ = O.target_forward(s, case.TwO, ti.v_tok[b], ti.v_pos[b], K32, V32, widx, vis, case.fl,
                                                  l, l + 1, h_in)
                r = assert_within_cascade(h_gpu[b], h_o, h_32, tol, f"layer {l} request {b}: h")
                say(f"  layer {l} request {b}: h max err {r[0]:.4g} (f32 variant {r[1]:.4g}), beyond tol {r[2]} "
                    f"(variant {r[3]}) of {h_o.size}")
            else:
                np.testing.assert_allclose(h_gpu[b], h_o, atol=tol[0], rtol=tol[1],
                                           err_msg=f"layer {l} request {b}: h")
            tk = case.cache.tk[l, b, :rows].float().cpu().numpy()
            tv = case.cache.tv[l, b, :rows].float().cpu().numpy()
            np.testing.assert_allclose(tk, Ks[l][cap:cap + rows], atol=tol[0], rtol=tol[1],
                                       err_msg=f"layer {l} request {b}: tree-slot keys")
            np.testing.assert_allclose(tv, Vs[l][cap:cap + rows], atol=tol[0], rtol=tol[1],
                                       err_msg=f"layer {l} request {b}: tree-slot values")
        # features of this layer: the dtype rounding of the GPU's own state
        for j, fl in enumerate(case.fl):
            if fl == l + 1:
                f = case.vf.feats[:, :, j].cpu()
                want = torch.as_tensor(h_gpu).to(f.dtype)
                assert torch.equal(f, want), f"feature {j} after layer {l + 1}"
        h_prev = h_gpu
    lg = case.vf.logits.cpu().numpy()
    for b in reqs:
        y = O._rnd(s, O.rmsnorm(h_prev[b].astype(np.float64), case.TwO["norm_out"], s.rms_eps))
        np.testing.assert_allclose(lg[b], O.matmul_wt(y, case.TwO["lm"]), atol=tol[0], rtol=tol[1],
                                   err_msg=f"request {b}: logits")
    return h_prev, case.vf.feats.cpu().clone(), lg


def check_one_call_equals_layerwise(case, layerwise):
    h_l, f_l, lg_l = layerwise
    case.run()
    assert np.array_equal(case.vf.hidden.cpu().numpy(), h_l)
    assert torch.equal(case.vf.feats.cpu(), f_l)
    assert np.array_equal(case.vf.logits.cpu().numpy(), lg_l)


SMALL_BF16 = tiny_shape(d=256, hq=4, hkv=2, hd=64, ffn=512, vocab=4096, dtype=BF16, theta=500000.0, name="tgt-bf16")
SMALL_F32 = tiny_shape(d=256, hq=4, hkv=4, hd=64, ffn=512, vocab=4096, dtype=F32, theta=10000.0, name="tgt-f32")


@pytest.mark.parametrize("dtype,pack,paged,batch", [(BF16, True, False, 2), (BF16, False, True, 3), (F32, False, False, 2)])
def test_target_forward_small(lib, dtype, pack, paged, batch):
    shape = SMALL_BF16 if dtype == BF16 else SMALL_F32
    w = Workload("target-small", shape, batch=batch, depth=4, topk=3, keep=11, prefix=70, paged=paged,
                 prefix_range=(5, 90) if paged else None)
    say("target small", dtype, "pack", pack, "paged", paged, "batch", batch)
    case = Case(w, 4, (1, 3, 4), pack=pack)
    tol = TOL_BF16 if dtype == BF16 else TOL_F32
    layerwise = check_layerwise(case, range(batch), tol)
    check_one_call_equals_layerwise(case, layerwise)
    # the oracle's independent run (no GPU state fed in)
    lg = case.vf.logits.cpu().numpy()
    feats = case.vf.feats.float().cpu().numpy()
    for b in range(batch):
        Ks, Vs = zip(*[case.oracle_kv(b, l) for l in range(case.L)])
        _, f_o, lg_o = O.target_verify_forward(shape, case.TwO, case.ti.v_tok[b], case.ti.v_pos[b],
                                               case.ti.v_anc[b], list(Ks), list(Vs), int(case.ti.ctx_len[b]), case.fl)
        np.testing.assert_allclose(lg[b], lg_o, atol=tol[0], rtol=tol[1], err_msg=f"request {b}: logits")
        np.testing.assert_allclose(feats[b], f_o, atol=tol[0], rtol=tol[1], err_msg=f"request {b}: features")


MID_BF16 = tiny_shape(d=512, hq=8, hkv=2, hd=64, ffn=1024, vocab=4096, dtype=BF16, theta=500000.0, name="tgt-bf16-512")


@pytest.mark.parametrize("shape,batch", [(SMALL_BF16, 20), (MID_BF16, 24), (MID_BF16, 32)],
                         ids=["d256-80rows-per-chunk", "d512-96rows-chunked", "d512-128rows-chunked"])
def test_target_forward_chain_rows_over_64(lib, shape, batch):
    """More than 64 verify rows in one call (batch x 4-row chains, paged).
    80 rows at width 256 end in a 16-row chunk, so every GEMM runs one launch
    per 64-row chunk; 96 and 128 rows at width 512 (every chunk 17..64 rows,
    split-K QKV, O and down) run all chunks of each GEMM and of the LM head
    in one launch."""
    w = Workload("target-chains", shape, batch=batch, depth=3, topk=1, keep=3, prefix=40, paged=True,
                 prefix_range=(1, 60))
    say("target chains", shape.name, "batch", batch, "rows", batch * 4)
    case = Case(w, 2, (1, 1, 2))
    layerwise = check_layerwise(case, [0, 7, batch - 1], TOL_BF16)
    check_one_call_equals_layerwise(case, layerwise)


def test_kv_commit(lib):
    """Root + accepted rows move to the committed rows of every layer bit for
    bit, features are gathered, lengths advance; a request that would not
    fit is left unchanged with status ECAPACITY."""
    w = Workload("target-commit", SMALL_BF16, batch=3, depth=4, topk=3, keep=11, prefix=30)
    case = Case(w, 3, (1, 2, 3))
    case.run()
    ti = case.ti
    Dmax = 5
    acc_len = np.array([3, 0, 2], np.int32)
    accepted = np.full((3, Dmax), -1, np.int32)
    for b in range(3):        # a root path of each tree
        node = int(np.nonzero(ti.v_parent[b] >= 0)[0][-1])
        path = []
        while node > 0:
            path.append(node)
            node = int(ti.v_parent[b, node])
        path = path[::-1][: acc_len[b]]
        acc_len[b] = len(path)
        accepted[b, : len(path)] = path
    # request 2 is made not to fit: its committed length sits at the capacity edge
    ctx = ti.ctx_len.copy()
    ctx[2] = ti.cap - int(acc_len[2])
    case.cache.ctx_len.copy_(torch.as_tensor(ctx))
    k_before = case.cache.k.clone()
    v_before = case.cache.v.clone()
    feats_next = torch.zeros(3, Dmax + 1, 3, SMALL_BF16.d, dtype=torch.bfloat16, device="cuda")
    status = torch.full((3,), 7, dtype=torch.int32, device="cuda")
    case.vf.commit(dev_i32(acc_len), dev_i32(accepted), Dmax, feats_next=feats_next,
                   ctx_len_out=case.cache.ctx_len, status=status)
    torch.cuda.synchronize()
    st = status.cpu().numpy()
    new_ctx = case.cache.ctx_len.cpu().numpy()
    assert list(st) == [0, 0, Bd.ECAPACITY]
    assert list(new_ctx) == [ctx[0] + acc_len[0] + 1, ctx[1] + acc_len[1] + 1, ctx[2]]
    for b in range(2):
        rows = O.commit_rows(int(acc_len[b]), accepted[b])
        for l in range(case.L):
            for j, i in enumerate(rows):
                assert torch.equal(case.cache.k[l, b, ctx[b] + j], case.cache.tk[l, b, i])
                assert torch.equal(case.cache.v[l, b, ctx[b] + j], case.cache.tv[l, b, i])
            # nothing else moved
            n = len(rows)
            assert torch.equal(case.cache.k[l, b, : ctx[b]], k_before[l, b, : ctx[b]])
            assert torch.equal(case.cache.k[l, b, ctx[b] + n:], k_before[l, b, ctx[b] + n:])
        for j, i in enumerate(rows):
            assert torch.equal(feats_next[b, j], case.vf.feats[b, i])
    assert torch.equal(case.cache.k[:, 2], k_before[:, 2]) and torch.equal(case.cache.v[:, 2], v_before[:, 2])


def test_greedy_cycles_on_the_target_reproduce_its_greedy_decode(lib):
    """(tree forward, greedy verify, KV commit) cycles on the GPU emit the
    oracle's sequential greedy decode of the same fp32 target; each tree
    holds the oracle's greedy continuation as one branch."""
    shape = SMALL_F32
    L = 2
    Tw = gen.gen_target_weights(shape, L, seed=5, gains="random", std=0.05)
    TwO = dict(emb=_f64(Tw["emb"]), lm=_f64(Tw["lm"]), norm_out=_f64(Tw["norm_out"]),
               layers=[{kk: _f64(vv) for kk, vv in Lw.items()} for Lw in Tw["layers"]])
    tw = TargetWeights(shape, Tw["layers"], Tw["emb"], Tw["lm"], Tw["norm_out"], (1, 2, 2))
    cap = 64
    cache = TargetCache(shape, L, 1, cap, torch.float32)
    rows = 8
    vf = VerifyForward(tw, cache, rows)
    prompt = [11, 400, 3071]
    n_new = 16

    def oracle_next(seq):
        Ks = [np.zeros((cap + O.MAX_TREE_SLOTS, shape.n_kv_heads, shape.head_dim)) for _ in range(L)]
        Vs = [np.zeros_like(k) for k in Ks]
        n = len(seq)
        vis = np.tril(np.ones((n, cap + O.MAX_TREE_SLOTS), bool))
        vis[:, n:] = False
        _, _, lg = O.target_forward(shape, TwO, np.array(seq), np.arange(n), Ks, Vs, np.arange(n), vis, (1, 2, 2))
        row = lg[-1].astype(np.float32)
        top2 = np.sort(row)[-2:]
        return int(np.argmax(row)), float(top2[1] - top2[0])

    ref, gaps = list(prompt), []
    while len(ref) < len(prompt) + n_new + 4:
        t, gap = oracle_next(ref)
        ref.append(t)
        gaps.append(gap)
    assert min(gaps) > 1e-3, "an oracle near-tie would make the comparison ambiguous"
    # the prompt's first tokens are committed by a chain forward + commit of all its rows
    rng = np.random.default_rng(3)
    seq = list(prompt)
    ws = torch.zeros(Bd.verify_workspace_size(1, rows - 1, shape.vocab), dtype=torch.uint8, device="cuda")
    # prefill: the prompt minus its last token as one chain, all committed
    n0 = len(prompt) - 1
    ch_tok = np.array(prompt[:n0] + [0] * (rows - n0), np.int32)
    par = np.arange(-1, rows - 1, dtype=np.int32)
    anc = gen.ancestor_bits(par)
    vf.run(dev_i32(ch_tok[None]), dev_i32(np.arange(rows)[None]), torch.as_tensor(anc.view(np.int64)[None]).cuda(),
           logits=False)
    acc = np.full((1, rows - 1), -1, np.int32)
    acc[0, : n0 - 1] = np.arange(1, n0)
    vf.commit(dev_i32([n0 - 1]), dev_i32(acc), rows - 1, ctx_len_out=cache.ctx_len)
    torch.cuda.synchronize()
    assert int(cache.ctx_len[0]) == n0
    accepted_total = 0
    while len(seq) < len(prompt) + n_new:
        ctx = len(seq) - 1
        spine = ref[len(seq): len(seq) + int(rng.integers(0, 4))]
        v_tok, v_par = [seq[-1]], [-1]
        for j, t in enumerate(spine):
            v_tok.append(t)
            v_par.append(j)
        while len(v_tok) < rows:
            p = int(rng.integers(0, len(v_tok)))
            t = int(rng.integers(0, shape.vocab))
            if any(v_par[c] == p and v_tok[c] == t for c in range(1, len(v_tok))):
                continue
            v_tok.append(t)
            v_par.append(p)
        v_par = np.array(v_par, np.int32)
        depth = np.zeros(rows, np.int32)
        for i in range(1, rows):
            depth[i] = depth[v_par[i]] + 1
        anc = gen.ancestor_bits(v_par)
        vf.run(dev_i32(np.array(v_tok)[None]), dev_i32((ctx + depth)[None]),
               torch.as_tensor(anc.view(np.int64)[None]).cuda())
        acc_len = torch.zeros(1, dtype=torch.int32, device="cuda")
        accepted = torch.full((1, rows - 1), -1, dtype=torch.int32, device="cuda")
        bonus = torch.zeros(1, dtype=torch.int32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        Bd.eagle3_verify(1, rows - 1, shape.vocab, rows - 1, dev_i32(np.array(v_tok)[None]), dev_i32(v_par[None]),
                         vf.logits, Bd.GREEDY, 1.0, None, None, acc_len, accepted, bonus, status, ws)
        vf.commit(acc_len, accepted, rows - 1, ctx_len_out=cache.ctx_len)
        torch.cuda.synchronize()
        a = int(acc_len[0])
        accepted_total += a
        seq += [v_tok[int(i)] for i in accepted[0, :a].cpu()] + [int(bonus[0])]
        assert int(cache.ctx_len[0]) == len(seq) - 1
    say("  accepted", accepted_total, "tokens over", len(seq) - len(prompt), "emitted")
    assert seq == ref[: len(seq)]
    assert accepted_total > 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("which", ["8b", "70b", "8b-chains"])
def test_target_forward_full_size_layers(lib, which):
    """Full-size layers: two 8B-shaped target layers over the 61 verify rows
    of the 8B tree (prefix 2048); one 70B-shaped layer over the 70B tree
    (prefix 4096); one 8B-shaped layer over the 64 x 4-row paged chains of
    the serving batch (256 rows).  Stage-isolated, sampled requests."""
    if which == "8b":
        w, L, fl, reqs = C2V_8B_TARGET_TREE, 2, (1, 2, 2), [0]
    elif which == "70b":
        w, L, fl, reqs = C4V_70B_TARGET_TREE, 1, (1, 1, 1), [0]
    else:
        w, L, fl, reqs = C3V_8B_TARGET_CHAIN, 1, (1, 1, 1), [0, 21, 63]
    say("target full size", which, "layers", L)
    case = Case(w, L, fl, pack=True, gains="ones")
    layerwise = check_layerwise(case, reqs, TOL_BF16, cascade=True)
    check_one_call_equals_layerwise(case, layerwise)
