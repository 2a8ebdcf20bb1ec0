"""CPU oracle for the gradients of the training-time-test loss.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

What is differentiated ("EAGLE-3 精读" (edgeai1 speculative-decoding
knowledge base) §1 and §2): the drafter is trained on the final-token CE of
its own rollout, about five self-fed steps built into one graph under the
training-time-test mask, with the target model and its LM head frozen.  The
forward is the one of ``eagle3_oracle.ttt_forward_full`` (rows (j, i), j =
1..R; step 1 feeds (g_i, x_i) at position i, step j >= 2 the previous step's
h2 and its argmax or forced token at position i + j - 1; query (j, i) sees
the step-1 keys i' <= i and its own chain keys (j', i), 2 <= j' <= j), here
written with PyTorch fp64 tensors so that autograd takes the derivative.

Readings (numbered after the forward oracle's R1..R41):

* R42 trained parameters: the fusion FC and the decoder layer's four
  matrices (qkv, o, gate_up, down) and four RMSNorm gains (norm_e, norm_s,
  norm_ffn, norm_out).  The token embedding and the LM head are the
  target's and stay frozen (§1: target and LM head frozen; R8: the
  drafter reads the target's embedding); the features are the frozen
  target's outputs and get no gradient.
* R43 the bf16 roundings of a bf16 workload (g, every GEMM input, q/k/v
  after RoPE, the attention output) are storage precision: the backward
  passes through them as the identity (straight-through), i.e. it is the
  derivative of the unrounded layer evaluated at the rounded values.  The
  CE reads float32 logits, as the forward does; the rounding to float32 is
  passed through the same way.
* R44 the fed token of step j >= 2 (an argmax, or a forced token) is an
  integer choice and carries no gradient; the gradient reaches earlier
  steps through the fed state s = h2 and through the keys and values every
  later query of the same position attends to.
* R45 the loss is the scalar the forward reports: the mean CE over the
  valid rows (i + j <= S - 1) of all B sequences.

Precision: fp64 throughout; decisions (argmax) on float32 logits with ties
to the lowest id, as in the forward oracle.
"""
from __future__ import annotations

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

TRAINED = ("fc", "qkv", "o", "gate_up", "down", "norm_e", "norm_s", "norm_ffn", "norm_out")


def _bf16(x):
    """Nearest bfloat16 value, ties to even, directly from fp64: x = m 2^e
    with 0.5 <= |m| < 1, round m 2^8 to an integer (torch.round is ties to
    even) and scale back."""
    m, e = torch.frexp(x)
    return torch.ldexp(torch.round(m * 256.0), e - 8)


def _st(x, r):
    """Value r(x), derivative of the identity (R43)."""
    return x + (r - x).detach()


def _rnd(cfg, x):
    return _st(x, _bf16(x.detach())) if cfg.dtype == BF16 else x


def _rms(v, gain, eps):
    return v / torch.sqrt((v * v).mean(dim=-1, keepdim=True) + eps) * gain


def _rope(x, pos, theta):
    """Rotate-half RoPE on [..., H, hd] at integer positions pos [...]."""
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-(2.0 * torch.arange(half, dtype=torch.float64)) / hd)
    ang = pos.to(torch.float64)[..., None, None] * inv
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


class _GradToBf16(torch.autograd.Function):
    """Identity whose backward rounds the gradient to bfloat16."""

    @staticmethod
    def forward(ctx, x):
        return x.view_as(x)

    @staticmethod
    def backward(ctx, g):
        return _bf16(g)


def _gq(on):
    """Gradient rounding at a GEMM's operand (the bf16-gradient variant)."""
    return _GradToBf16.apply if on else (lambda x: x)


def _mm_f32(a, b):
    """a @ b with float32 operands and accumulation (the f32 variant)."""
    return (a.to(torch.float32) @ b.to(torch.float32)).to(torch.float64)


def _es_f32(eq, *ops):
    return torch.einsum(eq, *(o.to(torch.float32) for o in ops)).to(torch.float64)


def _sequence(cfg, P, feats, tokens, R, forced, grad_bf16=False, gemm_f32=False):
    """Sum of the valid CE of one sequence plus its float32 predictions.

    feats [S, 3, d] (fp64 tensor), tokens [S] ints; forced [R-1, S] or None.
    P: parameters (fp64 tensors; the trained ones require grad).  grad_bf16:
    round to bf16 the gradients that reach a GEMM as an operand; gemm_f32:
    products and their gradients in float32 (see ttt_loss_and_grads)."""
    gq = _gq(grad_bf16)
    mm = _mm_f32 if gemm_f32 else (lambda a, b: a @ b)
    es = _es_f32 if gemm_f32 else torch.einsum
    S = len(tokens)
    d, Hq, Hkv, hd, F, eps = cfg.d, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.rms_eps
    grp = Hq // Hkv
    scale = 1.0 / np.sqrt(hd)
    g = _rnd(cfg, gq(mm(feats.reshape(S, 3 * d), P["fc"].T)))
    s = g
    t = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
    causal = torch.tril(torch.ones(S, S, dtype=torch.bool))
    k1 = v1 = None
    chain_k, chain_v = [], []              # keys/values of steps 2..j at every position
    ce_sum = torch.zeros((), dtype=torch.float64)
    ce = np.zeros((R, S))
    pred = np.zeros((R, S), np.int32)
    logits_all = []
    for j in range(1, R + 1):
        pos = torch.arange(S) + (j - 1)
        x = torch.cat([_rms(P["emb"][t], P["norm_e"], eps), _rms(s, P["norm_s"], eps)], dim=1)
        x = _rnd(cfg, x)
        qkv = gq(mm(x, P["qkv"].T))
        q = qkv[:, : Hq * hd].reshape(S, Hq, hd)
        k = qkv[:, Hq * hd: (Hq + Hkv) * hd].reshape(S, Hkv, hd)
        v = qkv[:, (Hq + Hkv) * hd:].reshape(S, Hkv, hd)
        q = _rnd(cfg, _rope(q, pos, cfg.rope_theta))
        k = _rnd(cfg, _rope(k, pos, cfg.rope_theta))
        v = _rnd(cfg, v)
        if j == 1:
            k1, v1 = k, v
        else:
            chain_k.append(k)
            chain_v.append(v)
        # query (j, i), head h of group h // grp: step-1 keys i' <= i, then the
        # chain keys (j', i) of its own position, 2 <= j' <= j
        qg = q.reshape(S, Hkv, grp, hd)
        sc1 = es("igcd,kgd->gcik", qg, k1) * scale            # [Hkv, grp, S, S]
        sc1 = sc1.masked_fill(~causal, float("-inf"))
        scs = [sc1]
        for kc in chain_k:
            scs.append((es("igcd,igd->gci", qg, kc) * scale)[..., None])
        p = torch.softmax(torch.cat(scs, dim=-1), dim=-1)
        a = es("gcik,kgd->igcd", p[..., :S], v1)
        for c, vc in enumerate(chain_v):
            a = a + es("gci,igd->igcd", p[..., S + c], vc)
        a = gq(_rnd(cfg, a.reshape(S, Hq * hd)))
        h1 = s + gq(mm(a, P["o"].T))
        u = _rnd(cfg, _rms(h1, P["norm_ffn"], eps))
        gu = gq(mm(u, P["gate_up"].T))
        gate, up = gu[:, :F], gu[:, F:]
        z = _rnd(cfg, gate * torch.sigmoid(gate) * up)
        h2 = h1 + gq(mm(z, P["down"].T))
        y = _rnd(cfg, _rms(h2, P["norm_out"], eps))
        logits = mm(y, P["lm"].T)
        l32 = gq(_st(logits, logits.detach().to(torch.float32).to(torch.float64)))   # R43: CE on float32 logits
        logits_all.append(l32.detach().numpy())
        pred[j - 1] = np.argmax(l32.detach().to(torch.float32).numpy(), axis=1)
        n_valid = max(S - j, 0)            # rows i <= S-1-j have the label x_{i+j}
        if n_valid:
            lab = torch.as_tensor(np.asarray(tokens[j:], dtype=np.int64))
            rows = l32[:n_valid]
            ce_rows = torch.logsumexp(rows, dim=1) - rows.gather(1, lab[:, None])[:, 0]
            ce_sum = ce_sum + ce_rows.sum()
            ce[j - 1, :n_valid] = ce_rows.detach().numpy()
        s = h2
        if j < R:
            nxt = pred[j - 1] if forced is None else np.asarray(forced[j - 1])
            t = torch.as_tensor(np.asarray(nxt, dtype=np.int64))        # R44: no gradient
    return ce_sum, ce, pred, logits_all


def ttt_loss_and_grads(cfg, W, feats, tokens, R, forced=None, want_grads=True, grad_bf16=False, gemm_f32=False):
    """Loss (R45) and its gradients w.r.t. the trained parameters (R42).

    grad_bf16 (a precision variant, not the reference): the gradients that
    reach a GEMM as an operand in a bf16 backward -- at the logits, at the
    outputs of the g, qkv, o, gate_up and down projections and at the
    attention output -- are rounded to bfloat16, as a backward with bf16 GEMM
    operands must; gemm_f32 (another precision variant) takes every product
    of the forward and the backward in float32.  Together they show how far
    a bf16-operand, fp32-accumulation training step may lie from the exact
    gradient (the forward's own bf16 roundings then differ now and then).

    W: drafter weights (arrays; row-major [out, in] matrices, gains [d]);
    feats [B, S, 3, d]; tokens [B, S]; forced [B, R-1, S] or None.
    Returns dict(loss, ce [B, R, S], pred [B, R, S], logits [B][R] arrays
    [S, V], grads {name: fp64 array of the parameter's shape}) -- grads only
    when want_grads."""
    feats = np.asarray(feats)
    tokens = np.asarray(tokens)
    Bn, S = tokens.shape
    P = {}
    for name in TRAINED + ("emb", "lm"):
        P[name] = _t(W[name])
        if want_grads and name in TRAINED:
            P[name].requires_grad_(True)
    count = Bn * sum(max(S - j, 0) for j in range(1, R + 1))
    total = torch.zeros((), dtype=torch.float64)
    ce = np.zeros((Bn, R, S))
    pred = np.zeros((Bn, R, S), np.int32)
    logits = []
    for b in range(Bn):
        s, ce[b], pred[b], lg = _sequence(cfg, P, _t(feats[b]), tokens[b], R,
                                          None if forced is None else forced[b], grad_bf16, gemm_f32)
        total = total + s
        logits.append(lg)
    loss = total / count if count else total
    out = dict(loss=float(loss.detach()), ce=ce, pred=pred, logits=logits)
    if want_grads:
        if count:
            gr = torch.autograd.grad(loss, [P[n] for n in TRAINED], allow_unused=True)
        else:
            gr = [None] * len(TRAINED)
        out["grads"] = {n: (np.zeros(np.shape(W[n])) if g is None else g.detach().numpy())
                        for n, g in zip(TRAINED, gr)}
    return out
