"""ctypes binding of ``libeagle3.so`` (the C ABI in include/eagle3.h).

Argument marshalling only: tensors are passed as device pointers, every step
runs in the library's HIP kernels on the caller's (torch current) stream.
There is no fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libeagle3.so")

EAGLE3_OK = 0
EINVAL, ECAPACITY, EUNSUPPORTED, EWORKSPACE, EHIP, ENUMERIC = -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
COMMIT, TREE = 0, 1
TOPK_ALL, TOPK_LAST = 0, 1
INIT, STEP, FINAL = 0, 1, 2
GREEDY, SAMPLE = 0, 1
MAX_TREE_SLOTS = 64
MAX_TOPK = 16

c_i32p = ctypes.POINTER(ctypes.c_int32)
vp = ctypes.c_void_p


class Dims(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


LAYOUT_ROWMAJOR, LAYOUT_PACKED = 0, 1


class Weights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("fc", "emb", "qkv", "o", "gate_up", "down", "lm",
                                  "norm_e", "norm_s", "norm_ffn", "norm_out")] + [("layout", ctypes.c_int32)] + \
               [(n, vp) for n in ("norm_fc", "norm_post_attn", "norm_post_ffn")]


GRAD_NAMES = ("fc", "qkv", "o", "gate_up", "down", "norm_e", "norm_s", "norm_ffn", "norm_out")


class Grads(ctypes.Structure):
    _fields_ = [(n, vp) for n in GRAD_NAMES]


class KV(ctypes.Structure):
    _fields_ = [("k", vp), ("v", vp), ("cap", ctypes.c_int32), ("block_table", vp),
                ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("ctx_len", vp), ("tk", vp), ("tv", vp)]


class LowrankHead(ctypes.Structure):
    _fields_ = [("a", vp), ("b", vp), ("rank", ctypes.c_int32), ("candidates", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class TargetLayer(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("qkv", "o", "gate_up", "down", "norm_attn", "norm_ffn")]


class Target(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("layers", ctypes.POINTER(TargetLayer)), ("emb", vp), ("lm", vp),
                ("norm_out", vp), ("layout", ctypes.c_int32), ("feat_layers", ctypes.c_int32 * 3)]


class CostTable(ctypes.Structure):
    _fields_ = [("n_batch", ctypes.c_int32), ("n_ctx", ctypes.c_int32), ("n_tok", ctypes.c_int32),
                ("batch", vp), ("ctx", vp), ("tok", vp), ("draft_ms", vp), ("verify_ms", vp)]


COST_DRAFT, COST_VERIFY = 0, 1


class Eagle3Error(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed: {code} ({msg})")
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} not built: run eagle_draft_tree_amd/build.py")
    # torch ships its own HIP runtime under the same soname; when torch is
    # used at all it must be loaded first, so that the library binds to that
    # runtime rather than bringing in a second one (which then finds no device)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I, SZ = vp, ctypes.c_int, ctypes.c_size_t
    sigs = {
        "eagle3_strerror": ([I], ctypes.c_char_p),
        "eagle3_last_error": ([], ctypes.c_char_p),
        "eagle3_version": ([], ctypes.c_char_p),
        "eagle3_workspace_size": ([P, I, I, I, ctypes.POINTER(SZ)], I),
        "eagle3_tree_state_size": ([I, I, I, ctypes.POINTER(SZ)], I),
        "eagle3_ttt_workspace_size": ([P, I, I, I, ctypes.POINTER(SZ)], I),
        "eagle3_fuse": ([P, P, P, I, P, P, SZ, P], I),
        "eagle3_draft_step": ([P, P, P, I, I, I, P, P, P, P, P, I, I, I, P, P, P, P, P, SZ, P], I),
        "eagle3_draft_step_lowrank": ([P, P, P, I, I, I, P, P, P, P, P, I, I, I, P, P, P, P, P, P, P, P, SZ, P], I),
        "eagle3_pack_matrix": ([P, I, I, P, SZ, P], I),
        "eagle3_tree_expand": ([I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P], I),
        "eagle3_verify": ([I, I, I, I, P, P, P, I, ctypes.c_float, P, P, P, P, P, P, P, SZ, P], I),
        "eagle3_verify_workspace_size": ([I, I, I, ctypes.POINTER(SZ)], I),
        "eagle3_verify_noalloc": ([I, I, I, I, P, P, P, I, ctypes.c_float, P, P, P, P, P, P, P], I),
        "eagle3_ttt_forward": ([P, P, P, P, I, I, I, P, P, P, P, P, SZ, P], I),
        "eagle3_ttt_train_workspace_size": ([P, I, I, I, ctypes.POINTER(SZ)], I),
        "eagle3_ttt_train": ([P, P, P, P, I, I, I, P, P, P, P, P, P, SZ, P], I),
        "eagle3_topk": ([P, I, I, I, P, P, P, P, SZ, P], I),
        "eagle3_timing_enable": ([I, I], I),
        "eagle3_packed_weights_size": ([P, ctypes.POINTER(SZ)], I),
        "eagle3_pack_weights": ([P, P, P, SZ, P, P], I),
        "eagle3_timing_read": ([I, P, P], I),
        "eagle3_timing_mode": ([I, I], I),
        "eagle3_target_layer_packed_size": ([P, ctypes.POINTER(SZ)], I),
        "eagle3_pack_target_layer": ([P, P, P, SZ, P, P], I),
        "eagle3_target_workspace_size": ([P, I, I, I, ctypes.POINTER(SZ)], I),
        "eagle3_target_forward": ([P, P, P, I, I, P, P, P, I, I, P, P, P, P, SZ, P], I),
        "eagle3_kv_commit": ([P, I, P, I, I, P, P, I, P, P, P, P, P], I),
        "eagle3_harness_cost": ([P, I, I, I, ctypes.c_float, P], I),
        "eagle3_harness_continue": ([P, I, I, I, I, P, ctypes.c_double, ctypes.c_double, P], I),
        "eagle3_harness_verify_count": ([P, I, I, I, P, ctypes.c_double, P], I),
        "eagle3_harness_branch_cap": ([P, I, I, P, ctypes.c_double, P], I),
        "eagle3_tree_confidence": ([I, I, I, I, P, P, P, P], I),
    }
    for name, (args, res) in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(fn, rc):
    if rc != EAGLE3_OK:
        lib = load()
        raise Eagle3Error(fn, rc, f"{lib.eagle3_strerror(rc).decode()}: {lib.eagle3_last_error().decode()}")


def ptr(t):
    """Device (or host) pointer of a tensor, or NULL for None."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def dims_of(shape) -> Dims:
    """eagle3_dims of a workloads.configs.DrafterShape-like object."""
    return Dims(shape.d, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn, shape.vocab,
                BF16 if shape.dtype == "bf16" else F32, shape.rms_eps, shape.rope_theta)


def weights_of(t: dict) -> Weights:
    """eagle3_weights from a dict of device tensors (keeps no references)."""
    opt = [t[n].data_ptr() if t.get(n) is not None else None for n in ("norm_fc", "norm_post_attn", "norm_post_ffn")]
    return Weights(*(t[n].data_ptr() for n in ("fc", "emb", "qkv", "o", "gate_up", "down", "lm",
                                                "norm_e", "norm_s", "norm_ffn", "norm_out")), LAYOUT_ROWMAJOR, *opt)


# ---------------------------------------------------------------- queries
def workspace_size(dims: Dims, B: int, max_rows: int, max_ctx: int) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_workspace_size", load().eagle3_workspace_size(ctypes.byref(dims), B, max_rows, max_ctx,
                                                                 ctypes.byref(out)))
    return out.value


def tree_state_size(B: int, k: int, D: int) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_tree_state_size", load().eagle3_tree_state_size(B, k, D, ctypes.byref(out)))
    return out.value


def ttt_workspace_size(dims: Dims, B: int, S: int, R: int) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_ttt_workspace_size", load().eagle3_ttt_workspace_size(ctypes.byref(dims), B, S, R,
                                                                         ctypes.byref(out)))
    return out.value


def packed_weights_size(dims: Dims) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_packed_weights_size", load().eagle3_packed_weights_size(ctypes.byref(dims), ctypes.byref(out)))
    return out.value


def eagle3_pack_weights(dims, weights, dst, stream=None) -> Weights:
    """Pack the GEMM matrices into `dst` (device uint8 tensor); returns the packed eagle3_weights."""
    packed = Weights()
    _check("eagle3_pack_weights", load().eagle3_pack_weights(
        ctypes.byref(dims), ctypes.byref(weights), ptr(dst), dst.numel() * dst.element_size(),
        ctypes.byref(packed), stream_ptr(stream)))
    return packed


# ---------------------------------------------------------------- the five calls (+ topk)
def eagle3_fuse(dims, weights, feats, n, g, ws=None, stream=None):
    _check("eagle3_fuse", load().eagle3_fuse(ctypes.byref(dims), ctypes.byref(weights), ptr(feats), n,
                                             ptr(g), ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                             stream_ptr(stream)))


def eagle3_draft_step(dims, weights, kv, mode, B, rows, state, parent_slot, tokens, pos, anc, slot_base,
                      k, topk_rows, h_tree, topk_id, topk_lp, logits_out, ws, stream=None):
    _check("eagle3_draft_step", load().eagle3_draft_step(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), mode, B, rows, ptr(state),
        ptr(parent_slot), ptr(tokens), ptr(pos), ptr(anc), slot_base, k, topk_rows, ptr(h_tree),
        ptr(topk_id), ptr(topk_lp), ptr(logits_out), ptr(ws), ws.numel() * ws.element_size(),
        stream_ptr(stream)))


def eagle3_draft_step_lowrank(dims, weights, kv, mode, B, rows, state, parent_slot, tokens, pos, anc, slot_base,
                              k, topk_rows, h_tree, topk_id, topk_lp, logits_out, head, cand_out, cand_logits_out, ws,
                              stream=None):
    _check("eagle3_draft_step_lowrank", load().eagle3_draft_step_lowrank(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), mode, B, rows, ptr(state),
        ptr(parent_slot), ptr(tokens), ptr(pos), ptr(anc), slot_base, k, topk_rows, ptr(h_tree),
        ptr(topk_id), ptr(topk_lp), ptr(logits_out), ctypes.byref(head), ptr(cand_out), ptr(cand_logits_out),
        ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)))


def eagle3_pack_matrix(src, n, k, dst, stream=None):
    """Pack a bf16 matrix src [n][k] into dst (device tensor, n*k*2 bytes) in MFMA fragment order."""
    _check("eagle3_pack_matrix", load().eagle3_pack_matrix(ptr(src), n, k, ptr(dst), dst.numel() * dst.element_size(),
                                                           stream_ptr(stream)))


def eagle3_tree_expand(phase, B, k, D, m, root_tok, root_pos, tree_state, topk_id, topk_lp,
                       next_tok, next_parent_slot, next_pos, next_anc,
                       v_tok=None, v_parent=None, v_depth=None, v_pos=None, v_anc=None, stream=None):
    _check("eagle3_tree_expand", load().eagle3_tree_expand(
        phase, B, k, D, m, ptr(root_tok), ptr(root_pos), ptr(tree_state), ptr(topk_id), ptr(topk_lp),
        ptr(next_tok), ptr(next_parent_slot), ptr(next_pos), ptr(next_anc), ptr(v_tok), ptr(v_parent),
        ptr(v_depth), ptr(v_pos), ptr(v_anc), stream_ptr(stream)))


def verify_workspace_size(B: int, m: int, V: int) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_verify_workspace_size", load().eagle3_verify_workspace_size(B, m, V, ctypes.byref(out)))
    return out.value


def eagle3_verify(B, m, V, Dmax, v_tok, v_parent, target_logits, mode, temperature, u_try, u_res,
                  accept_len, accepted, bonus, status, ws, stream=None):
    _check("eagle3_verify", load().eagle3_verify(
        B, m, V, Dmax, ptr(v_tok), ptr(v_parent), ptr(target_logits), mode, float(temperature),
        ptr(u_try), ptr(u_res), ptr(accept_len), ptr(accepted), ptr(bonus), ptr(status),
        ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)))


def eagle3_verify_noalloc(B, m, V, Dmax, v_tok, v_parent, target_logits, mode, temperature, u_try, u_res,
                          accept_len, accepted, bonus, status, stream=None):
    _check("eagle3_verify_noalloc", load().eagle3_verify_noalloc(
        B, m, V, Dmax, ptr(v_tok), ptr(v_parent), ptr(target_logits), mode, float(temperature),
        ptr(u_try), ptr(u_res), ptr(accept_len), ptr(accepted), ptr(bonus), ptr(status), stream_ptr(stream)))


def eagle3_ttt_forward(dims, weights, feats, tokens, B, S, R, forced_tokens, pred, ce, loss, ws,
                       stream=None):
    _check("eagle3_ttt_forward", load().eagle3_ttt_forward(
        ctypes.byref(dims), ctypes.byref(weights), ptr(feats), ptr(tokens), B, S, R, ptr(forced_tokens),
        ptr(pred), ptr(ce), ptr(loss), ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)))


def ttt_train_workspace_size(dims: Dims, B: int, S: int, R: int) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_ttt_train_workspace_size",
           load().eagle3_ttt_train_workspace_size(ctypes.byref(dims), B, S, R, ctypes.byref(out)))
    return out.value


def grads_struct(grads: dict) -> Grads:
    """eagle3_grads from a dict of fp32 device tensors keyed by GRAD_NAMES."""
    return Grads(*(grads[n].data_ptr() for n in GRAD_NAMES))


def eagle3_ttt_train(dims, weights, feats, tokens, B, S, R, forced_tokens, pred, ce, loss, grads, ws, stream=None):
    g = grads_struct(grads)
    _check("eagle3_ttt_train", load().eagle3_ttt_train(
        ctypes.byref(dims), ctypes.byref(weights), ptr(feats), ptr(tokens), B, S, R, ptr(forced_tokens),
        ptr(pred), ptr(ce), ptr(loss), ctypes.byref(g), ptr(ws), ws.numel() * ws.element_size(),
        stream_ptr(stream)))


def eagle3_topk(logits, rows, V, k, ids, lp, lse, ws, stream=None):
    _check("eagle3_topk", load().eagle3_topk(ptr(logits), rows, V, k, ptr(ids), ptr(lp), ptr(lse), ptr(ws),
                                             ws.numel() * ws.element_size(), stream_ptr(stream)))


# ---------------------------------------------------------------- the target's verification forward
def target_layer_packed_size(dims: Dims) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_target_layer_packed_size", load().eagle3_target_layer_packed_size(ctypes.byref(dims),
                                                                                     ctypes.byref(out)))
    return out.value


def eagle3_pack_target_layer(dims, layer: TargetLayer, dst, stream=None) -> TargetLayer:
    """Pack one target layer's matrices into `dst` (device uint8 tensor); returns the packed layer."""
    packed = TargetLayer()
    _check("eagle3_pack_target_layer", load().eagle3_pack_target_layer(
        ctypes.byref(dims), ctypes.byref(layer), ptr(dst), dst.numel() * dst.element_size(), ctypes.byref(packed),
        stream_ptr(stream)))
    return packed


def target_workspace_size(dims: Dims, B: int, rows: int, max_cap: int) -> int:
    out = ctypes.c_size_t(0)
    _check("eagle3_target_workspace_size", load().eagle3_target_workspace_size(ctypes.byref(dims), B, rows, max_cap,
                                                                               ctypes.byref(out)))
    return out.value


def kv_array(kvs):
    """A host array of eagle3_kv structs (one per layer)."""
    arr = (KV * len(kvs))()
    for i, k in enumerate(kvs):
        arr[i] = k
    return arr


def eagle3_target_forward(dims, target: Target, kv_arr, B, rows, tokens, pos, anc, layer_begin, layer_end, hidden,
                          feats, logits, ws, stream=None):
    _check("eagle3_target_forward", load().eagle3_target_forward(
        ctypes.byref(dims), ctypes.byref(target), kv_arr, B, rows, ptr(tokens), ptr(pos), ptr(anc), layer_begin,
        layer_end, ptr(hidden), ptr(feats), ptr(logits), ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)))


def eagle3_kv_commit(dims, n_layers, kv_arr, B, rows, accept_len, accepted, Dmax, feats, feats_next, ctx_len_out,
                     status, stream=None):
    _check("eagle3_kv_commit", load().eagle3_kv_commit(
        ctypes.byref(dims), n_layers, kv_arr, B, rows, ptr(accept_len), ptr(accepted), Dmax, ptr(feats),
        ptr(feats_next), ptr(ctx_len_out), ptr(status), stream_ptr(stream)))


# ---------------------------------------------------------------- EAGLE-4 Harness
class HarnessTable:
    """A warm-up cost table held in host arrays (kept alive here) plus its
    eagle3_cost_table struct.  draft_ms / verify_ms: [n_batch][n_ctx][n_tok]."""

    def __init__(self, batch, ctx, tok, draft_ms, verify_ms):
        import numpy as np
        self.batch = np.ascontiguousarray(batch, dtype=np.int32)
        self.ctx = np.ascontiguousarray(ctx, dtype=np.int32)
        self.tok = np.ascontiguousarray(tok, dtype=np.int32)
        self.draft_ms = np.ascontiguousarray(draft_ms, dtype=np.float32)
        self.verify_ms = np.ascontiguousarray(verify_ms, dtype=np.float32)
        shp = (len(self.batch), len(self.ctx), len(self.tok))
        assert self.draft_ms.shape == shp and self.verify_ms.shape == shp
        self.struct = CostTable(*shp, *(a.ctypes.data for a in (self.batch, self.ctx, self.tok, self.draft_ms,
                                                                 self.verify_ms)))

    def as_dict(self):
        """The same table in the oracle's form."""
        return dict(batch=self.batch.tolist(), ctx=self.ctx.tolist(), tok=self.tok.tolist(),
                    draft=self.draft_ms.astype(float).tolist(), verify=self.verify_ms.astype(float).tolist())


def _host_f32(a):
    import numpy as np
    return np.ascontiguousarray(a, dtype=np.float32)


def harness_cost(table: HarnessTable, kind, B, ctx, n):
    out = ctypes.c_double(0)
    _check("eagle3_harness_cost", load().eagle3_harness_cost(ctypes.byref(table.struct), kind, B, ctx, float(n),
                                                             ctypes.byref(out)))
    return out.value


def harness_continue(table: HarnessTable, B, ctx, k, depth, frontier_logconf, tau0, alpha):
    a = _host_f32(frontier_logconf)
    go = ctypes.c_int(0)
    _check("eagle3_harness_continue", load().eagle3_harness_continue(
        ctypes.byref(table.struct), B, ctx, k, depth, a.ctypes.data, float(tau0), float(alpha), ctypes.byref(go)))
    return bool(go.value)


def harness_verify_count(table: HarnessTable, B, ctx, logconf_sorted, tau):
    a = _host_f32(logconf_sorted)
    m = ctypes.c_int(0)
    _check("eagle3_harness_verify_count", load().eagle3_harness_verify_count(
        ctypes.byref(table.struct), B, ctx, a.shape[1], a.ctypes.data, float(tau), ctypes.byref(m)))
    return m.value


def harness_branch_cap(table: HarnessTable, B, ctx, root_lp, tau):
    a = _host_f32(root_lp)
    k = ctypes.c_int(0)
    _check("eagle3_harness_branch_cap", load().eagle3_harness_branch_cap(
        ctypes.byref(table.struct), B, ctx, a.ctypes.data, float(tau), ctypes.byref(k)))
    return k.value


def eagle3_tree_confidence(B, k, D, m_max, tree_state, frontier_logconf, pool_logconf, stream=None):
    _check("eagle3_tree_confidence", load().eagle3_tree_confidence(
        B, k, D, m_max, ptr(tree_state), ptr(frontier_logconf), ptr(pool_logconf), stream_ptr(stream)))


# ---------------------------------------------------------------- kernel timing
KC = dict(fuse=0, rowops=1, qkv=2, attn=3, o=4, gate_up=5, down=6, lm_head=7, topk=8, tree=9, verify=10,
          ttt_gemm=11, ttt_attn=12, ttt_ce=13, lr_scores=14, target=15, tgt_gate_up=16, tgt_lm_head=17,
          ttt_bwd_gemm=18, ttt_bwd_attn=19, ttt_wgrad=20, ttt_bwd_rows=21)


def timing_enable(kc: int, max_launches: int):
    _check("eagle3_timing_enable", load().eagle3_timing_enable(kc, max_launches))


def timing_mode(kc: int, mode: int):
    """0: events around each launch scope of the class; 1: the class's principal kernel's own start/stop."""
    _check("eagle3_timing_mode", load().eagle3_timing_mode(kc, mode))


def timing_read(kc: int):
    """(total milliseconds, launches) recorded for kernel class kc."""
    ms = ctypes.c_double(0)
    cnt = ctypes.c_int(0)
    _check("eagle3_timing_read", load().eagle3_timing_read(kc, ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value
