"""Host-side owner of a target model and its caches for the verification
forward through the C ABI (eagle3_target_forward, eagle3_kv_commit).

Device memory comes from torch; every step runs in the library's kernels on
torch's current stream.  Argument marshalling only.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import binding as B

_MATS = ("qkv", "o", "gate_up", "down")


def _dev(t, device):
    if isinstance(t, torch.Tensor):
        return t.to(device)
    if hasattr(t, "torch"):
        return t.torch(device)
    return torch.as_tensor(np.asarray(t, dtype=np.float32)).to(device)


class TargetWeights:
    """Device-resident target layers plus the eagle3_target struct.

    layers: per-layer dicts (qkv, o, gate_up, down, norm_attn, norm_ffn) of
    generator Tensors, arrays or device tensors; emb, lm, norm_out likewise
    (emb and lm may be the drafter's own device tensors).  pack=True (bf16)
    converts every layer into MFMA fragment order, one layer at a time, and
    drops the row-major copies (entries of `layers` are set to None as they
    are packed, so that device-resident inputs are freed one layer at a
    time); the LM head is packed too unless lm_packed (an already packed
    lm) is given."""

    def __init__(self, shape, layers, emb, lm, norm_out, feat_layers, device="cuda", pack=False, lm_packed=None):
        self.shape = shape
        self.dims = B.dims_of(shape)
        self.keep = []
        pack = pack and shape.dtype == "bf16"
        n = len(layers)
        self.layer_arr = (B.TargetLayer * n)()
        for l in range(n):
            t = {k: _dev(v, device) for k, v in layers[l].items()}
            lay = B.TargetLayer(*(t[k].data_ptr() for k in _MATS), t["norm_attn"].data_ptr(),
                                t["norm_ffn"].data_ptr())
            if pack:
                buf = torch.empty(B.target_layer_packed_size(self.dims), dtype=torch.uint8, device=device)
                lay = B.eagle3_pack_target_layer(self.dims, lay, buf)
                torch.cuda.synchronize()
                for k in _MATS:
                    del t[k]
                t["packed"] = buf
                layers[l] = None
            self.layer_arr[l] = lay
            self.keep.append(t)
        self.emb = _dev(emb, device)
        self.norm_out = _dev(norm_out, device)
        if lm_packed is not None:
            self.lm = lm_packed
        else:
            lm_t = _dev(lm, device)
            if pack:
                self.lm = torch.empty_like(lm_t)
                B.eagle3_pack_matrix(lm_t, lm_t.shape[0], lm_t.shape[1], self.lm)
                torch.cuda.synchronize()
                del lm_t
            else:
                self.lm = lm_t
        self.layout = B.LAYOUT_PACKED if pack or lm_packed is not None else B.LAYOUT_ROWMAJOR
        fl = (ctypes.c_int32 * 3)(*feat_layers)
        self.struct = B.Target(n, ctypes.cast(self.layer_arr, ctypes.POINTER(B.TargetLayer)), self.emb.data_ptr(),
                               self.lm.data_ptr(), self.norm_out.data_ptr(), self.layout, fl)
        self.n_layers = n


class TargetCache:
    """Per-layer K/V caches of B requests: contiguous [L][B][cap][Hkv][hd],
    or paged pools [L][n_blocks][block_size][Hkv][hd] behind one block table
    [B][max_blocks] shared by every layer; tree slots [L][B][64][Hkv][hd];
    committed lengths ctx_len [B] shared by every layer."""

    def __init__(self, shape, n_layers, Bn, cap, dtype, device="cuda", paged=False, block_size=16, n_blocks=0,
                 block_table=None, k=None, v=None):
        hkv, hd = shape.n_kv_heads, shape.head_dim
        self.n_layers, self.B = n_layers, Bn
        self.paged = paged
        if paged:
            self.k = k if k is not None else torch.zeros(n_layers, n_blocks, block_size, hkv, hd, dtype=dtype,
                                                         device=device)
            self.v = v if v is not None else torch.zeros_like(self.k)
            self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
            self.max_blocks = self.block_table.shape[1]
            self.block_size = block_size
            self.cap = 0
        else:
            self.k = k if k is not None else torch.zeros(n_layers, Bn, cap, hkv, hd, dtype=dtype, device=device)
            self.v = v if v is not None else torch.zeros_like(self.k)
            self.block_table = None
            self.max_blocks = self.block_size = 0
            self.cap = cap
        self.tk = torch.zeros(n_layers, Bn, B.MAX_TREE_SLOTS, hkv, hd, dtype=dtype, device=device)
        self.tv = torch.zeros_like(self.tk)
        self.ctx_len = torch.zeros(Bn, dtype=torch.int32, device=device)
        self.arr = B.kv_array([self._kv(l) for l in range(n_layers)])

    def _kv(self, l):
        bt = self.block_table.data_ptr() if self.block_table is not None else None
        return B.KV(self.k[l].data_ptr(), self.v[l].data_ptr(), self.cap, bt, self.max_blocks, self.block_size,
                    self.ctx_len.data_ptr(), self.tk[l].data_ptr(), self.tv[l].data_ptr())

    def cap_rows(self):
        return self.max_blocks * self.block_size if self.paged else self.cap


class VerifyForward:
    """Buffers of one verification forward of B x rows verify rows: the
    residual stream, the features, the logits and the workspace."""

    def __init__(self, tw: TargetWeights, cache: TargetCache, rows, device="cuda", keep_logits=True):
        s = tw.shape
        self.tw, self.cache, self.rows = tw, cache, rows
        Bn = cache.B
        dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
        self.hidden = torch.empty(Bn, rows, s.d, dtype=torch.float32, device=device)
        self.feats = torch.zeros(Bn, rows, 3, s.d, dtype=dt, device=device)
        self.logits = torch.empty(Bn, rows, s.vocab, dtype=torch.float32, device=device) if keep_logits else None
        nbytes = B.target_workspace_size(tw.dims, Bn, rows, max(cache.cap_rows(), 1))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def run(self, tokens, pos, anc, begin=0, end=None, logits=True):
        end = self.tw.n_layers if end is None else end
        B.eagle3_target_forward(self.tw.dims, self.tw.struct, self.cache.arr, self.cache.B, self.rows, tokens, pos,
                                anc, begin, end, self.hidden, self.feats, self.logits if logits else None, self.ws)

    def commit(self, accept_len, accepted, Dmax, feats_next=None, ctx_len_out=None, status=None):
        B.eagle3_kv_commit(self.tw.dims, self.tw.n_layers, self.cache.arr, self.cache.B, self.rows, accept_len,
                           accepted, Dmax, self.feats if feats_next is not None else None, feats_next,
                           ctx_len_out, status)
