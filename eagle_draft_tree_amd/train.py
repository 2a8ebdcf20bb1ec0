"""Host-side buffers of one training-time-test forward + backward through
the C ABI (eagle3_ttt_train).

Device memory comes from torch; every step runs in the library's kernels on
torch's current stream.  Argument marshalling only.
"""
from __future__ import annotations

import torch

from . import binding as B


def grad_shapes(shape) -> dict:
    """Logical shapes of the gradients eagle3_ttt_train writes."""
    d, F = shape.d, shape.ffn
    qd = shape.n_q_heads * shape.head_dim
    return dict(fc=(d, 3 * d), qkv=(shape.qkv_rows, 2 * d), o=(d, qd), gate_up=(2 * F, d), down=(d, F),
                norm_e=(d,), norm_s=(d,), norm_ffn=(d,), norm_out=(d,))


class TTTTrain:
    """Outputs, gradients and workspace of eagle3_ttt_train for B sequences
    of S tokens and R rollout steps of `drafter` (a cycle.Drafter)."""

    def __init__(self, drafter, Bn, S, R, device="cuda"):
        self.dr, self.B, self.S, self.R = drafter, Bn, S, R
        self.pred = torch.empty(Bn, R, S, dtype=torch.int32, device=device)
        self.ce = torch.empty(Bn, R, S, dtype=torch.float32, device=device)
        self.loss = torch.empty(1, dtype=torch.float32, device=device)
        self.grads = {n: torch.empty(shp, dtype=torch.float32, device=device)
                      for n, shp in grad_shapes(drafter.shape).items()}
        nbytes = B.ttt_train_workspace_size(drafter.dims, Bn, S, R)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def run(self, feats, tokens, forced=None):
        """feats [B][S][3][d] bf16, tokens [B][S] int32, forced [B][R-1][S]
        int32 or None (device tensors)."""
        B.eagle3_ttt_train(self.dr.dims, self.dr.weights, feats, tokens, self.B, self.S, self.R, forced, self.pred,
                           self.ce, self.loss, self.grads, self.ws)
