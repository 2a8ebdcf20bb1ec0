"""Workload shapes for the EAGLE-3 draft-and-verify path.

Pure data: drafter shapes, tree/verify parameters and synthetic-input
recipes.  Nothing here computes any step of the method.

Shapes follow the drafters the EAGLE-3 pages name (a Llama-3.1-8B-shaped and
a Llama-3.3-70B-shaped one-layer drafter, "EAGLE-3 精读" §4 结果与消融) plus a
tiny fp32 drafter small enough for exhaustive CPU checks.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class DrafterShape:
    """One-layer drafter dimensions ("EAGLE-3 精读" §1: fusion 3d -> d, one decoder layer)."""
    name: str
    d: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass(frozen=True)
class Workload:
    """A full synthetic workload: drafter shape + tree + verify + input recipe."""
    name: str
    shape: DrafterShape
    batch: int = 1
    depth: int = 3            # D: drafter rounds incl. the root round = max node depth
    topk: int = 2             # k: children per frontier node and beam width
    keep: int = 8             # m: drafted nodes sent to verification (plus the root)
    prefix: int = 64          # committed prefix length before the root
    commit_rows: int = 1      # rows the COMMIT step appends (root is the last)
    synthetic_prefix_kv: bool = True   # prefix K/V drawn N(0,1) instead of computed
    target_sigma: float = 2.0 # target logits N(0, sigma)
    planted_accept: Optional[float] = None  # planted per-node argmax agreement
    planted_accept_range: Optional[tuple] = None  # per-request U[lo,hi] (serving)
    paged: bool = False
    block_size: int = 16
    prefix_range: Optional[tuple] = None  # per-request prefix length U[lo,hi]
    verify_modes: tuple = ("greedy",)
    temperature: float = 1.0
    feat_scale: float = 1.0   # target features N(0,1) * feat_scale
    # TTT
    ttt_seq: int = 0
    ttt_steps: int = 5
    # efficient LM head (EAGLE-4): low-rank rank and candidates (0 = the full
    # head); the LM head is then drawn with a rank-`lowrank_rank` part holding
    # `lowrank_energy` of its entry variance, and that part is the low-rank head
    lowrank_rank: int = 0
    lowrank_candidates: int = 0
    lowrank_energy: float = 0.9
    # target verification forward: the target model scoring the m+1 verify rows
    target: Optional["TargetModel"] = None


@dataclass(frozen=True)
class TargetModel:
    """A target model: n_layers pre-norm decoder layers of `shape`'s layer
    shape with a d-wide attention input, sharing the drafter's embedding and
    LM head.  feat_layers: the low/mid/high feature layers, counted from 1
    (the hidden state after that many layers)."""
    name: str
    shape: DrafterShape
    n_layers: int
    feat_layers: tuple


TINY_SHAPE = DrafterShape("tiny-d256", d=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                          ffn=1024, vocab=4096, dtype=F32, rope_theta=10000.0)
L8B_SHAPE = DrafterShape("llama3.1-8b-drafter", d=4096, n_q_heads=32, n_kv_heads=8,
                         head_dim=128, ffn=14336, vocab=128256, dtype=BF16)
L70B_SHAPE = DrafterShape("llama3.3-70b-drafter", d=8192, n_q_heads=64, n_kv_heads=8,
                          head_dim=128, ffn=28672, vocab=128256, dtype=BF16)

# Tiny fp32 drafter: 64 committed prefix rows, the root is row 63.
C1_TINY = Workload(
    "tiny-fp32-b1-tree3x2-keep8", TINY_SHAPE, batch=1, depth=3, topk=2, keep=8,
    prefix=0, commit_rows=64, synthetic_prefix_kv=False, target_sigma=2.0,
    verify_modes=("greedy", "sample"), temperature=1.0, feat_scale=1.0 / 16.0)

# 8B-shaped drafter, batch 1, dynamic tree depth 6 / top-10 / 60 kept.
C2_8B_TREE = Workload(
    "llama3.1-8b-drafter-b1-tree6x10-keep60", L8B_SHAPE, batch=1, depth=6, topk=10,
    keep=60, prefix=2048, commit_rows=1, target_sigma=3.0, planted_accept=0.8,
    verify_modes=("greedy", "sample"))

# Serving: same drafter, batch 64, chain of 3 (k=1), paged 16-token KV.
C3_8B_CHAIN = Workload(
    "llama3.1-8b-drafter-b64-chain3-paged16", L8B_SHAPE, batch=64, depth=3, topk=1,
    keep=3, prefix=2048, commit_rows=1, target_sigma=3.0,
    planted_accept_range=(0.5, 0.9), paged=True, block_size=16,
    prefix_range=(256, 2048), verify_modes=("greedy",))

# 70B-shaped drafter, batch 1, tree 6/10/60, temperature-1 sampling verify.
C4_70B_TREE = Workload(
    "llama3.3-70b-drafter-b1-tree6x10-keep60", L70B_SHAPE, batch=1, depth=6, topk=10,
    keep=60, prefix=4096, commit_rows=1, target_sigma=3.0,
    verify_modes=("sample", "greedy"), temperature=1.0)

# Training-time-test forward, 8B-shaped drafter, 8 x 2048, 5 rollout steps.
C5_8B_TTT = Workload(
    "llama3.1-8b-drafter-ttt-b8x2048-r5", L8B_SHAPE, batch=8, ttt_seq=2048, ttt_steps=5)

CONFIGS = [C1_TINY, C2_8B_TREE, C3_8B_CHAIN, C4_70B_TREE, C5_8B_TTT]

# The 8B and 70B trees through EAGLE-4's efficient LM head: rank 256, the 64
# best low-rank scores re-scored exactly (an opt-in mode beside the full head).
C2E_8B_TREE_LOWRANK = replace(C2_8B_TREE, name="llama3.1-8b-drafter-b1-tree6x10-keep60-lowrank256-c64",
                              lowrank_rank=256, lowrank_candidates=64)
C4E_70B_TREE_LOWRANK = replace(C4_70B_TREE, name="llama3.3-70b-drafter-b1-tree6x10-keep60-lowrank256-c64",
                               lowrank_rank=256, lowrank_candidates=64)


# The targets of the two drafters: Llama-3.1-8B (32 layers) and Llama-3.3-70B
# (80 layers) layer stacks with the drafters' layer shapes; features after
# layers 2, L/2 and L-3.
L8B_TARGET = TargetModel("llama3.1-8b-target", L8B_SHAPE, 32, (2, 16, 29))
L70B_TARGET = TargetModel("llama3.3-70b-target", L70B_SHAPE, 80, (2, 40, 77))

# Target verification forward over the verify rows of the 8B/70B trees and of
# the batch-64 chains: root + kept nodes through every target layer, logits
# and the three feature layers out.
C2V_8B_TARGET_TREE = replace(C2_8B_TREE, name="llama3.1-8b-target32-b1-tree61rows-ctx2048", target=L8B_TARGET)
C3V_8B_TARGET_CHAIN = replace(C3_8B_CHAIN, name="llama3.1-8b-target32-b64-chain4rows-paged16", target=L8B_TARGET)
C4V_70B_TARGET_TREE = replace(C4_70B_TREE, name="llama3.3-70b-target80-b1-tree61rows-ctx4096", target=L70B_TARGET)


# The 8B tree with the EAGLE-3.1 norm variants EAGLE-4 keeps (FC norm and
# post-norm; gains 1 + 0.5 N(0,1)).
C2N_8B_TREE_NORMS = replace(C2_8B_TREE, name="llama3.1-8b-drafter-b1-tree6x10-keep60-fcnorm-postnorm")

# The 8B tree under the EAGLE-4 Harness (branch cap 8/4, up to 6 rounds, up
# to 60 verified nodes) with a warm-up table measured on the 8B drafter and
# the 8B target.  The drafter's final-norm gain is 5 (logit spread about 6.4
# instead of 1.3), so that draft confidences span the range the rules act on.
C2H_8B_TREE_HARNESS = replace(C2_8B_TREE, name="llama3.1-8b-drafter-b1-harness-d6-m60-target32", target=L8B_TARGET)


def tiny_shape(d=16, hq=2, hkv=1, hd=8, ffn=32, vocab=8, dtype=F32, theta=10000.0, name=None):
    """Very small drafters for exhaustive oracle checks."""
    return DrafterShape(name or f"micro-d{d}-v{vocab}-{dtype}", d=d, n_q_heads=hq,
                        n_kv_heads=hkv, head_dim=hd, ffn=ffn, vocab=vocab, dtype=dtype,
                        rope_theta=theta)


def scaled(w: Workload, **kw) -> Workload:
    return replace(w, **kw)
