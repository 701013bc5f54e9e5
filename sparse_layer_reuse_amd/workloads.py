"""Named decode workloads: shapes, top-k, layer policies and the planted
structure of their synthetic inputs.

The long-context settings stand in for the long-document benchmark and the
large models the HyLRA summary evaluates on (section 4: contexts of 8K-60K
tokens); the inputs are random with planted "hot" blocks instead of real
activations.  Shapes follow Llama-3-8B (32 query / 8 KV heads, head_dim 128,
32 layers) and Llama-3-70B (64 / 8, 80 layers) at 32K-128K context.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

BLOCK = 128


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16": element type of q, K and V
    ctx: int                        # context length of every sequence (tokens)
    topk: Tuple[int, ...]           # top-k blocks; the first entry is the default
    policy: str                     # "fixed" | "dp"
    resets: Tuple[int, ...] = ()    # reset layers of a fixed policy
    dp_theta: Tuple[float, ...] = ()  # thresholds of a DP policy (first = default)
    dp_decay: float = 0.0           # decay length of the synthetic similarity matrix
    dp_noise: float = 0.03          # std of the similarity matrix noise
    dp_force: Tuple[int, ...] = ()  # layers forced to reset
    hot_blocks: int = 0             # planted hot blocks per (layer, sequence)
    hot_alpha: float = 1.5          # key offset along the group's unit query direction
    hot_drift: float = 0.0          # fraction of the hot set swapped between layers (0 = independent)
    paged: bool = False             # randomly permuted physical pages
    seed: int = 0

    @property
    def blocks(self) -> int:
        return (self.ctx + BLOCK - 1) // BLOCK

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_layer(self) -> int:
        elt = 4 if self.dtype == "f32" else 2
        return 2 * self.batch * self.num_kv_heads * self.blocks * BLOCK * self.head_dim * elt


def round_half_up(x: float) -> int:
    return int(x + 0.5)


def src_from_resets(num_layers: int, resets) -> list:
    """Per-layer source list of a policy given its reset layers: a reset layer
    is its own source, any other layer keeps the previous layer's source."""
    resets = set(int(r) for r in resets)
    src = []
    for j in range(num_layers):
        src.append(j if (j == 0 or j in resets) else src[-1])
    return src


TINY_F32 = Workload(
    name="tiny_f32", batch=1, layers=4, num_q_heads=4, num_kv_heads=2, head_dim=64,
    dtype="f32", ctx=1024, topk=(2,), policy="fixed", resets=(0, 2),
    hot_blocks=2, hot_alpha=2.0, seed=1000)

LLAMA3_8B_32K = Workload(
    name="llama3_8b_32k", batch=1, layers=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
    dtype="bf16", ctx=32768, topk=(16,), policy="fixed",
    resets=tuple(sorted({0, 1, 2, 3} | {l for l in range(4, 32) if l % 4 == 0})),
    hot_blocks=round_half_up(0.05 * 256), hot_alpha=1.5, seed=2000)

LLAMA3_8B_B8_64K_DP = Workload(
    name="llama3_8b_b8_64k_dp", batch=8, layers=32, num_q_heads=32, num_kv_heads=8,
    head_dim=128, dtype="bf16", ctx=65536, topk=(32,), policy="dp", dp_theta=(0.8,),
    dp_decay=6.0, dp_force=(0, 1, 2, 3), hot_blocks=round_half_up(0.05 * 512),
    hot_alpha=1.5, hot_drift=0.10, seed=3000)

LLAMA3_8B_PAGED_128K = Workload(
    name="llama3_8b_paged_128k", batch=4, layers=32, num_q_heads=32, num_kv_heads=8,
    head_dim=128, dtype="bf16", ctx=131072, topk=(8, 32, 64), policy="fixed",
    resets=tuple(l for l in range(32) if l % 4 == 0),
    hot_blocks=round_half_up(0.03 * 1024), hot_alpha=1.5, paged=True, seed=4000)

LLAMA3_70B_128K_DP = Workload(
    name="llama3_70b_128k_dp", batch=1, layers=80, num_q_heads=64, num_kv_heads=8,
    head_dim=128, dtype="bf16", ctx=131072, topk=(32,), policy="dp",
    dp_theta=(0.8, 0.7, 0.9), dp_decay=10.0, dp_force=(0, 1, 2, 3),
    hot_blocks=round_half_up(0.05 * 1024), hot_alpha=1.5, hot_drift=0.10, seed=5000)

ALL = {w.name: w for w in (TINY_F32, LLAMA3_8B_32K, LLAMA3_8B_B8_64K_DP,
                           LLAMA3_8B_PAGED_128K, LLAMA3_70B_128K_DP)}


def get(name: str) -> Workload:
    try:
        return ALL[name]
    except KeyError:
        raise KeyError("unknown workload %r (have %s)" % (name, ", ".join(ALL))) from None
