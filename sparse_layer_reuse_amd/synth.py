"""Seeded synthetic inputs for the decode workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through the tests and the benchmark)
and the CPU oracle (through the tests) consume what it produces.

Recipe (per layer l of a workload with base seed S):
  * q, K, V ~ N(0, 1) in float32 from torch generators seeded S+16l+0/1/2;
  * hot blocks: per (layer, sequence) a set of ``hot_blocks`` logical blocks,
    drawn with numpy PCG64 seeded S+16l+3 (independent per layer), or, with
    drift, layer l+1's set is layer l's with round(drift*|set|) members
    replaced by uniform draws from the non-hot blocks;
  * every key of a hot block gets ``alpha * u`` added, u being the unit vector
    of the sum of the query heads of the key's KV group;
  * offsets are added in float32, then everything is rounded once to the
    workload's element type (round-to-nearest-even for bfloat16);
  * block table: identity (sequence b, block n -> page b*N+n) or, when paged,
    a PCG64 permutation (seed S+4) of all pages.
Layouts: q [B][Hq][d], K [pages][Hkv][128][d], V [pages][Hkv][4][d][32].
"""
from __future__ import annotations

import numpy as np
import torch

from .workloads import BLOCK, Workload

SUBTILE = 32  # tokens per V sub-tile

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def block_table(batch, max_blocks, *, paged=False, seed=0):
    """[B][max_blocks] int32 page ids (numpy): identity or a seeded permutation."""
    pages = np.arange(batch * max_blocks, dtype=np.int64)
    if paged:
        pages = np.random.Generator(np.random.PCG64(seed)).permutation(pages)
    return pages.reshape(batch, max_blocks).astype(np.int32)


def hot_sets(num_blocks_per_seq, count, seed, *, batch=1, drift=0.0, layers=1, drift_seed=None):
    """Hot block sets for ``layers`` consecutive layers of ``batch`` sequences.

    Returns a list (per layer) of lists (per sequence) of sorted numpy int arrays.
    ``num_blocks_per_seq`` is a list of per-sequence block counts.
    ``seed`` may be a callable layer -> seed for independent per-layer draws.
    """
    out = []
    prev = None
    for l in range(layers):
        s = seed(l) if callable(seed) else seed
        rng = np.random.Generator(np.random.PCG64(s))
        cur = []
        for b in range(batch):
            nb = int(num_blocks_per_seq[b])
            c = min(count, nb)
            if prev is None or drift <= 0.0:
                cur.append(np.sort(rng.choice(nb, size=c, replace=False)))
            else:
                old = prev[b]
                swap = min(int(round(drift * len(old))), len(old))
                keep = np.sort(rng.choice(len(old), size=len(old) - swap, replace=False))
                rest = np.setdiff1d(np.arange(nb), old)
                new = rng.choice(rest, size=min(swap, len(rest)), replace=False)
                cur.append(np.sort(np.concatenate([old[keep], new])))
        out.append(cur)
        if drift > 0.0:
            prev = cur
    return out


def make_layer(*, batch, num_q_heads, num_kv_heads, head_dim, dtype, ctx_lens,
               max_blocks=None, seed=0, paged=False, hot=None, alpha=0.0,
               device="cpu", table=None, num_pages=None):
    """One layer's q / K pool / V pool / block table / context lengths.

    ``ctx_lens``: per-sequence context lengths (ragged allowed).
    ``hot``: optional list (per sequence) of logical block ids that get the
    planted key offset ``alpha * u``.
    Returns a dict of torch tensors on ``device`` (table and ctx as int32).
    """
    ctx_lens = [int(t) for t in ctx_lens]
    if max_blocks is None:
        max_blocks = max(1, max((t + BLOCK - 1) // BLOCK for t in ctx_lens))
    if table is None:
        table = block_table(batch, max_blocks, paged=paged, seed=seed + 4)
    table = np.asarray(table, dtype=np.int32)
    if num_pages is None:
        num_pages = int(table.max()) + 1 if table.size else 1
    B, Hq, Hkv, d = batch, num_q_heads, num_kv_heads, head_dim
    G = Hq // Hkv
    q = torch.randn(B, Hq, d, generator=_gen(device, seed + 0), device=device)
    k = torch.randn(num_pages, Hkv, BLOCK, d, generator=_gen(device, seed + 1), device=device)
    v = torch.randn(num_pages, Hkv, BLOCK // SUBTILE, d, SUBTILE, generator=_gen(device, seed + 2),
                    device=device)
    if hot is not None and alpha != 0.0:
        u = q.view(B, Hkv, G, d).sum(dim=2)
        u = u / u.norm(dim=-1, keepdim=True)
        for b in range(B):
            blocks = np.asarray(hot[b], dtype=np.int64)
            if blocks.size == 0:
                continue
            pages = torch.as_tensor(table[b, blocks].astype(np.int64), device=device)
            k[pages] += alpha * u[b][None, :, None, :]
    dt = TORCH_DTYPE[dtype]
    return dict(q=q.to(dt).contiguous(), k_pool=k.to(dt).contiguous(),
                v_pool=v.to(dt).contiguous(),
                table=torch.as_tensor(table, device=device),
                ctx=torch.as_tensor(np.asarray(ctx_lens, dtype=np.int32), device=device))


def layer_seed(wl: Workload, layer: int) -> int:
    return wl.seed + 16 * layer


def workload_hot_sets(wl: Workload):
    """Hot sets of every layer of a workload (list over layers of lists over sequences)."""
    if wl.hot_blocks <= 0:
        return [[np.zeros(0, np.int64)] * wl.batch for _ in range(wl.layers)]
    return hot_sets([wl.blocks] * wl.batch, wl.hot_blocks,
                    (lambda l: layer_seed(wl, l) + 3), batch=wl.batch,
                    drift=wl.hot_drift, layers=wl.layers)


def workload_layer(wl: Workload, layer: int, *, device="cpu", hot=None, table=None):
    """Inputs of one layer of a named workload."""
    if hot is None:
        hot = workload_hot_sets(wl)[layer]
    if table is None:
        table = block_table(wl.batch, wl.blocks, paged=wl.paged, seed=wl.seed + 4)
    return make_layer(batch=wl.batch, num_q_heads=wl.num_q_heads,
                      num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, dtype=wl.dtype,
                      ctx_lens=[wl.ctx] * wl.batch, max_blocks=wl.blocks,
                      seed=layer_seed(wl, layer), hot=hot, alpha=wl.hot_alpha,
                      device=device, table=table, num_pages=wl.batch * wl.blocks)


def workload_layers(wl: Workload, *, device="cpu", layers=None):
    """Inputs of several layers (default: all) of a named workload."""
    hot = workload_hot_sets(wl)
    table = block_table(wl.batch, wl.blocks, paged=wl.paged, seed=wl.seed + 4)
    idx = range(wl.layers) if layers is None else layers
    return [workload_layer(wl, l, device=device, hot=hot[l], table=table) for l in idx]


def similarity_matrix(num_layers, decay, *, noise=0.03, seed=0):
    """Synthetic lower-triangular similarity matrix, stored row = target,
    column = source: M[j][i] = clip(exp(-(j-i)/decay) + N(0, noise), 0, 1)
    for i <= j, zero above the diagonal."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = int(num_layers)
    M = np.zeros((L, L), dtype=np.float64)
    for j in range(L):
        for i in range(j + 1):
            M[j, i] = min(1.0, max(0.0, np.exp(-(j - i) / decay) + rng.normal(0.0, noise)))
    return M.astype(np.float32)


def workload_similarity(wl: Workload):
    return similarity_matrix(wl.layers, wl.dp_decay, noise=wl.dp_noise, seed=wl.seed + 7)


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor with the exact bits the GPU reads:
    float32 stays float32, bfloat16 becomes its uint16 bit pattern."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError("unsupported dtype %s" % t.dtype)


def layer_to_oracle(layer: dict) -> dict:
    return {k: to_oracle(v) for k, v in layer.items()}
