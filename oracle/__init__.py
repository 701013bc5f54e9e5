"""HyLRA CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct reference of the hybrid decode attention path
of "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context Inference"
(technical summary sections 2.2-2.4).  Only ``tests/``, the smoke check and
the benchmark's CPU-baseline leg may import this package.  It shares no code
with the HIP path: the attention arithmetic lives in ``hylra_oracle.c`` (built
here with gcc into ``liboracle.so``), the policy dynamic program and its
brute-force check are plain Python below.

Array conventions (numpy): float32 arrays are fp32 data, uint16 arrays are
bfloat16 bit patterns.  K pages are ``[pages][Hkv][128][d]``, V pages are
``[pages][Hkv][4][d][32]`` (four 32-token sub-tiles, each dimension-major);
``table`` is ``[B][max_blocks]`` int32 and ``ctx`` ``[B]`` int32.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
library routines, closed forms, brute force or hand-derived fixtures.
"""
from __future__ import annotations

import ctypes
import itertools
import math
import os
import subprocess

import numpy as np

BLOCK = 128
SUB = 32  # tokens per V sub-tile
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hylra_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile ``hylra_oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_attend.argtypes = [I, I, I, I, I, ctypes.c_double, P, P, P, ctypes.c_int64,
                                      P, I, P, P, I, P, P, P]
        lib.oracle_attend.restype = I
        lib.oracle_block_score.argtypes = [I, I, I, I, P, P, P]
        lib.oracle_block_score.restype = None
        lib.oracle_topk.argtypes = [I, I, I, P, P, I, P, P]
        lib.oracle_topk.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError("oracle inputs are float32 or uint16 (bfloat16 bits), got %s" % a.dtype)


def set_threads(n: int) -> None:
    """Limit the OpenMP threads the C oracle uses (for single-core baselines)."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    try:
        libgomp = ctypes.CDLL("libgomp.so.1")
        libgomp.omp_set_num_threads(int(n))
    except OSError:
        pass


def attend(q, k_pool, v_pool, table, ctx, *, num_kv_heads, scale=None, sel=None, k=0,
           want_probs=False):
    """Full attention (``sel is None``) or attention restricted to the blocks in
    ``sel`` ([B][Hkv][k], -1 padded) -- HyLRA technical summary 2.3, sensitive
    and tolerant layers.  Returns ``(out [B][Hq][d] f64, lse [B][Hq] f64,
    probs [B][Hq][max_blocks*128] f64 or None)``."""
    q = np.ascontiguousarray(q)
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    table = np.ascontiguousarray(table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    dt = _dtype_code(q)
    if _dtype_code(k_pool) != dt or _dtype_code(v_pool) != dt:
        raise TypeError("q, K and V must share one element type")
    B, Hq, d = q.shape
    Hkv = int(num_kv_heads)
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    pages = k_pool.shape[0]
    if k_pool.shape != (pages, Hkv, BLOCK, d) or v_pool.shape != (pages, Hkv, BLOCK // SUB, d, SUB):
        raise ValueError("K pool must be [pages][Hkv][128][d], V pool [pages][Hkv][4][d][32]")
    max_blocks = table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        if sel.shape != (B, Hkv, k):
            raise ValueError("sel must be [B][Hkv][k]")
    out = np.zeros((B, Hq, d), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    probs = np.zeros((B, Hq, max_blocks * BLOCK), np.float64) if want_probs else None
    rc = _load().oracle_attend(B, Hq, Hkv, d, dt, float(scale), _ptr(q), _ptr(k_pool),
                               _ptr(v_pool), pages, _ptr(table), max_blocks, _ptr(ctx),
                               _ptr(sel), int(k), _ptr(out), _ptr(lse), _ptr(probs))
    if rc != 0:
        raise ValueError("block table names a page outside the pool")
    return out, lse, probs


def block_score(probs, ctx, *, num_kv_heads, max_blocks):
    """Block score: sum over the query heads of a KV group of the softmax
    probabilities of each 128-token block (summary 2.4 block granularity; the
    score itself is the specification's).  Returns [B][Hkv][max_blocks] f64."""
    probs = np.ascontiguousarray(probs, dtype=np.float64)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    B, Hq, _ = probs.shape
    score = np.zeros((B, num_kv_heads, max_blocks), np.float64)
    _load().oracle_block_score(B, Hq, num_kv_heads, max_blocks, _ptr(ctx), _ptr(probs),
                               _ptr(score))
    return score


def topk(score, ctx, k):
    """Top-k blocks per (b, g) by (score desc, id asc), emitted in ascending
    id order, -1 padded (summary 2.3 "top-k indices are extracted").
    Returns (idx [B][Hkv][k] int32, margin [B][Hkv] f64)."""
    score = np.ascontiguousarray(score, dtype=np.float64)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32)
    B, Hkv, max_blocks = score.shape
    idx = np.full((B, Hkv, k), -1, np.int32)
    margin = np.zeros((B, Hkv), np.float64)
    _load().oracle_topk(B, Hkv, max_blocks, _ptr(ctx), _ptr(score), int(k), _ptr(idx),
                        _ptr(margin))
    return idx, margin


def decode_full(q, k_pool, v_pool, table, ctx, *, num_kv_heads, scale=None):
    """Reset layer: full attention, block scores.  Returns (out, lse, score)."""
    out, lse, probs = attend(q, k_pool, v_pool, table, ctx, num_kv_heads=num_kv_heads,
                             scale=scale, want_probs=True)
    score = block_score(probs, ctx, num_kv_heads=num_kv_heads, max_blocks=table.shape[1])
    return out, lse, score


def check_policy(src):
    """A policy is valid when layer 0 resets and every later layer either
    resets (src[j] == j) or keeps the previous layer's source (summary 2.2:
    reset jumps go to the diagonal, vertical moves keep the source)."""
    src = [int(s) for s in src]
    if not src or src[0] != 0:
        return False
    return all(s == j or s == src[j - 1] for j, s in enumerate(src) if j > 0)


def run_policy(layers, src, k, *, num_kv_heads, scale=None):
    """One decode step of the hybrid policy (summary 2.3).

    ``layers`` is a list of dicts with keys q, k_pool, v_pool, table, ctx.
    Reset layer j: full attention, then top-k of the block scores becomes the
    carried index set.  Reuse layer j: attention restricted to the carried set
    of its source layer.  Returns a list of per-layer dicts with out, lse and
    idx (the set the layer computed or used) and margin (reset layers).
    """
    if not check_policy(src):
        raise ValueError("malformed policy %r" % (list(src),))
    res = []
    carried = None
    for j, layer in enumerate(layers):
        if src[j] == j:
            out, lse, score = decode_full(layer["q"], layer["k_pool"], layer["v_pool"],
                                          layer["table"], layer["ctx"],
                                          num_kv_heads=num_kv_heads, scale=scale)
            carried, margin = topk(score, layer["ctx"], k)
            res.append(dict(out=out, lse=lse, idx=carried.copy(), margin=margin,
                            score=score))
        else:
            out, lse, _ = attend(layer["q"], layer["k_pool"], layer["v_pool"],
                                 layer["table"], layer["ctx"], num_kv_heads=num_kv_heads,
                                 scale=scale, sel=carried, k=k)
            res.append(dict(out=out, lse=lse, idx=carried.copy(), margin=None, score=None))
    return res


# ---------------------------------------------------------------------------
# Offline profiling: the similarity matrix from logged index sets (summary 2.2)
# ---------------------------------------------------------------------------
def overlap_matrix(idx_log):
    """Similarity of the top-k index sets between layers, measured offline.

    Summary 2.2 builds a lower-triangular matrix M from the overlap ratio of
    the top-k indices of layer pairs on profiling data.  ``idx_log`` is
    ``[P][L][S][k]`` int (P profiling steps, L layers, S = sequences x KV
    heads, each row the layer's selected block ids, -1 padded).  Read here:
    one slice is (step, sequence, KV head); its ratio for source layer i and
    target layer j >= i is |I_i n I_j| / |I_j|, and M[j][i] is the mean of
    that ratio over the slices whose target set is not empty, summed in
    float64 in slice order (p, then s); 0 when every target set is empty,
    and 0 above the diagonal.  Returns a float32 [L][L] array.
    """
    idx = np.asarray(idx_log)
    P, L, S, _ = idx.shape
    sets = [[[set(int(x) for x in idx[p, l, s] if x >= 0) for s in range(S)]
             for l in range(L)] for p in range(P)]
    M = np.zeros((L, L), dtype=np.float32)
    for j in range(L):
        for i in range(j + 1):
            total, used = 0.0, 0
            for p in range(P):
                for s in range(S):
                    tgt = sets[p][j][s]
                    if not tgt:
                        continue
                    total += len(sets[p][i][s] & tgt) / len(tgt)
                    used += 1
            M[j, i] = np.float32(total / used) if used else np.float32(0.0)
    return M


# ---------------------------------------------------------------------------
# Offline policy optimisation (summary 2.2)
# ---------------------------------------------------------------------------
SIM_TIE = 1e-12


def _better(a, b):
    """Lexicographic objective: fewer resets first, then larger similarity."""
    if a[0] != b[0]:
        return a[0] < b[0]
    return a[1] > b[1]


def policy_dp(M, theta, force=None):
    """Dynamic program over states (i, j) = "layer j uses the indices of reset
    layer i" on the lower-triangular similarity matrix M, stored row = target,
    column = source (M[j][i] is the overlap of source i with target j).

    Summary 2.2: a reset jump goes to the diagonal state (j, j) and costs one
    full-attention layer; a vertical move (i, j) -> (i, j+1) reuses layer i's
    indices at layer j+1 and is allowed only when the similarity exceeds theta
    (strictly).  The objective minimises the number of resets, then maximises
    the summed similarity of the reuse moves.  Layer 0 always resets and
    layers with force[j] set always reset.  Among optimal policies (equal
    resets, similarity within 1e-12 of the best) the one that reuses at the
    earliest layer where they differ is returned.

    Returns (src list, num_resets, sim_sum).
    """
    M = np.asarray(M, dtype=np.float64)
    L = M.shape[0]
    if L < 1 or M.shape != (L, L):
        raise ValueError("M must be square with L >= 1")
    force = [False] * L if force is None else [bool(f) for f in force]
    theta = float(theta)

    def can_reuse(i, j):
        return (not force[j]) and M[j][i] > theta

    # best[(i, j)] = best (resets, sim) achievable by layers j+1 .. L-1
    best = {}
    for j in range(L - 1, -1, -1):
        for i in range(j + 1):
            if j == L - 1:
                best[(i, j)] = (0, 0.0)
                continue
            r = best[(j + 1, j + 1)]
            choice = (r[0] + 1, r[1])
            if can_reuse(i, j + 1):
                u = best[(i, j + 1)]
                cand = (u[0], u[1] + M[j + 1][i])
                if _better(cand, choice):
                    choice = cand
            best[(i, j)] = choice
    r_opt = 1 + best[(0, 0)][0]
    s_opt = best[(0, 0)][1]

    src = [0]
    i, acc_r, acc_s = 0, 1, 0.0
    for j in range(L - 1):
        take_reuse = False
        if can_reuse(i, j + 1):
            u = best[(i, j + 1)]
            if acc_r + u[0] == r_opt and acc_s + M[j + 1][i] + u[1] >= s_opt - SIM_TIE:
                take_reuse = True
        if take_reuse:
            acc_s += M[j + 1][i]
            src.append(i)
        else:
            acc_r += 1
            i = j + 1
            src.append(i)
    return src, acc_r, acc_s


def policy_cost(M, theta, src, force=None):
    """(resets, summed reuse similarity) of a policy, or None if it breaks the
    threshold or a forced reset."""
    M = np.asarray(M, dtype=np.float64)
    L = len(src)
    force = [False] * L if force is None else [bool(f) for f in force]
    if not check_policy(src):
        return None
    resets, sim = 0, 0.0
    for j, s in enumerate(src):
        if s == j:
            resets += 1
        else:
            if force[j] or not M[j][s] > theta:
                return None
            sim += M[j][s]
    return resets, sim


def brute_force_policy(M, theta, force=None):
    """Enumerate every reset/reuse choice of layers 1..L-1 (layer 0 resets,
    forced layers reset), keep the feasible ones, and pick by the same
    objective and tie rule as ``policy_dp``.  Exponential: L <= 16."""
    M = np.asarray(M, dtype=np.float64)
    L = M.shape[0]
    if L > 16:
        raise ValueError("brute force is for L <= 16")
    force = [False] * L if force is None else [bool(f) for f in force]
    free = [j for j in range(1, L) if not force[j]]
    feasible = []
    # reuse (True) enumerated before reset (False) at each free layer, so the
    # enumeration order is the tie-rule order (reuse earliest first).
    for choice in itertools.product([True, False], repeat=len(free)):
        reuse = [False] * L
        for j, c in zip(free, choice):
            reuse[j] = c
        src = []
        for j in range(L):
            src.append(src[-1] if (j > 0 and reuse[j]) else j)
        cost = policy_cost(M, theta, src, force)
        if cost is not None:
            feasible.append((src, cost))
    r_opt = min(c[0] for _, c in feasible)
    s_opt = max(c[1] for _, c in feasible if c[0] == r_opt)
    for src, c in feasible:
        if c[0] == r_opt and c[1] >= s_opt - SIM_TIE:
            return src, c[0], c[1]
    raise AssertionError("unreachable")
