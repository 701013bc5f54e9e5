"""ctypes binding of libhylra.so (include/hylra.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI.  Tensors are torch tensors on the GPU (PyTorch
provides device memory and streams); the binding checks dtypes, shapes and
contiguity, fills the C descriptors and passes raw pointers plus the current
HIP stream.  Importing this module loads the library and raises if it has not
been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("HYLRA_LIBRARY") or os.path.join(_HERE, "libhylra.so")

OK, E_INVALID_ARG, E_UNSUPPORTED, E_BAD_POLICY, E_WORKSPACE, E_DEVICE = range(6)
F32, BF16 = 0, 1
BLOCK = 128
SUBTILE = 32  # tokens per V sub-tile


class HylraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("hylra status %d (%s): %s" % (status, _status_str(status), message))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("scale", ctypes.c_float)]


class KV(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("ctx_lens", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libhylra.so is not built (%s); run __graft_entry__.build() or "
                          "python sparse_layer_reuse_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SP, KP = ctypes.POINTER(Shape), ctypes.POINTER(KV)
    sig = {
        "hylra_workspace_size": [SP, I32, ctypes.POINTER(SZ)],
        "hylra_decode_full": [SP, P, KP, P, P, P, P, SZ, P],
        "hylra_block_topk": [SP, P, P, I32, P, P],
        "hylra_decode_sparse": [SP, P, KP, P, I32, P, P, P, SZ, P],
        "hylra_run_policy": [SP, I32, P, I32, P, KP, P, P, P, P, SZ, P],
        "hylra_policy_dp": [I32, P, ctypes.c_float, P, P, P, P],
        "hylra_timer_start": [I32, I32],
        "hylra_timer_stop": [I32, P, P],
        "hylra_read_probe": [P, SZ, P, P],
        "hylra_overlap_matrix": [I32, I32, I32, I32, P, P, P],
        "hylra_gather_blocks": [SP, KP, P, I32, P, P, P],
        "hylra_append_kv": [SP, KP, P, P, P, P],
        "hylra_rope_append": [SP, KP, P, P, P, P, P, P],
        "hylra_silu_mul": [P, P, ctypes.c_int64, I32, P],
        "hylra_decode_staged": [SP, P, P, P, P, P, I32, P, P, P, SZ, P],
        "hylra_run_policy_offload": [SP, I32, P, I32, P, KP, P, P, P, P, P, P, P, SZ, P, P],
        "hylra_run_policy_noalloc": [SP, I32, P, I32, P, KP, P, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int32
    lib.hylra_status_str.argtypes = [ctypes.c_int32]
    lib.hylra_status_str.restype = ctypes.c_char_p
    lib.hylra_last_error.argtypes = []
    lib.hylra_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()

EXPORTED = ("hylra_workspace_size", "hylra_decode_full", "hylra_block_topk",
            "hylra_decode_sparse", "hylra_run_policy", "hylra_policy_dp", "hylra_timer_start",
            "hylra_timer_stop", "hylra_overlap_matrix", "hylra_read_probe", "hylra_gather_blocks",
            "hylra_decode_staged", "hylra_run_policy_offload", "hylra_append_kv",
            "hylra_rope_append", "hylra_silu_mul", "hylra_run_policy_noalloc",
            "hylra_status_str",
            "hylra_last_error")

KERNEL_FULL_ATTN, KERNEL_SPARSE_ATTN, KERNEL_TOPK, KERNEL_GATHER, KERNEL_FULL_SCORED = range(5)
KERNEL_NAMES = {KERNEL_FULL_ATTN: "attn_full_layer", KERNEL_SPARSE_ATTN: "attn_sparse_layer",
                KERNEL_TOPK: "score_topk", KERNEL_GATHER: "gather_blocks",
                KERNEL_FULL_SCORED: "attn_full_layer_scored"}


def _status_str(st: int) -> str:
    return _lib.hylra_status_str(int(st)).decode()


def last_error() -> str:
    return _lib.hylra_last_error().decode()


def _check(st: int):
    if st != OK:
        raise HylraError(st, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, cuda=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if cuda and not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s" % (name, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, has shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def make_shape(q: torch.Tensor, k_pool: torch.Tensor, table: torch.Tensor, scale: float = 0.0) -> Shape:
    _need(q, "q", tuple(_DTYPES), 3)
    _need(k_pool, "k_pool", q.dtype, 4)
    _need(table, "block_table", torch.int32, 2)
    B, Hq, d = q.shape
    return Shape(B, Hq, k_pool.shape[1], d, BLOCK, _DTYPES[q.dtype], table.shape[1], float(scale))


def check_pool_shapes(k_shape, v_shape):
    """Raises ValueError unless K is [pages][Hkv][128][d] and V the matching
    [pages][Hkv][4][d][32] (four 32-token sub-tiles per page, each
    dimension-major)."""
    k_shape, v_shape = tuple(k_shape), tuple(v_shape)
    ok = len(k_shape) == 4 and k_shape[2] == BLOCK
    if ok:
        P, Hkv, _, d = k_shape
        ok = v_shape == (P, Hkv, BLOCK // SUBTILE, d, SUBTILE)
    if not ok:
        raise ValueError("K pool must be [pages][Hkv][128][d] and V pool [pages][Hkv][4][d][32] "
                         "(got %s and %s)" % (k_shape, v_shape))


def _need_pool(t, name, dtype, ndim, host_ok):
    """A pool on the GPU, or (host_ok) in pinned host memory the GPU can read."""
    host = host_ok and isinstance(t, torch.Tensor) and not t.is_cuda
    if host and not t.is_pinned():
        raise ValueError("%s in host memory must be pinned (pin_memory=True)" % name)
    _need(t, name, dtype, ndim, cuda=not host)


def make_kv(k_pool, v_pool, table, ctx, *, host_ok=False) -> KV:
    _need_pool(k_pool, "k_pool", tuple(_DTYPES), 4, host_ok)
    _need_pool(v_pool, "v_pool", k_pool.dtype, 5, host_ok)
    _need(table, "block_table", torch.int32, 2)
    _need(ctx, "ctx_lens", torch.int32, 1)
    check_pool_shapes(k_pool.shape, v_pool.shape)
    P = k_pool.shape[0]
    if ctx.shape[0] != table.shape[0]:
        raise ValueError("ctx_lens and block_table disagree on the batch size")
    return KV(k_pool.data_ptr(), v_pool.data_ptr(), P, table.data_ptr(), ctx.data_ptr())


def workspace_size(shape: Shape, k: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.hylra_workspace_size(ctypes.byref(shape), int(k), ctypes.byref(n)))
    return int(n.value)


_ws_cache = {}


def workspace(shape: Shape, k: int, device) -> torch.Tensor:
    """A cached, zero-initialised device workspace big enough for `shape` and
    `k` (one per device; calls that share it must run on one stream)."""
    need = workspace_size(shape, k)
    dev = torch.device(device)
    key = (dev.type, dev.index)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def decode_full(q, k_pool, v_pool, table, ctx, *, scale=0.0, want_scores=False, out=None,
                lse=None, block_score=None, ws=None, stream=None):
    """Full decode attention of one layer; returns (out, lse, block_score or None)."""
    shape = make_shape(q, k_pool, table, scale)
    kv = make_kv(k_pool, v_pool, table, ctx)
    B, Hq, d = q.shape
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device) if out is None else out
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if lse is None else lse
    if want_scores and block_score is None:
        block_score = torch.empty(B, shape.num_kv_heads, shape.max_blocks_per_seq,
                                  dtype=torch.float32, device=q.device)
    ws = workspace(shape, 0, q.device) if ws is None else ws
    _check(_lib.hylra_decode_full(ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(out),
                                  _ptr(lse), _ptr(block_score), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return out, lse, block_score


def block_topk(block_score, ctx, k, *, idx=None, stream=None):
    """Top-k block ids of a [B][Hkv][max_blocks] float32 score array."""
    _need(block_score, "block_score", torch.float32, 3)
    _need(ctx, "ctx_lens", torch.int32, 1)
    B, Hkv, mb = block_score.shape
    shape = Shape(B, Hkv, Hkv, 128, BLOCK, BF16, mb, 0.0)
    idx = torch.empty(B, Hkv, int(k), dtype=torch.int32, device=block_score.device) \
        if idx is None else idx
    _check(_lib.hylra_block_topk(ctypes.byref(shape), _ptr(block_score), _ptr(ctx), int(k),
                                 _ptr(idx), _stream(stream)))
    return idx


def decode_sparse(q, k_pool, v_pool, table, ctx, idx, *, scale=0.0, out=None, lse=None,
                  ws=None, stream=None):
    """Decode attention restricted to the blocks in idx [B][Hkv][k]; returns (out, lse)."""
    shape = make_shape(q, k_pool, table, scale)
    kv = make_kv(k_pool, v_pool, table, ctx)
    _need(idx, "idx", torch.int32, 3)
    k = idx.shape[2]
    B, Hq, d = q.shape
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device) if out is None else out
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if lse is None else lse
    ws = workspace(shape, k, q.device) if ws is None else ws
    _check(_lib.hylra_decode_sparse(ctypes.byref(shape), _ptr(q), ctypes.byref(kv), _ptr(idx),
                                    int(k), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return out, lse


def staging_pools(k_pool, batch: int, k: int, device="cuda"):
    """Device staging pools for the selected blocks of one layer:
    K [B*k][Hkv][128][d] and V [B*k][Hkv][4][d][32]."""
    _, Hkv, _, d = k_pool.shape
    sk = torch.empty(batch * k, Hkv, BLOCK, d, dtype=k_pool.dtype, device=device)
    sv = torch.empty(batch * k, Hkv, BLOCK // SUBTILE, d, SUBTILE, dtype=k_pool.dtype, device=device)
    return sk, sv


def _check_staging(staged_k, staged_v, k_dtype, batch, k, Hkv, d):
    _need(staged_k, "staged_k", k_dtype, 4)
    _need(staged_v, "staged_v", k_dtype, 5)
    check_pool_shapes(staged_k.shape, staged_v.shape)
    if tuple(staged_k.shape) != (batch * k, Hkv, BLOCK, d):
        raise ValueError("staging pools must hold B*k = %d pages of %d KV heads, d = %d (got %s)"
                         % (batch * k, Hkv, d, tuple(staged_k.shape)))


def gather_blocks(k_pool, v_pool, table, ctx, idx, staged_k, staged_v, *, stream=None):
    """Copies the selected blocks idx [B][Hkv][k] of a layer (pools on the GPU
    or pinned in host memory) into staging pools (see staging_pools)."""
    kv = make_kv(k_pool, v_pool, table, ctx, host_ok=True)
    _need(idx, "idx", torch.int32, 3)
    B, Hkv, k = idx.shape
    _check_staging(staged_k, staged_v, k_pool.dtype, B, k, Hkv, k_pool.shape[3])
    if table.shape[0] != B or k_pool.shape[1] != Hkv:
        raise ValueError("idx, block_table and the pools disagree on the batch or KV heads")
    shape = Shape(B, Hkv, Hkv, k_pool.shape[3], BLOCK, _DTYPES[k_pool.dtype], table.shape[1], 0.0)
    _check(_lib.hylra_gather_blocks(ctypes.byref(shape), ctypes.byref(kv), _ptr(idx), int(k),
                                    _ptr(staged_k), _ptr(staged_v), _stream(stream)))


def append_kv(k_pool, v_pool, table, ctx, k_new, v_new, pos, *, stream=None):
    """Writes one decode step's k_new / v_new [B][Hkv][d] at positions pos [B]
    into a layer's pools (on the GPU or pinned in host memory)."""
    kv = make_kv(k_pool, v_pool, table, ctx, host_ok=True)
    _need(k_new, "k_new", k_pool.dtype, 3)
    _need(v_new, "v_new", k_pool.dtype, 3)
    _need(pos, "pos", torch.int32, 1)
    B, Hkv, d = k_new.shape
    if tuple(v_new.shape) != (B, Hkv, d) or pos.shape[0] != B or table.shape[0] != B \
            or k_pool.shape[1] != Hkv or k_pool.shape[3] != d:
        raise ValueError("k_new, v_new, pos, block_table and the pools disagree on B, Hkv or d")
    shape = Shape(B, Hkv, Hkv, d, BLOCK, _DTYPES[k_pool.dtype], table.shape[1], 0.0)
    _check(_lib.hylra_append_kv(ctypes.byref(shape), ctypes.byref(kv), _ptr(k_new), _ptr(v_new),
                                _ptr(pos), _stream(stream)))


def rope_append(qkv, cos_tab, sin_tab, pos, k_pool, v_pool, table, ctx, q_out, *,
                num_q_heads, stream=None):
    """Rotary embedding of the new q / k heads in qkv [B][(Hq + 2 Hkv) d]
    (cos_tab / sin_tab float32 [B][d/2]); rotated q into q_out [B][Hq][d],
    rotated k and v appended at pos [B] into the layer's pages."""
    kv = make_kv(k_pool, v_pool, table, ctx, host_ok=True)
    _need(qkv, "qkv", torch.bfloat16, 2)
    _need(q_out, "q_out", torch.bfloat16, 3)
    _need(cos_tab, "cos_tab", torch.float32)
    _need(sin_tab, "sin_tab", torch.float32)
    _need(pos, "pos", torch.int32, 1)
    B = qkv.shape[0]
    _, Hkv, _, d = k_pool.shape
    Hq = int(num_q_heads)
    if k_pool.dtype != torch.bfloat16 or qkv.shape[1] != (Hq + 2 * Hkv) * d \
            or tuple(q_out.shape) != (B, Hq, d) or pos.shape[0] != B or table.shape[0] != B \
            or cos_tab.numel() != B * (d // 2) or sin_tab.numel() != B * (d // 2):
        raise ValueError("rope_append: qkv, q_out, tables, pos and the pools disagree")
    shape = Shape(B, Hq, Hkv, d, BLOCK, BF16, table.shape[1], 0.0)
    _check(_lib.hylra_rope_append(ctypes.byref(shape), ctypes.byref(kv), _ptr(qkv), _ptr(cos_tab),
                                  _ptr(sin_tab), _ptr(pos), _ptr(q_out), _stream(stream)))


def silu_mul(gate_up, out=None, *, stream=None):
    """silu(gate) * up of gate_up [rows][2 width] (bf16) -> [rows][width]."""
    _need(gate_up, "gate_up", torch.bfloat16, 2)
    rows, w2 = gate_up.shape
    out = torch.empty(rows, w2 // 2, dtype=torch.bfloat16, device=gate_up.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    if w2 % 2 or tuple(out.shape) != (rows, w2 // 2):
        raise ValueError("silu_mul: gate_up must be [rows][2 width] and out [rows][width]")
    _check(_lib.hylra_silu_mul(_ptr(gate_up), _ptr(out), int(rows), int(w2 // 2), _stream(stream)))
    return out


def decode_staged(q, staged_k, staged_v, ctx, idx, max_blocks: int, *, scale=0.0, out=None,
                  lse=None, ws=None, stream=None):
    """Attention over staged blocks: the result of decode_sparse on the
    layer's own pools with the same idx.  max_blocks is the layer's block-table
    row length.  Returns (out, lse)."""
    _need(q, "q", tuple(_DTYPES), 3)
    _need(idx, "idx", torch.int32, 3)
    _need(ctx, "ctx_lens", torch.int32, 1)
    B, Hq, d = q.shape
    k = idx.shape[2]
    Hkv = staged_k.shape[1]
    _check_staging(staged_k, staged_v, q.dtype, B, k, Hkv, d)
    shape = Shape(B, Hq, Hkv, d, BLOCK, _DTYPES[q.dtype], int(max_blocks), float(scale))
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device) if out is None else out
    lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device) if lse is None else lse
    ws = workspace(shape, k, q.device) if ws is None else ws
    _check(_lib.hylra_decode_staged(ctypes.byref(shape), _ptr(q), _ptr(staged_k), _ptr(staged_v),
                                    _ptr(ctx), _ptr(idx), int(k), _ptr(out), _ptr(lse), _ptr(ws),
                                    ws.numel(), _stream(stream)))
    return out, lse


class PolicyPlan:
    """Pre-marshalled arguments of hylra_run_policy for a fixed set of layer
    tensors, so that repeated decode steps pay no Python marshalling."""

    def __init__(self, layers: Sequence[dict], src: Sequence[int], k: int, *, scale=0.0,
                 outs=None, lses=None, idx_log=None, ws=None, host_ok=None):
        first = layers[0]
        self.shape = make_shape(first["q"], first["k_pool"], first["table"], scale)
        L = len(layers)
        self.L = L
        self.k = int(k)
        B, Hq, d = first["q"].shape
        dev = first["q"].device
        self.src = (ctypes.c_int32 * L)(*[int(s) for s in src])
        host_ok = host_ok if host_ok is not None else [False] * L
        self.kvs = (KV * L)(*[make_kv(l["k_pool"], l["v_pool"], l["table"], l["ctx"],
                                      host_ok=bool(h)) for l, h in zip(layers, host_ok)])
        for l in layers:
            _need(l["q"], "q", first["q"].dtype, 3)
        self.qs = (ctypes.c_void_p * L)(*[l["q"].data_ptr() for l in layers])
        self.out = outs if outs is not None else [
            torch.empty(B, Hq, d, dtype=torch.float32, device=dev) for _ in range(L)]
        self.lse = lses if lses is not None else [
            torch.empty(B, Hq, dtype=torch.float32, device=dev) for _ in range(L)]
        self.outs = (ctypes.c_void_p * L)(*[o.data_ptr() for o in self.out])
        self.lses = (ctypes.c_void_p * L)(*[o.data_ptr() for o in self.lse])
        self.idx_log = idx_log
        self.ws = workspace(self.shape, self.k, dev) if ws is None else ws
        self._layers = layers  # keep tensors alive

    def run(self, stream=None):
        _check(_lib.hylra_run_policy(ctypes.byref(self.shape), self.L, self.src, self.k,
                                     self.qs, self.kvs, self.outs, self.lses,
                                     _ptr(self.idx_log), _ptr(self.ws), self.ws.numel(),
                                     _stream(stream)))
        return self.out, self.lse


NOALLOC_SCRATCH_BYTES = 32 << 20  # HYLRA_NOALLOC_SCRATCH_BYTES


def run_policy_noalloc(plan: PolicyPlan, stream=None):
    """hylra_run_policy_noalloc on a plan's pre-marshalled arguments: the same
    step as plan.run(), with the library's static device scratch in place of
    the plan's workspace.  Returns (outs, lses)."""
    _check(_lib.hylra_run_policy_noalloc(ctypes.byref(plan.shape), plan.L, plan.src, plan.k,
                                         plan.qs, plan.kvs, plan.outs, plan.lses,
                                         _ptr(plan.idx_log), _stream(stream)))
    return plan.out, plan.lse


class OffloadPlan(PolicyPlan):
    """Pre-marshalled arguments of hylra_run_policy_offload: layers whose
    entry in `offloaded` is true are reuse layers whose pools may be pinned
    host tensors; each gets device staging pools."""

    def __init__(self, layers: Sequence[dict], src: Sequence[int], k: int, offloaded, *,
                 scale=0.0, outs=None, lses=None, idx_log=None, ws=None, staging=None):
        L = len(layers)
        if len(offloaded) != L:
            raise ValueError("offloaded needs one entry per layer")
        super().__init__(layers, src, k, scale=scale, outs=outs, lses=lses, idx_log=idx_log,
                         ws=ws, host_ok=[bool(o) for o in offloaded])
        B = layers[0]["q"].shape[0]
        self.offloaded = (ctypes.c_uint8 * L)(*[1 if o else 0 for o in offloaded])
        self.staging = staging if staging is not None else [
            staging_pools(l["k_pool"], B, self.k) if off else (None, None)
            for l, off in zip(layers, offloaded)]
        for (sk, sv), l, off in zip(self.staging, layers, offloaded):
            if off:
                _check_staging(sk, sv, l["k_pool"].dtype, B, self.k, l["k_pool"].shape[1],
                               l["k_pool"].shape[3])
        self.sks = (ctypes.c_void_p * L)(*[sk.data_ptr() if sk is not None else 0
                                           for sk, _ in self.staging])
        self.svs = (ctypes.c_void_p * L)(*[sv.data_ptr() if sv is not None else 0
                                           for _, sv in self.staging])

    def run(self, stream=None, copy_stream=None):
        if copy_stream is None:
            raise ValueError("run needs a copy stream distinct from the compute stream")
        _check(_lib.hylra_run_policy_offload(
            ctypes.byref(self.shape), self.L, self.src, self.k, self.qs, self.kvs,
            self.offloaded, self.sks, self.svs, self.outs, self.lses, _ptr(self.idx_log),
            _ptr(self.ws), self.ws.numel(), _stream(stream), _stream(copy_stream)))
        return self.out, self.lse


def run_policy(layers, src, k, *, scale=0.0, idx_log=None, outs=None, lses=None, ws=None,
               stream=None):
    """One hybrid decode step over the layers (list of dicts with q, k_pool,
    v_pool, table, ctx).  Returns (outs, lses, idx_log)."""
    if idx_log is None:
        first = layers[0]
        B = first["q"].shape[0]
        idx_log = torch.full((len(layers), B, first["k_pool"].shape[1], int(k)), -2,
                             dtype=torch.int32, device=first["q"].device)
    plan = PolicyPlan(layers, src, k, scale=scale, outs=outs, lses=lses, idx_log=idx_log, ws=ws)
    outs, lses = plan.run(stream)
    return outs, lses, idx_log


def policy_dp(M, theta: float, force=None):
    """Offline policy DP on the host (row = target, column = source).
    Returns (src list, num_resets, sim_sum)."""
    M = np.ascontiguousarray(np.asarray(M, dtype=np.float32))
    L = M.shape[0]
    if M.shape != (L, L):
        raise ValueError("M must be square")
    f = None
    if force is not None:
        f = np.ascontiguousarray(np.asarray(force, dtype=np.uint8))
        if f.shape != (L,):
            raise ValueError("force must have one entry per layer")
    src = np.zeros(L, np.int32)
    nres = ctypes.c_int32(0)
    sim = ctypes.c_double(0.0)
    _check(_lib.hylra_policy_dp(L, M.ctypes.data_as(ctypes.c_void_p), ctypes.c_float(theta),
                                None if f is None else f.ctypes.data_as(ctypes.c_void_p),
                                src.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nres),
                                ctypes.byref(sim)))
    return src.tolist(), int(nres.value), float(sim.value)


def overlap_matrix(idx_log: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Offline similarity matrix M [L][L] (row = target layer) of logged index
    sets idx_log [P][L][S][k] int32 (P profiling steps, S slices)."""
    _need(idx_log, "idx_log", torch.int32, 4)
    t = idx_log.contiguous()
    P, L, S, k = t.shape
    if out is None:
        out = torch.empty(L, L, dtype=torch.float32, device=t.device)
    _check(_lib.hylra_overlap_matrix(P, L, S, k, t.data_ptr(), out.data_ptr(), _stream(stream)))
    return out


def profiling_log(policy_logs) -> torch.Tensor:
    """Stacks the idx_log tensors [L][B][Hkv][k] of several profiling steps
    of hylra_run_policy into the [P][L][B*Hkv][k] layout of overlap_matrix."""
    logs = [l.reshape(l.shape[0], -1, l.shape[-1]) for l in policy_logs]
    return torch.stack(logs).contiguous()


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream every byte of `buf` (a 16-byte aligned GPU tensor) once with the
    attention kernels' K/V load pattern (practical read-ceiling probe); `sink`
    is a one-word int32 GPU tensor."""
    _need(buf, "buf")
    _need(sink, "sink", torch.int32)
    _check(_lib.hylra_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(),
                                 sink.data_ptr(), _stream(stream)))


def profile_policy(step_layers, k, theta, force=None):
    """The offline loop of the technical summary 2.2 on profiling data: every
    layer resets and logs its top-k (one hylra_run_policy per profiling step
    in `step_layers`, a list of per-step layer lists), hylra_overlap_matrix
    turns the logs into M, and hylra_policy_dp solves the policy.
    Returns (src, num_resets, sim_sum, M as a host array)."""
    logs = []
    for layers in step_layers:
        L = len(layers)
        _, _, log = run_policy(layers, list(range(L)), k)
        logs.append(log)
    M = overlap_matrix(profiling_log(logs)).cpu().numpy()
    src, nres, sim = policy_dp(M, theta, force)
    return src, nres, sim, M


def timer_start(kind: int, capacity: int = 4096) -> None:
    """Start bracketing every launch of a kernel kind with HIP events."""
    _check(_lib.hylra_timer_start(int(kind), int(capacity)))


def timer_stop(kind: int):
    """Stop a kernel timer; returns (summed kernel milliseconds, launches)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    _check(_lib.hylra_timer_stop(int(kind), ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


class FullPlan:
    """Pre-marshalled hylra_decode_full calls over a list of layers (no block
    scores): the plain full-attention step used as the baseline policy."""

    def __init__(self, layers, *, scale=0.0, ws=None):
        first = layers[0]
        self.shape = make_shape(first["q"], first["k_pool"], first["table"], scale)
        B, Hq, d = first["q"].shape
        dev = first["q"].device
        self.kvs = [make_kv(l["k_pool"], l["v_pool"], l["table"], l["ctx"]) for l in layers]
        self.qs = [ctypes.c_void_p(l["q"].data_ptr()) for l in layers]
        self.out = [torch.empty(B, Hq, d, dtype=torch.float32, device=dev) for _ in layers]
        self.lse = [torch.empty(B, Hq, dtype=torch.float32, device=dev) for _ in layers]
        self.ws = workspace(self.shape, 0, dev) if ws is None else ws
        self._args = [(ctypes.byref(self.shape), q, ctypes.byref(kv), _ptr(o), _ptr(l), None,
                       _ptr(self.ws), self.ws.numel()) for q, kv, o, l in
                      zip(self.qs, self.kvs, self.out, self.lse)]
        self._layers = layers

    def run(self, stream=None):
        st = _stream(stream)
        for a in self._args:
            _check(_lib.hylra_decode_full(*a, st))
        return self.out, self.lse
