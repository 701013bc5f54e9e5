"""A decoder-only model step with random weights around the hybrid attention.

This is the integration harness that puts the attention-only measurements in
context (the pages report their speedup end to end, technical summary
section 4): every layer of a Llama-3-shaped decoder runs RMSNorm, the QKV
projection, rotary position embedding, the append of the new token's K and V
into the paged cache, attention, the output projection and a SwiGLU MLP.  The
projections and the MLP are plain library GEMMs (torch on hipBLASLt; each
weight is stored in the layout whose batch-1..8 GEMV kernel streams fastest,
and the residual adds ride in the GEMM's beta term) with torch's fused
RMSNorm; the rotary embedding of q and k together with the append of k and v
into the pages is one library launch (hylra_rope_append, with the step's
cos/sin computed once), and so is the SwiGLU product (hylra_silu_mul);
attention is this library: a reset
layer runs hylra_run_policy on that one layer (full attention, fused block
scores and top-k into the carried index buffer), a reuse layer runs
hylra_decode_sparse over the carried indices, and the full-attention baseline
runs hylra_decode_full on every layer.

Index-guided offloading (technical summary 2.4): offload() moves chosen reuse
layers' caches to pinned host memory.  In a hybrid step, right after a reset
layer has selected its blocks, the selected blocks of its offloaded reuse
layers are gathered to the device on a copy stream (hylra_gather_blocks), so
the transfers overlap with the projections, MLPs and attention of the layers
in between; each offloaded layer waits for its own gather and attends over
the staged blocks (hylra_decode_staged).

Weights are random (no trained model); the step's shapes are static, so it
can be captured as a HIP graph (the copy stream forks from and joins back
into the capturing stream).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import hylra, synth

@dataclass(frozen=True)
class DecoderShape:
    layers: int
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ffn: int
    rope_theta: float = 500000.0


LLAMA3_8B = DecoderShape(layers=32, hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         ffn=14336)
LLAMA3_70B = DecoderShape(layers=80, hidden=8192, num_q_heads=64, num_kv_heads=8, head_dim=128,
                          ffn=28672)


def shape_for(num_q_heads: int, num_kv_heads: int, head_dim: int):
    """The Llama-3 shape with these attention heads, or None."""
    for s in (LLAMA3_8B, LLAMA3_70B):
        if (s.num_q_heads, s.num_kv_heads, s.head_dim) == (num_q_heads, num_kv_heads, head_dim):
            return s
    return None


EPS = 1e-5


def rope_tables(pos: torch.Tensor, d: int, theta: float):
    """cos / sin tables [B][d/2] (float32, from float64 angles) of the
    rotate-half rotary embedding at positions pos [B]: dimension i < d/2
    pairs with i + d/2, both turned by the angle pos * theta^(-2i/d)."""
    inv = 1.0 / (theta ** (torch.arange(0, d, 2, device=pos.device, dtype=torch.float64) / d))
    ang = pos.double()[:, None] * inv[None, :]
    return torch.cos(ang).float().contiguous(), torch.sin(ang).float().contiguous()


class RandomDecoder:
    """Random-weight decoder with a paged KV cache holding `ctx` tokens per
    sequence (the last one is written by each step)."""

    def __init__(self, shape: DecoderShape, batch: int, ctx: int, *, seed: int = 0,
                 device="cuda", dtype=torch.bfloat16):
        self.shape, self.batch, self.ctx = shape, batch, ctx
        s = shape
        g = torch.Generator(device=device)
        g.manual_seed(seed)

        def w(*dims, fan_in):
            return (torch.randn(*dims, generator=g, device=device) / math.sqrt(fan_in)).to(dtype)

        qkv_out = (s.num_q_heads + 2 * s.num_kv_heads) * s.head_dim
        nq = s.num_q_heads * s.head_dim
        # [out][in] (F.linear / addmm with a transposed view) except the
        # gate/up weight, [in][out]
        self.w_qkv = [w(qkv_out, s.hidden, fan_in=s.hidden) for _ in range(s.layers)]
        self.w_o = [w(s.hidden, nq, fan_in=nq) for _ in range(s.layers)]
        self.w_gu = [w(s.hidden, 2 * s.ffn, fan_in=s.hidden) for _ in range(s.layers)]
        self.w_down = [w(s.hidden, s.ffn, fan_in=s.ffn) for _ in range(s.layers)]
        self.n1 = [torch.ones(s.hidden, device=device, dtype=dtype) for _ in range(s.layers)]
        self.n2 = [torch.ones(s.hidden, device=device, dtype=dtype) for _ in range(s.layers)]
        # the cache of every layer: seeded random history (the layer's q is unused)
        self.kv = [synth.make_layer(batch=batch, num_q_heads=s.num_kv_heads,
                                    num_kv_heads=s.num_kv_heads, head_dim=s.head_dim,
                                    dtype="bf16", ctx_lens=[ctx] * batch, seed=seed + 16 * (l + 1),
                                    device=device)
                   for l in range(s.layers)]
        t = ctx - 1  # position of the token this step appends
        self.pos = torch.full((batch,), t, dtype=torch.int32, device=device)
        self.rope_c, self.rope_s = rope_tables(self.pos, s.head_dim, s.rope_theta)  # [B][d/2]
        self.offloaded = [False] * s.layers
        self.staging = {}
        self.copy_stream = None
        self.gather_done = {}

    def offload(self, layers) -> None:
        """Moves the caches of `layers` (reuse layers of the policy the steps
        will run) to pinned host memory."""
        for l in layers:
            lay = self.kv[l]
            lay["k_pool"] = lay["k_pool"].cpu().pin_memory()
            lay["v_pool"] = lay["v_pool"].cpu().pin_memory()
            self.offloaded[l] = True
        if self.copy_stream is None:
            self.copy_stream = torch.cuda.Stream()
        torch.cuda.empty_cache()

    def dense(self, name: str, l: int) -> torch.Tensor:
        """Layer l's weight `name` (qkv, o, gu, down) as an [in][out] view."""
        w = getattr(self, "w_" + name)[l]
        return w if name == "gu" else w.t()

    def appended(self, l: int):
        """The k and v ([B][Hkv][d]) stored at position ctx - 1 of layer l's
        pages (K pages [page][Hkv][128][d], V pages [page][Hkv][4][d][32])."""
        lay = self.kv[l]
        t = self.ctx - 1
        dev = lay["k_pool"].device
        pages = lay["table"][:, t // 128].long().to(dev)
        k = lay["k_pool"][pages, :, t % 128, :]
        v = lay["v_pool"][pages, :, (t % 128) // 32, :, t % 32]
        return k.cuda(), v.cuda()

    def _staging(self, l: int, k: int):
        key = (l, k)
        if key not in self.staging:
            self.staging[key] = hylra.staging_pools(self.kv[l]["k_pool"], self.batch, k)
        return self.staging[key]

    def _gather_reusers(self, i: int, src, k: int, idx: torch.Tensor) -> None:
        """After reset layer i: gathers the selected blocks of its offloaded
        reuse layers on the copy stream, one event per layer."""
        users = [j for j in range(i + 1, self.shape.layers) if src[j] == i and self.offloaded[j]]
        if not users:
            return
        cs = self.copy_stream
        cs.wait_stream(torch.cuda.current_stream())
        idx.record_stream(cs)  # the allocator keeps idx until the gathers have read it
        with torch.cuda.stream(cs):
            for j in users:
                lay = self.kv[j]
                sk, sv = self._staging(j, k)
                hylra.gather_blocks(lay["k_pool"], lay["v_pool"], lay["table"], lay["ctx"], idx,
                                    sk, sv, stream=cs)
                ev = torch.cuda.Event()
                ev.record(cs)
                self.gather_done[j] = ev

    def attention(self, l: int, q: torch.Tensor, policy: str, src, k: int, carried):
        lay = self.kv[l]
        if policy == "full":
            if self.offloaded[l]:
                raise ValueError("full attention needs every cache on the device")
            out, _, _ = hylra.decode_full(q, lay["k_pool"], lay["v_pool"], lay["table"], lay["ctx"])
            return out, carried
        if src[l] == l:
            if self.offloaded[l]:
                raise ValueError("layer %d resets and needs its cache on the device" % l)
            idx = torch.empty(1, self.batch, self.shape.num_kv_heads, k, dtype=torch.int32,
                              device=q.device)
            layer = dict(lay, q=q)
            outs, _, _ = hylra.run_policy([layer], [0], k, idx_log=idx)
            self._gather_reusers(l, src, k, idx[0])
            return outs[0], idx[0]
        if self.offloaded[l]:
            torch.cuda.current_stream().wait_event(self.gather_done.pop(l))
            sk, sv = self._staging(l, k)
            out, _ = hylra.decode_staged(q, sk, sv, lay["ctx"], carried, lay["table"].shape[1])
            return out, carried
        out, _ = hylra.decode_sparse(q, lay["k_pool"], lay["v_pool"], lay["table"], lay["ctx"],
                                     carried)
        return out, carried

    def layer(self, l: int, x: torch.Tensor, policy: str, src, k: int, carried, trace=None):
        s = self.shape
        B = x.shape[0]
        x_in = x
        F = torch.nn.functional
        lay = self.kv[l]
        h = F.rms_norm(x, (s.hidden,), self.n1[l], EPS)
        qkv = F.linear(h, self.w_qkv[l])
        q = torch.empty(B, s.num_q_heads, s.head_dim, dtype=x.dtype, device=x.device)
        hylra.rope_append(qkv, self.rope_c, self.rope_s, self.pos, lay["k_pool"], lay["v_pool"],
                          lay["table"], lay["ctx"], q, num_q_heads=s.num_q_heads)
        att, carried = self.attention(l, q, policy, src, k, carried)
        # both residuals in place, except where x is the caller's or the trace's
        if l == 0 or trace is not None:
            x = torch.addmm(x, att.view(B, -1).to(x.dtype), self.w_o[l].t())
        else:
            x.addmm_(att.view(B, -1).to(x.dtype), self.w_o[l].t())
        gu = F.rms_norm(x, (s.hidden,), self.n2[l], EPS) @ self.w_gu[l]
        x.addmm_(hylra.silu_mul(gu), self.w_down[l].t())
        if trace is not None:
            torch.cuda.synchronize()
            kk, vv = self.appended(l)
            trace.append({"x": x_in, "q": q, "k": kk, "v": vv, "att": att, "idx": carried,
                          "out": x.clone()})
        return x, carried

    def step(self, x: torch.Tensor, policy: str = "hybrid", src=None, k: int = 16, trace=None):
        """One decode step of every layer for hidden states x [B][hidden]."""
        carried = None
        for l in range(self.shape.layers):
            x, carried = self.layer(l, x, policy, src, k, carried, trace)
        return x
