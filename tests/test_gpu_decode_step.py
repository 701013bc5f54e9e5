"""Integration of the hybrid attention into a random-weight decoder step
(the end-to-end harness): every layer's attention call against the oracle
on the layer's own q and KV cache (after the step appended its token), the
carried indices, and the surrounding projections, RoPE, KV append and MLP
against a float32 torch recomputation on the host."""
import numpy as np
import pytest
import torch

import oracle
from oracle.acceptance import check_topk_rows
from oracle_util import rope_pairs
from sparse_layer_reuse_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_layer_reuse_amd import decode_step
    return decode_step


def host_layer(D, dec, l, x):
    """The layer's non-attention math in float32 on the host from the same
    bf16 weights: returns (q, k, v) after RoPE, and a function of the
    attention output giving the layer output."""
    s = dec.shape
    cpu = lambda t: t.detach().float().cpu()
    xf = cpu(x)
    h = xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + 1e-5) * cpu(dec.n1[l])
    qkv = h @ cpu(dec.dense("qkv", l))
    B = x.shape[0]
    nq = s.num_q_heads * s.head_dim
    nk = s.num_kv_heads * s.head_dim
    q = qkv[:, :nq].view(B, s.num_q_heads, s.head_dim)
    k = qkv[:, nq:nq + nk].view(B, s.num_kv_heads, s.head_dim)
    v = qkv[:, nq + nk:].view(B, s.num_kv_heads, s.head_dim)
    pos = dec.pos.cpu()
    q = torch.from_numpy(rope_pairs(q.numpy(), pos.numpy(), s.rope_theta)).float()
    k = torch.from_numpy(rope_pairs(k.numpy(), pos.numpy(), s.rope_theta)).float()

    def finish(att):
        y = xf + cpu(att).reshape(B, -1) @ cpu(dec.dense("o", l))
        h2 = y * torch.rsqrt(y.pow(2).mean(-1, keepdim=True) + 1e-5) * cpu(dec.n2[l])
        gu = h2 @ cpu(dec.dense("gu", l))
        g, u = gu[:, : s.ffn], gu[:, s.ffn:]
        return y + (torch.nn.functional.silu(g) * u) @ cpu(dec.dense("down", l))
    return q, k, v, finish


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.abs(a - b).max() / max(1e-6, np.abs(b).max())


@pytest.mark.parametrize("policy", ["hybrid", "full", "hybrid-offload"])
def test_decode_step_layers(D, policy):
    shape = D.DecoderShape(layers=4, hidden=256, num_q_heads=8, num_kv_heads=2, head_dim=64,
                           ffn=512)
    B, ctx, k = 2, 1000, 3
    src = [0, 0, 2, 2]
    dec = D.RandomDecoder(shape, B, ctx, seed=5)
    if policy == "hybrid-offload":
        dec.offload([1, 3])  # the reuse layers' caches in pinned host memory
        policy = "hybrid"
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    x = torch.randn(B, shape.hidden, generator=g, device="cuda").to(torch.bfloat16)
    trace = []
    dec.step(x, policy=policy, src=src, k=k, trace=trace)
    torch.cuda.synchronize()
    carried = None
    for l, t in enumerate(trace):
        q, kk, vv, finish = host_layer(D, dec, l, t["x"])
        # projections and RoPE (bf16 GEMMs on the GPU vs float32 here)
        assert rel_err(t["q"].float().cpu(), q) < 2e-2, l
        assert rel_err(t["k"].float().cpu(), kk) < 2e-2, l
        assert rel_err(t["v"].float().cpu(), vv) < 2e-2, l
        # (t["k"], t["v"] are read back from position ctx - 1 of the cache, so
        # the checks above also cover the append)
        lay = dec.kv[l]
        # attention against the oracle on the layer's q and cache
        o = synth.layer_to_oracle(dict(lay, q=t["q"]))
        if policy == "full" or src[l] == l:
            r_out, r_lse, r_score = oracle.decode_full(o["q"], o["k_pool"], o["v_pool"], o["table"],
                                                       o["ctx"], num_kv_heads=shape.num_kv_heads)
            if policy == "hybrid":
                want, margin = oracle.topk(r_score, o["ctx"], k)
                got = t["idx"].cpu().numpy()
                check_topk_rows(got, want, r_score, margin, o["ctx"], k, what="layer %d" % l)
                carried = got
        else:
            np.testing.assert_array_equal(t["idx"].cpu().numpy(), carried)
            r_out, _, _ = oracle.attend(o["q"], o["k_pool"], o["v_pool"], o["table"], o["ctx"],
                                        num_kv_heads=shape.num_kv_heads, sel=carried, k=k)
        assert np.abs(t["att"].cpu().numpy() - r_out).max() <= 2e-3, l
        # output projection and MLP on the GPU's attention output
        assert rel_err(t["out"].float().cpu(), finish(t["att"])) < 3e-2, l


def test_offloaded_step_equals_device_step(D):
    """The same step with the reuse layers' caches in host memory (gathered
    on a copy stream) gives the very values of the step with every cache on
    the device, eager and as a replayed graph."""
    shape = D.DecoderShape(layers=6, hidden=256, num_q_heads=8, num_kv_heads=2, head_dim=128,
                           ffn=512)
    B, ctx, k = 2, 3000, 4
    src = [0, 0, 0, 3, 3, 3]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    x = torch.randn(B, shape.hidden, generator=g, device="cuda").to(torch.bfloat16)
    ref = D.RandomDecoder(shape, B, ctx, seed=8).step(x, "hybrid", src, k)
    dec = D.RandomDecoder(shape, B, ctx, seed=8)
    dec.offload([1, 2, 4, 5])
    out = dec.step(x, "hybrid", src, k)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dec.step(x, "hybrid", src, k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y = dec.step(x, "hybrid", src, k)
    for rep in range(3):
        y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), rep
        dec.step(x, "hybrid", src, k)  # eager work between replays
        torch.cuda.synchronize()
