"""Index-guided offloading on the GPU: the selected-block gather from pinned
host (and device) pools, attention over the staged blocks, and the policy run
with offloaded reuse layers, against the oracle and the layout of the pools."""
import numpy as np
import pytest
import torch

import oracle
from sparse_layer_reuse_amd import synth
from test_gpu_parity import (TOL, assert_close, check_policy_run, counters_are_zero, gpu_layer,
                             nan_out, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_layer_reuse_amd import hylra
    return hylra


def selection(ctx, Hkv, k, rng):
    """Ascending selected ids, -1 padded, with an id past the context and a
    negative id in some rows (both must be skipped)."""
    sel = np.full((len(ctx), Hkv, k), -1, np.int32)
    for b, T in enumerate(ctx):
        N = (T + 127) // 128
        for g in range(Hkv):
            c = min(N, k - 1)
            ids = list(np.sort(rng.choice(N, size=c, replace=False))) if c > 0 else []
            if (b + g) % 3 == 1:
                ids.append(N + 2)  # past the context
            sel[b, g, :len(ids)] = ids[:k]
    return sel


def host_copy(lay):
    """The layer with its K / V pools moved to pinned host memory."""
    return dict(lay, k_pool=lay["k_pool"].cpu().pin_memory(),
                v_pool=lay["v_pool"].cpu().pin_memory())


GATHER_CASES = [
    # dtype, ctx lens, Hq, Hkv, d, k, pools in host memory
    ("bf16", (1000, 777, 0, 129), 8, 2, 128, 3, True),
    ("bf16", (4096,), 32, 8, 128, 16, True),
    ("bf16", (2000, 300), 16, 4, 128, 6, False),
    ("bf16", (1500, 64), 8, 2, 64, 4, True),
    ("f32", (1024, 300), 4, 2, 64, 4, True),
    ("f32", (900,), 8, 2, 128, 5, True),
]


@pytest.mark.parametrize("case", GATHER_CASES, ids=lambda c: "%s-%s-%dx%d-d%d-k%d-%s" % (
    c[0], "_".join(map(str, c[1])), c[2], c[3], c[4], c[5], "host" if c[6] else "dev"))
def test_gather_and_staged_attention(H, case):
    dtype, ctx, Hq, Hkv, d, k, host = case
    say("gather + staged attention", case)
    lay = gpu_layer(dtype, ctx, Hq, Hkv, d, seed=41)
    src_lay = host_copy(lay) if host else lay
    sel = selection(ctx, Hkv, k, np.random.default_rng(d + k))
    idx = torch.from_numpy(sel).cuda()
    B = len(ctx)
    sk, sv = H.staging_pools(lay["k_pool"], B, k)
    sk.fill_(7.0)
    sv.fill_(-7.0)
    H.gather_blocks(src_lay["k_pool"], src_lay["v_pool"], lay["table"], lay["ctx"], idx, sk, sv)
    torch.cuda.synchronize()
    # every valid selection slot holds the selected page's tile, bit for bit;
    # skipped slots keep their previous contents
    table = lay["table"].cpu().numpy()
    kp, vp = lay["k_pool"].cpu(), lay["v_pool"].cpu()
    skc, svc = sk.cpu(), sv.cpu()
    for b, T in enumerate(ctx):
        N = (T + 127) // 128
        for g in range(Hkv):
            for r in range(k):
                n = sel[b, g, r]
                slot = b * k + r
                if 0 <= n < N:
                    page = table[b, n]
                    assert torch.equal(skc[slot, g], kp[page, g]), (b, g, r)
                    assert torch.equal(svc[slot, g], vp[page, g]), (b, g, r)
                else:
                    assert bool((skc[slot, g] == 7.0).all()) and bool((svc[slot, g] == -7.0).all())
    # attention over the staged blocks: the oracle's sparse attention
    o0, l0 = nan_out(lay["q"])
    out, lse = H.decode_staged(lay["q"], sk, sv, lay["ctx"], idx, lay["table"].shape[1],
                               out=o0, lse=l0)
    assert counters_are_zero(H, lay["q"], lay["k_pool"], lay["table"], k)
    o = synth.layer_to_oracle(lay)
    r_out, r_lse, _ = oracle.attend(o["q"], o["k_pool"], o["v_pool"], o["table"], o["ctx"],
                                    num_kv_heads=Hkv, sel=sel, k=k)
    assert_close(out.cpu().numpy(), r_out, TOL[dtype], "out")
    assert_close(lse.cpu().numpy(), r_lse, TOL[dtype], "lse")
    # and the very values of the selected-block kernel on the layer's own pools
    s_out, s_lse = H.decode_sparse(lay["q"], lay["k_pool"], lay["v_pool"], lay["table"],
                                   lay["ctx"], idx)
    assert torch.equal(out, s_out) and torch.equal(lse, s_lse)


def offload_layers(H, ctx, L, seed, dtype="bf16", Hq=32, Hkv=8, d=128):
    return [gpu_layer(dtype, ctx, Hq, Hkv, d, seed=seed + 16 * l,
                      hot=[[3, 9] if T > 9 * 128 else [] for T in ctx])
            for l in range(L)]


POLICY_CASES = [
    # src, offloaded, k, ctx, (dtype, Hq, Hkv, d)
    ([0, 0, 0, 3, 3, 5], [0, 1, 1, 0, 1, 0], 8, (5000, 1200), ("bf16", 32, 8, 128)),
    ([0, 0, 2, 2, 2, 2], [0, 1, 0, 1, 1, 1], 3, (5000, 1200), ("bf16", 32, 8, 128)),
    # k past the blocks of the shorter sequence
    ([0, 1, 1, 1, 4, 4], [0, 0, 1, 0, 0, 1], 40, (5000, 1200), ("bf16", 32, 8, 128)),
    # a sequence with no tokens
    ([0, 0, 0, 3, 3], [0, 1, 1, 0, 1], 6, (3000, 0, 700), ("bf16", 16, 4, 128)),
    # float32 K/V, d 64
    ([0, 0, 2, 2], [0, 1, 0, 1], 4, (2000, 900), ("f32", 8, 2, 64)),
]


@pytest.mark.parametrize("case", POLICY_CASES, ids=lambda c: "k%d-%s-%s-%s" % (
    c[2], "".join(map(str, c[1])), "_".join(map(str, c[3])), c[4][0]))
def test_run_policy_offload_matches_oracle(H, case):
    src, offloaded, k, ctx, (dtype, Hq, Hkv, d) = case
    say("run_policy_offload", case)
    layers = offload_layers(H, ctx, len(src), seed=500, dtype=dtype, Hq=Hq, Hkv=Hkv, d=d)
    host_layers = [host_copy(l) if off else l for l, off in zip(layers, offloaded)]
    copy = torch.cuda.Stream()
    L, B = len(src), len(ctx)

    def run(outs, lses):
        idx_log = torch.full((L, B, Hkv, k), -2, dtype=torch.int32, device="cuda")
        plan = H.OffloadPlan(host_layers, src, k, offloaded, outs=outs, lses=lses, idx_log=idx_log)
        return (*plan.run(copy_stream=copy), idx_log)

    checked, outs, lses, idx_log = check_policy_run(H, layers, src, k, dtype, Hkv, run=run)
    assert checked == L
    # the same values as the run with every pool on the device
    ref_out, ref_lse, ref_idx = H.run_policy(layers, src, k)
    torch.cuda.synchronize()
    assert torch.equal(idx_log, ref_idx)
    for a, b in zip(outs, ref_out):
        assert torch.equal(a, b)
    for a, b in zip(lses, ref_lse):
        assert torch.equal(a, b)


def test_run_policy_offload_graph_replays(H):
    """The offloaded step captured in a HIP graph (the copy stream forks from
    and joins back into the capturing stream): every replay, with eager work
    and synchronisations in between, equals the eager step."""
    say("run_policy_offload graph replay")
    src, offloaded, k = [0, 0, 0, 3, 3, 3], [0, 1, 1, 0, 1, 1], 8
    ctx = (4000, 900)
    layers = offload_layers(H, ctx, len(src), seed=700)
    host_layers = [host_copy(l) if off else l for l, off in zip(layers, offloaded)]
    copy = torch.cuda.Stream()
    mk = lambda: H.OffloadPlan(host_layers, src, k, offloaded,
                               idx_log=torch.full((6, 2, 8, k), -2, dtype=torch.int32, device="cuda"))
    eager = mk()
    ref_out, ref_lse = eager.run(copy_stream=copy)
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in ref_out]
    ref_lse = [l.clone() for l in ref_lse]
    ref_idx = eager.idx_log.clone()
    plan = mk()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(copy_stream=copy)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(copy_stream=copy)
    for rep in range(4):
        for o in plan.out:
            o.fill_(float("nan"))
        for sk, sv in plan.staging:
            if sk is not None:
                sk.fill_(0.0)
                sv.fill_(0.0)
        plan.idx_log.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(plan.out, ref_out):
            assert torch.equal(a, b), "replay %d out" % rep
        for a, b in zip(plan.lse, ref_lse):
            assert torch.equal(a, b), "replay %d lse" % rep
        assert torch.equal(plan.idx_log, ref_idx), "replay %d idx" % rep
        eager.run(copy_stream=copy)  # eager work between replays
        torch.cuda.synchronize()


def test_offload_llama3_8b_32k_layers(H):
    """Three layers of the 8B shape at 32K context (one reset, two offloaded
    reuse layers with 128 MiB of pinned host KV each), two sampled sequences
    of the oracle's check -- here the batch is 1."""
    from sparse_layer_reuse_amd import workloads as W
    say("offload at the 8B 32K shape")
    wl = W.get("llama3_8b_32k")
    layers = synth.workload_layers(wl, device="cuda", layers=range(3))
    src, offloaded, k = [0, 0, 0], [0, 1, 1], wl.topk[0]
    host_layers = [host_copy(l) if off else l for l, off in zip(layers, offloaded)]
    copy = torch.cuda.Stream()

    def run(outs, lses):
        idx_log = torch.full((3, 1, 8, k), -2, dtype=torch.int32, device="cuda")
        plan = H.OffloadPlan(host_layers, src, k, offloaded, outs=outs, lses=lses, idx_log=idx_log)
        return (*plan.run(copy_stream=copy), idx_log)

    checked, _, _, _ = check_policy_run(H, layers, src, k, "bf16", 8, run=run)
    assert checked == 3


def test_gather_rejects_pageable_host_pools(H):
    """Pools in ordinary (pageable) host memory are refused on the host, so
    the gather kernel never dereferences an address the device does not map."""
    import ctypes
    say("gather refuses pageable pools")
    lay = gpu_layer("bf16", (300,), 8, 2, 128, seed=3)
    kp = np.zeros(tuple(lay["k_pool"].shape), np.uint16)  # pageable
    vp = np.zeros(tuple(lay["v_pool"].shape), np.uint16)
    kv = H.KV(kp.ctypes.data, vp.ctypes.data, kp.shape[0], lay["table"].data_ptr(),
              lay["ctx"].data_ptr())
    shape = H.Shape(1, 8, 2, 128, 128, H.BF16, lay["table"].shape[1], 0.0)
    idx = torch.zeros(1, 2, 2, dtype=torch.int32, device="cuda")
    sk, sv = H.staging_pools(lay["k_pool"], 1, 2)
    st = H._lib.hylra_gather_blocks(ctypes.byref(shape), ctypes.byref(kv), H._ptr(idx), 2,
                                    H._ptr(sk), H._ptr(sv), None)
    assert st == H.E_INVALID_ARG and "pinned" in H.last_error()
