"""hylra_run_policy_noalloc (static device scratch, no caller workspace)
against hylra_run_policy (caller workspace) through the C ABI: two calls in a
row, the second on a smaller shape, each bit-identical to the workspace
entry point on the same inputs (the same kernels run in the same order), and
a shape too large for the static scratch refused with HYLRA_E_WORKSPACE."""
import numpy as np
import pytest
import torch

from sparse_layer_reuse_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_layer_reuse_amd import hylra
    return hylra


def _layers(ctx, Hq, Hkv, d, n, seed, hot=None):
    return [synth.make_layer(batch=len(ctx), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                             dtype="bf16", ctx_lens=ctx, seed=seed + 16 * l, paged=True,
                             hot=hot, alpha=1.5, device="cuda")
            for l in range(n)]


def _plan(H, layers, src, k, fill):
    B, Hq, d = layers[0]["q"].shape
    Hkv = layers[0]["k_pool"].shape[1]
    L = len(layers)
    outs = [torch.full((B, Hq, d), fill, device="cuda") for _ in range(L)]
    lses = [torch.full((B, Hq), fill, device="cuda") for _ in range(L)]
    log = torch.full((L, B, Hkv, k), -7, dtype=torch.int32, device="cuda")
    return H.PolicyPlan(layers, src, k, outs=outs, lses=lses, idx_log=log)


CASES = [
    # contexts, Hq, Hkv, d, policy, k  (the second is the smaller input)
    ((5000, 1200), 32, 8, 128, [0, 0, 0, 3, 3, 5], 8),
    ((900,), 16, 4, 64, [0, 1, 1, 1], 4),
]


def test_noalloc_matches_workspace_entry_point_twice(H):
    for i, (ctx, Hq, Hkv, d, src, k) in enumerate(CASES):
        print("[case] noalloc call %d: ctx %s Hq %d Hkv %d d %d src %s k %d"
              % (i, ctx, Hq, Hkv, d, src, k), flush=True)
        layers = _layers(ctx, Hq, Hkv, d, len(src), seed=600 + 100 * i, hot=[[1, 3]] * len(ctx))
        ref = _plan(H, layers, src, k, 0.0)
        ref.run()
        got = _plan(H, layers, src, k, float("nan"))
        H.run_policy_noalloc(got)
        torch.cuda.synchronize()
        for j in range(len(src)):
            assert torch.equal(got.out[j], ref.out[j]), "call %d layer %d out" % (i, j)
            assert torch.equal(got.lse[j], ref.lse[j]), "call %d layer %d lse" % (i, j)
        assert torch.equal(got.idx_log, ref.idx_log), "call %d idx" % i
        assert bool((got.idx_log[0] >= -1).all())


def test_noalloc_refuses_shape_beyond_scratch(H):
    # 4096 sequences x 16 KV heads x 64 splits of d = 128 partials: far more
    # than the static scratch holds
    layers = _layers((128,) * 2, 32, 16, 128, 1, seed=9)
    plan = _plan(H, layers, [0], 4, 0.0)
    plan.shape.batch = 4096
    plan.shape.max_blocks_per_seq = 8192
    need = H.workspace_size(plan.shape, 4)
    assert need > H.NOALLOC_SCRATCH_BYTES
    with pytest.raises(H.HylraError) as e:
        H.run_policy_noalloc(plan)
    assert e.value.status == H.E_WORKSPACE
