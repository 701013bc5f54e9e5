"""Seeded random shapes through the whole policy step, against the oracle:
batch, group size (1-16), head_dim 64/128, float32/bf16, ragged and empty
contexts, contiguous or paged tables, k from 1 past the block count, and
random valid reset/reuse policies.  Each case is small enough for the
oracle; together they cover the planner's and the kernels' shape space
beyond the fixed cases."""
import numpy as np
import pytest
import torch

from test_gpu_parity import check_policy_run, gpu_layer, say

pytestmark = pytest.mark.gpu

N_CASES = 40


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_layer_reuse_amd import hylra
    return hylra


def random_case(i):
    rng = np.random.default_rng(7000 + i)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    B = int(rng.integers(1, 5))
    ctx = [int(rng.choice([0, 1, 31, 127, 128, 129])) if rng.random() < 0.25
           else int(rng.integers(1, 3000)) for _ in range(B)]
    if max(ctx) == 0:
        ctx[0] = 500
    L = int(rng.integers(2, 6))
    src = [0]
    for j in range(1, L):
        src.append(j if rng.random() < 0.4 else src[-1])
    k = int(rng.choice([1, 2, 5, 16, 40]))
    paged = bool(rng.random() < 0.5)
    return dict(Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, ctx=tuple(ctx), src=src, k=k,
                paged=paged, seed=100 * i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_policy_step(H, i):
    c = random_case(i)
    say("random shape", i, c)
    layers = [gpu_layer(c["dtype"], c["ctx"], c["Hq"], c["Hkv"], c["d"], seed=c["seed"] + 16 * l,
                        paged=c["paged"], hot=[[1] if T > 256 else [] for T in c["ctx"]])
              for l in range(len(c["src"]))]
    checked, _, _, _ = check_policy_run(H, layers, c["src"], c["k"], c["dtype"], c["Hkv"])
    assert checked == len(c["src"])


@pytest.mark.parametrize("i", range(0, N_CASES, 4))
def test_random_offloaded_step(H, i):
    """The same shapes with every reuse layer's pools in pinned host memory:
    the oracle's values, and the very values of the all-device step."""
    c = random_case(i)
    say("random shape, offloaded", i, c)
    src, k = c["src"], c["k"]
    layers = [gpu_layer(c["dtype"], c["ctx"], c["Hq"], c["Hkv"], c["d"], seed=c["seed"] + 16 * l,
                        paged=c["paged"], hot=[[1] if T > 256 else [] for T in c["ctx"]])
              for l in range(len(src))]
    offloaded = [s != j for j, s in enumerate(src)]
    host_layers = [dict(l, k_pool=l["k_pool"].cpu().pin_memory(),
                        v_pool=l["v_pool"].cpu().pin_memory()) if off else l
                   for l, off in zip(layers, offloaded)]
    copy = torch.cuda.Stream()
    L, B = len(src), len(c["ctx"])

    def run(outs, lses):
        idx_log = torch.full((L, B, c["Hkv"], k), -2, dtype=torch.int32, device="cuda")
        plan = H.OffloadPlan(host_layers, src, k, offloaded, outs=outs, lses=lses, idx_log=idx_log)
        return (*plan.run(copy_stream=copy), idx_log)

    checked, outs, lses, idx_log = check_policy_run(H, layers, src, k, c["dtype"], c["Hkv"],
                                                    run=run)
    assert checked == L
    ref_out, ref_lse, ref_idx = H.run_policy(layers, src, k)
    torch.cuda.synchronize()
    assert torch.equal(idx_log, ref_idx)
    for a, b in zip(outs, ref_out):
        assert torch.equal(a, b)
    for a, b in zip(lses, ref_lse):
        assert torch.equal(a, b)
