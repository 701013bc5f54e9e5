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
