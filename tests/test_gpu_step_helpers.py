"""Decode-step helpers on the GPU: the token append into device and pinned
host pages, the fused rotary embedding + append, and the SwiGLU product,
against their definitions on the host."""
import numpy as np
import pytest
import torch

from oracle_util import rope_pairs
from test_gpu_parity import gpu_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_layer_reuse_amd import hylra
    return hylra


def bf16_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def expected_pages(lay, pos, k_new, v_new):
    """The pools after writing k_new / v_new [B][Hkv][d] at positions pos
    (positions outside the table write nothing), built on the host."""
    kp, vp = lay["k_pool"].cpu().clone(), lay["v_pool"].cpu().clone()
    table = lay["table"].cpu().numpy()
    mb = table.shape[1]
    for b, t in enumerate(pos):
        if not 0 <= t < 128 * mb:
            continue
        page = table[b, t // 128]
        kp[page, :, t % 128, :] = k_new[b].cpu()
        vp[page, :, (t % 128) // 32, :, t % 32] = v_new[b].cpu()
    return kp, vp


@pytest.mark.parametrize("host", [False, True], ids=["device", "pinned-host"])
def test_append_kv(H, host):
    say("append_kv", "host" if host else "device")
    lay = gpu_layer("bf16", (1000, 300, 129, 500), 8, 2, 128, seed=61)
    pos = [999, 0, 128, 128 * lay["table"].shape[1]]  # the last is past the table
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    k_new = torch.randn(4, 2, 128, generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn(4, 2, 128, generator=g, device="cuda").to(torch.bfloat16)
    want_k, want_v = expected_pages(lay, pos, k_new, v_new)
    kp, vp = lay["k_pool"], lay["v_pool"]
    if host:
        kp, vp = kp.cpu().pin_memory(), vp.cpu().pin_memory()
    H.append_kv(kp, vp, lay["table"], lay["ctx"], k_new, v_new,
                torch.tensor(pos, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(kp.cpu(), want_k)
    assert torch.equal(vp.cpu(), want_v)


@pytest.mark.parametrize("host", [False, True], ids=["device", "pinned-host"])
def test_rope_append(H, host):
    from sparse_layer_reuse_amd import decode_step as DS
    say("rope_append", "host" if host else "device")
    Hq, Hkv, d = 8, 2, 128
    lay = gpu_layer("bf16", (1000, 40000), Hq, Hkv, d, seed=71)
    pos = [999, 39999]
    B = 2
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    qkv = torch.randn(B, (Hq + 2 * Hkv) * d, generator=g, device="cuda").to(torch.bfloat16)
    pos_t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    cos_t, sin_t = DS.rope_tables(pos_t, d, 500000.0)
    q_out = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    x = bf16_f64(qkv).reshape(B, Hq + 2 * Hkv, d)
    want_q = rope_pairs(x[:, :Hq], pos, 500000.0)
    want_k = rope_pairs(x[:, Hq:Hq + Hkv], pos, 500000.0)
    kp, vp = lay["k_pool"], lay["v_pool"]
    if host:
        kp, vp = kp.cpu().pin_memory(), vp.cpu().pin_memory()
    H.rope_append(qkv, cos_t, sin_t, pos_t, kp, vp, lay["table"], lay["ctx"], q_out,
                  num_q_heads=Hq)
    torch.cuda.synchronize()
    # one bf16 rounding of a float32 rotation: within 2^-8 of the value
    tol = lambda w: 2.0 ** -8 * np.abs(w) + 1e-6
    got_q = bf16_f64(q_out)
    assert np.all(np.abs(got_q - want_q) <= tol(want_q))
    table = lay["table"].cpu().numpy()
    for b, t in enumerate(pos):
        page = table[b, t // 128]
        got_k = kp[page, :, t % 128, :].float().cpu().numpy()
        assert np.all(np.abs(got_k - want_k[b]) <= tol(want_k[b]))
        got_v = vp[page, :, (t % 128) // 32, :, t % 32].cpu()
        assert torch.equal(got_v, qkv[b, (Hq + Hkv) * d:].view(Hkv, d).cpu())


def test_silu_mul(H):
    say("silu_mul")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    gu = (3 * torch.randn(5, 2 * 1000, generator=g, device="cuda")).to(torch.bfloat16)
    out = H.silu_mul(gu)
    torch.cuda.synchronize()
    x = bf16_f64(gu)
    gate, up = x[:, :1000], x[:, 1000:]
    want = gate / (1.0 + np.exp(-gate)) * up
    got = bf16_f64(out)
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-5)
