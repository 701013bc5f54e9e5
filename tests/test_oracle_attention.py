"""Pins of the oracle's attention, block scores and sparse attention against
library routines, closed forms and hand-derived values (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_layer_reuse_amd import synth
from oracle_util import BLOCK, as_f64, dense_kv, pools_from_dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ragged_layer(dtype="f32", ctx=(300, 1, 129, 640), Hq=8, Hkv=2, d=64, seed=7, paged=True,
                 hot=None, alpha=0.0):
    B = len(ctx)
    lay = synth.make_layer(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, dtype=dtype,
                           ctx_lens=ctx, seed=seed, paged=paged, hot=hot, alpha=alpha)
    return synth.layer_to_oracle(lay)


def sdpa_reference(lay, b, Hkv, scale, mask=None):
    """torch scaled_dot_product_attention in float64 on one sequence."""
    q = torch.from_numpy(as_f64(lay["q"][b]))            # [Hq][d]
    K, V = dense_kv(lay, b, Hkv)                          # [Hkv][T][d]
    Hq = q.shape[0]
    G = Hq // Hkv
    Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)  # [Hq][T][d]
    Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
    attn_mask = None
    if mask is not None:
        attn_mask = torch.from_numpy(mask).repeat_interleave(G, dim=0)[:, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], Kt, Vt, attn_mask=attn_mask, scale=scale)[:, 0, :]
    logits = torch.einsum("hd,htd->ht", q, Kt) * scale
    if mask is not None:
        logits = logits.masked_fill(~torch.from_numpy(mask).repeat_interleave(G, dim=0),
                                    float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return out.numpy(), lse.numpy(), torch.softmax(logits, dim=-1).numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_matches_sdpa(dtype):
    Hkv = 2
    lay = ragged_layer(dtype)
    d = lay["q"].shape[-1]
    scale = 1 / math.sqrt(d)
    out, lse, probs = oracle.attend(lay["q"], lay["k_pool"], lay["v_pool"], lay["table"],
                                    lay["ctx"], num_kv_heads=Hkv, want_probs=True)
    for b in range(len(lay["ctx"])):
        ro, rl, rp = sdpa_reference(lay, b, Hkv, scale)
        np.testing.assert_allclose(out[b], ro, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(lse[b], rl, atol=1e-12, rtol=1e-12)
        T = int(lay["ctx"][b])
        np.testing.assert_allclose(probs[b][:, :T], rp, atol=1e-14)
        assert np.all(probs[b][:, T:] == 0)
        # softmax rows sum to 1
        np.testing.assert_allclose(probs[b].sum(-1), 1.0, atol=1e-12)


def test_sparse_matches_masked_sdpa():
    Hkv = 2
    lay = ragged_layer("bf16", ctx=(700, 1000, 128), seed=11)
    B = 3
    rng = np.random.default_rng(0)
    k = 3
    sel = np.full((B, Hkv, k), -1, np.int32)
    for b in range(B):
        N = (int(lay["ctx"][b]) + BLOCK - 1) // BLOCK
        for g in range(Hkv):
            c = rng.choice(N, size=min(k, N), replace=False)
            sel[b, g, :len(c)] = np.sort(c)
    out, lse, _ = oracle.attend(lay["q"], lay["k_pool"], lay["v_pool"], lay["table"], lay["ctx"],
                                num_kv_heads=Hkv, sel=sel, k=k)
    d = lay["q"].shape[-1]
    for b in range(B):
        T = int(lay["ctx"][b])
        mask = np.zeros((Hkv, T), bool)
        for g in range(Hkv):
            for n in sel[b, g]:
                if n >= 0:
                    mask[g, n * BLOCK:min(T, (n + 1) * BLOCK)] = True
        ro, rl, _ = sdpa_reference(lay, b, Hkv, 1 / math.sqrt(d), mask=mask)
        np.testing.assert_allclose(out[b], ro, atol=1e-12, rtol=1e-10)
        np.testing.assert_allclose(lse[b], rl, atol=1e-12)


def test_sparse_with_all_blocks_equals_full():
    Hkv = 2
    lay = ragged_layer("f32", ctx=(513, 256), seed=3)
    full_out, full_lse, _ = oracle.attend(lay["q"], lay["k_pool"], lay["v_pool"], lay["table"],
                                          lay["ctx"], num_kv_heads=Hkv)
    k = 8
    sel = np.full((2, Hkv, k), -1, np.int32)
    sel[0, :, :5] = np.arange(5)
    sel[1, :, :2] = np.arange(2)
    sp_out, sp_lse, _ = oracle.attend(lay["q"], lay["k_pool"], lay["v_pool"], lay["table"],
                                      lay["ctx"], num_kv_heads=Hkv, sel=sel, k=k)
    np.testing.assert_allclose(sp_out, full_out, atol=1e-12)
    np.testing.assert_allclose(sp_lse, full_lse, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(5)
    Hkv, G, d, T = 2, 3, 16, 300
    q = rng.standard_normal((1, Hkv * G, d)).astype(np.float32)
    # constant V rows -> out equals that row
    K = rng.standard_normal((Hkv, T, d))
    row = rng.standard_normal((Hkv, 1, d))
    V = np.repeat(row, T, axis=1)
    kp, vp, table = pools_from_dense(K, V)
    ctx = np.array([T], np.int32)
    out, _, _ = oracle.attend(q, kp, vp, table, ctx, num_kv_heads=Hkv)
    want = np.repeat(row[:, 0, :].astype(np.float32).astype(np.float64), G, axis=0)
    np.testing.assert_allclose(out[0], want, atol=1e-12)
    # K == 0 -> uniform softmax: out = mean of V, lse = ln T
    V = rng.standard_normal((Hkv, T, d))
    kp, vp, table = pools_from_dense(np.zeros((Hkv, T, d)), V)
    out, lse, _ = oracle.attend(q, kp, vp, table, ctx, num_kv_heads=Hkv)
    want = np.repeat(V.astype(np.float32).astype(np.float64).mean(axis=1), G, axis=0)
    np.testing.assert_allclose(out[0], want, atol=1e-12)
    np.testing.assert_allclose(lse[0], math.log(T), atol=1e-12)
    # T == 1 -> out = V_0, lse = s_0
    kp, vp, table = pools_from_dense(K[:, :1], V[:, :1])
    out, lse, _ = oracle.attend(q, kp, vp, table, np.array([1], np.int32), num_kv_heads=Hkv)
    want = np.repeat(V[:, 0, :].astype(np.float32).astype(np.float64), G, axis=0)
    np.testing.assert_allclose(out[0], want, atol=1e-12)
    s0 = (q[0].astype(np.float64) * np.repeat(K[:, 0, :].astype(np.float32), G, axis=0)).sum(-1)
    np.testing.assert_allclose(lse[0], s0 / math.sqrt(d), atol=1e-12)
    # empty context -> zeros and -inf
    out, lse, _ = oracle.attend(q, kp, vp, table, np.array([0], np.int32), num_kv_heads=Hkv)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_golden_worked_examples():
    spec = json.load(open(os.path.join(GOLDEN, "attention_worked.json")))
    for case in spec["cases"]:
        d = case["d"]
        q = np.array(case["q"], np.float32)[None]          # [1][Hq][d]
        Kd = np.array(case["keys"], np.float64)[None]       # [1][T][d] (one KV head)
        Vd = np.array(case["values"], np.float64)[None]
        kp, vp, table = pools_from_dense(Kd, Vd)
        ctx = np.array([Kd.shape[1]], np.int32)
        out, lse, probs = oracle.attend(q, kp, vp, table, ctx, num_kv_heads=1,
                                        scale=case["scale"], want_probs=True)
        np.testing.assert_allclose(out[0], np.array(case["out"]), atol=case["tol"] * 10,
                                   err_msg=case["name"])
        np.testing.assert_allclose(lse[0], np.array(case["lse"]), atol=case["tol"] * 10,
                                   err_msg=case["name"])
        score = oracle.block_score(probs, ctx, num_kv_heads=1, max_blocks=1)
        np.testing.assert_allclose(score[0, 0, 0], q.shape[1], atol=1e-12)


def test_block_scores_sum_to_group_size_and_match_bruteforce():
    Hkv, Hq = 2, 8
    lay = ragged_layer("bf16", ctx=(300, 1, 129, 640), Hq=Hq, Hkv=Hkv)
    out, lse, score = oracle.decode_full(lay["q"], lay["k_pool"], lay["v_pool"], lay["table"],
                                         lay["ctx"], num_kv_heads=Hkv)
    G = Hq // Hkv
    d = lay["q"].shape[-1]
    for b, T in enumerate(lay["ctx"]):
        N = (int(T) + BLOCK - 1) // BLOCK
        np.testing.assert_allclose(score[b].sum(-1), G, atol=1e-12)
        assert np.all(score[b][:, N:] == 0)
        _, _, p = sdpa_reference(lay, b, Hkv, 1 / math.sqrt(d))   # torch softmax, float64
        for g in range(Hkv):
            for n in range(N):
                want = p[g * G:(g + 1) * G, n * BLOCK:min(int(T), (n + 1) * BLOCK)].sum()
                assert abs(score[b, g, n] - want) < 1e-12


def test_planted_blocks_score_highest():
    from sparse_layer_reuse_amd import workloads as W
    wl = W.TINY_F32
    hot = synth.workload_hot_sets(wl)
    for l, lay in enumerate(synth.workload_layers(wl)):
        o = synth.layer_to_oracle(lay)
        _, _, score = oracle.decode_full(o["q"], o["k_pool"], o["v_pool"], o["table"], o["ctx"],
                                         num_kv_heads=wl.num_kv_heads)
        for g in range(wl.num_kv_heads):
            top = set(np.argsort(-score[0, g])[:2].tolist())
            assert top == set(hot[l][0].tolist()), (l, g, score[0, g])
