"""Host-side checks of the end-to-end decoder harness: its RoPE tables
against the rotary embedding written out pair by pair, and its shape table."""
import numpy as np
import torch

from oracle_util import rope_pairs
from sparse_layer_reuse_amd import decode_step as DS


def apply_tables(x, pos, theta):
    """The rotation the tables feed (the GPU kernel applies the same per pair)."""
    d = x.shape[-1]
    c, s = DS.rope_tables(torch.as_tensor(pos), d, theta)
    c, s = c.double().numpy()[:, None, :], s.double().numpy()[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def test_rope_tables_match_pairwise_rotation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 4, 64))
    pos = np.array([0, 999, 131071])
    got = apply_tables(x, pos, 500000.0)
    np.testing.assert_allclose(got, rope_pairs(x, pos, 500000.0), atol=2e-5)


def test_rope_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 3, 128))
    r = rope_pairs(x, [0, 0], 500000.0)
    np.testing.assert_allclose(r, x, atol=0)
    r = rope_pairs(x, [17, 40000], 500000.0)
    d = 128
    pair_norm = lambda a: a[..., : d // 2] ** 2 + a[..., d // 2:] ** 2
    np.testing.assert_allclose(pair_norm(r), pair_norm(x), rtol=1e-12)
    # the first pair turns by exactly pos radians
    a = 17.0
    np.testing.assert_allclose(r[0, :, 0], x[0, :, 0] * np.cos(a) - x[0, :, d // 2] * np.sin(a),
                               rtol=1e-12)


def test_shape_table():
    assert DS.shape_for(32, 8, 128) == DS.LLAMA3_8B
    assert DS.shape_for(64, 8, 128) == DS.LLAMA3_70B
    assert DS.shape_for(4, 2, 64) is None
