"""Test-side helpers shared by oracle and parity tests (plumbing only)."""
import numpy as np

BLOCK = 128
SUB = 32  # tokens per V sub-tile: V pages are [Hkv][4][d][32]


def dense_kv(layer_np, b, num_kv_heads):
    """Gather sequence b's K and V into dense [Hkv][T][d] float64 arrays by
    walking its block table (layout plumbing, no attention arithmetic)."""
    k_pool, v_pool, table, ctx = (layer_np["k_pool"], layer_np["v_pool"], layer_np["table"],
                                  layer_np["ctx"])
    T = int(ctx[b])
    d = k_pool.shape[-1]
    K = np.zeros((num_kv_heads, T, d))
    V = np.zeros((num_kv_heads, T, d))
    kf, vf = as_f64(k_pool), as_f64(v_pool)
    for t in range(T):
        page = table[b, t // BLOCK]
        K[:, t, :] = kf[page, :, t % BLOCK, :]
        V[:, t, :] = vf[page, :, (t % BLOCK) // SUB, :, t % SUB]
    return K, V


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def pools_from_dense(K, V, dtype=np.float32):
    """Pack dense [Hkv][T][d] K/V into one sequence's pages (identity table)."""
    Hkv, T, d = K.shape
    nb = max(1, (T + BLOCK - 1) // BLOCK)
    kp = np.zeros((nb, Hkv, BLOCK, d), dtype)
    vp = np.zeros((nb, Hkv, BLOCK // SUB, d, SUB), dtype)
    for t in range(T):
        kp[t // BLOCK, :, t % BLOCK, :] = K[:, t, :]
        vp[t // BLOCK, :, (t % BLOCK) // SUB, :, t % SUB] = V[:, t, :]
    table = np.arange(nb, dtype=np.int32)[None, :]
    return kp, vp, table


def rope_pairs(x, pos, theta):
    """Rotary position embedding written out pair by pair (rotate-half
    pairing, as in Llama-3): dimensions i < d/2 and i + d/2 of every head
    vector of sequence b are rotated by the angle pos[b] * theta^(-2i/d).
    x is [B][H][d]; float64 result."""
    x = np.asarray(x, np.float64)
    B, H, d = x.shape
    out = x.copy()
    for b in range(B):
        for i in range(d // 2):
            a = float(pos[b]) * theta ** (-2.0 * i / d)
            c, s = np.cos(a), np.sin(a)
            x1, x2 = x[b, :, i], x[b, :, i + d // 2]
            out[b, :, i] = x1 * c - x2 * s
            out[b, :, i + d // 2] = x1 * s + x2 * c
    return out
