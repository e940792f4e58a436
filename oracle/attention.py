"""fp64 split-half RoPE and single-query decode attention (test oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Attention as the pages define it for one head: score s_i = (q . k_i) / sqrt(D)
([nalar] "Error pada key mengubah input softmax"), probabilities p = softmax(s),
output = sum_i p_i v_i ([nalar] "Error pada value masuk setelah attention
probability").  Several query heads share one key/value head under grouped-query
attention ([trefon] "Bajty na token"); the reading here is the consecutive
mapping kv_head = q_head // (Hq / Hkv).

Keys may be stored before RoPE and rotated when used ([troisinh] "Tại sao Key
và Value lại khác nhau?", paragraph "RoPE — Cái bẫy tinh vi", and "Tại sao nó
hoạt động", item 3); the supported models use split-half RoPE ([nexus] "Các mô
hình được hỗ trợ").  Reading: channel pairs (j, j + 64), frequency
theta_j = base ** (-2 j / 128), angle = position * theta_j, token i at
position i, the decode query at position q_pos; everything in float64.
"""

import numpy as np

D = 128


def rope_freqs(base, dim=D):
    j = np.arange(dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / dim)


def rope_f64(x, positions, base):
    """Rotate x [..., n, 128] whose rows sit at ``positions`` [n] (split-half)."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * rope_freqs(base)[None, :]          # [n, 64]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :64], x[..., 64:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def softmax_f64(s):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def decode_f64(q, K, V, sm_scale=None):
    """q [B, Hq, 128]; K, V [B, T, Hkv, 128] (already in the attended domain).

    Returns out [B, Hq, 128] float64.  Every cached token is attended; no mask.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, Hq, Dq = q.shape
    _, T, Hkv, _ = K.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(Dq) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    out = np.zeros((B, Hq, Dq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            s = (K[b, :, kv, :] @ q[b, h]) * scale
            p = softmax_f64(s)
            out[b, h] = p @ V[b, :, kv, :]
    return out
