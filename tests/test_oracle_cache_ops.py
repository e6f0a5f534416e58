"""Pins of the oracle's inference-mode attention and Shift.

Inference attention (cross-attention reuse page, 6.4, inference mode) is
pinned to PyTorch's scaled_dot_product_attention (float64, GQA, additive
float mask built independently), to the degenerate case, to the GQA head
map and to "no write-back".  Shift (Budgeted KV-Cache Repair, section 7.1,
Eq. 2) is pinned to its defining property (a key rotated at i and shifted
equals the same raw key rotated at i - d), to an independent complex-number
rotation by -d, and to pure-Python brute force.  A slip such as a wrong
rotation sign, the pairing (i, i+1) instead of (i, i+d/2), h % Hkv instead
of h // G, exclusive instead of inclusive causality, or moving the prefix
fails one of these."""
import math
from dataclasses import dataclass

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from tests import refs


@dataclass
class Cfg:
    n_q_heads: int = 6
    n_kv_heads: int = 2
    head_dim: int = 8
    rope_theta: float = 10000.0
    alpha: float = -1.0
    beta: float = -2.0


def _flags(N, block):
    f = np.zeros(N, dtype=np.uint8)
    f[block:] |= oracle.FLAG_LOCAL
    f[np.arange(block, N, block)] |= oracle.FLAG_SINK
    return f


def _sdpa_rows(c, q, pos, K, V, flags):
    """Library reference: SDPA with GQA and a [B, N] additive mask that holds
    -inf past each query's position plus the metadata bias."""
    B, N = len(pos), K.shape[0]
    bias = np.where(flags & 1, c.alpha, 0.0) + np.where(flags & 2, c.beta, 0.0)
    m = np.full((B, N), -np.inf)
    for r, u in enumerate(pos):
        m[r, :u + 1] = bias[:u + 1]
    out = F.scaled_dot_product_attention(
        torch.tensor(q).transpose(0, 1), torch.tensor(K).transpose(0, 1).contiguous(),
        torch.tensor(V).transpose(0, 1).contiguous(), attn_mask=torch.tensor(m)[None],
        enable_gqa=True)
    return out.transpose(0, 1).numpy()


# ---------------------------------------------------------- inference mode
def test_inference_unbiased_prefill_is_causal_sdpa():
    c = Cfg(alpha=0.0, beta=0.0)
    rng = np.random.default_rng(10)
    N = 37
    q = rng.standard_normal((N, c.n_q_heads, c.head_dim))
    K = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    V = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    got = oracle.inference_attention(c, q, np.arange(N), K, V, _flags(N, 8))
    want = F.scaled_dot_product_attention(
        torch.tensor(q).transpose(0, 1), torch.tensor(K).transpose(0, 1).contiguous(),
        torch.tensor(V).transpose(0, 1).contiguous(), is_causal=True, enable_gqa=True)
    assert np.allclose(got, want.transpose(0, 1).numpy(), atol=1e-12)


def test_inference_biased_matches_masked_sdpa_on_sparse_positions():
    c = Cfg(alpha=-1.5, beta=-3.0)
    rng = np.random.default_rng(11)
    N = 64
    pos = np.array([0, 5, 8, 9, 31, 32, 33, 63])
    q = rng.standard_normal((len(pos), c.n_q_heads, c.head_dim))
    K = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    V = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    fl = _flags(N, 16)
    got = oracle.inference_attention(c, q, pos, K, V, fl)
    assert np.allclose(got, _sdpa_rows(c, q, pos, K, V, fl), atol=1e-12)


def test_inference_no_write_back_and_gqa_head_map():
    c = Cfg()
    rng = np.random.default_rng(12)
    N = 40
    pos = np.array([3, 20, 39])
    q = rng.standard_normal((3, c.n_q_heads, c.head_dim))
    K = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    V = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    fl = _flags(N, 10)
    K0, V0, f0 = K.copy(), V.copy(), fl.copy()
    a = oracle.inference_attention(c, q, pos, K, V, fl)
    assert np.array_equal(K, K0) and np.array_equal(V, V0) and np.array_equal(fl, f0)
    # heads 0..2 read KV head 0 only, heads 3..5 KV head 1 only
    K2, V2 = K.copy(), V.copy()
    K2[:, 1] += 5.0
    V2[:, 1] *= -2.0
    b = oracle.inference_attention(c, q, pos, K2, V2, fl)
    assert np.array_equal(a[:, :3], b[:, :3])
    assert not np.allclose(a[:, 3:], b[:, 3:])


def test_inference_degenerates_without_local_or_sink_keys():
    rng = np.random.default_rng(13)
    N = 30
    q = rng.standard_normal((4, 6, 8))
    K, V = rng.standard_normal((N, 2, 8)), rng.standard_normal((N, 2, 8))
    pos = [0, 7, 15, 29]
    z = np.zeros(N, dtype=np.uint8)
    a = oracle.inference_attention(Cfg(alpha=-4.0, beta=-9.0), q, pos, K, V, z)
    b = oracle.inference_attention(Cfg(alpha=0.0, beta=0.0), q, pos, K, V, z)
    assert np.array_equal(a, b)


def test_inference_brute_force_python():
    c = Cfg(n_q_heads=2, n_kv_heads=1, head_dim=4, alpha=-0.7, beta=-1.3)
    rng = np.random.default_rng(14)
    N = 12
    K, V = rng.standard_normal((N, 1, 4)), rng.standard_normal((N, 1, 4))
    fl = _flags(N, 4)
    pos = [2, 4, 11]
    q = rng.standard_normal((3, 2, 4))
    got = oracle.inference_attention(c, q, pos, K, V, fl)
    for r, u in enumerate(pos):
        for h in range(2):
            sc = [sum(q[r, h, i] * K[j, 0, i] for i in range(4)) / 2.0
                  + (c.alpha if fl[j] & 1 else 0.0) + (c.beta if fl[j] & 2 else 0.0)
                  for j in range(u + 1)]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            want = [sum(e[j] * V[j, 0, i] for j in range(u + 1)) / sum(e) for i in range(4)]
            assert np.allclose(got[r, h], want, atol=1e-13)


# ------------------------------------------------------------------- shift
def test_shift_keys_equal_raw_keys_rotated_at_new_positions():
    """Eq. 2's purpose: a key stored as R_i k is, after the shift, R_{i-d} k."""
    c = Cfg()
    rng = np.random.default_rng(20)
    N, a, d = 50, 12, 7
    raw = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    K = oracle.rope(raw, np.arange(N), c.rope_theta)
    V = rng.standard_normal((N, c.n_kv_heads, c.head_dim))
    K2, V2, _, _ = oracle.shift_cache(c, K, V, np.zeros(N, np.uint8), None, a, d)
    keep = np.r_[0:a, a + d:N]
    want = oracle.rope(raw[keep], np.arange(N - d), c.rope_theta)
    assert K2.shape == (N - d, c.n_kv_heads, c.head_dim)
    assert np.allclose(K2, want, atol=1e-12)
    assert np.array_equal(V2, V[keep])


def test_shift_is_rotation_by_minus_d_complex_form():
    c = Cfg(rope_theta=1e6, head_dim=16)
    rng = np.random.default_rng(21)
    N, a, d = 40, 5, 9
    K = rng.standard_normal((N, 2, 16))
    V = rng.standard_normal((N, 2, 16))
    K2, _, _, _ = oracle.shift_cache(c, K, V, np.zeros(N, np.uint8), None, a, d)
    suffix = torch.tensor(K[a + d:])
    want = refs.rope_complex(suffix, torch.full((N - a - d,), -d), c.rope_theta).numpy()
    assert np.array_equal(K2[:a], K[:a])
    assert np.allclose(K2[a:], want, atol=1e-12)
    assert np.allclose(np.linalg.norm(K2[a:], axis=-1), np.linalg.norm(K[a + d:], axis=-1))


def test_shift_metadata_and_edges():
    c = Cfg()
    rng = np.random.default_rng(22)
    N = 20
    K, V = rng.standard_normal((N, 2, 8)), rng.standard_normal((N, 2, 8))
    fl = _flags(N, 5)
    blk = (np.arange(N) // 5).astype(np.int32)
    K2, V2, f2, b2 = oracle.shift_cache(c, K, V, fl, blk, 5, 3, mark=oracle.FLAG_LOCAL)
    assert f2.tolist() == fl[:5].tolist() + (fl[8:] | 1).tolist()
    assert b2.tolist() == blk[:5].tolist() + blk[8:].tolist()
    # d = 0: identity up to the rotation by zero
    K3, V3, f3, _ = oracle.shift_cache(c, K, V, fl, None, 7, 0)
    assert np.allclose(K3, K, atol=1e-15) and np.array_equal(V3, V) and np.array_equal(f3, fl)
    # deleting the whole suffix leaves the prefix
    K4, V4, f4, _ = oracle.shift_cache(c, K, V, fl, None, 6, N - 6)
    assert K4.shape[0] == 6 and np.array_equal(K4, K[:6]) and np.array_equal(V4, V[:6])


def test_shift_brute_force_python():
    c = Cfg(n_kv_heads=1, head_dim=4, rope_theta=100.0)
    rng = np.random.default_rng(23)
    N, a, d = 9, 2, 3
    K, V = rng.standard_normal((N, 1, 4)), rng.standard_normal((N, 1, 4))
    K2, _, _, _ = oracle.shift_cache(c, K, V, np.zeros(N, np.uint8), None, a, d)
    for i in range(a + d, N):
        for j in range(2):                       # pairs (j, j + 2)
            ang = -d * 100.0 ** (-2.0 * j / 4)
            x, y = K[i, 0, j], K[i, 0, j + 2]
            assert math.isclose(K2[i - d, 0, j], x * math.cos(ang) - y * math.sin(ang), abs_tol=1e-12)
            assert math.isclose(K2[i - d, 0, j + 2], y * math.cos(ang) + x * math.sin(ang), abs_tol=1e-12)
