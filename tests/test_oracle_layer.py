"""Pins of the oracle's float side: closed forms, library routines the
operator reduces to, invariants the pages state, and pure-Python brute force.
Each is chosen so that a plausible slip in the oracle (a dropped bias term,
a wrong sign or pairing in RoPE, a transposed operand, attention that is not
inclusive of the query's own position, write-back after instead of before
attention) fails at least one of them."""
import math
from dataclasses import dataclass

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import refs


@dataclass
class Cfg:
    hidden: int = 32
    n_q_heads: int = 4
    n_kv_heads: int = 2
    head_dim: int = 8
    intermediate: int = 48
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    alpha: float = -1.0
    beta: float = -2.0


def rand_layer(rng, c: Cfg, scale=0.3, bias=False):
    h, qd, kd, it = c.hidden, c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim, c.intermediate
    w = {
        "attn_norm": 1 + 0.1 * rng.standard_normal(h),
        "wq": scale * rng.standard_normal((qd, h)),
        "wk": scale * rng.standard_normal((kd, h)),
        "wv": scale * rng.standard_normal((kd, h)),
        "wo": scale * rng.standard_normal((h, qd)),
        "mlp_norm": 1 + 0.1 * rng.standard_normal(h),
        "w_gate": scale * rng.standard_normal((it, h)),
        "w_up": scale * rng.standard_normal((it, h)),
        "w_down": scale * rng.standard_normal((h, it)),
    }
    if bias:
        w["bq"] = rng.standard_normal(qd)
        w["bk"] = rng.standard_normal(kd)
        w["bv"] = rng.standard_normal(kd)
    return w


def mixed_flags(N, block):
    s = np.arange(0, N, block)
    f = np.zeros(N, dtype=np.uint8)
    f[block:] |= oracle.FLAG_LOCAL
    f[s[1:]] |= oracle.FLAG_SINK
    return f


# --------------------------------------------------------------- elementwise
def test_rms_norm_closed_form():
    x = np.full((2, 16), -3.0)
    g = np.arange(16) + 1.0
    y = oracle.rms_norm(x, g, 0.0)
    assert np.allclose(y, -g[None, :], rtol=0, atol=1e-15)
    # eps enters under the square root: mean(x^2)=1 -> 1/sqrt(1+eps)
    y = oracle.rms_norm(np.ones((1, 4)), np.ones(4), 0.25)
    assert np.allclose(y, 1 / math.sqrt(1.25))


def test_rope_two_dims_is_plane_rotation():
    # d = 2: one pair, inv_freq = 1, the angle is the position itself
    x = np.array([[[0.6, -0.8]]])
    for p in (0, 1, 5, 1000):
        y = oracle.rope(x, [p], 1e6)[0, 0]
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(y, [0.6 * c + 0.8 * s, -0.8 * c + 0.6 * s], atol=1e-12)


def test_rope_matches_complex_formulation_and_properties():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((9, 3, 16))
    pos = np.array([0, 1, 2, 7, 100, 511, 4095, 16383, 32767])
    y = oracle.rope(x, pos, 1e6)
    want = refs.rope_complex(torch.tensor(x), torch.tensor(pos), 1e6).numpy()
    assert np.allclose(y, want, atol=1e-10)
    assert np.allclose(y[0], x[0])                                   # position 0 = identity
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    # <R_m q, R_n k> depends only on m - n
    q, k = rng.standard_normal((1, 1, 16)), rng.standard_normal((1, 1, 16))
    dots = [float(np.sum(oracle.rope(q, [m], 1e4) * oracle.rope(k, [m - 5], 1e4)))
            for m in (5, 17, 300)]
    assert np.allclose(dots, dots[0], atol=1e-10)


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    y = oracle.silu(z)
    assert y[0] == 0.0
    assert math.isclose(y[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(y[2], -1 / (1 + math.e), rel_tol=1e-15)
    assert math.isclose(y[3], 40.0, rel_tol=1e-15) and abs(y[4]) < 1e-15


# ----------------------------------------------------------------- attention
def test_attention_bias_terms():
    f = np.array([0, 1, 2, 3], dtype=np.uint8)
    assert oracle.attention_bias(f, -1.5, -3.0).tolist() == [0.0, -1.5, -3.0, -4.5]


def test_attention_unbiased_is_causal_sdpa():
    rng = np.random.default_rng(1)
    N, G, d = 40, 3, 16
    K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    Q = rng.standard_normal((N, G, d))
    zero = np.zeros(N)
    got = np.stack([oracle.biased_attention_row(Q[u], K, V, zero, u) for u in range(N)])
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Q).transpose(0, 1), torch.tensor(K)[None].expand(G, N, d).contiguous(),
        torch.tensor(V)[None].expand(G, N, d).contiguous(), is_causal=True).transpose(0, 1)
    assert np.allclose(got, want.numpy(), atol=1e-12)


def test_attention_biased_is_sdpa_with_additive_mask():
    rng = np.random.default_rng(2)
    N, G, d = 33, 2, 8
    K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    flags = mixed_flags(N, 8)
    bias = oracle.attention_bias(flags, -1.0, -2.0)
    for u in (0, 7, 8, 9, 20, 32):
        q = rng.standard_normal((G, d))
        got = oracle.biased_attention_row(q, K, V, bias, u)
        assert np.allclose(got, refs.sdpa_biased(q, K, V, bias, u), atol=1e-12)


def test_attention_two_key_closed_form():
    # equal scores, key 0 global, key 1 local: weight of the local key is
    # e^alpha / (1 + e^alpha); sink adds beta on top
    d = 4
    q = np.zeros((1, d))
    K = np.zeros((2, d))
    V = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    for a, b, fl in ((-1.0, 0.0, 1), (-1.0, -2.0, 3), (0.7, -2.0, 2)):
        bias = oracle.attention_bias(np.array([0, fl], dtype=np.uint8), a, b)
        o = oracle.biased_attention_row(q, K, V, bias, 1)[0]
        t = (a if fl & 1 else 0.0) + (b if fl & 2 else 0.0)
        assert np.allclose(o[:2], [1 / (1 + math.exp(t)), math.exp(t) / (1 + math.exp(t))])


def test_attention_shift_invariance_all_local():
    rng = np.random.default_rng(3)
    N, d = 20, 8
    K, V, q = rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((2, d))
    f = np.full(N, oracle.FLAG_LOCAL, dtype=np.uint8)
    a = oracle.biased_attention_row(q, K, V, oracle.attention_bias(f, -3.0, -2.0), N - 1)
    b = oracle.biased_attention_row(q, K, V, np.zeros(N), N - 1)
    assert np.allclose(a, b, atol=1e-13)


def test_attention_brute_force_python():
    rng = np.random.default_rng(4)
    N, d = 24, 6
    K, V, q = rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((1, d))
    flags = mixed_flags(N, 6)
    for u in (0, 5, 6, 13, 23):
        got = oracle.biased_attention_row(q, K, V, oracle.attention_bias(flags, -1.2, -0.4), u)[0]
        sc = [sum(q[0, c] * K[j, c] for c in range(d)) / math.sqrt(d)
              - 1.2 * (flags[j] & 1) - 0.4 * ((flags[j] >> 1) & 1) for j in range(u + 1)]
        mx = max(sc)
        e = [math.exp(s - mx) for s in sc]
        want = [sum(e[j] * V[j, c] for j in range(u + 1)) / sum(e) for c in range(d)]
        assert np.allclose(got, want, atol=1e-13)


# --------------------------------------------------------------- layer/stack
def _stack_inputs(seed, c: Cfg, N, L, bias=False, scale=0.3):
    rng = np.random.default_rng(seed)
    layers = [rand_layer(rng, c, scale, bias) for _ in range(L)]
    caches = [(rng.standard_normal((N, c.n_kv_heads, c.head_dim)),
               rng.standard_normal((N, c.n_kv_heads, c.head_dim))) for _ in range(L)]
    X = rng.standard_normal((N, c.hidden))
    return layers, caches, X


def _copy(caches):
    return [(K.copy(), V.copy()) for K, V in caches]


def test_stack_matches_pure_python_brute_force():
    c = Cfg()
    N, L = 20, 2
    for bias in (False, True):
        layers, caches, X = _stack_inputs(5, c, N, L, bias)
        flags = mixed_flags(N, 5)
        T = [4, 5, 6, 11, 15, 19]
        cc = _copy(caches)
        f1 = flags.copy()
        got = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cc)], f1, T, X)
        # pure python
        Kp = [K.tolist() for K, _ in caches]
        Vp = [V.tolist() for _, V in caches]
        fp = flags.tolist()
        xs = [X[t].tolist() for t in T]
        for li in range(L):
            fl = list(fp)
            xs = refs.py_layer(c, layers[li], Kp[li], Vp[li], fl, T, xs)
            fp = fl
        assert np.allclose(got, np.array(xs), atol=1e-11, rtol=1e-11)
        for li in range(L):
            assert np.allclose(cc[li][0], np.array(Kp[li]), atol=1e-12)
            assert np.allclose(cc[li][1], np.array(Vp[li]), atol=1e-12)
        assert f1.tolist() == fp


@pytest.mark.parametrize("alpha,beta", [(0.0, 0.0), (-1.0, -2.0)])
def test_degeneration_equals_full_prefill(alpha, beta):
    # tau >= |B|/2 covers B_2..B_m: after write-back no local keys and no
    # sinks remain, so F is plain causal softmax attention (6.4), and the
    # repaired rows equal one full prefill.  B_1's cache comes from a
    # repair over B_1 itself (its rows see only themselves).
    c = Cfg(alpha=alpha, beta=beta)
    N, L, blk = 48, 3, 12
    layers, caches, X = _stack_inputs(6, c, N, L, bias=True)
    flags = mixed_flags(N, blk)
    s = list(range(0, N, blk))
    e = s[1:] + [N]
    T = oracle.seam_set(s, e, blk // 2, True)
    assert T.tolist() == list(range(blk, N))
    cc = _copy(caches)
    stack = lambda TT: oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cc)],
                                           flags, TT, X)
    y1 = stack(np.arange(blk))
    y2 = stack(T)
    want, kvs = refs.full_prefill(c, layers, X)
    assert np.allclose(y1, want[:blk], atol=1e-11)
    assert np.allclose(y2, want[blk:], atol=1e-11)
    for li in range(L):
        assert np.allclose(cc[li][0], kvs[li][0], atol=1e-11)
        assert np.allclose(cc[li][1], kvs[li][1], atol=1e-11)
    assert np.all(flags == 0)


def test_layer_major_equals_interval_major():
    c = Cfg()
    N, L = 64, 3
    layers, caches, X = _stack_inputs(8, c, N, L)
    flags = mixed_flags(N, 16)
    T = np.array([3, 4, 5, 17, 18, 30, 31, 32, 33, 47, 60, 61, 62, 63])
    ca, cb = _copy(caches), _copy(caches)
    fa, fb = flags.copy(), flags.copy()
    ya = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, ca)], fa, T, X)
    yb = oracle.interval_major(c, [(w, K, V) for w, (K, V) in zip(layers, cb)], fb, T, X)
    assert np.allclose(ya, yb, atol=1e-12)
    for (Ka, Va), (Kb, Vb) in zip(ca, cb):
        assert np.allclose(Ka, Kb, atol=1e-12) and np.allclose(Va, Vb, atol=1e-12)
    assert np.array_equal(fa, fb)


def test_packing_order_and_untouched_rows():
    c = Cfg()
    N, L = 50, 2
    layers, caches, X = _stack_inputs(9, c, N, L)
    flags = mixed_flags(N, 10)
    T = np.array([10, 11, 25, 26, 27, 40, 49])
    perm = np.array([4, 0, 6, 2, 1, 5, 3])
    ca, cb = _copy(caches), _copy(caches)
    fa, fb = flags.copy(), flags.copy()
    ya = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, ca)], fa, T, X)
    yb = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cb)], fb, T[perm], X)
    assert np.allclose(yb, ya[perm], atol=1e-13)
    keep = np.setdiff1d(np.arange(N), T)
    for (K0, V0), (Ka, Va) in zip(caches, ca):
        assert np.array_equal(Ka[keep], K0[keep]) and np.array_equal(Va[keep], V0[keep])
        assert not np.allclose(Ka[T], K0[T])
    assert np.array_equal(fa[keep], flags[keep]) and np.all(fa[T] == 0)


def test_causal_prefix_of_support_is_self_contained():
    # the first k selected rows depend only on keys <= their positions, so a
    # repair over T[:k] reproduces their rows of the repair over T exactly
    # (this is what the sampled full-size parity checks rely on)
    c = Cfg()
    N, L = 60, 2
    layers, caches, X = _stack_inputs(10, c, N, L)
    flags = mixed_flags(N, 12)
    T = np.array([12, 13, 14, 24, 25, 36, 40, 41, 59])
    for k in (1, 4, 6):
        ca, cb = _copy(caches), _copy(caches)
        ya = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, ca)], flags.copy(), T, X)
        yb = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cb)], flags.copy(),
                                 T[:k], X)
        assert np.allclose(ya[:k], yb, atol=1e-13)


def test_bias_alpha_beta_zero_is_exactly_unbiased():
    c0, c1 = Cfg(alpha=0.0, beta=0.0), Cfg(alpha=0.0, beta=0.0)
    N = 30
    layers, caches, X = _stack_inputs(11, c0, N, 1)
    T = [10, 20, 21]
    a = oracle.stack_repair(c0, [(layers[0], *_copy(caches)[0])], mixed_flags(N, 10), T, X)
    b = oracle.stack_repair(c1, [(layers[0], *_copy(caches)[0])], np.zeros(N, np.uint8), T, X)
    assert np.array_equal(a, b)


def test_workload_tiny_layer_runs():
    # the oracle runs on the tiny workload's real generated inputs
    w = wl.TINY
    s, e = wl.blocks(w)
    T = oracle.seam_set(s, e, w.tau, True)
    K, V = wl.kv_cache(w, 0)
    K, V = K.astype(np.float64), V.astype(np.float64)
    flags = wl.initial_flags(w)
    X = wl.hidden_states(w)
    y = oracle.stack_repair(w, [(wl.layer_weights(w, 0), K, V)], flags, T, X)
    assert y.shape == (24, 256) and np.all(np.isfinite(y))
    assert np.all(flags[T] == 0)


# ------------------------------------------------------- global positions g_t


def _gapped_positions(N, rng):
    """A strictly increasing position map with gaps (as a cache that lost
    spans without being shifted would have)."""
    return np.cumsum(rng.integers(1, 5, size=N)) + 7


def test_identity_position_map_is_bitwise_the_default():
    c = Cfg()
    N = 30
    layers, caches, X = _stack_inputs(12, c, N, 2)
    T = [10, 11, 20, 29]
    ca, cb = _copy(caches), _copy(caches)
    a = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, ca)], mixed_flags(N, 10),
                            T, X)
    b = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cb)], mixed_flags(N, 10),
                            T, X, gpos=np.arange(N))
    assert np.array_equal(a, b)
    for (Ka, Va), (Kb, Vb) in zip(ca, cb):
        assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)


def test_position_map_matches_pure_python_brute_force():
    c = Cfg()
    N, L = 18, 2
    rng = np.random.default_rng(13)
    g = _gapped_positions(N, rng)
    layers, caches, X = _stack_inputs(13, c, N, L, bias=True)
    flags = mixed_flags(N, 6)
    T = [5, 6, 7, 12, 17]
    cc = _copy(caches)
    f1 = flags.copy()
    got = oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cc)], f1, T, X, gpos=g)
    Kp = [K.tolist() for K, _ in caches]
    Vp = [V.tolist() for _, V in caches]
    fp = flags.tolist()
    xs = [X[t].tolist() for t in T]
    for li in range(L):
        xs = refs.py_layer(c, layers[li], Kp[li], Vp[li], fp, T, xs, pos=g)
    assert np.allclose(got, np.array(xs), atol=1e-11, rtol=1e-11)
    for li in range(L):
        assert np.allclose(cc[li][0], np.array(Kp[li]), atol=1e-12)


def test_position_map_degeneration_equals_full_prefill_at_those_positions():
    # a full recompute with alpha = beta = 0 and a gapped position map is a
    # textbook prefill whose RoPE uses those positions
    c = Cfg(alpha=0.0, beta=0.0)
    N, L, blk = 40, 2, 10
    rng = np.random.default_rng(14)
    g = _gapped_positions(N, rng)
    layers, caches, X = _stack_inputs(14, c, N, L, bias=False)
    cc = _copy(caches)
    flags = mixed_flags(N, blk)
    run = lambda TT: oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cc)], flags,
                                         TT, X, gpos=g)
    y1 = run(np.arange(blk))
    y2 = run(np.arange(blk, N))
    want, kvs = refs.full_prefill(c, layers, X, pos=g)
    assert np.allclose(y1, want[:blk], atol=1e-11)
    assert np.allclose(y2, want[blk:], atol=1e-11)
    for li in range(L):
        assert np.allclose(cc[li][0], kvs[li][0], atol=1e-11)
    # and it is not the identity-position prefill
    other, _ = refs.full_prefill(c, layers, X)
    assert not np.allclose(y2, other[blk:], atol=1e-6)


def test_constant_position_offset_leaves_a_full_recompute_unchanged():
    # RoPE scores depend only on position differences, so shifting every
    # position by one constant changes nothing once all keys are recomputed
    c = Cfg(alpha=0.0, beta=0.0)
    N = 24
    layers, caches, X = _stack_inputs(15, c, N, 2)
    outs = []
    for off in (0, 1000):
        cc = _copy(caches)
        outs.append(oracle.stack_repair(c, [(w, K, V) for w, (K, V) in zip(layers, cc)],
                                        np.zeros(N, np.uint8), np.arange(N), X,
                                        gpos=np.arange(N) + off))
    assert np.allclose(outs[0], outs[1], atol=1e-10)
