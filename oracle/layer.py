"""Floating-point side of the oracle: one decoder layer of the packed
selective recompute over the mixed cache, the layer stack, and sequential
maximal-interval replay.  float64 throughout.

TEST INFRASTRUCTURE (see the package docstring).

Shape parameters are read from any object with the attributes ``hidden,
n_q_heads, n_kv_heads, head_dim, intermediate, rms_eps, rope_theta, alpha,
beta``.  Weights follow the PyTorch Linear layout [out, in]; query heads are
row-major in W_q (head h owns rows h*d .. h*d+d-1), likewise W_k / W_v.
"""
from __future__ import annotations

import os
from typing import Callable, Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

FLAG_LOCAL = 1
FLAG_SINK = 2


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def row_threads() -> int:
    """Threads over which independent rows are spread (OMP_NUM_THREADS if set,
    else the usable cores, at most 16)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return min(16, int(env))
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def for_each_row(fn: Callable[[int], None], n: int) -> None:
    """fn(r) for r = 0..n-1.  Rows are independent (each writes only its own
    outputs), so large counts are spread over threads; every row runs the
    same operations whatever the thread count (BLAS is held to one thread
    inside, so a row's products do not depend on how BLAS splits them)."""
    nt = row_threads()
    if n < 32 or nt == 1:
        for r in range(n):
            fn(r)
        return
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(nt) as ex:
        list(ex.map(fn, range(n)))


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row: x / sqrt(mean(x^2) + eps) * gain."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gain)


def rope(x: np.ndarray, pos: Sequence[int], theta: float) -> np.ndarray:
    """Rotary embedding at global positions ``pos`` (the position g_t that the
    cross-attention reuse page, 6.2, says drives RoPE), rotate-half pairing:
    for i < d/2, angle phi_i = g * theta^(-2i/d) and
    (a_i, a_{i+d/2}) -> (a_i cos phi - a_{i+d/2} sin phi,
                         a_{i+d/2} cos phi + a_i sin phi).
    x: [B, H, d]."""
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    phi = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def attention_bias(flags: np.ndarray, alpha: float, beta: float) -> np.ndarray:
    """Per-key additive logit term alpha*1[type=local] + beta*1[key in S']
    (cross-attention reuse page, 6.4, logit form)."""
    f = np.asarray(flags)
    local = ((f & FLAG_LOCAL) != 0).astype(np.float64)
    sink = ((f & FLAG_SINK) != 0).astype(np.float64)
    return alpha * local + beta * sink


def biased_attention_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, bias: np.ndarray,
                         u: int) -> np.ndarray:
    """Output of the query rows ``q`` [G, d] (all at position u) over keys
    0..u inclusive: s_j = <q, k_j>/sqrt(d) + bias_j, o = sum_j softmax_j(s) v_j
    (Budgeted KV-Cache Repair, section 13.2, Eq. 22 with the logit form of the
    cross-attention reuse page, 6.4).  K, V: [N, d] of one KV head."""
    q = _f64(q)
    d = q.shape[-1]
    Kj = _f64(K[:u + 1])
    Vj = _f64(V[:u + 1])
    s = q @ Kj.T / np.sqrt(d) + bias[None, :u + 1]
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ Vj


def write_back_flags(flags: np.ndarray, T: Sequence[int]) -> None:
    """Write-back turns every refreshed position global and takes it out of
    the spurious-sink set (cross-attention reuse page, 6.4: write-back sets
    the type to global; after physical repair no spurious sink remains among
    the repaired keys).  ``flags`` is updated in place."""
    flags[np.asarray(T, dtype=np.int64)] &= np.uint8(~(FLAG_LOCAL | FLAG_SINK) & 0xFF)


def layer_repair(cfg, w: Dict[str, np.ndarray], K: np.ndarray, V: np.ndarray,
                 flags: np.ndarray, T: Sequence[int], x: np.ndarray,
                 return_qkv: bool = False, gpos: Optional[Sequence[int]] = None):
    """One layer of the layer-major packed recurrence (Budgeted KV-Cache
    Repair, section 13.2) for the packed rows ``x`` [B, hidden] at positions T.

    1. n = RMSNorm(x) * gain_attn; q, k, v = n W_q^T (+b_q), n W_k^T (+b_k),
       n W_v^T (+b_v); RoPE on q and k at each row's global position
       g_{u_r} (``gpos[u_r]``, or u_r itself when ``gpos`` is None; the
       cross-attention reuse page, 6.2, has g_t drive RoPE and F).
    2. Before attention, write the fresh k, v into the cache rows T
       (Eq. 21) and mark those positions global with the sink bit cleared
       (write-back sets type <- global, cross-attention reuse page 6.4).
    3. Each query head h attends causally, by global position (keys j with
       g_j <= g_{u_r}), over KV head h // (Hq/Hkv) with the metadata bias
       (Eq. 22 + 6.4 logit form).
    4. h1 = x + O W_o^T; y = h1 + W_down(SiLU(n2 W_gate^T) * (n2 W_up^T))
       with n2 = RMSNorm(h1) * gain_mlp.

    K, V ([N, Hkv, d], float64) and flags ([N], uint8) are updated in place.
    Returns y [B, hidden] (and the post-RoPE q, k and v when asked).
    """
    T = np.asarray(T, dtype=np.int64)
    B = len(T)
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = Hq // Hkv
    N = K.shape[0]
    g = np.arange(N, dtype=np.int64) if gpos is None else np.asarray(gpos, dtype=np.int64)
    x = _f64(x)
    n = rms_norm(x, w["attn_norm"], cfg.rms_eps)
    q = n @ _f64(w["wq"]).T
    k = n @ _f64(w["wk"]).T
    v = n @ _f64(w["wv"]).T
    if w.get("bq") is not None:
        q = q + _f64(w["bq"])
        k = k + _f64(w["bk"])
        v = v + _f64(w["bv"])
    q = rope(q.reshape(B, Hq, d), g[T], cfg.rope_theta)
    k = rope(k.reshape(B, Hkv, d), g[T], cfg.rope_theta)
    v = v.reshape(B, Hkv, d)

    K[T] = k
    V[T] = v
    write_back_flags(flags, T)

    bias = attention_bias(flags, cfg.alpha, cfg.beta)
    # each KV head's keys and values as contiguous [N, d] arrays (a copy for
    # faster row slices; the values are the cache's)
    Kh = [np.ascontiguousarray(K[:, kv]) for kv in range(Hkv)]
    Vh = [np.ascontiguousarray(V[:, kv]) for kv in range(Hkv)]
    o = np.empty((B, Hq, d), dtype=np.float64)

    def attend(r: int) -> None:
        visible = np.flatnonzero(g <= g[T[r]])     # keys at or before the query's position
        u = int(visible[-1])
        assert len(visible) == u + 1, "position map must be strictly increasing"
        for kv in range(Hkv):
            o[r, kv * G:(kv + 1) * G] = biased_attention_row(q[r, kv * G:(kv + 1) * G],
                                                             Kh[kv], Vh[kv], bias, u)

    for_each_row(attend, B)
    h1 = x + o.reshape(B, Hq * d) @ _f64(w["wo"]).T
    n2 = rms_norm(h1, w["mlp_norm"], cfg.rms_eps)
    m = silu(n2 @ _f64(w["w_gate"]).T) * (n2 @ _f64(w["w_up"]).T)
    y = h1 + m @ _f64(w["w_down"]).T
    if return_qkv:
        return y, q, k, v
    return y


def stack_repair(cfg, layers: Iterable[Tuple[Dict[str, np.ndarray], np.ndarray, np.ndarray]],
                 flags: np.ndarray, T: Sequence[int], x: np.ndarray,
                 x_is_full: bool = True,
                 on_layer: Optional[Callable[[int, np.ndarray], None]] = None,
                 gpos: Optional[Sequence[int]] = None) -> np.ndarray:
    """Layer-major traversal (Budgeted KV-Cache Repair, section 3.3): the
    selected rows are gathered once from ``x`` (full [N, hidden] input when
    ``x_is_full``, else already packed) and advance through every layer
    together.  ``layers`` yields (weights, K, V) per layer; each K / V is
    updated in place.  ``on_layer(l, y)`` sees every layer's packed output.
    """
    T = np.asarray(T, dtype=np.int64)
    y = _f64(x)[T] if x_is_full else _f64(x)
    for li, (w, K, V) in enumerate(layers):
        y = layer_repair(cfg, w, K, V, flags, T, y, gpos=gpos)
        if on_layer is not None:
            on_layer(li, y)
    return y


def interval_major(cfg, layers: List[Tuple[Dict[str, np.ndarray], np.ndarray, np.ndarray]],
                   flags: np.ndarray, T: Sequence[int], x_full: np.ndarray) -> np.ndarray:
    """Sequential maximal-interval replay (Budgeted KV-Cache Repair, section
    7.1): each maximal interval [a, b) of T, in order, is forwarded through
    all layers against the current cache, and its K/V rows replace rows
    [a, b) at every layer before the next interval runs.  Returns the final
    hidden states of all selected rows in the order of T."""
    from .repair_set import runs
    T = np.asarray(T, dtype=np.int64)
    starts, lens = runs(T)
    out = []
    for a, ln in zip(starts, lens):
        rows = np.arange(a, a + ln, dtype=np.int64)
        out.append(stack_repair(cfg, layers, flags, rows, x_full, x_is_full=True))
    if not out:
        return np.zeros((0, cfg.hidden), dtype=np.float64)
    return np.concatenate(out, axis=0)
