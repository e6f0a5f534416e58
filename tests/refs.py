"""Independent references used to pin the oracle (never the GPU path).

* ``full_prefill``: a textbook dense causal decoder built from PyTorch CPU
  float64 library routines (F.rms_norm, complex-multiplication RoPE,
  scaled_dot_product_attention with GQA, F.silu, F.linear).  It is what
  the biased operator must reduce to in the degenerate case (cross-attention
  reuse page, 6.4, "Degeneration").
* ``py_*``: pure-Python brute force (lists, ``math``) for tiny inputs.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def rope_complex(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """RoPE as multiplication of z_i = a_i + i*a_{i+d/2} by exp(i*pos*theta^(-2i/d))."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-(torch.arange(half, dtype=torch.float64) * 2.0) / d)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def full_prefill(cfg, layers: Sequence[Dict[str, np.ndarray]], X: np.ndarray, pos=None):
    """Dense causal decoder over all rows of X [N, hidden]; returns the final
    hidden states and every layer's (K, V) [N, Hkv, d] (post-RoPE keys).
    ``pos`` (default 0..N-1) are the rows' positions for RoPE; the causal
    mask is the row order (positions must increase with the row)."""
    N = X.shape[0]
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pos = torch.arange(N) if pos is None else torch.as_tensor(np.asarray(pos, dtype=np.int64))
    x = _t(X)
    kvs = []
    for w in layers:
        n = F.rms_norm(x, (cfg.hidden,), weight=_t(w["attn_norm"]), eps=cfg.rms_eps)
        q = F.linear(n, _t(w["wq"]), None if w.get("bq") is None else _t(w["bq"]))
        k = F.linear(n, _t(w["wk"]), None if w.get("bk") is None else _t(w["bk"]))
        v = F.linear(n, _t(w["wv"]), None if w.get("bv") is None else _t(w["bv"]))
        q = rope_complex(q.view(N, Hq, d), pos, cfg.rope_theta)
        k = rope_complex(k.view(N, Hkv, d), pos, cfg.rope_theta)
        v = v.view(N, Hkv, d)
        kvs.append((k.numpy().copy(), v.numpy().copy()))
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1).contiguous(),
                                           v.transpose(0, 1).contiguous(), is_causal=True,
                                           enable_gqa=True)
        h1 = x + F.linear(o.transpose(0, 1).reshape(N, Hq * d), _t(w["wo"]))
        n2 = F.rms_norm(h1, (cfg.hidden,), weight=_t(w["mlp_norm"]), eps=cfg.rms_eps)
        m = F.silu(F.linear(n2, _t(w["w_gate"]))) * F.linear(n2, _t(w["w_up"]))
        x = h1 + F.linear(m, _t(w["w_down"]))
    return x.numpy(), kvs


def sdpa_biased(q, K, V, bias, u):
    """Library attention of query rows q [G, d] at position u over keys
    0..u with an additive float mask equal to ``bias``."""
    q = _t(q)[None]                          # [1, G, d]
    k = _t(K[:u + 1])[None]
    v = _t(V[:u + 1])[None]
    m = _t(bias[:u + 1])[None, None, :]      # broadcast over the G rows
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m)[0].numpy()


# ----------------------------------------------------------------------------
# pure Python
# ----------------------------------------------------------------------------
def py_matvec(W: List[List[float]], x: List[float]) -> List[float]:
    return [sum(wi * xi for wi, xi in zip(row, x)) for row in W]


def py_rms(x: List[float], g: List[float], eps: float) -> List[float]:
    r = math.sqrt(sum(v * v for v in x) / len(x) + eps)
    return [v / r * gi for v, gi in zip(x, g)]


def py_rope(a: List[float], p: int, theta: float) -> List[float]:
    d = len(a)
    h = d // 2
    out = list(a)
    for i in range(h):
        ang = p * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = a[i] * c - a[i + h] * s
        out[i + h] = a[i + h] * c + a[i] * s
    return out


def py_layer(cfg, w, K, V, flags, T, X, pos=None):
    """One packed layer with lists: K, V are lists [N][Hkv][d] (mutated),
    flags a list of ints (mutated), X a list of packed rows; ``pos`` maps a
    row to its RoPE position (default: the row itself)."""
    P = (lambda t: t) if pos is None else (lambda t: int(pos[t]))
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = Hq // Hkv
    tolist = lambda a: np.asarray(a, dtype=np.float64).tolist()
    Wq, Wk, Wv, Wo = tolist(w["wq"]), tolist(w["wk"]), tolist(w["wv"]), tolist(w["wo"])
    Wg, Wu, Wd = tolist(w["w_gate"]), tolist(w["w_up"]), tolist(w["w_down"])
    ga, gm = tolist(w["attn_norm"]), tolist(w["mlp_norm"])
    Q = []
    for r, t in enumerate(T):
        n = py_rms(X[r], ga, cfg.rms_eps)
        q, k, v = py_matvec(Wq, n), py_matvec(Wk, n), py_matvec(Wv, n)
        if w.get("bq") is not None:
            q = [a + b for a, b in zip(q, tolist(w["bq"]))]
            k = [a + b for a, b in zip(k, tolist(w["bk"]))]
            v = [a + b for a, b in zip(v, tolist(w["bv"]))]
        Q.append([py_rope(q[h * d:(h + 1) * d], P(t), cfg.rope_theta) for h in range(Hq)])
        K[t] = [py_rope(k[g * d:(g + 1) * d], P(t), cfg.rope_theta) for g in range(Hkv)]
        V[t] = [v[g * d:(g + 1) * d] for g in range(Hkv)]
        flags[t] = 0
    out = []
    for r, t in enumerate(T):
        o = []
        for h in range(Hq):
            g = h // G
            sc = []
            for j in range(t + 1):
                s = sum(a * b for a, b in zip(Q[r][h], K[j][g])) / math.sqrt(d)
                s += cfg.alpha * (1 if flags[j] & 1 else 0) + cfg.beta * (1 if flags[j] & 2 else 0)
                sc.append(s)
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            o.extend(sum(e[j] / z * V[j][g][c] for j in range(t + 1)) for c in range(d))
        h1 = [a + b for a, b in zip(X[r], py_matvec(Wo, o))]
        n2 = py_rms(h1, gm, cfg.rms_eps)
        gt, up = py_matvec(Wg, n2), py_matvec(Wu, n2)
        mm = [a / (1.0 + math.exp(-a)) * b for a, b in zip(gt, up)]
        out.append([a + b for a, b in zip(h1, py_matvec(Wd, mm))])
    return out
