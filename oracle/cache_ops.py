"""Two operations on the mixed cache beside the repair itself.  float64.

TEST INFRASTRUCTURE (see the package docstring).

* ``inference_attention``: the operator F in inference mode (cross-attention
  reuse page, 6.4, "Prefill / decode, inference mode"): attention only, with
  the metadata logit bias, and no write-back.
* ``shift_cache``: the positional correction applied after a span is deleted
  from the cached sequence ("Budgeted KV-Cache Repair", section 7.1, Eq. 2):
  every retained suffix key moves d positions down and is re-rotated from
  its old position to its new one; values move unchanged.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .layer import _f64, attention_bias, biased_attention_row, rope


def inference_attention(cfg, q: np.ndarray, pos: Sequence[int], K: np.ndarray, V: np.ndarray,
                        flags: np.ndarray) -> np.ndarray:
    """Biased attention of query rows over the mixed cache (6.4, inference
    mode): for row r at position u = pos[r] and query head h (KV head
    h // (Hq/Hkv)), s_j = <q, k_j>/sqrt(d) + alpha*1[local_j] + beta*1[sink_j]
    over keys j = 0..u inclusive, o = sum_j softmax_j(s) v_j.

    Reading: the query at u sees its own position, as the repair's attention
    does (Eq. 22); in decode use the caller has written the new token's K/V
    at u beforehand.  Nothing is written: K, V and flags are left as they are.

    q: [B, Hq, d] post-RoPE; K, V: [N, Hkv, d]; flags: [N].  Returns [B, Hq, d].
    """
    pos = np.asarray(pos, dtype=np.int64)
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = cfg.n_kv_heads
    G = Hq // Hkv
    bias = attention_bias(flags, cfg.alpha, cfg.beta)
    o = np.empty((B, Hq, d), dtype=np.float64)
    for r in range(B):
        u = int(pos[r])
        for g in range(Hkv):
            o[r, g * G:(g + 1) * G] = biased_attention_row(q[r, g * G:(g + 1) * G], K[:, g],
                                                           V[:, g], bias, u)
    return o


def shift_cache(cfg, K: np.ndarray, V: np.ndarray, flags: np.ndarray,
                block_id: Optional[np.ndarray], del_start: int, del_len: int,
                mark: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Cache of x^- = p + s after deleting the span e = [a, a + d) of x = p + e + s
    (section 7.1): rows [0, a) are kept; the suffix key at old position i
    (i >= a + d) becomes the key at i - d,

        K~_{i-d} = R_{i-d} (R_i)^{-1} K_i,   V~_{i-d} = V_i     (Eq. 2),

    with R_i the rotary map of the oracle's ``rope`` at position i and
    (R_i)^{-1} = R_{-i} (a rotation).  Metadata moves with its row.

    Reading: the pages say the shifted suffix still carries the deleted
    span's influence; a caller that tracks this in the type bit passes
    ``mark`` (e.g. the local bit), which is OR-ed into every moved row's
    flags.  K, V: [N, Hkv, d].  Returns (K~, V~, flags~, block_id~) with
    N - d rows; the inputs are not modified.
    """
    N = K.shape[0]
    a, d = int(del_start), int(del_len)
    if a < 0 or d < 0 or a + d > N:
        raise ValueError("deleted span outside the cache")
    old = np.arange(a + d, N, dtype=np.int64)
    Ks = _f64(K[a + d:])
    Kt = rope(rope(Ks, -old, cfg.rope_theta), old - d, cfg.rope_theta)
    K2 = np.concatenate([_f64(K[:a]), Kt], axis=0)
    V2 = np.concatenate([_f64(V[:a]), _f64(V[a + d:])], axis=0)
    f = np.asarray(flags, dtype=np.uint8)
    f2 = np.concatenate([f[:a], f[a + d:] | np.uint8(mark)]).astype(np.uint8)
    b2 = None
    if block_id is not None:
        b = np.asarray(block_id, dtype=np.int32)
        b2 = np.concatenate([b[:a], b[a + d:]]).astype(np.int32)
    return K2, V2, f2, b2
