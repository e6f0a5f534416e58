"""Numeric core of Semantic-Unit Refresh ("Budgeted KV-Cache Repair",
section 3.2 and Appendix 7.3, Eq. 1 / 7, Eq. 8, Algorithm 1): token
relevance from the frozen embedding table, unit scores and ranking, the
exact-budget fill with a forward-envelope window for the unit that does not
fit, and the sort-and-coalesce into positions.

TEST INFRASTRUCTURE (see the package docstring).

Precision: the page runs embedding normalisation and cosine scoring in
float32, so token scores are computed in float32 here (numpy float32
arithmetic, BLAS float32 matmul as the library step).  Unit scores and the
envelope are float32 too: they are computed from the float32 scores and
decide which positions are selected.

Readings where the page leaves a step open:
* Unit boundaries come from text (messages, containers, paragraphs,
  sentences) and a tokenizer, neither of which is here: the partition of the
  suffix into units is an input (sorted unit starts, first 0; unit u covers
  [start[u], start[u+1]) with start[n_units] = S).
* A zero-norm embedding row has no direction: its cosine is taken as 0.
* "s_i in q" means token identity: the suffix token id occurs among the
  query token ids.
* The envelope starts from u_0 = 0 before the unit's first token, so the
  first token's envelope value is e^(r_1 - r_max).
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

SUR_BONUS = np.float32(0.25)
ENVELOPE_DECAY = np.float32(math.exp(-1.0 / 16.0))


def token_scores(E: np.ndarray, suffix_ids: Sequence[int], query_ids: Sequence[int]) -> np.ndarray:
    """Eq. 7: r_i = max_j <E(s_i), E(q_j)> / (||E(s_i)||_2 ||E(q_j)||_2)
    + 0.25 * 1[s_i in q], in float32.  E: [vocab, hidden] (any float dtype,
    read as float32).  Returns r [S] float32."""
    s = np.asarray(suffix_ids, dtype=np.int64)
    qi = np.asarray(query_ids, dtype=np.int64)
    Es = np.asarray(E, dtype=np.float32)[s]
    Eq = np.asarray(E, dtype=np.float32)[qi]
    ns = np.sqrt(np.sum(Es * Es, axis=1, dtype=np.float32), dtype=np.float32)
    nq = np.sqrt(np.sum(Eq * Eq, axis=1, dtype=np.float32), dtype=np.float32)
    dots = (Es @ Eq.T).astype(np.float32)
    den = (ns[:, None] * nq[None, :]).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        cos = np.where(den > 0, dots / den, np.float32(0.0)).astype(np.float32)
    bonus = np.isin(s, qi).astype(np.float32) * SUR_BONUS
    return (np.max(cos, axis=1) + bonus).astype(np.float32)


def unit_bounds(starts: Sequence[int], S: int) -> List[Tuple[int, int]]:
    """[(a, b)] of each unit from the sorted starts (first 0) and suffix length S."""
    st = [int(x) for x in starts]
    if not st or st[0] != 0 or any(b <= a for a, b in zip(st, st[1:])) or st[-1] >= S:
        raise ValueError("unit starts must be strictly increasing from 0 and below S")
    return list(zip(st, st[1:] + [S]))


def unit_scores(r: np.ndarray, starts: Sequence[int]) -> np.ndarray:
    """Appendix 7.3: each unit scores the mean of its four largest token
    scores, or of all of them when it has fewer than four (float32)."""
    r = np.asarray(r, dtype=np.float32)
    out = []
    for a, b in unit_bounds(starts, len(r)):
        top = np.sort(r[a:b])[::-1][:4]
        out.append(np.float32(np.sum(top, dtype=np.float32) / np.float32(len(top))))
    return np.array(out, dtype=np.float32)


def rank_units(scores: np.ndarray, starts: Sequence[int]) -> List[int]:
    """Units by score, highest first; the earlier unit wins a tie."""
    return sorted(range(len(scores)), key=lambda u: (-float(scores[u]), int(starts[u])))


def envelope(r_unit: np.ndarray) -> np.ndarray:
    """Eq. 8 over one unit's tokens in order: u_0 = 0,
    u_t = max(e^(r_t - r_max), e^(-1/16) u_{t-1}), r_max the unit's maximum
    (float32)."""
    r_unit = np.asarray(r_unit, dtype=np.float32)
    rmax = np.max(r_unit)
    u = np.empty(len(r_unit), dtype=np.float32)
    prev = np.float32(0.0)
    for t in range(len(r_unit)):
        prev = max(np.float32(np.exp(r_unit[t] - rmax)), np.float32(ENVELOPE_DECAY * prev))
        u[t] = prev
    return u


def best_window(u: np.ndarray, w: int) -> int:
    """Start of the width-w window with the largest sum of u, the earliest
    maximiser on ties (float32 sums, accumulated left to right)."""
    best, best_s = -1, None
    for a in range(len(u) - w + 1):
        s = np.float32(0.0)
        for x in u[a:a + w]:
            s = np.float32(s + x)
        if best_s is None or s > best_s:
            best, best_s = a, s
    return best


def select(r: np.ndarray, starts: Sequence[int], B: int, pos0: int = 0) -> np.ndarray:
    """The selection part of Algorithm 1 (section 7.3): rank units, admit
    whole units in ranked order while they fit the remaining allowance
    w = B - |A|; the first unit that does not fit contributes its best
    width-w envelope window, which fills the allowance exactly; the chosen
    suffix indices are sorted.  Returns global positions pos0 + i (int32,
    ascending)."""
    r = np.asarray(r, dtype=np.float32)
    S = len(r)
    if not 0 <= B <= S:
        raise ValueError("budget outside [0, S]")
    bounds = unit_bounds(starts, S)
    order = rank_units(unit_scores(r, starts), starts)
    chosen: List[int] = []
    for u in order:
        w = B - len(chosen)
        if w == 0:
            break
        a, b = bounds[u]
        if b - a <= w:
            chosen.extend(range(a, b))
        else:
            s0 = best_window(envelope(r[a:b]), w)
            chosen.extend(range(a + s0, a + s0 + w))
    return (pos0 + np.sort(np.array(chosen, dtype=np.int64))).astype(np.int32)
