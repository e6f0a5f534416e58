"""Integer side of the oracle: blocks, the seam set T_tau, execution
intervals, the exact budget, support checks and the attention tile plan.

TEST INFRASTRUCTURE (see the package docstring).
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np


class BadBlocks(ValueError):
    pass


class BadSupport(ValueError):
    pass


def validate_blocks(s: Sequence[int], e: Sequence[int], n_tokens: int) -> None:
    """The blocks must tile [0, N) exactly (cross-attention reuse page, 6.1:
    the sequence is the concatenation B_1 + ... + B_m of half-open spans
    x[s_i:e_i)).  Empty blocks, gaps, overlaps and a wrong total are errors."""
    m = len(s)
    if m < 1 or len(e) != m:
        raise BadBlocks("need m >= 1 blocks with one start and one end each")
    if s[0] != 0 or e[m - 1] != n_tokens:
        raise BadBlocks("blocks must start at 0 and end at N")
    for i in range(m):
        if not s[i] < e[i]:
            raise BadBlocks(f"block {i} is empty")
        if i + 1 < m and e[i] != s[i + 1]:
            raise BadBlocks(f"blocks {i} and {i + 1} are not adjacent")


def seam_set(s: Sequence[int], e: Sequence[int], tau: int, asymmetric: bool = True,
             n_tokens: int | None = None) -> np.ndarray:
    """Recomputation set T_tau (cross-attention reuse page, 6.3).

    The window at seam B_i | B_{i+1} is the last tau positions of B_i and the
    first tau positions of B_{i+1}, each intersected with its own block.
    The asymmetric true-prefix rule drops B_1's trailing window at seam
    B_1 | B_2 and adds the trailing tau positions of B_m instead.  T is the
    set union of all windows, returned ascending (a set; sorted as in
    Budgeted KV-Cache Repair, section 3.2).  m = 1 or tau = 0 gives the
    empty set.
    """
    m = len(s)
    validate_blocks(s, e, n_tokens if n_tokens is not None else (e[-1] if m else 0))
    if tau < 0:
        raise ValueError("tau must be >= 0")
    chosen = set()
    for i in range(m - 1):                      # seam between block i and i+1 (0-based)
        if not (asymmetric and i == 0):
            chosen.update(range(max(s[i], e[i] - tau), e[i]))
        chosen.update(range(s[i + 1], min(e[i + 1], s[i + 1] + tau)))
    if asymmetric and m >= 2:
        chosen.update(range(max(s[m - 1], e[m - 1] - tau), e[m - 1]))
    return np.array(sorted(chosen), dtype=np.int64)


def runs(T: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Maximal runs of consecutive positions of a sorted set (the execution
    intervals of Budgeted KV-Cache Repair, section 3.2 / Algorithm 1:
    "sort and coalesce").  Returns (start, length) arrays."""
    starts: List[int] = []
    lens: List[int] = []
    for t in T:
        t = int(t)
        if starts and t == starts[-1] + lens[-1]:
            lens[-1] += 1
        else:
            starts.append(t)
            lens.append(1)
    return np.array(starts, dtype=np.int64), np.array(lens, dtype=np.int64)


def budget(S: int, b) -> int:
    """Exact allowance B(S, b) = min{S, ceil(S*b/100)} (Budgeted KV-Cache
    Repair, section 7.1, Eq. 3), evaluated in exact rational arithmetic."""
    b = Fraction(str(b)) if isinstance(b, float) else Fraction(b)
    if not 0 <= b <= 100:
        raise ValueError("0 <= b <= 100")
    return min(S, math.ceil(Fraction(S) * b / 100))


def check_support(T: Sequence[int], n_tokens: int, first_selectable: int, B: int) -> None:
    """A support is executable when it is strictly increasing (hence unique),
    lies in [first_selectable, N) (only retained-suffix positions are
    selectable, section 7.1) and holds exactly B positions."""
    T = list(map(int, T))
    if len(T) != B:
        raise BadSupport(f"support has {len(T)} positions, expected {B}")
    for k, t in enumerate(T):
        if not max(first_selectable, 0) <= t < n_tokens:     # a position is a cache row
            raise BadSupport(f"position {t} outside [{first_selectable}, {n_tokens})")
        if k and T[k - 1] >= t:
            raise BadSupport("support is not strictly increasing")


def kv_tile_first_query(T: Sequence[int], n_tokens: int, kv_tile: int) -> np.ndarray:
    """Key-tile-major view of the plan: for each key tile c (keys
    [c*W, (c+1)*W) of an n_tokens cache), the index of the first packed row r
    whose position T[r] is at or after the tile's first key -- the first
    query of a sorted support that sees any key of the tile (every later row
    sees it too) -- or len(T) when no row reaches the tile.

    This is the inverse of the query-tile plan of Budgeted KV-Cache Repair,
    section 13.2 (Eq. 24): a query tile touches key tile c exactly when its
    last row index is at or past first[c].  The index is a left insertion
    point of c*W into the sorted support (a library search serves as the
    step).
    """
    T = np.asarray(T, dtype=np.int64)
    n_kv = -(-int(n_tokens) // kv_tile)
    return np.searchsorted(T, np.arange(n_kv, dtype=np.int64) * kv_tile, side="left").astype(np.int64)


def attn_tile_plan(T: Sequence[int], group: int, rows_per_tile: int,
                   kv_tile: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-query-tile key-tile counts (Budgeted KV-Cache Repair, section 13.2,
    Eq. 23-24): with u_min, u_max the first and last selected positions of a
    query tile, n_full = floor((u_min+1)/W) tiles are visible to every row
    and n_total = ceil((u_max+1)/W) tiles are touched at all.

    Query tiles here run over (packed row, query head of one KV group) pairs:
    pair p = r*group + h, and tile t holds pairs [t*rows_per_tile,
    min(B*group, (t+1)*rows_per_tile)).
    """
    B = len(T)
    P = B * group
    nt = (P + rows_per_tile - 1) // rows_per_tile
    n_full = np.zeros(nt, dtype=np.int64)
    n_total = np.zeros(nt, dtype=np.int64)
    for t in range(nt):
        p0 = t * rows_per_tile
        p1 = min(P, p0 + rows_per_tile) - 1
        u_min = int(T[p0 // group])
        u_max = int(T[p1 // group])
        n_full[t] = (u_min + 1) // kv_tile
        n_total[t] = -(-(u_max + 1) // kv_tile)
    return n_full, n_total


def initial_meta(s: Sequence[int], e: Sequence[int], n_tokens: int) -> Tuple[np.ndarray, np.ndarray]:
    """Load-time metadata of the mixed cache (cross-attention reuse page,
    6.2, and the sink term of F in 6.4): the first block B_1 was encoded as
    a true prefix, so its positions are global; every position of a later
    block was encoded locally, so its type is local; the spurious-sink set
    S' is the first position s_i of every block after the first (each such
    block began its own local encoding there).  Returns (flags uint8 [N],
    block id int32 [N]) with flags bit 0 = local, bit 1 = spurious sink and
    block ids counted from 0."""
    validate_blocks(s, e, n_tokens)
    flags = np.zeros(n_tokens, dtype=np.uint8)
    block = np.zeros(n_tokens, dtype=np.int32)
    for i in range(len(s)):
        for t in range(int(s[i]), int(e[i])):
            block[t] = i
            if i >= 1:
                flags[t] |= 1            # local: not part of the true prefix
        if i >= 1:
            flags[int(s[i])] |= 2        # spurious sink: head of a local block
    return flags, block


def check_positions(gpos: Sequence[int], n_tokens: int) -> None:
    """A global-position map g_t (cross-attention reuse page, 6.2) is usable
    when it has one entry per cache row, is non-negative and strictly
    increasing: causal visibility by position (g_j <= g_u) is then a prefix
    of the rows."""
    g = list(map(int, gpos))
    if len(g) != n_tokens:
        raise ValueError(f"position map has {len(g)} entries, expected {n_tokens}")
    for t, x in enumerate(g):
        if x < 0 or (t and g[t - 1] >= x):
            raise ValueError("position map is not non-negative and strictly increasing")
