"""Pins of the oracle's integer side against what the pages fix: hand-derived
seam sets, closed forms, the degeneration coverage statement, an independent
per-position reading of the seam rule, the page's budget examples and
brute-force counting for the tile plan."""
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "seam_sets.txt")


def _parse_ranges(txt):
    if txt.strip() == "-":
        return []
    out = []
    for tok in txt.split():
        a, b = tok.split("-")
        out.extend(range(int(a), int(b) + 1))
    return out


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, ends, tau, mode, T, runs = [c.strip() for c in line.split("|")]
            e = [int(v) for v in ends.split()]
            s = [0] + e[:-1]
            rs = [] if runs == "-" else [tuple(map(int, r.split(":"))) for r in runs.split()]
            cases.append((name, s, e, int(tau), mode == "asym", _parse_ranges(T), rs))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_seam_set_golden(case):
    name, s, e, tau, asym, T, rs = case
    got = oracle.seam_set(s, e, tau, asymmetric=asym)
    assert got.tolist() == T
    st, ln = oracle.runs(got)
    assert list(zip(st.tolist(), ln.tolist())) == rs


def _member(t, s, e, tau, asym):
    """Independent per-position reading of the seam rule: position t, at
    offset o inside block i of length L, is recomputed when it is one of the
    first tau tokens of a non-first block, one of the last tau tokens of a
    block that has a right neighbour (except B_1 under the asymmetric rule),
    or, under the asymmetric rule, one of the last tau tokens of B_m."""
    m = len(s)
    i = next(k for k in range(m) if s[k] <= t < e[k])
    o = t - s[i]
    L = e[i] - s[i]
    lead = i >= 1 and o < tau
    trail_seam = i < m - 1 and not (asym and i == 0) and o >= L - tau
    trail_last = asym and m >= 2 and i == m - 1 and o >= L - tau
    return lead or trail_seam or trail_last


def test_seam_set_per_position_reading_random_partitions():
    rng = np.random.default_rng(7)
    n_cases = 0
    for m in range(1, 6):
        for _ in range(60):
            sizes = rng.integers(1, 13, size=m)
            e = np.cumsum(sizes).tolist()
            s = [0] + e[:-1]
            for tau in range(0, 9):
                for asym in (True, False):
                    want = [t for t in range(e[-1]) if _member(t, s, e, tau, asym)]
                    assert oracle.seam_set(s, e, tau, asym).tolist() == want
                    n_cases += 1
    assert n_cases > 4000


@pytest.mark.parametrize("w", [wl.TINY, wl.QWEN15_LAYER, wl.QWEN7_LAYER_SEAMS],
                         ids=lambda w: w.name)
def test_seam_set_closed_form_count(w):
    # Uniform blocks with tau <= |B|/2: every seam contributes 2*tau, the
    # asymmetric rule moves tau from B_1 to B_m: |T| = 2*tau*(m-1).
    s, e = wl.blocks(w)
    T = oracle.seam_set(s, e, w.tau, True)
    assert len(T) == 2 * w.tau * (len(s) - 1)
    assert {wl.TINY.name: 24, wl.QWEN15_LAYER.name: 240,
            wl.QWEN7_LAYER_SEAMS.name: 756}[w.name] == len(T)
    # recompute ratio |T|/N near the 5% engineering target (4.7%, 5.9%, 4.6%)
    assert 0.04 <= len(T) / w.n_tokens <= 0.06


def test_seam_set_7b_runs_layout():
    s, e = wl.blocks(wl.QWEN7_LAYER_SEAMS)
    st, ln = oracle.runs(oracle.seam_set(s, e, 6, True))
    assert len(st) == 64
    assert ln[0] == 6 and ln[-1] == 6 and all(ln[1:-1] == 12)
    assert st[0] == 256 and st[-1] == 16384 - 6


@pytest.mark.parametrize("block,tau", [(256, 128), (256, 200), (16, 8), (10, 5), (7, 4)])
def test_seam_set_degeneration_covers_suffix(block, tau):
    # tau >= |B|/2 with asymmetric coverage covers all of B_2..B_m (6.4 degeneration)
    N = block * 9
    s = list(range(0, N, block))
    e = s[1:] + [N]
    T = oracle.seam_set(s, e, tau, True)
    assert T.tolist() == list(range(block, N))


def test_degenerate_config_support():
    w = wl.QWEN15_STACK_DEGENERATE
    s, e = wl.blocks(w)
    T = oracle.seam_set(s, e, w.tau, True)
    assert T[0] == 256 and T[-1] == 16383 and len(T) == 16128


@pytest.mark.parametrize("s,e,N", [([0], [0], 0), ([1, 4], [4, 8], 8), ([0, 4], [4, 7], 8),
                                   ([0, 3], [4, 8], 8), ([0, 4], [3, 8], 8), ([], [], 0)])
def test_validate_blocks_errors(s, e, N):
    with pytest.raises(oracle.BadBlocks):
        oracle.validate_blocks(s, e, N)


def test_runs_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(300):
        N = int(rng.integers(1, 60))
        T = np.flatnonzero(rng.random(N) < rng.random())
        st, ln = oracle.runs(T)
        # rebuild membership from runs; check maximality
        rebuilt = [a + k for a, l in zip(st, ln) for k in range(l)]
        assert rebuilt == T.tolist()
        for a, l in zip(st, ln):
            assert a - 1 not in set(T.tolist()) and a + l not in set(T.tolist())


def test_budget_page_examples():
    # section 13.1: a 10,000-token suffix at 2-5% refreshes 200-500 positions
    assert oracle.budget(10000, 2) == 200
    assert oracle.budget(10000, 5) == 500
    # ceiling, cap at S, endpoints (Eq. 3)
    assert oracle.budget(32256, 2) == 646      # 645.12 -> 646
    assert oracle.budget(101, 1) == 2
    assert oracle.budget(7, 100) == 7
    assert oracle.budget(7, 0) == 0
    assert oracle.budget(3, 40) == 2
    with pytest.raises(ValueError):
        oracle.budget(10, 101)


def test_isolated_support_is_budgeted_and_non_adjacent():
    w = wl.QWEN7_STACK_ISOLATED
    T = wl.isolated_support(w)
    S = w.n_tokens - w.block_size
    assert len(T) == oracle.budget(S, 2) == 646
    oracle.check_support(T, w.n_tokens, w.block_size, 646)
    assert np.all(np.diff(T) >= 2)
    st, ln = oracle.runs(T)
    assert len(st) == 646 and np.all(ln == 1)


@pytest.mark.parametrize("T,first,B", [([5, 5, 6], 0, 3), ([6, 5], 0, 2), ([2, 9], 3, 2),
                                        ([3, 10], 3, 2), ([3, 4], 3, 3), ([-1, 2], -5, 2)])
def test_check_support_errors(T, first, B):
    with pytest.raises(oracle.BadSupport):
        oracle.check_support(T, 10, first, B)


def test_check_support_ok():
    oracle.check_support([3, 4, 9], 10, 3, 3)
    oracle.check_support([], 10, 3, 0)


def test_tile_plan_brute_force_counting():
    rng = np.random.default_rng(11)
    for _ in range(200):
        N = int(rng.integers(1, 700))
        B = int(rng.integers(1, min(N, 90) + 1))
        T = np.sort(rng.choice(N, size=B, replace=False))
        G = int(rng.integers(1, 8))
        rows = int(rng.choice([16, 32, 128]))
        W = int(rng.choice([16, 64]))
        n_full, n_total = oracle.attn_tile_plan(T, G, rows, W)
        P = B * G
        assert len(n_full) == -(-P // rows)
        for t in range(len(n_full)):
            us = [int(T[p // G]) for p in range(t * rows, min(P, (t + 1) * rows))]
            # tiles fully visible to every row / touched by some row, by counting
            full = sum(1 for c in range(N // W + 2) if (c + 1) * W - 1 <= min(us))
            touched = sum(1 for c in range(N // W + 2) if c * W <= max(us))
            assert n_full[t] == full and n_total[t] == touched


def test_kv_tile_first_query_brute_force_and_plan_inverse():
    """The key-tile map against a per-tile scan of the support, and against
    Eq. 24's n_total: query tile t touches key tile c iff its last row is at
    or past first[c]."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        N = int(rng.integers(1, 900))
        B = int(rng.integers(0, min(N, 120) + 1))
        T = np.sort(rng.choice(N, size=B, replace=False))
        W = int(rng.choice([16, 64]))
        first = oracle.kv_tile_first_query(T, N, W)
        assert len(first) == -(-N // W)
        for c in range(len(first)):
            scan = next((r for r in range(B) if T[r] >= c * W), B)
            assert first[c] == scan
        if B == 0:
            continue
        G = int(rng.integers(1, 8))
        rows = int(rng.choice([16, 32, 128]))
        _, n_total = oracle.attn_tile_plan(T, G, rows, W)
        for t in range(len(n_total)):
            last_row = (min(B * G, (t + 1) * rows) - 1) // G
            for c in range(len(first)):
                assert (c < n_total[t]) == (last_row >= first[c])


def test_kv_tile_first_query_edges():
    assert list(oracle.kv_tile_first_query([], 130, 64)) == [0, 0, 0]
    assert list(oracle.kv_tile_first_query([0, 63, 64, 200], 256, 64)) == [0, 2, 3, 3]
    assert list(oracle.kv_tile_first_query([5], 64, 64)) == [0]
