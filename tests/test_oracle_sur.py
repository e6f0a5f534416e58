"""Pins of the Semantic-Unit Refresh oracle (Budgeted KV-Cache Repair,
section 3.2 and Appendix 7.3, Eq. 1 / 7, Eq. 8, Algorithm 1).

Token scores are pinned to closed forms (a token scored against itself,
orthogonal and opposite directions, scale invariance, the identity bonus
depending on the id and not on the vector) and to pure-Python float64 brute
force; unit scores, ranking, the envelope recurrence, the window argmax and
the exact-budget fill to hand-worked cases and brute force.  A slip such as
dividing by one norm only, max over the wrong axis, a bonus keyed on the
embedding, a top-3 or top-5 mean, the later unit winning a tie, a growing
instead of decaying envelope, or the latest maximiser fails one of these."""
import math

import numpy as np
import pytest

import oracle
from oracle import sur


def test_token_scores_closed_forms():
    H = 8
    E = np.zeros((10, H), dtype=np.float32)
    E[0, 0] = 2.0              # query token 0
    E[1, 1] = 0.5              # query token 1
    E[2, 0] = 7.0              # same direction as token 0, other id
    E[3, 2] = 1.0              # orthogonal to both queries
    E[4, 0] = -3.0             # opposite to token 0, orthogonal to token 1
    E[4, 1] = -3.0
    E[5] = 0.0                 # zero row
    r = sur.token_scores(E, [0, 2, 3, 4, 5, 1], [0, 1])
    assert r.dtype == np.float32
    assert abs(r[0] - 1.25) < 1e-6                 # itself + identity bonus
    assert abs(r[1] - 1.0) < 1e-6                  # parallel, different id: no bonus
    assert abs(r[2]) < 1e-7                        # orthogonal
    assert abs(r[3] + 1 / math.sqrt(2)) < 1e-6     # max(-1/sqrt2, -1/sqrt2)
    E2 = E.copy()
    E2[4] = 0.0
    E2[4, 0] = -1.0
    assert abs(sur.token_scores(E2, [4], [0])[0] + 1.0) < 1e-6   # opposite: -1
    assert r[4] == 0.0                             # zero-norm row reads as cosine 0
    assert abs(r[5] - 1.25) < 1e-6


def test_token_scores_scale_invariance_and_brute_force():
    rng = np.random.default_rng(0)
    V, H = 40, 16
    E = rng.standard_normal((V, H)).astype(np.float32)
    s = rng.integers(0, V, size=30)
    q = rng.integers(0, V, size=5)
    r = sur.token_scores(E, s, q)
    scale = rng.uniform(0.1, 10.0, size=(V, 1)).astype(np.float32)
    assert np.allclose(sur.token_scores(E * scale, s, q), r, atol=2e-6)
    for i, si in enumerate(s):
        best = -2.0
        for qj in q:
            dot = math.fsum(float(E[si, k]) * float(E[qj, k]) for k in range(H))
            na = math.sqrt(math.fsum(float(E[si, k]) ** 2 for k in range(H)))
            nb = math.sqrt(math.fsum(float(E[qj, k]) ** 2 for k in range(H)))
            best = max(best, dot / (na * nb))
        best += 0.25 if si in set(q.tolist()) else 0.0
        assert abs(r[i] - best) < 2e-6


def test_unit_scores_top_four_mean():
    r = np.array([1, 5, 3, 2, 4, 2, 7, 0.5, 0.5, 0.5, 0.5, 9], dtype=np.float32)
    starts = [0, 5, 7, 11]
    got = sur.unit_scores(r, starts)
    assert got.tolist() == [3.5, 4.5, 0.5, 9.0]     # (5+4+3+2)/4, (2+7)/2, all 0.5, 9
    rng = np.random.default_rng(1)
    r = rng.standard_normal(200).astype(np.float32)
    starts = [0] + sorted(rng.choice(np.arange(1, 200), size=30, replace=False).tolist())
    b = starts[1:] + [200]
    want = [sum(sorted(r[a:z].tolist(), reverse=True)[:4]) / min(4, z - a) for a, z in zip(starts, b)]
    assert np.allclose(sur.unit_scores(r, starts), want, atol=1e-6)


def test_rank_ties_break_by_earlier_unit():
    assert sur.rank_units(np.array([1.0, 2.0, 2.0, 0.5], np.float32), [0, 3, 6, 9]) == [1, 2, 0, 3]


def test_envelope_recurrence():
    c = math.exp(-1 / 16)
    assert np.allclose(sur.envelope(np.zeros(5)), 1.0)            # flat: every token at the max
    r = np.array([-50, -50, 0, -50, -50, -50, -1], dtype=np.float32)
    u = sur.envelope(r)
    assert u[0] < 1e-20 and u[1] < 1e-20 and u[2] == 1.0
    assert np.allclose(u[3:6], [c, c * c, c ** 3], rtol=1e-6)     # decays after the peak
    assert np.isclose(u[6], max(math.exp(-1), c ** 4), rtol=1e-6)
    rng = np.random.default_rng(2)
    r = rng.standard_normal(64).astype(np.float32)
    u = sur.envelope(r)
    prev, mx = 0.0, float(np.max(r))
    for t in range(64):
        prev = max(math.exp(float(r[t]) - mx), c * prev)
        assert abs(u[t] - prev) <= 1e-6 * prev


def test_best_window_argmax_earliest():
    assert sur.best_window(np.ones(6, np.float32), 3) == 0
    u = np.array([0.1, 0.2, 0.9, 0.8, 0.1, 0.9, 0.8], np.float32)
    assert sur.best_window(u, 2) == 2            # (0.9+0.8) at 2 and at 5: earliest
    rng = np.random.default_rng(3)
    u = rng.random(40).astype(np.float32)
    for w in (1, 5, 17, 40):
        sums = [math.fsum(u[a:a + w].tolist()) for a in range(40 - w + 1)]
        assert sur.best_window(u, w) == int(np.argmax(sums))


def test_select_hand_worked():
    # units [0,3) [3,5) [5,9) [9,12); scores 3.0, 8.5, 4.0, 0.5
    r = np.array([3, 3, 3, 8, 9, 1, 2, 9, 4, 0.5, 0.5, 0.5], dtype=np.float32)
    starts = [0, 3, 5, 9]
    assert sur.unit_scores(r, starts).tolist() == [3.0, 8.5, 4.0, 0.5]
    # B = 2: unit 1 exactly
    assert sur.select(r, starts, 2).tolist() == [3, 4]
    # B = 5: unit 1, then unit 2 does not fit (4 > 3): its best width-3 window
    u = sur.envelope(r[5:9])
    s0 = sur.best_window(u, 3)
    assert s0 == 1                                   # [2, 9, 4] beats [1, 2, 9]
    assert sur.select(r, starts, 5).tolist() == [3, 4, 6, 7, 8]
    # B = 9: units 1, 2, 0 whole (2 + 4 + 3)
    assert sur.select(r, starts, 9, pos0=100).tolist() == [100, 101, 102, 103, 104, 105, 106, 107, 108]
    assert sur.select(r, starts, 0).tolist() == []
    assert sur.select(r, starts, 12).tolist() == list(range(12))


def test_select_invariants_random():
    rng = np.random.default_rng(4)
    for trial in range(20):
        S = int(rng.integers(20, 300))
        r = rng.standard_normal(S).astype(np.float32)
        k = int(rng.integers(1, max(2, S // 4)))
        starts = [0] + sorted(rng.choice(np.arange(1, S), size=min(k, S - 1), replace=False).tolist())
        B = int(rng.integers(0, S + 1))
        A = sur.select(r, starts, B, pos0=7)
        assert len(A) == B and np.all(np.diff(A) > 0) and (B == 0 or (A[0] >= 7 and A[-1] < 7 + S))
        # units inside A are a prefix of the ranking plus at most one partial unit
        bounds = sur.unit_bounds(starts, S)
        order = sur.rank_units(sur.unit_scores(r, starts), starts)
        sel = set((A - 7).tolist())
        full = [u for u in order if all(i in sel for i in range(*bounds[u]))]
        part = [u for u in order if u not in full and any(i in sel for i in range(*bounds[u]))]
        assert len(part) <= 1
        assert full == order[:len(full)]
        if part:
            assert order[len(full)] == part[0]
            a, b = bounds[part[0]]
            idx = sorted(i - a for i in sel if a <= i < b)
            assert idx == list(range(idx[0], idx[0] + len(idx)))       # one contiguous window


def test_select_rejects_bad_units_and_budget():
    r = np.zeros(10, np.float32)
    with pytest.raises(ValueError):
        sur.select(r, [1, 5], 3)
    with pytest.raises(ValueError):
        sur.select(r, [0, 5, 5], 3)
    with pytest.raises(ValueError):
        sur.select(r, [0, 5], 11)
