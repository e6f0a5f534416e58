"""Pins of the oracle's load-time metadata and global-position rules, and of
the input generators that reproduce them, against what the pages fix:
hand-derived metadata (tests/golden/initial_meta.txt), the page's example
block B_1 = [0, 384), closed-form counts over random partitions, and the
exact budget of Eq. 3 over a sweep."""
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "initial_meta.txt")


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, ends, flags, bids = [c.strip() for c in line.split("|")]
            e = [int(v) for v in ends.split()]
            s = [0] + e[:-1]
            cases.append((name, s, e, [int(v) for v in flags.split()],
                          [int(v) for v in bids.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_initial_meta_golden(case):
    name, s, e, flags, bids = case
    f, b = oracle.initial_meta(s, e, e[-1])
    assert f.tolist() == flags
    assert b.tolist() == bids


def test_initial_meta_page_example_block():
    # the page's example first block s_1 = 0, e_1 = 384 covers 0..383: all
    # global; the next block starts locally with a sink at 384
    f, b = oracle.initial_meta([0, 384], [384, 512], 512)
    assert np.all(f[:384] == 0) and f[384] == 3 and np.all(f[385:] == 1)
    assert np.all(b[:384] == 0) and np.all(b[384:] == 1)


def test_initial_meta_counts_random_partitions():
    rng = np.random.default_rng(31)
    for _ in range(300):
        N = int(rng.integers(1, 400))
        m = int(rng.integers(1, N + 1))
        s, e = wl.random_partition(rng, N, m)
        f, b = oracle.initial_meta(s, e, N)
        assert int(np.count_nonzero(f & 2)) == m - 1           # one sink per later block
        assert int(np.count_nonzero(f & 1)) == N - int(e[0])   # everything after B_1 is local
        assert np.all(f[: e[0]] == 0)
        assert np.all((f & 2) <= 2 * (f & 1))                  # a sink is always local
        assert np.array_equal(np.flatnonzero(np.diff(b)) + 1, s[1:])
        assert b[0] == 0 and b[-1] == m - 1


def test_initial_meta_rejects_bad_blocks():
    with pytest.raises(oracle.BadBlocks):
        oracle.initial_meta([0, 4], [4, 7], 8)


def test_generators_reproduce_the_oracle_metadata():
    """The seeded generators hand the load-time flags to both sides as an
    input; they must be the oracle's."""
    rng = np.random.default_rng(32)
    for w in (wl.TINY, wl.QWEN15_LAYER, wl.QWEN7_LAYER_SEAMS, wl.QWEN7_STACK_ISOLATED,
              wl.QWEN15_STACK_DEGENERATE, wl.QWEN7_DECODE_32K):
        s, e = wl.blocks(w)
        f, b = oracle.initial_meta(s, e, w.n_tokens)
        assert np.array_equal(wl.initial_flags(w), f)
        assert np.array_equal(wl.block_ids(w), b)
    for _ in range(100):
        N = int(rng.integers(2, 3000))
        m = int(rng.integers(1, min(N, 200) + 1))
        s, e = wl.random_partition(rng, N, m)
        f, _ = oracle.initial_meta(s, e, N)
        assert np.array_equal(wl.initial_flags(wl.TINY.with_(n_tokens=N), s, e), f)


def test_generator_budget_is_eq3_over_a_sweep():
    for b in (0.5, 1.0, 2.0, 2.5, 3.0, 5.0, 12.5, 33.3, 50.0, 100.0):
        for S in list(range(0, 600)) + [4095, 16128, 16384, 32256, 100003]:
            assert wl.budget_count(S, b) == oracle.budget(S, b), (S, b)


def test_check_positions():
    oracle.check_positions([0, 1, 5, 9], 4)
    for g in ([0, 1, 1, 2], [3, 2, 4, 5], [-1, 0, 1, 2], [0, 1, 2]):
        with pytest.raises(ValueError):
            oracle.check_positions(g, 4)
