"""The seeded workloads reproduce the sizes the pages and the stated
configurations fix."""
import numpy as np

import oracle
import workloads as wl


def test_table18_supports_match_the_stated_pair_counts():
    # Budgeted KV-Cache Repair, section 13.3: B = 64, R = 1/4/16, and the
    # causal pair count sum(u+1): 65568 for the 2K cache, 262176 for the 8K one.
    for w in wl.TABLE18:
        T = wl.explicit_support(w)
        assert len(T) == 64
        st, ln = oracle.runs(T)
        assert len(st) == w.n_intervals and np.all(ln == 64 // w.n_intervals)
        want = {2048: 65568, 8192: 262176}[w.n_tokens]
        assert int(np.sum(T.astype(np.int64) + 1)) == want


def test_equal_budget_supports_of_the_7b_layer():
    s, e = wl.blocks(wl.QWEN7_LAYER_SEAMS)
    seams = oracle.seam_set(s, e, 6, True)
    contig = wl.explicit_support(wl.QWEN7_LAYER_CONTIG)
    matched = wl.explicit_support(wl.QWEN7_LAYER_MATCHED)
    assert len(seams) == len(contig) == len(matched) == 756
    assert contig[0] == e[0]
    pairs = lambda T: int(np.sum(np.asarray(T, np.int64) + 1))
    assert pairs(matched) == pairs(seams) == 6290298


def test_generation_is_deterministic_and_thread_independent():
    w = wl.QWEN15_LAYER
    a = wl.normal(w, 3, wl.T_WQ, (1 << 23) + 5, 0.02, threads=1)
    b = wl.normal(w, 3, wl.T_WQ, (1 << 23) + 5, 0.02, threads=7)
    assert np.array_equal(a, b)
    assert np.array_equal(wl.bf16_round(a), a)          # bf16-representable
    assert abs(float(np.std(a)) - 0.02) < 1e-3


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], dtype=np.float32)
    r = wl.bf16_round(x)
    assert r.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5]
