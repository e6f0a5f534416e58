"""GPU parity of the Semantic-Unit Refresh numeric core (kvr_sur_scores,
kvr_sur_select) against the oracle.

Token scores: float32 on both sides, different summation order, compared
within 2e-5 absolute (cosines lie in [-1, 1]).  Unit scores: bit-exact
given the same token scores (same float32 operations in the same order).
Selection: given the GPU's token scores, T and its runs equal the oracle's
bit for bit, except where two windows of the cut unit tie to within the
envelope's exponential rounding; then the GPU's window must be one of the
near-best ones (several answers are valid)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle import sur
from tests.gpu_harness import kvr, log

pytestmark = pytest.mark.gpu

SCORE_TOL = 2e-5


def _table(w):
    E = wl.embedding_table(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return E, torch.from_numpy(E).to(tdt).cuda()


def _gpu_scores(m, w, dE, s, q):
    r = torch.full((len(s),), float("nan"), dtype=torch.float32, device="cuda")
    m.kvr_sur_scores(dE, m.KVR_BF16 if w.dtype == "bf16" else m.KVR_F32,
                     torch.from_numpy(s).cuda(), torch.from_numpy(q).cuda(), r)
    torch.cuda.synchronize()
    return r


def _gpu_select(m, r, starts, B, pos0):
    S = r.numel()
    U = len(starts)
    us = torch.from_numpy(np.asarray(starts, dtype=np.int32)).cuda()
    uscore = torch.empty(U, dtype=torch.float32, device="cuda")
    cap = max(B, 1)
    T = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
    rs = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
    rl = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
    counts = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(2 * S, dtype=torch.float32, device="cuda")
    n, R, st = m.kvr_sur_select(r, us, B, pos0, uscore, T, rs, rl, counts, ws)
    return (T[:n].cpu().numpy(), rs[:R].cpu().numpy(), rl[:R].cpu().numpy(),
            uscore.cpu().numpy())


def _check_select(r_np, starts, B, pos0, T, rs, rl, uscore):
    assert np.array_equal(uscore, sur.unit_scores(r_np, starts))
    want = sur.select(r_np, starts, B, pos0)
    if not np.array_equal(T, want):
        # only the cut unit's window may differ, and only between near-equal windows
        assert len(T) == len(want) == B and np.all(np.diff(T) > 0)
        bounds = sur.unit_bounds(starts, len(r_np))
        order = sur.rank_units(sur.unit_scores(r_np, starts), starts)
        diff = set(T.tolist()) ^ set(want.tolist())
        units = {next(u for u, (a, b) in enumerate(bounds) if a <= i - pos0 < b) for i in diff}
        assert len(units) == 1
        u = units.pop()
        a, b = bounds[u]
        # the GPU's positions in the cut unit must be one contiguous window
        # of the oracle's width, which starts at the GPU's first position
        g_pos = sorted(int(x) - pos0 - a for x in T if a <= x - pos0 < b)
        w_pos = sorted(int(x) - pos0 - a for x in want if a <= x - pos0 < b)
        wlen = len(w_pos)
        assert wlen > 0 and w_pos == list(range(w_pos[0], w_pos[0] + wlen))
        assert g_pos == list(range(g_pos[0], g_pos[0] + wlen)), "GPU window not contiguous"
        assert 0 <= g_pos[0] and g_pos[-1] < b - a
        env = sur.envelope(r_np[a:b])
        g0, w0 = g_pos[0], w_pos[0]
        sg, so = float(np.sum(env[g0:g0 + wlen])), float(np.sum(env[w0:w0 + wlen]))
        log(f"  window tie in unit {u}: gpu start {g0} sum {sg:.8g}, oracle start {w0} sum {so:.8g}")
        assert abs(sg - so) <= 1e-5 * max(1.0, abs(so))
        want = np.asarray(T)
    starts_o, lens_o = oracle.runs(want)
    assert np.array_equal(rs, starts_o) and np.array_equal(rl, lens_o)


def test_sur_scores_tiny_f32_and_select():
    m = kvr()
    w = wl.SUR_TINY
    E, dE = _table(w)
    s, q, starts = wl.sur_ids(w)
    log(f"[sur] {w.name}: S={len(s)} Q={len(q)} units={len(starts)}")
    r = _gpu_scores(m, w, dE, s, q)
    ref = sur.token_scores(E, s, q)
    err = float(np.max(np.abs(r.cpu().numpy() - ref)))
    log(f"  scores max|d|={err:.2e}")
    assert err <= SCORE_TOL
    r_np = r.cpu().numpy()
    for B in (0, 1, wl.sur_budget(w), len(s) // 2, len(s)):
        T, rs, rl, us = _gpu_select(m, r, starts, B, w.pos0)
        _check_select(r_np, starts, B, w.pos0, T, rs, rl, us)


# (Q, hidden, S): hidden a multiple of 256 with Q <= 128 takes the
# query-stationary kernel (16-query blocks 1, 2, 3, 4, 6, 8; ragged last
# workgroup of 64 tokens); other hidden sizes and Q > 128 take the general
# kernel (32-query blocks).
@pytest.mark.parametrize("Q,hidden,S", [
    (1, 1024, 1000), (17, 1024, 1000), (48, 1024, 1000), (64, 1024, 1000), (65, 512, 777),
    (96, 256, 64), (128, 1024, 1000), (5, 256, 5),
    (129, 1024, 1000), (200, 1024, 1000), (48, 320, 1000),
])
def test_sur_scores_bf16_query_blocks(Q, hidden, S):
    m = kvr()
    w = wl.SurWorkload(f"sur-bf16-q{Q}-h{hidden}-s{S}", 42, vocab=5000, hidden=hidden, n_suffix=S,
                       n_query=Q, budget_percent=5.0)
    E, dE = _table(w)
    s, q, _ = wl.sur_ids(w)
    r = _gpu_scores(m, w, dE, s, q)
    ref = sur.token_scores(E, s, q)
    err = float(np.max(np.abs(r.cpu().numpy() - ref)))
    log(f"[sur] Q={Q}: scores max|d|={err:.2e}, bonus tokens {int(np.sum(np.isin(s, q)))}")
    assert err <= SCORE_TOL


@pytest.mark.parametrize("hidden", [64, 256])
def test_sur_scores_bad_ids_are_nan(hidden):
    m = kvr()
    w = wl.SurWorkload(f"sur-bad-ids-h{hidden}", 43, vocab=200, hidden=hidden, n_suffix=130,
                       n_query=3, budget_percent=5.0)
    E, dE = _table(w)
    s, q, _ = wl.sur_ids(w)
    s = s.copy()
    s[[0, 77, 129]] = [-1, 200, 10 ** 6]
    r = _gpu_scores(m, w, dE, s, q).cpu().numpy()
    assert np.isnan(r[[0, 77, 129]]).all()
    ok = np.ones(len(s), bool)
    ok[[0, 77, 129]] = False
    ref = sur.token_scores(E, s[ok], q)
    assert np.max(np.abs(r[ok] - ref)) <= SCORE_TOL


def test_sur_select_random_partitions_and_ties():
    m = kvr()
    rng = np.random.default_rng(7)
    for trial in range(12):
        S = int(rng.integers(50, 3000))
        # quantised scores create many exact ties between units and tokens
        r_np = (np.round(rng.standard_normal(S) * 4) / 4).astype(np.float32)
        k = int(rng.integers(1, max(2, S // 10)))
        starts = [0] + sorted(rng.choice(np.arange(1, S), size=min(k, S - 1), replace=False).tolist())
        B = int(rng.integers(0, S + 1))
        pos0 = int(rng.integers(0, 5000))
        T, rs, rl, us = _gpu_select(m, torch.from_numpy(r_np).cuda(), starts, B, pos0)
        _check_select(r_np, starts, B, pos0, T, rs, rl, us)


@pytest.mark.parametrize("S,n_units,B", [(20000, 1500, 900), (40000, 5000, 23457), (3000, 1024, 1500),
                                         (3000, 1025, 1499)])
def test_sur_select_many_units(S, n_units, B):
    """Above 1024 units the ranking is a bitonic sort and T is written per
    unit; at or below, ranking by counting and T by binary search."""
    m = kvr()
    rng = np.random.default_rng(S + n_units)
    r_np = (np.round(rng.standard_normal(S) * 8) / 8).astype(np.float32)
    starts = [0] + sorted(rng.choice(np.arange(1, S), size=n_units - 1, replace=False).tolist())
    T, rs, rl, us = _gpu_select(m, torch.from_numpy(r_np).cuda(), starts, B, 11)
    _check_select(r_np, starts, B, 11, T, rs, rl, us)


def test_sur_select_rejects_bad_units():
    m = kvr()
    r = torch.zeros(50, dtype=torch.float32, device="cuda")
    with pytest.raises(m.KvrError):
        _gpu_select(m, r, [0, 10, 10, 20], 5, 0)
    with pytest.raises(m.KvrError):
        _gpu_select(m, r, [3, 10], 5, 0)


@pytest.mark.timeout(600)
def test_sur_qwen7_16k_end_to_end():
    """Full-size vocabulary and suffix: GPU scores against the oracle on a
    sample of 2048 tokens, and the selection against the oracle on the
    GPU's scores."""
    m = kvr()
    w = wl.SUR_QWEN7_16K
    E, dE = _table(w)
    s, q, starts = wl.sur_ids(w)
    log(f"[sur] {w.name}: vocab={w.vocab} S={len(s)} Q={len(q)} units={len(starts)}")
    r = _gpu_scores(m, w, dE, s, q)
    r_np = r.cpu().numpy()
    idx = np.random.default_rng(0).choice(len(s), size=2048, replace=False)
    ref = sur.token_scores(E, s[idx], q)
    err = float(np.max(np.abs(r_np[idx] - ref)))
    log(f"  sampled scores max|d|={err:.2e}")
    assert err <= SCORE_TOL
    B = wl.sur_budget(w)
    T, rs, rl, us = _gpu_select(m, r, starts, B, w.pos0)
    _check_select(r_np, starts, B, w.pos0, T, rs, rl, us)
