"""GPU parity of the integer side: T_tau, runs, load-time metadata, support
checks and the attention plan are bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_harness import build_seams_gpu, kvr, log

pytestmark = pytest.mark.gpu

SEAM_WORKLOADS = [wl.TINY, wl.QWEN15_LAYER, wl.QWEN7_LAYER_SEAMS, wl.QWEN7_STACK_ISOLATED.with_(tau=3),
                  wl.QWEN15_STACK_DEGENERATE]


@pytest.mark.parametrize("w", SEAM_WORKLOADS, ids=lambda w: w.name)
def test_seam_set_and_meta_match_oracle(w):
    log(f"[index] seam set {w.name} tau={w.tau}")
    T, (rs, rl), h, flags, bid = build_seams_gpu(w)
    s, e = wl.blocks(w)
    ref = oracle.seam_set(s, e, w.tau, True)
    st, ln = oracle.runs(ref)
    assert h[2] == 0 and h[0] == len(ref) and h[1] == len(st)
    assert np.array_equal(T.cpu().numpy(), ref)
    assert np.array_equal(rs, st) and np.array_equal(rl, ln)
    f_ref, b_ref = oracle.initial_meta(s, e, w.n_tokens)
    assert np.array_equal(flags.cpu().numpy(), f_ref)
    assert np.array_equal(bid.cpu().numpy(), b_ref)


def _run_build(s, e, N, tau, asym, cap=None):
    m = kvr()
    cap = N if cap is None else cap
    ds, de = torch.from_numpy(np.asarray(s, np.int32)).cuda(), torch.from_numpy(np.asarray(e, np.int32)).cuda()
    T = torch.empty(max(cap, 4), dtype=torch.int32, device="cuda")[:cap]
    rs = torch.empty(max(cap, 4), dtype=torch.int32, device="cuda")
    rl = torch.empty(max(cap, 4), dtype=torch.int32, device="cuda")
    counts = torch.empty(4, dtype=torch.int32, device="cuda")
    h = m.kvr_build_repair_set(ds, de, N, tau, m.KVR_SEAM_ASYMMETRIC if asym else 0, T, rs, rl,
                               counts)
    return h, T[:h[0]].cpu().numpy(), rs[:h[1]].cpu().numpy(), rl[:h[1]].cpu().numpy()


def test_seam_set_random_partitions():
    rng = np.random.default_rng(20)
    for it in range(60):
        N = int(rng.integers(1, 40000))
        m = int(rng.integers(1, min(N, 3000) + 1))
        s, e = wl.random_partition(rng, N, m)
        tau = int(rng.integers(0, 40))
        asym = bool(rng.integers(0, 2))
        if it % 20 == 0:
            log(f"[index] random partition it={it} N={N} m={m} tau={tau} asym={asym}")
        h, T, rs, rl = _run_build(s, e, N, tau, asym)
        ref = oracle.seam_set(s, e, tau, asym)
        st, ln = oracle.runs(ref)
        assert h == (len(ref), len(st), 0)
        assert np.array_equal(T, ref) and np.array_equal(rs, st) and np.array_equal(rl, ln)


def test_seam_set_edge_cases():
    # one block, tau 0, single-token blocks, every position its own block
    for s, e, N, tau in (([0], [10], 10, 3), ([0, 4], [4, 8], 8, 0),
                         (list(range(64)), list(range(1, 65)), 64, 1),
                         (list(range(2500)), list(range(1, 2501)), 2500, 2)):
        h, T, rs, rl = _run_build(s, e, N, tau, True)
        ref = oracle.seam_set(s, e, tau, True)
        assert np.array_equal(T, ref), (N, tau)
        assert h[1] == len(oracle.runs(ref)[0])


def test_bad_blocks_and_capacity():
    m = kvr()
    with pytest.raises(m.KvrError) as ei:
        _run_build([0, 5], [4, 8], 8, 1, True)              # gap
    assert ei.value.status == -3
    with pytest.raises(m.KvrError) as ei:
        _run_build([0, 4], [4, 7], 8, 1, True)              # does not reach N
    assert ei.value.status == -3
    with pytest.raises(m.KvrError) as ei:
        _run_build([0, 4, 4], [4, 4, 8], 8, 1, True)        # empty block
    assert ei.value.status == -3
    with pytest.raises(m.KvrError) as ei:
        _run_build([0, 4], [4, 8], 8, 2, True, cap=3)       # |T| = 4 > cap
    assert ei.value.status == -5


def test_check_support():
    m = kvr()
    res = torch.empty(4, dtype=torch.int32, device="cuda")
    ok = torch.tensor([3, 4, 9, 15], dtype=torch.int32, device="cuda")
    m.kvr_check_support(ok, 16, 3, res)
    m.kvr_check_support(ok[:0], 16, 3, res)
    for bad, first in (([3, 3, 9], 0), ([5, 4], 0), ([2, 9], 3), ([3, 16], 0)):
        with pytest.raises(m.KvrError) as ei:
            m.kvr_check_support(torch.tensor(bad, dtype=torch.int32, device="cuda"), 16, first, res)
        assert ei.value.status == -4
    big = torch.arange(5000, 40000, 3, dtype=torch.int32, device="cuda")
    m.kvr_check_support(big, 40000, 5000, res)


def test_plan_matches_oracle():
    m = kvr()
    rng = np.random.default_rng(21)
    for _ in range(40):
        N = int(rng.integers(1, 40000))
        B = int(rng.integers(1, min(N, 3000) + 1))
        T = np.sort(rng.choice(N, size=B, replace=False)).astype(np.int32)
        G = int(rng.choice([1, 2, 6, 7]))
        nt = -(-B * G // m.KVR_ATTN_QROWS)
        nf = torch.empty(nt, dtype=torch.int32, device="cuda")
        ntot = torch.empty(nt, dtype=torch.int32, device="cuda")
        m.kvr_build_plan(torch.from_numpy(T).cuda(), G, nf, ntot)
        rf, rt = oracle.attn_tile_plan(T, G, m.KVR_ATTN_QROWS, m.KVR_ATTN_KV_TILE)
        assert np.array_equal(nf.cpu().numpy(), rf) and np.array_equal(ntot.cpu().numpy(), rt)


def test_tile_map_matches_oracle():
    """The key-tile map of random, workload and edge supports, bit-exact."""
    m = kvr()
    rng = np.random.default_rng(22)
    cases = []
    for _ in range(30):
        N = int(rng.integers(1, 40000))
        B = int(rng.integers(1, min(N, 3000) + 1))
        cases.append((np.sort(rng.choice(N, size=B, replace=False)).astype(np.int32), N))
    for w in (wl.QWEN7_STACK_ISOLATED, wl.QWEN7_LAYER_MATCHED, *wl.TABLE18):
        cases.append((wl.explicit_support(w).astype(np.int32), w.n_tokens))
    cases += [(np.arange(0, 64, dtype=np.int32), 100),        # every row in the first tile
              (np.array([99], dtype=np.int32), 100),           # the last position only
              (np.zeros(0, dtype=np.int32), 130)]              # empty support
    for T, N in cases:
        n_kv = -(-N // m.KVR_ATTN_KV_TILE)
        out = torch.full((n_kv,), -7, dtype=torch.int32, device="cuda")
        m.kvr_build_tile_map(torch.from_numpy(T).cuda(), N, out)
        ref = oracle.kv_tile_first_query(T, N, m.KVR_ATTN_KV_TILE)
        assert np.array_equal(out.cpu().numpy(), ref), (len(T), N)


def test_seam_set_with_more_runs_than_the_lds_holds():
    """40,000 positions in blocks of 4 with tau = 1: about 10,000 runs, so the
    run lengths are fixed up from global memory instead of LDS."""
    N, blk = 40000, 4
    s = np.arange(0, N, blk, dtype=np.int32)
    e = (s + blk).astype(np.int32)
    for asym in (True, False):
        log(f"[index] many runs N={N} blocks of {blk} tau=1 asym={asym}")
        h, T, rs, rl = _run_build(s, e, N, 1, asym)
        ref = oracle.seam_set(s, e, 1, asym)
        st, ln = oracle.runs(ref)
        assert len(st) > 4096
        assert h == (len(ref), len(st), 0)
        assert np.array_equal(T, ref) and np.array_equal(rs, st) and np.array_equal(rl, ln)


def _runs_gpu(T, N, first, sync=True):
    m = kvr()
    B = len(T)
    dT = torch.from_numpy(np.asarray(T, np.int32)).cuda() if B else \
        torch.empty(0, dtype=torch.int32, device="cuda")
    cap = max(B, 4)
    rs = torch.full((cap,), -9, dtype=torch.int32, device="cuda")
    rl = torch.full((cap,), -9, dtype=torch.int32, device="cuda")
    counts = torch.full((4,), -9, dtype=torch.int32, device="cuda")
    h = m.kvr_build_runs(dT, N, first, rs, rl, counts, sync=sync)
    if not sync:
        torch.cuda.synchronize()
        h = tuple(counts[:3].cpu().tolist())
    return h, rs[:h[1]].cpu().numpy(), rl[:h[1]].cpu().numpy()


def _support_cases():
    cases = []
    for w in (wl.QWEN7_STACK_ISOLATED, wl.QWEN7_LAYER_CONTIG, wl.QWEN7_LAYER_MATCHED,
              *wl.TABLE18):
        s, e = wl.blocks(w)
        first = int(e[0]) if len(s) > 1 else 0      # the retained suffix starts after B_1
        cases.append((w.name, wl.explicit_support(w), w.n_tokens, first))
    rng = np.random.default_rng(22)
    # every third position: 11,667 runs of length 1 (global-memory run pass)
    cases.append(("every-third", np.arange(5000, 40000, 3), 40000, 5000))
    # pairs of neighbours every fifth position: 6,000 runs of length 2
    cases.append(("pairs", np.sort(np.concatenate([np.arange(0, 30000, 5),
                                                     np.arange(1, 30000, 5)])), 30000, 0))
    for i in range(20):
        N = int(rng.integers(1, 30000))
        B = int(rng.integers(0, min(N, 5000) + 1))
        T = np.sort(rng.choice(N, size=B, replace=False))
        cases.append((f"random-{i}", T, N, 0))
    cases.append(("empty", np.zeros(0, np.int64), 100, 0))
    cases.append(("all", np.arange(777), 777, 0))
    return cases


def test_build_runs_matches_oracle():
    for name, T, N, first in _support_cases():
        ref_s, ref_l = oracle.runs(T)
        oracle.check_support(T, N, first, len(T))
        for sync in (True, False):
            h, rs, rl = _runs_gpu(T, N, first, sync)
            assert h == (len(T), len(ref_s), 0), (name, h)
            assert np.array_equal(rs, ref_s) and np.array_equal(rl, ref_l), name
        if len(ref_s) > 4096:
            log(f"[index] build runs {name}: B={len(T)} R={len(ref_s)} (global-memory run pass)")


def test_build_runs_rejects_bad_supports():
    m = kvr()
    for bad, first in (([3, 3, 9], 0), ([5, 4], 0), ([2, 9], 3), ([3, 16], 0), ([-1, 2], -5)):
        with pytest.raises(m.KvrError) as ei:
            _runs_gpu(bad, 16, first)
        assert ei.value.status == -4
        h, _, _ = _runs_gpu(bad, 16, first, sync=False)
        assert h[2] == -4


def test_check_support_position_map():
    """The global-position map of the metadata (cross-attention reuse page,
    6.2) is checked with the support: identity and gapped maps pass, a map
    that is not strictly increasing or negative is an invalid argument."""
    m = kvr()
    res = torch.empty(4, dtype=torch.int32, device="cuda")
    T = torch.tensor([3, 4, 9, 15], dtype=torch.int32, device="cuda")
    N = 5000
    ident = torch.arange(N, dtype=torch.int32, device="cuda")
    gapped = torch.from_numpy((np.arange(N) + 3 * (np.arange(N) >= 1000)).astype(np.int32)).cuda()
    m.kvr_check_support(T, N, 3, res, gpos=ident)
    m.kvr_check_support(T, N, 3, res, gpos=gapped)
    m.kvr_check_support(T[:0], N, 0, res, gpos=gapped)
    for bad in (ident.clone().index_fill_(0, torch.tensor([4321], device="cuda"), 4320),
                ident.clone().index_fill_(0, torch.tensor([0], device="cuda"), -1),
                torch.flip(ident, [0])):
        with pytest.raises(m.KvrError) as ei:
            m.kvr_check_support(T, N, 3, res, gpos=bad)
        assert ei.value.status == -1
    # a bad support is reported as such even with a valid map
    with pytest.raises(m.KvrError) as ei:
        m.kvr_check_support(torch.tensor([5, 4], dtype=torch.int32, device="cuda"), N, 0, res,
                            gpos=ident)
    assert ei.value.status == -4
