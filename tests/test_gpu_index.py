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
    assert np.array_equal(flags.cpu().numpy(), wl.initial_flags(w))
    assert np.array_equal(bid.cpu().numpy(), wl.block_ids(w))


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
