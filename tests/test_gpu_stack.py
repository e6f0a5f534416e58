"""GPU parity of the layer stack (kvr_stack_repair).

Both stack workloads are checked at full size against the oracle on every
row through their first two layers.  Through all 28 layers the oracle cannot
run every row in seconds, so there the checks are (a) exact oracle parity on
the first k packed rows (a repair's first k rows depend only on keys at or
before their positions, so the oracle's repair of T[:k] is exactly their
value; pinned on the CPU by test_causal_prefix_of_support_is_self_contained),
and (b) properties that hold at any size: untouched rows bit-identical, flags
exact, finite outputs, and agreement of two schedules of the same
computation.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_harness import (assert_close, build_seams_gpu, cfg_of, cpu, dev_cache,
                               dev_weights, kvr, log, workspace)

pytestmark = pytest.mark.gpu


def _upload_layers(w, oracle_rows_upto=None):
    """Generate every layer once; returns device weights/caches, and host
    float64 copies (optionally truncated to the rows the oracle needs)."""
    dws, dcs, host = [], [], []
    for li in range(w.n_layers):
        wnp = wl.layer_weights(w, li)
        K0, V0 = wl.kv_cache(w, li)
        dws.append(dev_weights(w, wnp))
        dcs.append(dev_cache(w, K0, V0))
        n = w.n_tokens if oracle_rows_upto is None else oracle_rows_upto
        host.append((wnp, K0[:n].astype(np.float64), V0[:n].astype(np.float64)))
    return dws, dcs, host


def test_small_stack_seams_bf16():
    w = wl.Workload("small-stack-bf16", 102, hidden=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                    intermediate=512, n_layers=4, n_tokens=1024, block_size=128, dtype="bf16",
                    alpha=-1.0, beta=-2.0, tau=7)
    log(f"[stack] {w.name}")
    m = kvr()
    dT, _, h, flags, _ = build_seams_gpu(w)
    T = dT.cpu().numpy().astype(np.int64)
    dws, dcs, host = _upload_layers(w)
    X = wl.hidden_states(w)
    x_out = torch.empty((len(T), w.hidden), dtype=torch.float32, device="cuda")
    cfg = cfg_of(w)
    m.kvr_stack_repair(cfg, dws, dcs, flags, dT, torch.from_numpy(X).cuda(), x_out,
                       workspace(cfg, len(T), w.n_tokens))
    torch.cuda.synchronize()
    f = _oracle_flags(w)
    y = oracle.stack_repair(cfg, host, f, T, X)
    assert_close(w, cpu(x_out), y, "stack output")
    for li, ((_, K, V), (kc, vc)) in enumerate(zip(host, dcs)):
        assert_close(w, cpu(kc[dT.long()]), K[T], f"layer {li} K rows")
        assert_close(w, cpu(vc[dT.long()]), V[T], f"layer {li} V rows")
    assert np.array_equal(flags.cpu().numpy(), f)


def _oracle_flags(w, upto=None):
    s, e = wl.blocks(w)
    f = oracle.initial_meta(s, e, w.n_tokens)[0]
    return f if upto is None else f[:upto].copy()


def _run_stack_gpu(w, cfg, dws, dcs, flags, dT, dX):
    x_out = torch.empty((dT.numel(), w.hidden), dtype=torch.float32, device="cuda")
    kvr().kvr_stack_repair(cfg, dws, dcs, flags, dT, dX, x_out,
                           workspace(cfg, dT.numel(), w.n_tokens))
    torch.cuda.synchronize()
    return x_out


@pytest.mark.timeout(900)
def test_qwen7_isolated_32k_two_layers_every_row():
    """The fragmented extreme at full size (N = 32768, all 646 isolated rows,
    alpha = -1.5, beta = -3 with live sinks) through the first two layers of
    the 7B stack: every packed output row, every refreshed K/V row of both
    layers and every flag against the oracle."""
    w = wl.QWEN7_STACK_ISOLATED.with_(n_layers=2)
    T = wl.isolated_support(w)
    s, e = wl.blocks(w)
    oracle.check_support(T, w.n_tokens, int(e[0]), oracle.budget(w.n_tokens - int(e[0]), 2))
    log(f"[stack] {w.name} x{w.n_layers}: B={len(T)} N={w.n_tokens}; oracle on every row")
    dT = torch.from_numpy(T).cuda()
    dws, dcs, host = _upload_layers(w)
    kc0 = [(kc.clone(), vc.clone()) for kc, vc in dcs]
    X = wl.hidden_states(w)
    flags = torch.from_numpy(_oracle_flags(w)).cuda()
    cfg = cfg_of(w)
    out = cpu(_run_stack_gpu(w, cfg, dws, dcs, flags, dT, torch.from_numpy(X).cuda()))
    log("  gpu stack done; oracle")
    f = _oracle_flags(w)
    y = oracle.stack_repair(cfg, host, f, T, X,
                            on_layer=lambda li, _: log(f"  oracle layer {li} done"))
    assert_close(w, out, y, "stack output, all 646 rows")
    keep = torch.ones(w.n_tokens, dtype=torch.bool, device="cuda")
    keep[dT.long()] = False
    for li, (_, K, V) in enumerate(host):
        assert_close(w, cpu(dcs[li][0][dT.long()]), K[T], f"layer {li} K rows")
        assert_close(w, cpu(dcs[li][1][dT.long()]), V[T], f"layer {li} V rows")
        assert torch.equal(dcs[li][0][keep], kc0[li][0][keep])
        assert torch.equal(dcs[li][1][keep], kc0[li][1][keep])
    assert np.array_equal(flags.cpu().numpy(), f)


@pytest.mark.timeout(900)
def test_qwen7_stack28_32k_isolated_sampled():
    """All 28 layers at full size: oracle parity on the first k packed rows
    (exact: a repair's first rows depend only on keys at or before their
    positions), flags and untouched rows on all of them."""
    w = wl.QWEN7_STACK_ISOLATED
    m = kvr()
    T = wl.isolated_support(w)
    k = 64
    log(f"[stack] {w.name}: B={len(T)} layers={w.n_layers}; oracle on first {k} rows")
    dT = torch.from_numpy(T).cuda()
    res = torch.empty(4, dtype=torch.int32, device="cuda")
    m.kvr_check_support(dT, w.n_tokens, w.block_size, res)
    dws, dcs, host = _upload_layers(w, oracle_rows_upto=int(T[k - 1]) + 1)
    log("  inputs on device")
    X = wl.hidden_states(w)
    flags = torch.from_numpy(_oracle_flags(w)).cuda()
    keep = torch.ones(w.n_tokens, dtype=torch.bool, device="cuda")
    keep[dT.long()] = False
    k_keep0 = [kc[keep].clone() for kc, _ in dcs[:2]]
    cfg = cfg_of(w)
    out = cpu(_run_stack_gpu(w, cfg, dws, dcs, flags, dT, torch.from_numpy(X).cuda()))
    log("  gpu stack done")
    assert np.all(np.isfinite(out))
    for li in range(2):
        assert torch.equal(dcs[li][0][keep], k_keep0[li])
    f_ref = _oracle_flags(w)
    oracle.write_back_flags(f_ref, T)
    assert np.array_equal(flags.cpu().numpy(), f_ref)
    f = _oracle_flags(w, upto=int(T[k - 1]) + 1)
    y = oracle.stack_repair(cfg, host, f, T[:k], X)
    assert_close(w, out[:k], y, f"stack output rows 0..{k - 1}")
    for li in (0, 13, w.n_layers - 1):
        _, K, V = host[li]
        assert_close(w, cpu(dcs[li][0][dT[:k].long()]), K[T[:k]], f"layer {li} K rows")
        assert_close(w, cpu(dcs[li][1][dT[:k].long()]), V[T[:k]], f"layer {li} V rows")


@pytest.mark.timeout(900)
def test_qwen15_degenerate_16k_two_layers_every_row():
    """Degeneration at full size (N = 16384, tau = 128: T = [256, N), 16,128
    rows) through the first two layers of the 1.5B stack: B_1's cache is
    produced by a repair over B_1, then T is repaired; every packed row,
    every cache row of both layers and every flag against the oracle's same
    two-phase repair."""
    w = wl.QWEN15_STACK_DEGENERATE.with_(n_layers=2)
    dT, _, h, flags, _ = build_seams_gpu(w)
    T = dT.cpu().numpy().astype(np.int64)
    s, e = wl.blocks(w)
    assert np.array_equal(T, oracle.seam_set(s, e, w.tau, True))
    log(f"[stack] {w.name} x{w.n_layers}: B={len(T)}; oracle on every row")
    dws, dcs, host = _upload_layers(w)
    X = wl.hidden_states(w)
    dX = torch.from_numpy(X).cuda()
    cfg = cfg_of(w)
    TA = torch.arange(w.block_size, dtype=torch.int32, device="cuda")
    xa = cpu(_run_stack_gpu(w, cfg, dws, dcs, flags, TA, dX))
    xb = cpu(_run_stack_gpu(w, cfg, dws, dcs, flags, dT, dX))
    log("  gpu two-phase done; oracle")
    f = _oracle_flags(w)
    ya = oracle.stack_repair(cfg, host, f, np.arange(w.block_size), X)
    yb = oracle.stack_repair(cfg, host, f, T, X,
                             on_layer=lambda li, _: log(f"  oracle layer {li} done"))
    assert_close(w, xa, ya, "B_1 output")
    assert_close(w, xb, yb, f"T output, all {len(T)} rows")
    for li, (_, K, V) in enumerate(host):
        assert_close(w, cpu(dcs[li][0]), K, f"layer {li} K, all rows")
        assert_close(w, cpu(dcs[li][1]), V, f"layer {li} V, all rows")
    assert np.all(f == 0) and np.array_equal(flags.cpu().numpy(), f)


@pytest.mark.timeout(900)
def test_qwen15_stack28_16k_degenerate():
    """Degeneration (tau >= |B|/2) through all 28 layers: T covers B_2..B_m,
    no local key and no sink survives write-back, so the repair equals a
    full causal prefill.  B_1's cache is itself produced by a repair over
    B_1 (a prefix sees only itself).  Checks: oracle parity on B_1 and the
    first k rows of T; and at full size, the two-phase result equals one
    repair over all N positions."""
    w = wl.QWEN15_STACK_DEGENERATE
    m = kvr()
    k = 64
    dT, _, h, flags, _ = build_seams_gpu(w)
    T = dT.cpu().numpy().astype(np.int64)
    assert T[0] == w.block_size and len(T) == w.n_tokens - w.block_size
    log(f"[stack] {w.name}: B={len(T)} layers={w.n_layers}; oracle on B_1 + first {k} rows")
    upto = w.block_size + k
    dws, dcs, host = _upload_layers(w, oracle_rows_upto=upto)
    fresh = [(kc.clone(), vc.clone()) for kc, vc in dcs]
    X = wl.hidden_states(w)
    dX = torch.from_numpy(X).cuda()
    cfg = cfg_of(w)
    TA = torch.arange(w.block_size, dtype=torch.int32, device="cuda")
    xa = _run_stack_gpu(w, cfg, dws, dcs, flags, TA, dX)
    xb = _run_stack_gpu(w, cfg, dws, dcs, flags, dT, dX)
    log("  gpu two-phase done")
    assert np.all(flags.cpu().numpy() == 0)

    # (a) oracle on B_1 then on the first k rows of T
    f = _oracle_flags(w, upto=upto)
    ya = oracle.stack_repair(cfg, host, f, np.arange(w.block_size), X)
    yb = oracle.stack_repair(cfg, host, f, T[:k], X)
    assert_close(w, cpu(xa), ya, "B_1 output")
    assert_close(w, cpu(xb[:k]), yb, f"T output rows 0..{k - 1}")
    for li in (0, w.n_layers - 1):
        _, K, V = host[li]
        assert_close(w, cpu(dcs[li][0][:upto]), K[:upto], f"layer {li} K rows 0..{upto - 1}")
        assert_close(w, cpu(dcs[li][1][:upto]), V[:upto], f"layer {li} V rows 0..{upto - 1}")

    # (b) full size: one repair over [0, N) with alpha = beta = 0 is the same
    # full prefill; compare every row of the two-phase result against it
    flags2 = torch.from_numpy(_oracle_flags(w)).cuda()
    T_all = torch.arange(w.n_tokens, dtype=torch.int32, device="cuda")
    x_all = _run_stack_gpu(w, cfg, dws, fresh, flags2, T_all, dX)
    log("  gpu single-call prefill done")
    assert_close(w, cpu(xb), cpu(x_all[w.block_size:]), "two-phase vs one-call, all rows")
    for li in (0, 13, w.n_layers - 1):
        assert_close(w, cpu(dcs[li][0]), cpu(fresh[li][0]), f"layer {li} K, all rows")
        assert_close(w, cpu(dcs[li][1]), cpu(fresh[li][1]), f"layer {li} V, all rows")


def test_interval_wise_replay_equals_packed():
    """Sequential maximal-interval replay (Budgeted KV-Cache Repair, section
    7.1), one kvr_stack_repair call per run, equals the packed layer-major
    call (section 13.2 argues they agree in real arithmetic) and the oracle's
    interval-major replay."""
    w = wl.Workload("small-stack-intervals", 103, hidden=256, n_q_heads=8, n_kv_heads=2,
                    head_dim=64, intermediate=512, n_layers=3, n_tokens=768, block_size=128,
                    dtype="bf16", alpha=-1.0, beta=-2.0, tau=5)
    log(f"[stack] {w.name}: packed vs interval-wise")
    m = kvr()
    dT, (starts, lens), h, flags, _ = build_seams_gpu(w)
    T = dT.cpu().numpy().astype(np.int64)
    ref_s, ref_l = oracle.runs(T)
    assert np.array_equal(starts, ref_s) and np.array_equal(lens, ref_l)
    X = wl.hidden_states(w)
    dX = torch.from_numpy(X).cuda()
    cfg = cfg_of(w)
    dws, dcs, host = _upload_layers(w)
    caches_b = [(k.clone(), v.clone()) for k, v in dcs]
    flags_b = flags.clone()
    x_p = torch.empty((len(T), w.hidden), dtype=torch.float32, device="cuda")
    m.kvr_stack_repair(cfg, dws, dcs, flags, dT, dX, x_p, workspace(cfg, len(T), w.n_tokens))
    outs = []
    for a, ln in zip(starts, lens):
        Tr = torch.arange(int(a), int(a) + int(ln), dtype=torch.int32, device="cuda")
        o = torch.empty((int(ln), w.hidden), dtype=torch.float32, device="cuda")
        m.kvr_stack_repair(cfg, dws, caches_b, flags_b, Tr, dX, o, workspace(cfg, int(ln), w.n_tokens))
        outs.append(o)
    x_i = torch.cat(outs)
    torch.cuda.synchronize()
    assert len(starts) == 6
    yi = oracle.interval_major(cfg, host, _oracle_flags(w), T, X)
    assert_close(w, cpu(x_i), yi, "interval-wise vs oracle interval-major")
    assert_close(w, cpu(x_p), cpu(x_i), "packed vs interval-wise")
    assert torch.equal(flags, flags_b)
    for li in range(w.n_layers):
        assert_close(w, cpu(dcs[li][0][dT.long()]), cpu(caches_b[li][0][dT.long()]), f"layer {li} K")
