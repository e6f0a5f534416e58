"""Validation mode (KVR_VALIDATE in the environment): the repair and
attention entries check their support (and position map) on the device
before any other launch and return the check's error with the cache, flags
and outputs untouched; a valid support gives results bit-identical to the
unchecked call.  Every bad support used here stays inside [0, N), so the
kernels would stay in bounds even if a check let one through."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_harness import cfg_of, dev_cache, dev_weights, kvr, log, workspace

pytestmark = pytest.mark.gpu

BAD_SUPPORT, INVALID_ARGUMENT = -4, -1   # kvr_status codes (include/kvr.h)

W = wl.Workload("validate-bf16", 120, hidden=384, n_q_heads=6, n_kv_heads=2, head_dim=64,
                intermediate=640, n_layers=1, n_tokens=600, block_size=100, dtype="bf16",
                alpha=-1.0, beta=-2.0, tau=5)


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("KVR_VALIDATE", "1")


def _layer_setup():
    m = kvr()
    cfg = cfg_of(W)
    wnp = wl.layer_weights(W, 0)
    K0, V0 = wl.kv_cache(W, 0)
    X = wl.hidden_states(W)
    flags0 = wl.initial_flags(W)
    return m, cfg, dev_weights(W, wnp), K0, V0, X, flags0


def _run_layer(T, gpos=None):
    """Runs one layer on fresh copies of the inputs; returns (outcome, x_out,
    cache, flags, untouched copies)."""
    m, cfg, dw, K0, V0, X, flags0 = _layer_setup()
    kc, vc = dev_cache(W, K0, V0)
    kc0, vc0 = kc.clone(), vc.clone()
    flags = torch.from_numpy(flags0).cuda()
    dT = torch.from_numpy(np.asarray(T, np.int32)).cuda()
    dg = None if gpos is None else torch.from_numpy(np.asarray(gpos, np.int32)).cuda()
    x_in = torch.from_numpy(X).cuda()
    x_out = torch.full((len(T), W.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = workspace(cfg, len(T), W.n_tokens)
    err = None
    try:
        m.kvr_layer_repair(cfg, dw, kc, vc, flags, dT, x_in, x_out, ws, gpos=dg)
    except m.KvrError as e:
        err = e
    torch.cuda.synchronize()
    return err, x_out, (kc, vc, flags), (kc0, vc0, flags0)


def _assert_untouched(x_out, cur, orig):
    kc, vc, flags = cur
    kc0, vc0, flags0 = orig
    assert torch.isnan(x_out).all()
    assert torch.equal(kc, kc0) and torch.equal(vc, vc0)
    assert np.array_equal(flags.cpu().numpy(), flags0)


@pytest.mark.parametrize("case", ["unsorted", "duplicate"])
def test_validate_rejects_bad_support_before_any_launch(validate, case):
    T = np.arange(100, 600, 7, dtype=np.int32)
    if case == "unsorted":
        T[[3, 4]] = T[[4, 3]]
    else:
        T[5] = T[4]
    log(f"[validate] layer, {case} support, B={len(T)}")
    err, x_out, cur, orig = _run_layer(T)
    assert err is not None and err.status == BAD_SUPPORT, err
    _assert_untouched(x_out, cur, orig)


def test_validate_rejects_bad_position_map(validate):
    T = np.arange(100, 600, 7, dtype=np.int32)
    g = np.arange(W.n_tokens, dtype=np.int32) * 2
    g[300] = g[299]                                  # not strictly increasing
    log("[validate] layer, bad position map")
    err, x_out, cur, orig = _run_layer(T, gpos=g)
    assert err is not None and err.status == INVALID_ARGUMENT, err
    _assert_untouched(x_out, cur, orig)


def test_validate_valid_support_matches_unchecked_call(monkeypatch):
    T = np.arange(100, 600, 7, dtype=np.int32)
    g = np.arange(W.n_tokens, dtype=np.int32) * 2 + 5
    log("[validate] layer, valid support, checked vs unchecked")
    monkeypatch.setenv("KVR_VALIDATE", "1")
    err1, x1, cur1, _ = _run_layer(T, gpos=g)
    monkeypatch.setenv("KVR_VALIDATE", "0")
    err0, x0, cur0, _ = _run_layer(T, gpos=g)
    assert err1 is None and err0 is None
    assert torch.equal(x1, x0)
    for a, b in zip(cur1[:2], cur0[:2]):
        assert torch.equal(a, b)
    assert torch.equal(cur1[2], cur0[2])


@pytest.mark.parametrize("B", [3, 40])   # decode kernel, then the packed path
def test_validate_attention_rejects_unsorted_positions(validate, B):
    m = kvr()
    cfg = cfg_of(W)
    K0, V0 = wl.kv_cache(W, 0)
    kc, vc = dev_cache(W, K0, V0)
    flags = torch.from_numpy(wl.initial_flags(W)).cuda()
    pos = np.arange(W.n_tokens - B, W.n_tokens, dtype=np.int32)
    pos[[0, 1]] = pos[[1, 0]]
    log(f"[validate] attention, unsorted positions, B={B}")
    q = torch.from_numpy(wl.queries(W, B)).cuda()
    o = torch.full((B, W.n_q_heads, W.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty((m.kvr_attention_workspace_bytes(cfg, B, W.n_tokens),), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(m.KvrError) as ei:
        m.kvr_biased_attention(cfg, kc, vc, flags, q, torch.from_numpy(pos).cuda(), o, ws)
    assert ei.value.status == BAD_SUPPORT
    with pytest.raises(m.KvrError) as ei:
        m.kvr_biased_attention_noalloc(cfg, kc, vc, flags, q, torch.from_numpy(pos).cuda(), o)
    assert ei.value.status == BAD_SUPPORT
    torch.cuda.synchronize()
    assert torch.isnan(o).all()
