"""The workspace entry points launch kernels only (no allocation, no
synchronisation, no memset), so a caller can capture them into a HIP graph.
Each test captures one call on a side stream after an eager call on the
same inputs, then replays the graph several times with eager work and
synchronisations in between; every replay must reproduce the eager result
bit for bit (a repair is idempotent for a fixed support and inputs, and
inference attention does not write the cache).  Two streams running
different repairs at once must also give their sequential results."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_harness import cfg_of, dev_cache, dev_weights, kvr, log, workspace

pytestmark = pytest.mark.gpu

W = wl.Workload("graph-bf16", 130, hidden=384, n_q_heads=6, n_kv_heads=2, head_dim=128,
                intermediate=640, n_layers=1, n_tokens=900, block_size=100, dtype="bf16",
                alpha=-1.0, beta=-2.0, tau=5)


def _layer_inputs(T):
    m = kvr()
    cfg = cfg_of(W)
    wnp = wl.layer_weights(W, 0)
    K0, V0 = wl.kv_cache(W, 0)
    kc, vc = dev_cache(W, K0, V0)
    flags = torch.from_numpy(wl.initial_flags(W)).cuda()
    dT = torch.from_numpy(np.asarray(T, np.int32)).cuda()
    x_in = torch.from_numpy(wl.hidden_states(W)).cuda()
    x_out = torch.empty((len(T), W.hidden), dtype=torch.float32, device="cuda")
    ws = workspace(cfg, len(T), W.n_tokens)
    return m, cfg, dev_weights(W, wnp), kc, vc, flags, dT, x_in, x_out, ws


def _replays_match(g, out, ref, noise):
    for rep in range(3):
        out.fill_(float("nan"))
        noise.add_(1.0)                          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"


def test_layer_repair_in_a_graph_replays_bit_exact():
    T = np.arange(100, 900, 9, dtype=np.int32)
    m, cfg, dw, kc, vc, flags, dT, x_in, x_out, ws = _layer_inputs(T)
    log(f"[graph] layer repair, B={len(T)}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.kvr_layer_repair(cfg, dw, kc, vc, flags, dT, x_in, x_out, ws, stream=s)
    s.synchronize()
    ref = x_out.clone()
    k_ref, v_ref, f_ref = kc.clone(), vc.clone(), flags.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        m.kvr_layer_repair(cfg, dw, kc, vc, flags, dT, x_in, x_out, ws, stream=s)
    noise = torch.zeros(1024, device="cuda")
    _replays_match(g, x_out, ref, noise)
    assert torch.equal(kc, k_ref) and torch.equal(vc, v_ref) and torch.equal(flags, f_ref)


@pytest.mark.parametrize("B", [2, 48])     # decode kernel, then the packed path
def test_inference_attention_in_a_graph_replays_bit_exact(B):
    m = kvr()
    cfg = cfg_of(W)
    K0, V0 = wl.kv_cache(W, 0)
    kc, vc = dev_cache(W, K0, V0)
    flags = torch.from_numpy(wl.initial_flags(W)).cuda()
    pos = torch.from_numpy(np.arange(W.n_tokens - B, W.n_tokens, dtype=np.int32)).cuda()
    q = torch.from_numpy(wl.queries(W, B)).cuda()
    o = torch.empty((B, W.n_q_heads, W.head_dim), dtype=torch.float32, device="cuda")
    ws = torch.empty((m.kvr_attention_workspace_bytes(cfg, B, W.n_tokens),), dtype=torch.uint8,
                     device="cuda")
    log(f"[graph] inference attention, B={B}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for noalloc in (False, True):
        call = (lambda: m.kvr_biased_attention_noalloc(cfg, kc, vc, flags, q, pos, o, stream=s)) \
            if noalloc else (lambda: m.kvr_biased_attention(cfg, kc, vc, flags, q, pos, o, ws, stream=s))
        with torch.cuda.stream(s):
            call()
        s.synchronize()
        ref = o.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call()
        _replays_match(g, o, ref, torch.zeros(1024, device="cuda"))


def test_two_streams_at_once_match_their_sequential_results():
    Ta = np.arange(100, 900, 7, dtype=np.int32)
    Tb = np.arange(150, 900, 11, dtype=np.int32)
    log("[graph] two repairs on two streams")
    runs = {}
    for name, T in (("a", Ta), ("b", Tb)):
        args = _layer_inputs(T)
        m, cfg, dw, kc, vc, flags, dT, x_in, x_out, ws = args
        m.kvr_layer_repair(cfg, dw, kc, vc, flags, dT, x_in, x_out, ws)
        torch.cuda.synchronize()
        runs[name] = (x_out.clone(), kc.clone(), vc.clone())
    ia, ib = _layer_inputs(Ta), _layer_inputs(Tb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for st in (sa, sb):
        st.wait_stream(torch.cuda.current_stream())
    for (m, cfg, dw, kc, vc, flags, dT, x_in, x_out, ws), st in ((ia, sa), (ib, sb)):
        m.kvr_layer_repair(cfg, dw, kc, vc, flags, dT, x_in, x_out, ws, stream=st)
    torch.cuda.synchronize()
    for name, inp in (("a", ia), ("b", ib)):
        x_out, kc, vc = inp[8], inp[3], inp[4]
        ref = runs[name]
        assert torch.equal(x_out, ref[0]) and torch.equal(kc, ref[1]) and torch.equal(vc, ref[2])
