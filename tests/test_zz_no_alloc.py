"""The allocation-free inference-mode entry point (kvr_biased_attention_noalloc)
against kvr_biased_attention on the same inputs, through the C ABI: two
calls in a row on the shared static scratch, the second with a smaller
input, both bit-identical to the workspace entry point and within the bf16
tolerance of the oracle; shapes needing more scratch than the library holds
are rejected before any device work."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_harness import assert_close, cfg_of, cpu, dev_cache, kvr, log

pytestmark = pytest.mark.gpu


def _inputs(w, B):
    K0, V0 = wl.kv_cache(w, 0)
    s, e = wl.blocks(w)
    flags0 = oracle.initial_meta(s, e, w.n_tokens)[0]
    pos = np.arange(w.n_tokens - B, w.n_tokens, dtype=np.int32)
    q = wl.queries(w, B)
    return K0, V0, flags0, pos, q


def _both(w, B):
    m = kvr()
    cfg = cfg_of(w)
    K0, V0, flags0, pos, q = _inputs(w, B)
    kc, vc = dev_cache(w, K0, V0)
    flags = torch.from_numpy(flags0).cuda()
    dq, dpos = torch.from_numpy(q).cuda(), torch.from_numpy(pos).cuda()
    o_ws = torch.full((B, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                      device="cuda")
    o_na = torch.full_like(o_ws, float("nan"))
    ws = torch.full((m.kvr_attention_workspace_bytes(cfg, B, w.n_tokens),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    m.kvr_biased_attention(cfg, kc, vc, flags, dq, dpos, o_ws, ws)
    m.kvr_biased_attention_noalloc(cfg, kc, vc, flags, dq, dpos, o_na)
    torch.cuda.synchronize()
    return cfg, o_ws, o_na, (K0, V0, flags0, pos, q)


def test_noalloc_matches_workspace_entry_two_calls_shrinking():
    w_big = wl.QWEN7_DECODE_16K
    w_small = wl.QWEN7_DECODE_16K.with_(n_tokens=4096, cfg_id=70)
    for w, B in ((w_big, 8), (w_small, 1), (wl.TINY.with_(dtype="bf16"), 24),
                 (wl.TINY.with_(dtype="bf16"), 40)):
        log(f"[noalloc] {w.name} N={w.n_tokens} B={B}")
        cfg, o_ws, o_na, (K0, V0, flags0, pos, q) = _both(w, B)
        assert torch.equal(o_na, o_ws), "noalloc output differs from the workspace entry point"
        ref = oracle.inference_attention(cfg, q, pos, K0.astype(np.float64),
                                         V0.astype(np.float64), flags0)
        assert_close(w, cpu(o_na), ref, "noalloc output vs oracle")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    m = kvr()
    # 64 query rows of the 7B shape over N = 16384 take the packed attention
    # path, whose plan, scaled queries and partials need more than the
    # static scratch holds
    w = wl.QWEN7_DECODE_16K
    cfg = cfg_of(w)
    B, N = 64, w.n_tokens
    need = m.kvr_attention_workspace_bytes(cfg, B, N) - 256
    assert need > m.KVR_NOALLOC_SCRATCH_BYTES
    kc = torch.zeros((N, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    flags = torch.zeros(N, dtype=torch.uint8, device="cuda")
    q = torch.zeros((B, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    pos = torch.arange(N - B, N, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(m.KvrError) as ei:
        m.kvr_biased_attention_noalloc(cfg, kc, vc, flags, q, pos, o)
    assert ei.value.status == -6
