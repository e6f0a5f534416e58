"""GPU parity of inference-mode attention (kvr_biased_attention) and Shift
(kvr_shift_cache) against the oracle on the same seeded inputs.

Inference mode: every query row against oracle.inference_attention within
the dtype's tolerance; the cache and flags stay bit-identical.  Shift:
moved keys within half a storage ulp of the float64 rotation (plus float32
rounding), values, prefix rows and metadata bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_harness import assert_close, cfg_of, cpu, dev_cache, kvr, log

pytestmark = pytest.mark.gpu


def _small(name, cfg_id, dtype, hq, hkv, d, n, block, alpha=-1.0, beta=-2.0):
    return wl.Workload(name, cfg_id, hidden=hq * d, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                       intermediate=64, n_layers=1, n_tokens=n, block_size=block, dtype=dtype,
                       alpha=alpha, beta=beta)


def run_inference(w: wl.Workload, pos: np.ndarray, check_rows=None):
    m = kvr()
    cfg = cfg_of(w)
    pos = np.asarray(pos, dtype=np.int32)
    B = len(pos)
    log(f"[inference] {w.name} dtype={w.dtype} N={w.n_tokens} B={B}")
    K0, V0 = wl.kv_cache(w, 0)
    flags0 = wl.initial_flags(w)
    q = wl.queries(w, B)
    kc, vc = dev_cache(w, K0, V0)
    kc0, vc0 = kc.clone(), vc.clone()
    flags = torch.from_numpy(flags0).cuda()
    dq = torch.from_numpy(q).cuda()
    dpos = torch.from_numpy(pos).cuda()
    o = torch.full((B, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    # 0xFF bytes (float32 NaN): a read of workspace not written in this call shows
    ws = torch.full((m.kvr_attention_workspace_bytes(cfg, B, w.n_tokens),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    m.kvr_biased_attention(cfg, kc, vc, flags, dq, dpos, o, ws)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc0) and torch.equal(vc, vc0)
    assert np.array_equal(flags.cpu().numpy(), flags0)
    rows = np.arange(B) if check_rows is None else np.asarray(check_rows)
    ref = oracle.inference_attention(cfg, q[rows], pos[rows], K0.astype(np.float64),
                                     V0.astype(np.float64), flags0)
    assert_close(w, cpu(o)[rows], ref, "inference output")


def test_inference_tiny_f32_sparse_rows():
    w = _small("inf-tiny-f32", 201, "f32", 4, 2, 64, 512, 128)
    rng = np.random.default_rng(0)
    pos = np.sort(rng.choice(np.arange(1, 511), size=22, replace=False))
    run_inference(w, np.r_[0, pos, 511])


def test_inference_tiny_bf16_group6_multi_tile():
    w = _small("inf-tiny-bf16-g6", 202, "bf16", 6, 1, 128, 700, 100)
    rng = np.random.default_rng(1)
    pos = np.sort(rng.choice(700, size=50, replace=False))   # 300 pairs: 3 query tiles
    run_inference(w, pos)


def test_inference_bf16_head_dim_64_prefill_all_positions():
    w = _small("inf-prefill-d64", 203, "bf16", 8, 2, 64, 1024, 256, alpha=-0.5, beta=-4.0)
    run_inference(w, np.arange(1024), check_rows=np.r_[0:40, 250:260, 1000:1024])


def test_inference_alpha_beta_zero_without_metadata_is_plain_attention():
    w = _small("inf-unbiased", 204, "bf16", 4, 4, 128, 300, 300, alpha=0.0, beta=0.0)
    run_inference(w, np.arange(0, 300, 7))


@pytest.mark.parametrize("hq,hkv,d,n,pos", [
    (8, 2, 64, 1000, [5, 300, 999]),                 # d = 64, ragged last chunk
    (32, 8, 128, 2048, list(range(2040, 2048))),     # 32 pairs: one column block
    (32, 8, 128, 2048, list(range(2039, 2048))),     # 36 pairs: two column blocks
    (28, 4, 128, 4096, [100, 3000]),                 # chunks past the last query skipped
    (8, 8, 128, 513, list(range(0, 513, 9))),        # G = 1, 58 pairs
    (4, 1, 128, 777, [10, 400, 776]),                # one KV head; last step holds 9 keys
    (12, 2, 128, 20000, list(range(19995, 20000))),  # 30 pairs, 157 steps over 79 workgroups
])
def test_inference_decode_path_shapes(hq, hkv, d, n, pos):
    w = _small(f"inf-decode-{hq}-{hkv}-{d}-{n}", 205, "bf16", hq, hkv, d, n, 128)
    run_inference(w, np.asarray(pos))


def test_inference_stream_k_short_ranges_odd_tile_count():
    # 7B heads over a 16K cache, queries at positions 0..299: the launch takes
    # the stream-K pair kernel (sized by the cache length) although every
    # query sees at most 5 KV tiles, so workgroups get 4-tile pieces; 2100
    # pairs make 17 query tiles, the last pair holding one.
    w = _small("inf-sk-short", 206, "bf16", 28, 4, 128, 16384, 256)
    run_inference(w, np.arange(300))


def test_inference_stream_k_group6_scattered():
    # 1.5B heads (G = 6) over a 16K cache, 600 scattered queries (29 query
    # tiles): segments of very different lengths split over workgroups.
    w = _small("inf-sk-g6", 207, "bf16", 12, 2, 128, 16384, 512, alpha=-0.7, beta=-3.0)
    rng = np.random.default_rng(7)
    pos = np.sort(rng.choice(16384, size=600, replace=False))
    run_inference(w, pos, check_rows=np.r_[0:8, 290:300, 590:600])


@pytest.mark.parametrize("B", [1, 8])
def test_inference_qwen7_decode_16k(B):
    w = wl.QWEN7_DECODE_16K
    run_inference(w, np.arange(w.n_tokens - B, w.n_tokens))


def test_inference_qwen7_decode_32k():
    w = wl.QWEN7_DECODE_32K
    run_inference(w, wl.explicit_support(w))


# --------------------------------------------------------------------- shift
def run_shift(w: wl.Workload, n_layers: int, a: int, d: int, mark: int, check_layers=None):
    m = kvr()
    cfg = cfg_of(w)
    N = w.n_tokens
    n_out = N - d
    log(f"[shift] {w.name} dtype={w.dtype} layers={n_layers} N={N} delete [{a}, {a + d})")
    host, src, dst = [], [], []
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    for li in range(n_layers):
        K0, V0 = wl.kv_cache(w, li)
        host.append((K0, V0))
        src.append(dev_cache(w, K0, V0))
        dst.append((torch.full((n_out, w.n_kv_heads, w.head_dim), float("nan"), dtype=tdt,
                               device="cuda"),
                    torch.full((n_out, w.n_kv_heads, w.head_dim), float("nan"), dtype=tdt,
                               device="cuda")))
    f0 = wl.initial_flags(w)
    b0 = wl.block_ids(w)
    fs, bs = torch.from_numpy(f0).cuda(), torch.from_numpy(b0).cuda()
    fd = torch.full((n_out,), 0xEE, dtype=torch.uint8, device="cuda")
    bd = torch.full((n_out,), -7, dtype=torch.int32, device="cuda")
    src0 = [(k.clone(), v.clone()) for k, v in src]
    m.kvr_shift_cache(cfg, src, dst, a, d, flags_src=fs, flags_dst=fd, block_src=bs,
                      block_dst=bd, mark=mark)
    torch.cuda.synchronize()
    for (k, v), (k0, v0) in zip(src, src0):
        assert torch.equal(k, k0) and torch.equal(v, v0)
    layers = range(n_layers) if check_layers is None else check_layers
    for li in layers:
        K0, V0 = host[li]
        Kr, Vr, fr, br = oracle.shift_cache(cfg, K0, V0, f0, b0, a, d, mark)
        kg, vg = dst[li]
        # prefix and values: bit-exact moves
        assert torch.equal(kg[:a], src[li][0][:a]), f"layer {li}: prefix keys"
        assert torch.equal(vg, torch.cat([src[li][1][:a], src[li][1][a + d:]])), f"layer {li}: values"
        got = cpu(kg[a:]).astype(np.float64)
        ref = Kr[a:]
        # half an ulp of the storage format plus float32 arithmetic
        half_ulp = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -23
        err = np.abs(got - ref)
        bound = half_ulp * np.abs(ref) + 1e-6 * (np.abs(ref) + 1.0)
        worst = float(np.max(err - bound)) if err.size else -1.0
        log(f"  layer {li}: max|d|={float(err.max()) if err.size else 0:.3e} (worst margin {worst:.2e})")
        assert worst <= 0.0
    dummy = np.zeros((N, 1, 2))
    _, _, fr, br = oracle.shift_cache(cfg, dummy, dummy, f0, b0, a, d, mark)
    assert np.array_equal(fd.cpu().numpy(), fr)
    assert np.array_equal(bd.cpu().numpy(), br)


def test_shift_tiny_f32_two_layers():
    w = _small("shift-tiny-f32", 211, "f32", 4, 2, 64, 300, 50)
    run_shift(w, 2, 37, 50, oracle.FLAG_LOCAL)


def test_shift_bf16_head_dim_64_many_layers_two_launches():
    w = _small("shift-40-layers", 212, "bf16", 8, 2, 64, 257, 64)
    run_shift(w, 40, 100, 3, 0, check_layers=[0, 31, 32, 39])


@pytest.mark.parametrize("a,d", [(0, 17), (200, 0), (150, 106), (0, 0)])
def test_shift_edges(a, d):
    w = _small("shift-edges", 213, "bf16", 4, 2, 128, 256, 64)
    run_shift(w, 1, a, d, oracle.FLAG_LOCAL)


def test_shift_zero_span_copies_bit_for_bit():
    m = kvr()
    w = _small("shift-copy", 214, "bf16", 4, 2, 128, 256, 64)
    K0, V0 = wl.kv_cache(w, 0)
    src = [dev_cache(w, K0, V0)]
    dst = [(torch.empty_like(src[0][0]), torch.empty_like(src[0][1]))]
    m.kvr_shift_cache(cfg_of(w), src, dst, 77, 0)
    torch.cuda.synchronize()
    assert torch.equal(dst[0][0], src[0][0]) and torch.equal(dst[0][1], src[0][1])


@pytest.mark.timeout(600)
def test_shift_qwen7_28_layers_16k():
    w = wl.QWEN7_SHIFT
    run_shift(w, w.n_layers, w.support_start, w.support_len, oracle.FLAG_LOCAL,
              check_layers=[0, 13, 27])
