"""Helpers for the GPU parity tests: move seeded workload inputs to the
device, run the HIP path through the C ABI, and compare with the oracle.

Tolerances (written here, applied per output tensor):
* float32 storage: max|gpu - ref| <= 1e-4 * max|ref| + 1e-5
* bf16 storage / float32 accumulation: max|gpu - ref| <= 2e-2 * max|ref| + 1e-3
Integer outputs (T, runs, plan tables, flags) and untouched cache rows are
compared bit for bit.
"""
from __future__ import annotations

import sys
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import workloads as wl


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def kvr():
    import packed_partial_prefill_amd as m
    return m


def tdtype(w: wl.Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def cfg_of(w: wl.Workload, **over):
    m = kvr()
    c = m.Config(hidden=w.hidden, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                 head_dim=w.head_dim, intermediate=w.intermediate, rms_eps=w.rms_eps,
                 rope_theta=w.rope_theta, alpha=w.alpha, beta=w.beta,
                 dtype=m.KVR_BF16 if w.dtype == "bf16" else m.KVR_F32)
    for k, v in over.items():
        setattr(c, k, v)
    return c


F32_KEYS = ("attn_norm", "mlp_norm", "bq", "bk", "bv")


def dev_weights(w: wl.Workload, wnp: Dict[str, np.ndarray]) -> Dict[str, torch.Tensor]:
    out = {}
    for k, a in wnp.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        out[k] = (t if k in F32_KEYS else t.to(tdtype(w))).cuda()
    return out


def dev_cache(w: wl.Workload, K: np.ndarray, V: np.ndarray) -> Tuple[torch.Tensor, torch.Tensor]:
    return (torch.from_numpy(K).to(tdtype(w)).cuda(), torch.from_numpy(V).to(tdtype(w)).cuda())


def workspace(cfg, B: int, n_tokens: int) -> torch.Tensor:
    n = kvr().kvr_workspace_bytes(cfg, B, n_tokens)
    # all bytes 0xFF (float32 NaN): a kernel that reads workspace it has not
    # written in the same call shows up as NaN, not as a stale value
    return torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")


def build_seams_gpu(w: wl.Workload, tau: Optional[int] = None, asym: bool = True,
                    init_meta: bool = True):
    """Run kvr_build_repair_set on the workload's blocks; returns (T, runs,
    counts, flags, block_id) as device tensors / host tuple."""
    m = kvr()
    s, e = wl.blocks(w)
    ds = torch.from_numpy(s).cuda()
    de = torch.from_numpy(e).cuda()
    cap = w.n_tokens
    T = torch.empty(cap, dtype=torch.int32, device="cuda")
    rs = torch.empty(cap, dtype=torch.int32, device="cuda")
    rl = torch.empty(cap, dtype=torch.int32, device="cuda")
    counts = torch.empty(4, dtype=torch.int32, device="cuda")
    flags = torch.full((w.n_tokens,), 0xAB, dtype=torch.uint8, device="cuda")
    bid = torch.full((w.n_tokens,), -1, dtype=torch.int32, device="cuda")
    mode = (m.KVR_SEAM_ASYMMETRIC if asym else 0) | (m.KVR_INIT_META if init_meta else 0)
    h = m.kvr_build_repair_set(ds, de, w.n_tokens, w.tau if tau is None else tau, mode, T, rs, rl,
                               counts, flags=flags if init_meta else None,
                               block_id=bid if init_meta else None)
    n, R, st = h
    return T[:n].clone(), (rs[:R].cpu().numpy(), rl[:R].cpu().numpy()), h, flags, bid


def tol(w: wl.Workload, ref: np.ndarray) -> float:
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    return (1e-4 * mx + 1e-5) if w.dtype == "f32" else (2e-2 * mx + 1e-3)


def assert_close(w: wl.Workload, got, ref, what: str) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    bound = tol(w, ref)
    log(f"  {what}: max|d|={err:.3e} bound={bound:.3e} max|ref|={np.max(np.abs(ref)):.3e}")
    assert err <= bound, f"{what}: max|d|={err:.3e} > {bound:.3e}"
    return err


def cpu(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()
