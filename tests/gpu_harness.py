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
from workloads.device import cfg_of, dev_cache, dev_weights, kvr, tdtype, workspace  # noqa: F401


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


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
