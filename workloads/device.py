"""Device copies of the seeded inputs, for the GPU tests and the benchmark.

Moves generated weights and caches to the GPU in the workload's storage type,
builds the library's config for a workload, and allocates a workspace.  Like
the rest of ``workloads`` it holds none of the method's arithmetic.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np
import torch

from . import Workload

# per-layer tensors that stay float32 whatever the storage type
F32_KEYS = ("attn_norm", "mlp_norm", "bq", "bk", "bv")


def kvr():
    import packed_partial_prefill_amd as m
    return m


def tdtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def cfg_of(w: Workload, **over):
    """The library config of a workload (fields overridable)."""
    m = kvr()
    c = m.Config(hidden=w.hidden, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                 head_dim=w.head_dim, intermediate=w.intermediate, rms_eps=w.rms_eps,
                 rope_theta=w.rope_theta, alpha=w.alpha, beta=w.beta,
                 dtype=m.KVR_BF16 if w.dtype == "bf16" else m.KVR_F32)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def dev_weights(w: Workload, wnp: Dict[str, np.ndarray]) -> Dict[str, torch.Tensor]:
    out = {}
    for k, a in wnp.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        out[k] = (t if k in F32_KEYS else t.to(tdtype(w))).cuda()
    return out


def dev_cache(w: Workload, K: np.ndarray, V: np.ndarray) -> Tuple[torch.Tensor, torch.Tensor]:
    return (torch.from_numpy(K).to(tdtype(w)).cuda(), torch.from_numpy(V).to(tdtype(w)).cuda())


def workspace(cfg, B: int, n_tokens: int) -> torch.Tensor:
    """kvr_workspace_bytes() bytes, all 0xFF (float32 NaN): a kernel that
    reads workspace it has not written in the same call shows up as NaN, not
    as a stale value."""
    n = kvr().kvr_workspace_bytes(cfg, B, n_tokens)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
