"""Seeded synthetic inputs for the packed selective-recompute path.

This module only draws numbers and lays out inputs (block partitions,
initial per-position metadata, weights, caches, hidden states and explicit
supports).  It holds none of the method's arithmetic, so both the CPU
oracle and the GPU path may take their inputs from it.

Recipe
------
* Every tensor is identified by (config id, layer, tensor id) and drawn in
  fixed chunks of ``CHUNK`` elements; chunk ``c`` comes from
  ``Generator(PCG64(SeedSequence([1234, cfg, layer, tensor, c])))`` with
  ``standard_normal(dtype=float32)``.  The result does not depend on how many
  threads draw it.
* Scales: cache K/V ~ N(0,1), hidden states ~ N(0,1), linear weights
  ~ N(0, 0.02), RMSNorm gains 1 + N(0, 0.02).
* bf16 workloads round every drawn value to bfloat16 with
  round-to-nearest-even once; both sides then see identical bits (the
  oracle widens them to float64, the GPU path stores them as bf16).
* Tensor ids: 0 K cache, 1 V cache, 2 hidden states X, 3 attention-norm
  gain, 4 W_q, 5 W_k, 6 W_v, 7 W_o, 8 MLP-norm gain, 9 W_gate, 10 W_up,
  11 W_down, 12 support sampling, 13-15 q/k/v biases (only when asked for).
* Metadata at load (mixed-cache statement, Budgeted/Cross-attention page
  section 6.2): block 1 is global, every later block is local; the spurious
  sink set is the first token of every block after the first.
"""
from __future__ import annotations

import math
import threading
from dataclasses import dataclass, replace
from typing import Dict, Optional, Tuple

import numpy as np

FLAG_LOCAL = 1
FLAG_SINK = 2

CHUNK = 1 << 22
SEED_ROOT = 1234

T_KCACHE, T_VCACHE, T_X, T_ATTN_NORM, T_WQ, T_WK, T_WV, T_WO, T_MLP_NORM, \
    T_WGATE, T_WUP, T_WDOWN, T_SUPPORT, T_BQ, T_BK, T_BV, T_QUERY = range(17)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    n_layers: int
    n_tokens: int
    block_size: int
    dtype: str                      # "f32" or "bf16": weights + KV cache storage
    alpha: float
    beta: float
    tau: int = 0                    # seam half-width (support == "seams")
    support: str = "seams"          # seams | contiguous | matched | isolated | intervals | suffix | span
    budget_percent: float = 0.0     # isolated supports: B = min(S, ceil(S*b/100))
    support_start: int = 0          # contiguous / matched supports: first position
    support_len: int = 0            # contiguous / matched / intervals supports: length B
    n_intervals: int = 1            # intervals supports: number of equal runs R
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    qkv_bias: bool = False

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_blocks(self) -> int:
        return self.n_tokens // self.block_size

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: shapes follow the Qwen2.5 1.5B / 7B families the pages
# evaluate on; sizes, budgets, tau, alpha and beta are the stated configs.
TINY = Workload("tiny-f32", 1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                intermediate=512, n_layers=1, n_tokens=512, block_size=128, dtype="f32",
                alpha=-1.0, beta=-2.0, tau=4)
QWEN15_LAYER = Workload("qwen2.5-1.5b-layer", 2, hidden=1536, n_q_heads=12, n_kv_heads=2,
                        head_dim=128, intermediate=8960, n_layers=1, n_tokens=4096,
                        block_size=256, dtype="bf16", alpha=-1.0, beta=-2.0, tau=8)
QWEN7_LAYER_SEAMS = Workload("qwen2.5-7b-layer-16k-seams", 3, hidden=3584, n_q_heads=28,
                             n_kv_heads=4, head_dim=128, intermediate=18944, n_layers=1,
                             n_tokens=16384, block_size=256, dtype="bf16", alpha=-1.0,
                             beta=-2.0, tau=6)
# Equal budget as one interval at the suffix start: |T_seams| = 2*tau*(m-1) = 756.
QWEN7_LAYER_CONTIG = QWEN7_LAYER_SEAMS.with_(name="qwen2.5-7b-layer-16k-contiguous",
                                             support="contiguous", support_start=256,
                                             support_len=756)
# Equal budget, one interval whose mean position (8319.5) equals the seam set's,
# so the causal pair count sum(u+1) is identical (matched work).
QWEN7_LAYER_MATCHED = QWEN7_LAYER_SEAMS.with_(name="qwen2.5-7b-layer-16k-matched",
                                              support="matched", support_start=7942,
                                              support_len=756)
QWEN7_STACK_ISOLATED = Workload("qwen2.5-7b-stack28-32k-isolated", 4, hidden=3584,
                                n_q_heads=28, n_kv_heads=4, head_dim=128,
                                intermediate=18944, n_layers=28, n_tokens=32768,
                                block_size=512, dtype="bf16", alpha=-1.5, beta=-3.0,
                                support="isolated", budget_percent=2.0)
QWEN15_STACK_DEGENERATE = Workload("qwen2.5-1.5b-stack28-16k-degenerate", 5, hidden=1536,
                                   n_q_heads=12, n_kv_heads=2, head_dim=128,
                                   intermediate=8960, n_layers=28, n_tokens=16384,
                                   block_size=256, dtype="bf16", alpha=0.0, beta=0.0,
                                   tau=128)

# Qwen3-8B-shaped stacks at the execution-benchmark geometry of Budgeted
# KV-Cache Repair, section 13.3 (Table 18): 36 layers, B = 64 selected
# positions in R = 1, 4 or 16 equal intervals, N = 2048 or 8192.  The
# intervals are centred at (k + 1/2) N / R, so the mean selected position is
# (N - 1) / 2 and sum(u + 1) is the same for every R at one N (65,568 at 2K,
# 262,176 at 8K, as the section states).  Q/K normalisation of that model is
# not part of this path's operator set; the shape is used for timing.
def _qwen3_8b(n_tokens: int, n_intervals: int) -> Workload:
    return Workload(f"qwen3-8b-stack36-{n_tokens // 1024}k-b64-r{n_intervals}", 6, hidden=4096,
                    n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=12288, n_layers=36,
                    n_tokens=n_tokens, block_size=n_tokens, dtype="bf16", alpha=-1.0, beta=-2.0,
                    support="intervals", support_len=64, n_intervals=n_intervals)


TABLE18 = [_qwen3_8b(n, r) for n in (2048, 8192) for r in (1, 4, 16)]

# Inference mode (attention only, no write-back) at decode sizes: the last
# B = support_len positions query the 7B mixed cache (seam geometry flags).
QWEN7_DECODE_16K = Workload("qwen2.5-7b-decode-16k", 7, hidden=3584, n_q_heads=28, n_kv_heads=4,
                            head_dim=128, intermediate=18944, n_layers=1, n_tokens=16384,
                            block_size=256, dtype="bf16", alpha=-1.0, beta=-2.0,
                            support="suffix", support_len=8)
QWEN7_DECODE_32K = Workload("qwen2.5-7b-decode-32k", 8, hidden=3584, n_q_heads=28, n_kv_heads=4,
                            head_dim=128, intermediate=18944, n_layers=1, n_tokens=32768,
                            block_size=512, dtype="bf16", alpha=-1.5, beta=-3.0,
                            support="suffix", support_len=8)
# Shift (deletion + positional correction) over a 28-layer 7B cache: the
# span [support_start, support_start + support_len) is deleted.
QWEN7_SHIFT = Workload("qwen2.5-7b-shift28-16k", 9, hidden=3584, n_q_heads=28, n_kv_heads=4,
                       head_dim=128, intermediate=18944, n_layers=28, n_tokens=16384,
                       block_size=256, dtype="bf16", alpha=-1.0, beta=-2.0, support="span",
                       support_start=4096, support_len=1024)

WORKLOADS = {w.name: w for w in (TINY, QWEN15_LAYER, QWEN7_LAYER_SEAMS, QWEN7_LAYER_CONTIG,
                                 QWEN7_LAYER_MATCHED, QWEN7_STACK_ISOLATED,
                                 QWEN15_STACK_DEGENERATE, *TABLE18, QWEN7_DECODE_16K,
                                 QWEN7_DECODE_32K, QWEN7_SHIFT)}


# ----------------------------------------------------------------------------
# bf16 helpers (storage format of the generated values, not method arithmetic)
# ----------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Chunked, thread-parallel standard normals
# ----------------------------------------------------------------------------
def _normal_chunks(key: Tuple[int, ...], n: int, out: np.ndarray, threads: int,
                   scale: float = 1.0, offset: float = 0.0, bf16: bool = False) -> None:
    """Fill ``out`` with N(offset, scale^2) draws chunk by chunk (optionally
    bf16-rounded); chunks are spread over threads, numpy releases the GIL."""
    nchunks = (n + CHUNK - 1) // CHUNK
    nthreads = max(1, min(threads, nchunks))

    def work(c0: int) -> None:
        for c in range(c0, nchunks, nthreads):
            lo = c * CHUNK
            hi = min(n, lo + CHUNK)
            g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key) + [c])))
            x = g.standard_normal(hi - lo, dtype=np.float32)
            if scale != 1.0:
                x *= np.float32(scale)
            if offset != 0.0:
                x += np.float32(offset)
            out[lo:hi] = bf16_round(x) if bf16 else x

    if nthreads == 1:
        work(0)
        return
    ts = [threading.Thread(target=work, args=(i,)) for i in range(nthreads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()


def default_threads() -> int:
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(w: Workload, layer: int, tensor: int, shape, scale: float = 1.0,
           offset: float = 0.0, threads: Optional[int] = None) -> np.ndarray:
    """Seeded N(offset, scale^2) tensor in float32, bf16-rounded for bf16 workloads."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _normal_chunks((SEED_ROOT, w.cfg_id, layer, tensor), n, out,
                   threads if threads is not None else default_threads(), scale, offset,
                   w.dtype == "bf16")
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# Inputs of one workload
# ----------------------------------------------------------------------------
def blocks(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Uniform block partition of [0, N): starts s_i and (exclusive) ends e_i."""
    s = np.arange(0, w.n_tokens, w.block_size, dtype=np.int32)
    e = np.minimum(s + w.block_size, w.n_tokens).astype(np.int32)
    return s, e


def initial_flags(w: Workload, s: Optional[np.ndarray] = None,
                  e: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-position metadata bits at load: LOCAL outside block 1, SINK on the
    first token of every block after the first."""
    if s is None:
        s, e = blocks(w)
    f = np.zeros(w.n_tokens, dtype=np.uint8)
    f[e[0]:] |= FLAG_LOCAL
    f[s[1:]] |= FLAG_SINK
    return f


def block_ids(w: Workload) -> np.ndarray:
    s, e = blocks(w)
    b = np.zeros(w.n_tokens, dtype=np.int32)
    for i, (a, z) in enumerate(zip(s, e)):
        b[a:z] = i
    return b


def hidden_states(w: Workload, threads: Optional[int] = None) -> np.ndarray:
    """Layer-0 input X [N, hidden] ~ N(0,1).  Activations are float32 at the
    boundary, so X is never bf16-rounded."""
    n = w.n_tokens * w.hidden
    out = np.empty(n, dtype=np.float32)
    _normal_chunks((SEED_ROOT, w.cfg_id, 0, T_X), n, out,
                   threads if threads is not None else default_threads())
    return out.reshape(w.n_tokens, w.hidden)


def queries(w: Workload, B: int, threads: Optional[int] = None) -> np.ndarray:
    """Post-RoPE queries [B, Hq, d] ~ N(0,1) handed to inference-mode
    attention; float32 at the boundary (never bf16-rounded)."""
    n = B * w.n_q_heads * w.head_dim
    out = np.empty(n, dtype=np.float32)
    _normal_chunks((SEED_ROOT, w.cfg_id, 0, T_QUERY), n, out,
                   threads if threads is not None else default_threads())
    return out.reshape(B, w.n_q_heads, w.head_dim)


def kv_cache(w: Workload, layer: int, threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Retained cache of one layer: K, V [N, Hkv, d] ~ N(0,1)."""
    shp = (w.n_tokens, w.n_kv_heads, w.head_dim)
    return (normal(w, layer, T_KCACHE, shp, threads=threads),
            normal(w, layer, T_VCACHE, shp, threads=threads))


def layer_weights(w: Workload, layer: int, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Weights of one decoder layer, PyTorch Linear layout [out, in]."""
    h, qd, kd, it = w.hidden, w.q_dim, w.kv_dim, w.intermediate
    f32 = w.with_(dtype="f32")   # norm gains and biases stay float32
    d = {
        "attn_norm": normal(f32, layer, T_ATTN_NORM, (h,), 0.02, 1.0, threads),
        "wq": normal(w, layer, T_WQ, (qd, h), 0.02, threads=threads),
        "wk": normal(w, layer, T_WK, (kd, h), 0.02, threads=threads),
        "wv": normal(w, layer, T_WV, (kd, h), 0.02, threads=threads),
        "wo": normal(w, layer, T_WO, (h, qd), 0.02, threads=threads),
        "mlp_norm": normal(f32, layer, T_MLP_NORM, (h,), 0.02, 1.0, threads),
        "w_gate": normal(w, layer, T_WGATE, (it, h), 0.02, threads=threads),
        "w_up": normal(w, layer, T_WUP, (it, h), 0.02, threads=threads),
        "w_down": normal(w, layer, T_WDOWN, (h, it), 0.02, threads=threads),
    }
    if w.qkv_bias:
        d["bq"] = normal(f32, layer, T_BQ, (qd,), 0.5, threads=threads)
        d["bk"] = normal(f32, layer, T_BK, (kd,), 0.5, threads=threads)
        d["bv"] = normal(f32, layer, T_BV, (kd,), 0.5, threads=threads)
    return d


def budget_count(S: int, percent: float) -> int:
    """Size of a budgeted support over an S-position suffix: the exact budget
    min(S, ceil(S * percent / 100)) of Budgeted KV-Cache Repair, section 7.1,
    Eq. 3, in integers (percent with at most three decimals)."""
    num = S * int(round(percent * 1000))
    return min(S, -(-num // 100000))


def isolated_support(w: Workload) -> np.ndarray:
    """Budgeted set of pairwise non-adjacent single positions after block 1.

    B = min(S, ceil(S*b/100)) with S = N - |B_1| (budget on the retained
    suffix).  A uniformly random non-adjacent B-subset of [e_1, N) is drawn
    through the stars-and-bars bijection: B distinct values from
    [0, S - B + 1), sorted, then position = e_1 + value + rank.
    """
    s, e = blocks(w)
    S = w.n_tokens - int(e[0])
    B = budget_count(S, w.budget_percent)
    if B > (S + 1) // 2:
        raise ValueError("budget too large for a non-adjacent support")
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_ROOT, w.cfg_id, 0, T_SUPPORT])))
    v = np.sort(g.choice(S - B + 1, size=B, replace=False))
    return (int(e[0]) + v + np.arange(B)).astype(np.int32)


def explicit_support(w: Workload) -> Optional[np.ndarray]:
    """Support of workloads that do not use seam windows (None for seams)."""
    if w.support == "seams":
        return None
    if w.support in ("contiguous", "matched"):
        return np.arange(w.support_start, w.support_start + w.support_len, dtype=np.int32)
    if w.support == "isolated":
        return isolated_support(w)
    if w.support == "intervals":
        return interval_support(w.n_tokens, w.support_len, w.n_intervals)
    if w.support == "suffix":
        return np.arange(w.n_tokens - w.support_len, w.n_tokens, dtype=np.int32)
    raise ValueError(w.support)


def interval_support(n_tokens: int, B: int, R: int) -> np.ndarray:
    """R equal runs of B/R positions centred at (k + 1/2) * N / R."""
    ln = B // R
    if ln * R != B or (n_tokens // R) < ln:
        raise ValueError("B must split into R runs that fit their N/R slots")
    out = []
    for k in range(R):
        c = (2 * k + 1) * n_tokens // (2 * R)
        out.extend(range(c - ln // 2, c - ln // 2 + ln))
    return np.array(out, dtype=np.int32)


def random_partition(rng: np.random.Generator, n_tokens: int, m: int) -> Tuple[np.ndarray, np.ndarray]:
    """A random partition of [0, n_tokens) into m non-empty blocks."""
    cuts = np.sort(rng.choice(np.arange(1, n_tokens), size=m - 1, replace=False)) if m > 1 else \
        np.zeros(0, dtype=np.int64)
    s = np.concatenate([[0], cuts]).astype(np.int32)
    e = np.concatenate([cuts, [n_tokens]]).astype(np.int32)
    return s, e


# ----------------------------------------------------------------------------
# Semantic-Unit Refresh scoring inputs
# ----------------------------------------------------------------------------
T_EMBED, T_SUR_IDS = 32, 33


@dataclass(frozen=True)
class SurWorkload:
    """Synthetic stand-in for SUR's inputs (Budgeted KV-Cache Repair, 7.3):
    a frozen embedding table, the retained suffix's token ids, the query's
    token ids and the suffix's partition into units.  Units have lengths in
    [8, 128], the range the page's split / merge rules leave."""
    name: str
    cfg_id: int
    vocab: int
    hidden: int
    n_suffix: int
    n_query: int
    budget_percent: float
    dtype: str = "bf16"
    pos0: int = 0


SUR_TINY = SurWorkload("sur-tiny-f32", 40, vocab=300, hidden=128, n_suffix=700, n_query=5,
                       budget_percent=10.0, dtype="f32", pos0=64)
SUR_QWEN7_16K = SurWorkload("sur-qwen2.5-7b-16k", 41, vocab=152064, hidden=3584, n_suffix=16384,
                            n_query=48, budget_percent=5.0, pos0=0)
SUR_WORKLOADS = {w.name: w for w in (SUR_TINY, SUR_QWEN7_16K)}


def embedding_table(w: SurWorkload, threads: Optional[int] = None) -> np.ndarray:
    """[vocab, hidden] ~ N(0, 1), bf16-rounded for bf16 workloads."""
    n = w.vocab * w.hidden
    out = np.empty(n, dtype=np.float32)
    _normal_chunks((SEED_ROOT, w.cfg_id, 0, T_EMBED), n, out,
                   threads if threads is not None else default_threads(), 1.0, 0.0,
                   w.dtype == "bf16")
    return out.reshape(w.vocab, w.hidden)


def sur_ids(w: SurWorkload) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(suffix ids [S], query ids [Q], unit starts): uniform token ids; half
    of the query tokens are copied from the suffix (so some suffix tokens
    occur in the query); unit lengths uniform in [8, 128]."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_ROOT, w.cfg_id, 0, T_SUR_IDS])))
    s = g.integers(0, w.vocab, size=w.n_suffix, dtype=np.int64).astype(np.int32)
    q = g.integers(0, w.vocab, size=w.n_query, dtype=np.int64).astype(np.int32)
    k = w.n_query // 2
    q[:k] = s[g.choice(w.n_suffix, size=k, replace=False)]
    starts = [0]
    while True:
        nxt = starts[-1] + int(g.integers(8, 129))
        if nxt >= w.n_suffix:
            break
        starts.append(nxt)
    return s, q, np.array(starts, dtype=np.int32)


def sur_budget(w: SurWorkload) -> int:
    """Budget of the SUR workload over its suffix (see budget_count)."""
    return budget_count(w.n_suffix, w.budget_percent)
