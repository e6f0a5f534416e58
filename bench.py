"""Benchmark of the packed selective-recompute path on one MI355X.

Default: a step is one pass of the whole hot path over one batch — the
repair-set build (T_tau and its runs from the block boundaries) followed by
one repaired layer (plan, gather, RMSNorm, QKV, RoPE + K/V write-back, packed
biased attention, O projection, RMSNorm, gate/up + SwiGLU, down) — on the
7B-shaped single layer at 16K context with seam windows (tau = 6, B = 756,
5% budget).  Inputs are seeded synthetic data, resident in HBM before the
timed region.  The layer is idempotent (the same T is rewritten with the same
fresh K/V each step), so steps repeat the same work.  Prints one JSON line on
stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --schedule interval --workload NAME   # sequential maximal-interval replay
    python bench.py --table18                              # packed vs interval-wise sweep
    python bench.py --op inference                         # inference-mode F at decode sizes
    python bench.py --op shift                             # Shift over the 28-layer 7B cache
    python bench.py --op sur                               # SUR scoring + selection, 16K suffix
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
METRIC = "repaired tokens/sec per layer @5% budget, 16K ctx; attn HBM GB/s vs peak"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def flop_counts(w: wl.Workload, T: np.ndarray):
    """Algorithmic FLOPs per launch of each kernel and KV bytes of attention."""
    B = len(T)
    h, qd, kd, it, d = w.hidden, w.q_dim, w.kv_dim, w.intermediate, w.head_dim
    pairs = int(np.sum(T.astype(np.int64) + 1))          # M(U) = sum(u+1) per head
    es = 2 if w.dtype == "bf16" else 4
    kv_bytes = (int(T.max()) + 1) * w.n_kv_heads * d * 2 * es   # K and V read once
    return {
        "qkv": 2.0 * B * h * (qd + 2 * kd),
        "oproj": 2.0 * B * qd * h,
        "gateup": 2.0 * B * h * 2 * it,
        "down": 2.0 * B * it * h,
        "attn": 4.0 * d * w.n_q_heads * pairs,
        "attn_kv_bytes": float(kv_bytes),
        "attn_q_o_bytes": float(2 * B * qd * es),
        "pairs": pairs,
    }


def profiled_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summaries under profiles/ (scaled by a plain-copy
    calibration), or None when none matches the current kernel sources (each
    summary records the SHA-256 of the sources its counters were taken on)."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        for line in open(path):
            if not line.startswith("traffic "):
                continue
            kv = dict(item.split("=", 1) for item in line.split()[1:])
            if kv.get("kernel") != kernel:
                continue
            h = hashlib.sha256()
            for f in kv["sources"].split(","):
                fp = os.path.join(ROOT, f)
                if not os.path.exists(fp):
                    break
                h.update(open(fp, "rb").read())
            else:
                if h.hexdigest() == kv["sources_sha256"]:
                    return float(kv["bytes_per_launch"])
    return None


def cpu_baseline(w: wl.Workload, T: np.ndarray, min_seconds: float = 10.0, max_reps: int = 12,
                 max_rows: int = 1024) -> dict:
    """The oracle (float64 numpy) on the same workload, on this host's cores:
    one repaired layer (layer 0 of a stack) over the support's first
    min(B, max_rows) rows — exact for those rows, since a repair's first rows
    depend only on keys at or before their positions — repeated until about
    min_seconds of CPU work; the median repetition gives repaired tokens/s
    per layer."""
    import oracle
    from threadpoolctl import threadpool_info
    rows = T[:max_rows].astype(np.int64)
    n = int(rows[-1]) + 1
    wnp = wl.layer_weights(w, 0)
    K0, V0 = wl.kv_cache(w, 0)
    X = wl.hidden_states(w)
    times = []
    t_start = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_start) < min_seconds:
        K, V = K0[:n].astype(np.float64), V0[:n].astype(np.float64)
        f = wl.initial_flags(w)[:n].copy()
        t0 = time.perf_counter()
        oracle.stack_repair(w, [(wnp, K, V)], f, rows, X)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    threads = max(blas, oracle.layer.row_threads())
    what = "all" if len(rows) == len(T) else f"the first {len(rows)} of"
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "nproc": os.cpu_count(), "usable_cpus": usable,
            "cpu_model": cpu_model(),
            "sample": f"{len(times)} one-layer repairs of {w.name} over {what} B={len(T)} rows, "
                      f"float64 numpy oracle ({blas} BLAS threads, attention rows over "
                      f"{oracle.layer.row_threads()} threads), median {dt:.2f} s, "
                      f"{sum(times):.1f} s total"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def first_selectable(w: wl.Workload) -> int:
    """First retained-suffix position (only those are selectable): the end of
    B_1, or 0 for a single-block workload."""
    s, e = wl.blocks(w)
    return int(e[0]) if len(s) > 1 else 0


class Setup:
    """Device inputs of one workload (weights and caches of every layer), its
    support and that support's runs, all taken from the library."""

    def __init__(self, w: wl.Workload, dws=None):
        import torch
        import packed_partial_prefill_amd as kvr
        from workloads.device import cfg_of, dev_cache, dev_weights, workspace
        self.w, self.kvr, self.torch = w, kvr, torch
        self.workspace = workspace
        self.L = w.n_layers
        s, e = wl.blocks(w)
        self.ds, self.de = torch.from_numpy(s).cuda(), torch.from_numpy(e).cuda()
        cap = w.n_tokens
        self.dT_all = torch.empty(cap, dtype=torch.int32, device="cuda")
        self.rs, self.rl = torch.empty_like(self.dT_all), torch.empty_like(self.dT_all)
        self.counts = torch.empty(4, dtype=torch.int32, device="cuda")
        self.flags = torch.from_numpy(wl.initial_flags(w)).cuda()
        self.seams = w.support == "seams"
        self.first = first_selectable(w)
        if self.seams:
            n, R, _ = kvr.kvr_build_repair_set(self.ds, self.de, w.n_tokens, w.tau,
                                               kvr.KVR_SEAM_ASYMMETRIC, self.dT_all, self.rs,
                                               self.rl, self.counts)
            self.dT = self.dT_all[:n]
        else:
            self.dT = torch.from_numpy(wl.explicit_support(w)).cuda()
            n, R, _ = kvr.kvr_build_runs(self.dT, w.n_tokens, self.first, self.rs, self.rl,
                                         self.counts)
        self.T = self.dT.cpu().numpy()
        self.B = len(self.T)
        # the support's maximal runs, as the library coalesced them
        self.runs = [(int(a), int(b)) for a, b in zip(self.rs[:R].cpu().tolist(),
                                                       self.rl[:R].cpu().tolist())]
        self.R = R
        if dws is None:
            dws = []
            for li in range(self.L):
                wnp = wl.layer_weights(w, li)
                dws.append(dev_weights(w, wnp))
                del wnp
        self.dws = dws
        self.caches = []
        for li in range(self.L):
            K0, V0 = wl.kv_cache(w, li)
            self.caches.append(dev_cache(w, K0, V0))
            del K0, V0
        self.X = torch.from_numpy(wl.hidden_states(w)).cuda()
        self.x_out = torch.empty((self.B, w.hidden), dtype=torch.float32, device="cuda")
        self.cfg = cfg_of(w)
        self.ws = workspace(self.cfg, self.B, w.n_tokens)
        self.stream = torch.cuda.current_stream()
        # interval-wise replay: one support tensor and output per run
        self.run_T = [torch.arange(a, a + ln, dtype=torch.int32, device="cuda")
                      for a, ln in self.runs]
        self.run_out = [torch.empty((ln, w.hidden), dtype=torch.float32, device="cuda")
                        for _, ln in self.runs]
        self.run_ws = workspace(self.cfg, max(ln for _, ln in self.runs), w.n_tokens)

    def repair(self, dT, x_out, ws):
        kvr = self.kvr
        if self.L == 1:
            kvr.kvr_layer_repair(self.cfg, self.dws[0], self.caches[0][0], self.caches[0][1],
                                 self.flags, dT, self.X, x_out, ws, stream=self.stream)
        else:
            kvr.kvr_stack_repair(self.cfg, self.dws, self.caches, self.flags, dT, self.X, x_out,
                                 ws, stream=self.stream)

    def step_packed(self):
        """One pass of the hot path: the support and its runs (seam set from
        the block boundaries, or an explicit support checked and coalesced),
        then the repair."""
        kvr = self.kvr
        if self.seams:
            kvr.kvr_build_repair_set(self.ds, self.de, self.w.n_tokens, self.w.tau,
                                     kvr.KVR_SEAM_ASYMMETRIC, self.dT_all, self.rs, self.rl,
                                     self.counts, sync=False, stream=self.stream)
        else:
            kvr.kvr_build_runs(self.dT, self.w.n_tokens, self.first, self.rs, self.rl,
                               self.counts, sync=False, stream=self.stream)
        self.repair(self.dT, self.x_out, self.ws)

    def explicit_step(self, T: np.ndarray):
        """A packed step over another explicit support of the same layer (its
        own output and workspace), for equal-budget comparisons."""
        torch, kvr = self.torch, self.kvr
        dT = torch.from_numpy(np.asarray(T, np.int32)).cuda()
        rs, rl = torch.empty_like(dT), torch.empty_like(dT)
        counts = torch.empty(4, dtype=torch.int32, device="cuda")
        out = torch.empty((len(T), self.w.hidden), dtype=torch.float32, device="cuda")
        ws = self.workspace(self.cfg, len(T), self.w.n_tokens)
        n, R, _ = kvr.kvr_build_runs(dT, self.w.n_tokens, self.first, rs, rl, counts)

        def step():
            kvr.kvr_build_runs(dT, self.w.n_tokens, self.first, rs, rl, counts, sync=False,
                               stream=self.stream)
            self.repair(dT, out, ws)
        return step, R

    def step_interval(self):
        """Sequential maximal-interval replay (Budgeted KV-Cache Repair,
        section 7.1): one full traversal of the layers per run, in order."""
        for dT, out in zip(self.run_T, self.run_out):
            self.repair(dT, out, self.run_ws)

    def time_steps(self, step, steps: int, warmup: int) -> float:
        torch = self.torch
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps



def flushed_trials(st: "Setup", w: wl.Workload, torch, warmup: int = 10, rounds: int = 20,
                   flush_mib: int = 512) -> dict:
    """Median ms per step with the Infinity Cache flushed before every trial
    (a 512 MiB read), for the workload's support and, on the 7B 16K seam
    layer, its two equal-budget contiguous companions on the same layer
    weights and cache (suffix start and matched work), trials of the
    variants in a random order each round (Budgeted KV-Cache Repair,
    section 13.3 protocol: ten warmups, twenty interleaved trials, medians)."""
    import random
    variants = {"packed": (st.step_packed, st.R)}
    if w.name == wl.QWEN7_LAYER_SEAMS.name:
        for comp in (wl.QWEN7_LAYER_CONTIG, wl.QWEN7_LAYER_MATCHED):
            fn, R = st.explicit_step(wl.explicit_support(comp))
            variants[comp.support] = (fn, R)
    scratch = torch.ones((flush_mib << 20) // 4, dtype=torch.int32, device="cuda")
    for fn, _ in variants.values():
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    rng = random.Random(1234)
    times = {k: [] for k in variants}
    names = list(variants)
    for _ in range(rounds):
        rng.shuffle(names)
        for k in names:
            scratch.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            variants[k][0]()
            e1.record()
            e1.synchronize()
            times[k].append(e0.elapsed_time(e1))
    del scratch
    out = {k: {"ms_median": round(float(np.median(v)), 4), "ms_min": round(float(np.min(v)), 4),
               "R": variants[k][1],
               "tokens_per_s": round(st.B / (float(np.median(v)) * 1e-3), 1)}
           for k, v in times.items()}
    out["protocol"] = (f"{warmup} warmups each, {rounds} rounds of randomly ordered trials, "
                       f"{flush_mib} MiB read before every trial, HIP events, medians")
    return out

def run_table18(a) -> int:
    """Packed vs interval-wise refresh at the Table 18 geometry (Qwen3-8B
    shape, 36 layers, B = 64, R = 1/4/16, N = 2K/8K, M(U) matched)."""
    dws = None
    for w in wl.TABLE18:
        log(f"[table18] {w.name}")
        st = Setup(w, dws)
        dws = st.dws
        t_packed = st.time_steps(st.step_packed, a.steps, a.warmup)
        t_interval = st.time_steps(st.step_interval, a.steps, a.warmup)
        print(json.dumps({"workload": w.name, "N": w.n_tokens, "B": st.B, "R": st.R,
                          "layers": st.L, "pairs_per_head": int(np.sum(st.T.astype(np.int64) + 1)),
                          "packed_ms": round(t_packed, 4), "interval_ms": round(t_interval, 4),
                          "interval_over_packed": round(t_interval / t_packed, 3),
                          "unit": "ms per full refresh"}), flush=True)
        del st
    return 0


def _event_trials(torch, fn, trials: int, warmup: int, flush_bytes: int = 0):
    """Median microseconds of fn() over `trials` runs, each bracketed by HIP
    events on the current stream; when flush_bytes > 0 a scratch buffer of
    that size is read before every run (outside the events) so that the
    256 MB Infinity Cache holds none of the operands.  The scratch is read,
    not written: written lines would be dirty, and their write-back as the
    timed call evicts them would be charged to that call."""
    scratch = None
    if flush_bytes:
        scratch = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda")
        scratch.max()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(trials):
        if scratch is not None:
            scratch.max()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    return float(np.median(times))


def run_inference_bench(a) -> int:
    """Inference-mode F (cross-attention reuse page, 6.4): biased attention
    of the last B positions over the 7B mixed cache, no write-back.  HBM-bound
    at decode sizes: the K/V rows 0..u_max are read once per call.  The
    Infinity Cache is flushed before every trial."""
    import torch
    import packed_partial_prefill_amd as kvr
    from workloads.device import cfg_of, dev_cache
    for w in (wl.QWEN7_DECODE_16K, wl.QWEN7_DECODE_32K):
        K0, V0 = wl.kv_cache(w, 0)
        kc, vc = dev_cache(w, K0, V0)
        del K0, V0
        flags = torch.from_numpy(wl.initial_flags(w)).cuda()
        cfg = cfg_of(w)
        for B in (1, 8, 64):
            pos = np.arange(w.n_tokens - B, w.n_tokens, dtype=np.int32)
            dq = torch.from_numpy(wl.queries(w, B)).cuda()
            dpos = torch.from_numpy(pos).cuda()
            o = torch.empty((B, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
            ws = torch.empty(kvr.kvr_attention_workspace_bytes(cfg, B, w.n_tokens),
                             dtype=torch.uint8, device="cuda")
            fn = lambda: kvr.kvr_biased_attention(cfg, kc, vc, flags, dq, dpos, o, ws)
            us = _event_trials(torch, fn, a.steps, a.warmup, flush_bytes=512 << 20)
            kvr.kvr_timing_begin((1 << kvr.KVR_KERNEL_COUNT) - 1)
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            kms, kn = kvr.kvr_timing_end()
            parts = {n: round(kms[i] / kn[i] * 1e3, 2) for i, n in enumerate(kvr.KERNEL_NAMES) if kn[i]}
            kv_bytes = (int(pos.max()) + 1) * w.n_kv_heads * w.head_dim * 2 * 2
            qo_bytes = 2 * B * w.n_q_heads * w.head_dim * 4
            gbs = (kv_bytes + qo_bytes) / (us * 1e-6) / 1e9
            print(json.dumps({"op": "inference_attention", "workload": w.name, "N": w.n_tokens,
                              "B": B, "us": round(us, 2), "hbm_gbps": round(gbs, 1),
                              "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                              "bytes": kv_bytes + qo_bytes, "kernel_us": parts,
                              "flush": "512 MiB read before each trial"}), flush=True)
        del kc, vc
    return 0


def run_shift_bench(a) -> int:
    """Shift (Budgeted KV-Cache Repair, 7.1, Eq. 2) over the 28-layer 7B cache:
    delete [support_start, support_start + support_len), re-rotate the
    suffix keys, move values and metadata.  Pure HBM stream."""
    import torch
    import packed_partial_prefill_amd as kvr
    from workloads.device import cfg_of, dev_cache
    w = wl.QWEN7_SHIFT
    cfg = cfg_of(w)
    a0, d = w.support_start, w.support_len
    n_out = w.n_tokens - d
    src, dst = [], []
    for li in range(w.n_layers):
        K0, V0 = wl.kv_cache(w, li)
        src.append(dev_cache(w, K0, V0))
        dst.append((torch.empty((n_out, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16,
                                device="cuda"),
                    torch.empty((n_out, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16,
                                device="cuda")))
    fs = torch.from_numpy(wl.initial_flags(w)).cuda()
    fd = torch.empty(n_out, dtype=torch.uint8, device="cuda")
    fn = lambda: kvr.kvr_shift_cache(cfg, src, dst, a0, d, flags_src=fs, flags_dst=fd,
                                     mark=kvr.KVR_FLAG_LOCAL)
    us = _event_trials(torch, fn, a.steps, a.warmup)
    row = w.n_kv_heads * w.head_dim * 2 * 2              # K and V bytes of one position
    nbytes = 2 * n_out * row * w.n_layers + 2 * n_out    # read + write, plus flags
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({"op": "shift_cache", "workload": w.name, "N": w.n_tokens,
                      "deleted": [a0, a0 + d], "layers": w.n_layers, "us": round(us, 2),
                      "hbm_gbps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                      "bytes": nbytes}), flush=True)
    return 0


def run_sur_bench(a) -> int:
    """Semantic-Unit Refresh numeric core (Budgeted KV-Cache Repair, 7.3):
    token relevance over the 16K suffix against a Qwen2.5-7B-sized bf16
    embedding table (the gathered rows dominate the traffic), then the
    exact-budget selection.  Infinity Cache flushed before every trial."""
    import torch
    import packed_partial_prefill_amd as kvr
    w = wl.SUR_QWEN7_16K
    log(f"[bench] {w.name}: generating the embedding table")
    dE = torch.from_numpy(wl.embedding_table(w)).to(torch.bfloat16).cuda()
    s, q, starts = wl.sur_ids(w)
    ds, dq = torch.from_numpy(s).cuda(), torch.from_numpy(q).cuda()
    dus = torch.from_numpy(starts).cuda()
    S, U, B = len(s), len(starts), wl.sur_budget(w)
    r = torch.empty(S, dtype=torch.float32, device="cuda")
    uscore = torch.empty(U, dtype=torch.float32, device="cuda")
    T = torch.empty(B, dtype=torch.int32, device="cuda")
    rs, rl = torch.empty_like(T), torch.empty_like(T)
    counts = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = torch.empty(2 * S, dtype=torch.float32, device="cuda")
    score = lambda: kvr.kvr_sur_scores(dE, kvr.KVR_BF16, ds, dq, r)
    select = lambda: kvr.kvr_sur_select(r, dus, B, w.pos0, uscore, T, rs, rl, counts, ws,
                                        sync=False)
    us_score = _event_trials(torch, score, a.steps, a.warmup, flush_bytes=512 << 20)
    us_select = _event_trials(torch, select, a.steps, a.warmup, flush_bytes=512 << 20)
    both = lambda: (score(), select())
    us_both = _event_trials(torch, both, a.steps, a.warmup, flush_bytes=512 << 20)
    row_bytes = w.hidden * 2
    nbytes = S * row_bytes + len(q) * row_bytes + S * 4
    gbs = nbytes / (us_score * 1e-6) / 1e9
    flops = 2.0 * S * len(q) * w.hidden
    print(json.dumps({"op": "sur", "workload": w.name, "vocab": w.vocab, "hidden": w.hidden,
                      "S": S, "Q": len(q), "units": U, "budget": B,
                      "us_scores": round(us_score, 2), "us_select": round(us_select, 2),
                      "us_total": round(us_both, 2), "scores_hbm_gbps": round(gbs, 1),
                      "scores_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                      "scores_tflops": round(flops / (us_score * 1e-6) / 1e12, 2),
                      "bytes": nbytes, "flush": "512 MiB read before each trial"}), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=wl.QWEN7_LAYER_SEAMS.name, choices=sorted(wl.WORKLOADS))
    ap.add_argument("--schedule", default="packed", choices=("packed", "interval"))
    ap.add_argument("--table18", action="store_true")
    ap.add_argument("--op", default="repair", choices=("repair", "inference", "shift", "sur"),
                    help="repair (default, the one-line contract), or the inference-mode "
                         "attention / Shift measurements (JSON lines)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(reference dispatch for scaling FETCH_SIZE / WRITE_SIZE counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the repair path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    torch.cuda.set_device(0)
    if a.table18:
        return run_table18(a)
    if a.op == "inference":
        return run_inference_bench(a)
    if a.op == "shift":
        return run_shift_bench(a)
    if a.op == "sur":
        return run_sur_bench(a)

    w = wl.WORKLOADS[a.workload]
    log(f"[bench] workload {w.name}: generating inputs")
    st = Setup(w)
    kvr = st.kvr
    B, L, T = st.B, st.L, st.T
    step = st.step_packed if a.schedule == "packed" else st.step_interval

    log(f"[bench] B={B} R={st.R} layers={L} schedule={a.schedule}: warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    fc = flop_counts(w, T)
    # per-kernel breakdown from an instrumented pass outside the timed region
    kvr.kvr_timing_begin((1 << kvr.KVR_KERNEL_COUNT) - 1)
    for _ in range(max(3, min(a.steps, 10))):
        step()
    torch.cuda.synchronize()
    kms, klaunch = kvr.kvr_timing_end()
    per_kernel = {name: round(kms[i] / klaunch[i] * 1e3, 2)
                  for i, name in enumerate(kvr.KERNEL_NAMES) if klaunch[i]}   # us per launch
    dom = max((n for n in ("qkv", "oproj", "gateup", "down", "attn") if n in per_kernel),
              key=lambda n: per_kernel[n])
    dom_id = kvr.KERNEL_NAMES.index(dom)

    # timed region: exactly K steps; the dominant kernel's launches are
    # bracketed live by HIP events on the launch stream (library probe)
    kvr.kvr_timing_begin(1 << dom_id)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms, klaunch = kvr.kvr_timing_end()
    ms_per_step = (t1 - t0) * 1e3 / a.steps
    value = B * L / (ms_per_step * 1e-3)      # repaired token-layers per second

    t_dom = kms[dom_id] / klaunch[dom_id] * 1e-3
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    per_layer_dom = kms[dom_id] * 1e-3 / (a.steps * L)   # seconds of the dominant kernel per layer
    achieved = fc[dom] / per_layer_dom / 1e12
    traffic = profiled_traffic(dom) if (a.schedule == "packed" and
                                        w.name == wl.QWEN7_LAYER_SEAMS.name) else None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None if traffic is None else round(traffic),
                "us_per_launch": round(t_dom * 1e6, 2)}

    # attention and the projections, each timed live in its own pass of K
    # steps with only its launches bracketed (HIP events on the launch stream)
    def bracketed(names):
        ids = [kvr.KERNEL_NAMES.index(n) for n in names]
        kvr.kvr_timing_begin(sum(1 << i for i in ids))
        for _ in range(a.steps):
            step()
        torch.cuda.synchronize()
        ms, nl = kvr.kvr_timing_end()
        return {n: ms[i] * 1e3 / (a.steps * L) for n, i in zip(names, ids) if nl[i]}  # us/layer

    attn = None
    t_attn = 0.0
    if a.schedule == "packed":
        at = bracketed(["attn", "attn_merge"])
        t_attn = sum(at.values()) * 1e-6
        gbs = (fc["attn_kv_bytes"] + fc["attn_q_o_bytes"]) / t_attn / 1e9
        tf = fc["attn"] / t_attn / 1e12
        attn = {"us_per_layer": round(t_attn * 1e6, 2),
                "launches_us": {n: round(v, 2) for n, v in at.items()},
                "hbm_gbps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "tflops": round(tf, 2), "mfma_frac": round(tf / peak, 4),
                "pairs_per_head": fc["pairs"], "timing": "live HIP events, attention only"}
    gm = bracketed(["qkv", "oproj", "gateup", "down"])
    gemm_t = sum(gm.values()) * 1e-6
    gemm_tf = (fc["qkv"] + fc["oproj"] + fc["gateup"] + fc["down"]) / gemm_t / 1e12 if gemm_t else 0
    gemm = {"us_per_layer": round(gemm_t * 1e6, 1),
            "launches_us": {n: round(v, 2) for n, v in gm.items()},
            "tflops": round(gemm_tf, 1), "mfma_frac": round(gemm_tf / peak, 4),
            "timing": "live HIP events, projections only"}

    # the pages' protocol with a cold Infinity Cache: ten warmups, then
    # twenty rounds in which the seam step and its two equal-budget
    # contiguous companions run in a random order, each trial after a
    # 512 MiB read flush; medians
    flushed = None
    if a.schedule == "packed" and L == 1:
        flushed = flushed_trials(st, w, torch)
    if a.copy_calib_mib:
        n = a.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {a.copy_calib_mib} MiB read + {a.copy_calib_mib} MiB written")
        del src, dst

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(w, T)

    out = {
        "metric": METRIC,
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "hidden": w.hidden, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "intermediate": w.intermediate, "n_tokens": w.n_tokens, "B": B, "R": st.R,
                   "layers": L, "schedule": a.schedule},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "attn": attn,
        "gemm": gemm,
        "gemm_mfma_frac": round(gemm_tf / peak, 4),
        "flushed": flushed,
        "kernel_us_instrumented": per_kernel,
        "stack_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
