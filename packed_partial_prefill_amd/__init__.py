"""Python binding of libkvr (layer-packed selective recompute on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libkvr.so``.  Tensors are PyTorch device tensors (torch is used for device
memory and streams); each function here has the name of the C entry point it
calls (see include/kvr.h for the full contract) and raises ``KvrError`` on a
non-OK status.  There is no CPU fallback: importing this package without a
built ``libkvr.so`` raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvr.so")

KVR_OK = 0
STATUS_NAMES = {0: "KVR_OK", -1: "KVR_ERR_INVALID_ARGUMENT", -2: "KVR_ERR_UNSUPPORTED",
                -3: "KVR_ERR_BAD_BLOCKS", -4: "KVR_ERR_BAD_SUPPORT", -5: "KVR_ERR_CAPACITY",
                -6: "KVR_ERR_WORKSPACE", -7: "KVR_ERR_HIP"}
KVR_F32, KVR_BF16 = 0, 1
KVR_FLAG_LOCAL, KVR_FLAG_SINK = 1, 2
KVR_SEAM_ASYMMETRIC, KVR_INIT_META = 1, 2
KVR_ATTN_QROWS, KVR_ATTN_KV_TILE = 128, 64
KVR_NOALLOC_SCRATCH_BYTES = 32 << 20
KERNEL_NAMES = ["plan", "norm", "qkv", "rope", "attn", "attn_merge", "oproj", "gateup", "down",
                "final", "qprep", "shift", "sur_score", "sur_select"]
KVR_KERNEL_COUNT = len(KERNEL_NAMES)


class KvrError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m packed_partial_prefill_amd.build`")
_lib = C.CDLL(LIB_PATH)


# ----------------------------------------------------------------- structs
class kvr_config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("intermediate", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_double), ("alpha", C.c_float), ("beta", C.c_float),
                ("dtype", C.c_int)]


class kvr_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo",
                                          "mlp_norm", "w_gate", "w_up", "w_down")]


class kvr_kv(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p)]


class kvr_meta(C.Structure):
    _fields_ = [("flags", C.c_void_p), ("block_id", C.c_void_p), ("gpos", C.c_void_p),
                ("n_tokens", C.c_int32)]


class kvr_repair_set(C.Structure):
    _fields_ = [("T", C.c_void_p), ("run_start", C.c_void_p), ("run_len", C.c_void_p),
                ("counts", C.c_void_p), ("cap", C.c_int32)]


_P = C.c_void_p
_I = C.c_int32
_sigs = {
    "kvr_build_repair_set": (C.c_int, [_P, _P, _I, _I, _I, C.c_uint32, C.POINTER(kvr_meta),
                                       C.POINTER(kvr_repair_set), _P, _P]),
    "kvr_check_support": (C.c_int, [_P, _I, _I, _I, _P, _P, _P]),
    "kvr_build_runs": (C.c_int, [_P, _I, _I, _I, C.POINTER(kvr_repair_set), _P, _P]),
    "kvr_build_plan": (C.c_int, [_P, _I, _I, _P, _P, _P]),
    "kvr_build_tile_map": (C.c_int, [_P, _I, _I, _P, _P]),
    "kvr_workspace_bytes": (C.c_size_t, [C.POINTER(kvr_config), _I, _I]),
    "kvr_layer_repair": (C.c_int, [C.POINTER(kvr_config), C.POINTER(kvr_layer_weights), kvr_kv,
                                   C.POINTER(kvr_meta), _P, _I, _P, _I, _P, _P, C.c_size_t, _P]),
    "kvr_stack_repair": (C.c_int, [C.POINTER(kvr_config), _I, C.POINTER(kvr_layer_weights),
                                   C.POINTER(kvr_kv), C.POINTER(kvr_meta), _P, _I, _P, _I, _P,
                                   _P, C.c_size_t, _P]),
    "kvr_attention_workspace_bytes": (C.c_size_t, [C.POINTER(kvr_config), _I, _I]),
    "kvr_biased_attention": (C.c_int, [C.POINTER(kvr_config), kvr_kv, _P, _I, _P, _P, _I, _P, _P,
                                       C.c_size_t, _P]),
    "kvr_biased_attention_noalloc": (C.c_int, [C.POINTER(kvr_config), kvr_kv, _P, _I, _P, _P, _I,
                                               _P, _P]),
    "kvr_shift_cache": (C.c_int, [C.POINTER(kvr_config), _I, C.POINTER(kvr_kv), C.POINTER(kvr_kv),
                                  _P, _P, _P, _P, _I, _I, _I, C.c_uint8, _P]),
    "kvr_sur_scores": (C.c_int, [_P, C.c_int, _I, _I, _P, _I, _P, _I, _P, _P]),
    "kvr_sur_select": (C.c_int, [_P, _I, _P, _I, _I, _I, _P, C.POINTER(kvr_repair_set), _P,
                                 C.c_size_t, _P, _P]),
    "kvr_status_string": (C.c_char_p, [C.c_int]),
    "kvr_last_error": (C.c_char_p, []),
    "kvr_timing_begin": (C.c_int, [C.c_uint32]),
    "kvr_timing_end": (C.c_int, [C.POINTER(C.c_double), C.POINTER(C.c_int32)]),
}
for _n, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _n)
    _f.restype = _res
    _f.argtypes = _args


def _check(st: int) -> None:
    if st != KVR_OK:
        raise KvrError(st, _lib.kvr_last_error().decode())


# ----------------------------------------------------------------- helpers
def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None for None)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class Config:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    alpha: float = 0.0
    beta: float = 0.0
    dtype: int = KVR_BF16

    def c(self) -> kvr_config:
        return kvr_config(self.hidden, self.n_q_heads, self.n_kv_heads, self.head_dim,
                          self.intermediate, self.rms_eps, self.rope_theta, self.alpha,
                          self.beta, self.dtype)


def _weights_c(w: dict) -> kvr_layer_weights:
    names = ("attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "wo", "mlp_norm", "w_gate", "w_up",
             "w_down")
    return kvr_layer_weights(*[_ptr(w.get(n)) for n in names])


def _meta_c(flags, n_tokens: int, block_id=None, gpos=None) -> kvr_meta:
    return kvr_meta(_ptr(flags), _ptr(block_id), _ptr(gpos), n_tokens)


# ----------------------------------------------------------------- API
def kvr_build_repair_set(d_s, d_e, n_tokens: int, tau: int, mode: int, T, run_start, run_len,
                         counts, flags=None, block_id=None, sync: bool = True,
                         stream=None) -> Optional[Tuple[int, int, int]]:
    """Seam set T_tau, its runs and optional load-time metadata.  Returns
    (|T|, R, status) when ``sync``; otherwise None (counts stay on device)."""
    out = kvr_repair_set(_ptr(T), _ptr(run_start), _ptr(run_len), _ptr(counts), T.numel())
    meta = _meta_c(flags, n_tokens, block_id) if flags is not None else None
    h = (C.c_int32 * 3)() if sync else None
    st = _lib.kvr_build_repair_set(_ptr(d_s), _ptr(d_e), d_s.numel(), n_tokens, tau, mode,
                                   C.byref(meta) if meta is not None else None, C.byref(out),
                                   C.cast(h, C.c_void_p) if h is not None else None,
                                   _stream(stream))
    _check(st)
    return (h[0], h[1], h[2]) if h is not None else None


def kvr_check_support(d_T, n_tokens: int, first_selectable: int, d_result, gpos=None,
                      stream=None) -> None:
    """Support strictly increasing inside [first_selectable, n_tokens) and,
    when given, the global position map non-negative and strictly increasing.
    Synchronises."""
    _check(_lib.kvr_check_support(_ptr(d_T), d_T.numel(), n_tokens, first_selectable,
                                  _ptr(gpos), _ptr(d_result), _stream(stream)))


def kvr_build_runs(d_T, n_tokens: int, first_selectable: int, run_start, run_len, counts,
                   sync: bool = True, stream=None) -> Optional[Tuple[int, int, int]]:
    """Checks an explicit support and coalesces it into maximal runs.
    Returns (B, R, status) when ``sync``; otherwise None."""
    out = kvr_repair_set(None, _ptr(run_start), _ptr(run_len), _ptr(counts),
                         min(run_start.numel(), run_len.numel()))
    h = (C.c_int32 * 3)() if sync else None
    _check(_lib.kvr_build_runs(_ptr(d_T), d_T.numel(), n_tokens, first_selectable, C.byref(out),
                               C.cast(h, C.c_void_p) if h is not None else None,
                               _stream(stream)))
    return (h[0], h[1], h[2]) if h is not None else None


def kvr_build_plan(d_T, group: int, d_n_full, d_n_total, stream=None) -> None:
    _check(_lib.kvr_build_plan(_ptr(d_T), d_T.numel(), group, _ptr(d_n_full), _ptr(d_n_total),
                               _stream(stream)))


def kvr_build_tile_map(d_T, n_tokens: int, d_first_q, stream=None) -> None:
    _check(_lib.kvr_build_tile_map(_ptr(d_T), d_T.numel(), n_tokens, _ptr(d_first_q),
                                   _stream(stream)))


def kvr_workspace_bytes(cfg: Config, B: int, n_tokens: int) -> int:
    c = cfg.c()
    n = _lib.kvr_workspace_bytes(C.byref(c), B, n_tokens)
    if n == 0:
        raise KvrError(-1, "invalid shape for kvr_workspace_bytes")
    return int(n)


def kvr_layer_repair(cfg: Config, weights: dict, k_cache, v_cache, flags, d_T, x_in, x_out, ws,
                     gpos=None, stream=None) -> None:
    c = cfg.c()
    w = _weights_c(weights)
    meta = _meta_c(flags, k_cache.shape[0], gpos=gpos)
    _check(_lib.kvr_layer_repair(C.byref(c), C.byref(w), kvr_kv(_ptr(k_cache), _ptr(v_cache)),
                                 C.byref(meta), _ptr(d_T), d_T.numel(), _ptr(x_in),
                                 x_in.shape[0], _ptr(x_out), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)))


def kvr_stack_repair(cfg: Config, weights: Sequence[dict], caches: Sequence[Tuple], flags, d_T,
                     x_in, x_out, ws, gpos=None, stream=None) -> None:
    c = cfg.c()
    L = len(weights)
    if len(caches) != L:
        raise ValueError("one (k, v) cache per layer")
    ws_arr = (kvr_layer_weights * L)(*[_weights_c(w) for w in weights])
    kv_arr = (kvr_kv * L)(*[kvr_kv(_ptr(k), _ptr(v)) for k, v in caches])
    meta = _meta_c(flags, caches[0][0].shape[0], gpos=gpos)
    _check(_lib.kvr_stack_repair(C.byref(c), L, ws_arr, kv_arr, C.byref(meta), _ptr(d_T),
                                 d_T.numel(), _ptr(x_in), x_in.shape[0], _ptr(x_out), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)))


def kvr_attention_workspace_bytes(cfg: Config, B: int, n_tokens: int) -> int:
    c = cfg.c()
    n = _lib.kvr_attention_workspace_bytes(C.byref(c), B, n_tokens)
    if n == 0:
        raise KvrError(-1, "invalid shape for kvr_attention_workspace_bytes")
    return int(n)


def kvr_biased_attention(cfg: Config, k_cache, v_cache, flags, q, d_pos, o, ws,
                         stream=None) -> None:
    """Inference-mode F: o [B, Hq, d] (float32) = biased attention of the
    post-RoPE queries q [B, Hq, d] (float32) at positions d_pos over the
    cache, without write-back."""
    c = cfg.c()
    _check(_lib.kvr_biased_attention(C.byref(c), kvr_kv(_ptr(k_cache), _ptr(v_cache)),
                                     _ptr(flags), k_cache.shape[0], _ptr(q), _ptr(d_pos),
                                     d_pos.numel(), _ptr(o), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def kvr_biased_attention_noalloc(cfg: Config, k_cache, v_cache, flags, q, d_pos, o,
                                 stream=None) -> None:
    """kvr_biased_attention without a workspace: the library's static
    per-GPU scratch is used (calls that overlap on one GPU race)."""
    c = cfg.c()
    _check(_lib.kvr_biased_attention_noalloc(C.byref(c), kvr_kv(_ptr(k_cache), _ptr(v_cache)),
                                             _ptr(flags), k_cache.shape[0], _ptr(q), _ptr(d_pos),
                                             d_pos.numel(), _ptr(o), _stream(stream)))


def kvr_shift_cache(cfg: Config, src: Sequence[Tuple], dst: Sequence[Tuple], del_start: int,
                    del_len: int, flags_src=None, flags_dst=None, block_src=None,
                    block_dst=None, mark: int = 0, stream=None) -> None:
    """Shift (Eq. 2): dst caches (n_tokens - del_len rows) from src caches
    with [del_start, del_start + del_len) deleted and the suffix keys
    re-rotated; flags / block ids move with their rows."""
    c = cfg.c()
    L = len(src)
    if len(dst) != L:
        raise ValueError("one destination (k, v) per source layer")
    s_arr = (kvr_kv * L)(*[kvr_kv(_ptr(k), _ptr(v)) for k, v in src])
    d_arr = (kvr_kv * L)(*[kvr_kv(_ptr(k), _ptr(v)) for k, v in dst])
    _check(_lib.kvr_shift_cache(C.byref(c), L, s_arr, d_arr, _ptr(flags_src), _ptr(flags_dst),
                                _ptr(block_src), _ptr(block_dst), src[0][0].shape[0], del_start,
                                del_len, mark, _stream(stream)))


def kvr_sur_scores(E, dtype: int, suffix_ids, query_ids, r, stream=None) -> None:
    """Eq. 7 token relevance: r [S] (float32) from the embedding table E
    [vocab, hidden] (bf16 or float32, `dtype`)."""
    _check(_lib.kvr_sur_scores(_ptr(E), dtype, E.shape[0], E.shape[1], _ptr(suffix_ids),
                               suffix_ids.numel(), _ptr(query_ids), query_ids.numel(), _ptr(r),
                               _stream(stream)))


def kvr_sur_select(r, unit_start, budget: int, pos0: int, unit_scores, T, run_start, run_len,
                   counts, ws, sync: bool = True, stream=None) -> Optional[Tuple[int, int, int]]:
    """The selection part of Algorithm 1: returns (|T|, R, status) when ``sync``."""
    out = kvr_repair_set(_ptr(T), _ptr(run_start), _ptr(run_len), _ptr(counts), T.numel())
    h = (C.c_int32 * 3)() if sync else None
    _check(_lib.kvr_sur_select(_ptr(r), r.numel(), _ptr(unit_start), unit_start.numel(), budget,
                               pos0, _ptr(unit_scores), C.byref(out), _ptr(ws),
                               ws.numel() * ws.element_size(),
                               C.cast(h, C.c_void_p) if h is not None else None,
                               _stream(stream)))
    return (h[0], h[1], h[2]) if h is not None else None


def kvr_status_string(st: int) -> str:
    return _lib.kvr_status_string(st).decode()


def kvr_last_error() -> str:
    return _lib.kvr_last_error().decode()


def kvr_timing_begin(mask: int) -> None:
    _check(_lib.kvr_timing_begin(mask))


def kvr_timing_end() -> Tuple[List[float], List[int]]:
    ms = (C.c_double * KVR_KERNEL_COUNT)()
    n = (C.c_int32 * KVR_KERNEL_COUNT)()
    _check(_lib.kvr_timing_end(ms, n))
    return list(ms), list(n)


def lib():
    """The loaded ctypes library (for ABI tests)."""
    return _lib
