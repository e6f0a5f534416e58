"""The C-ABI library loads, exports every entry point include/kvr.h declares,
and rejects bad arguments on the host before any device work (these calls
pass fake, aligned addresses that the library must never dereference)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvr.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kvr_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("kvr_build_repair_set", "kvr_check_support", "kvr_build_plan",
              "kvr_workspace_bytes", "kvr_layer_repair", "kvr_stack_repair",
              "kvr_attention_workspace_bytes", "kvr_biased_attention", "kvr_shift_cache",
              "kvr_sur_scores", "kvr_sur_select", "kvr_build_runs", "kvr_build_tile_map",
              "kvr_status_string", "kvr_last_error", "kvr_timing_begin", "kvr_timing_end"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import packed_partial_prefill_amd as kvr
    out = subprocess.run(["nm", "-D", "--defined-only", kvr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        getattr(kvr.lib(), n)


@pytest.fixture(scope="module")
def kvr():
    import packed_partial_prefill_amd as m
    return m


FAKE = 1 << 20   # aligned, never dereferenced: validation fails first


def _cfg(kvr, **kw):
    c = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512,
             rms_eps=1e-6, rope_theta=1e6, alpha=-1.0, beta=-2.0, dtype=kvr.KVR_F32)
    c.update(kw)
    return kvr.kvr_config(**c)


def _w(kvr, **over):
    vals = {n: FAKE for n, _ in kvr.kvr_layer_weights._fields_}
    vals.update(bq=None, bk=None, bv=None)
    vals.update(over)
    return kvr.kvr_layer_weights(**vals)


def _layer(kvr, cfg=None, w=None, B=4, x_rows=4, n_tokens=512, ws_bytes=1 << 40, T=FAKE,
           x_in=FAKE, x_out=FAKE + 4096, flags=FAKE, gpos=None):
    lib = kvr.lib()
    cfg = cfg or _cfg(kvr)
    w = w or _w(kvr)
    meta = kvr.kvr_meta(flags=flags, block_id=None, gpos=gpos, n_tokens=n_tokens)
    return lib.kvr_layer_repair(C.byref(cfg), C.byref(w), kvr.kvr_kv(FAKE, FAKE), C.byref(meta),
                                T, B, x_in, x_rows, x_out, FAKE, ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=96), -2), (dict(n_q_heads=5), -2), (dict(hidden=200), -2),
    (dict(intermediate=500), -2), (dict(alpha=float("nan")), -1), (dict(beta=float("inf")), -1),
    (dict(rms_eps=float("nan")), -1), (dict(dtype=7), -1), (dict(rope_theta=0.0), -1)])
def test_layer_repair_rejects_bad_config(kvr, over, status):
    assert _layer(kvr, cfg=_cfg(kvr, **over)) == status
    assert kvr.kvr_last_error() != ""


def test_layer_repair_rejects_bad_arguments(kvr):
    assert _layer(kvr, B=-1) == -1
    assert _layer(kvr, B=600) == -1                        # B > N
    assert _layer(kvr, x_rows=7) == -1                     # neither B nor N
    assert _layer(kvr, T=None) == -1
    assert _layer(kvr, T=FAKE + 4) == -1                   # misaligned
    assert _layer(kvr, x_in=FAKE, x_out=FAKE, x_rows=512) == -1   # gather into x_in itself
    assert _layer(kvr, w=_w(kvr, wq=None)) == -1
    assert _layer(kvr, w=_w(kvr, bq=FAKE)) == -1           # partial biases
    assert _layer(kvr, ws_bytes=1024) == -6
    assert _layer(kvr, gpos=FAKE + 4, ws_bytes=1024) == -1   # misaligned position map
    assert _layer(kvr, B=0, x_rows=0) == 0                 # no-op success
    assert _layer(kvr, B=0, x_rows=512) == 0


def test_workspace_bytes(kvr):
    lib = kvr.lib()
    c = _cfg(kvr)
    a = lib.kvr_workspace_bytes(C.byref(c), 24, 512)
    b = lib.kvr_workspace_bytes(C.byref(c), 48, 512)
    assert 0 < a < b
    assert lib.kvr_workspace_bytes(C.byref(_cfg(kvr, head_dim=80)), 24, 512) == 0
    assert lib.kvr_workspace_bytes(C.byref(c), 600, 512) == 0


def test_build_repair_set_host_validation(kvr):
    lib = kvr.lib()
    out = kvr.kvr_repair_set(FAKE, FAKE, FAKE, FAKE, 16)
    f = lambda m=2, n=8, tau=1, mode=1, meta=None, s=FAKE: lib.kvr_build_repair_set(
        s, FAKE, m, n, tau, mode, meta, C.byref(out), None, None)
    assert f(m=0) == -3
    assert f(tau=-1) == -1
    assert f(mode=8) == -1
    assert f(s=None) == -1
    assert f(mode=3) == -1                                 # INIT_META without meta
    bad_meta = kvr.kvr_meta(flags=FAKE, block_id=None, gpos=None, n_tokens=9)
    assert f(mode=3, meta=C.byref(bad_meta)) == -1         # meta for another N


def test_check_support_and_plan_host_validation(kvr):
    lib = kvr.lib()
    assert lib.kvr_check_support(FAKE, 5, 4, 0, None, FAKE, None) == -1      # B > N
    assert lib.kvr_check_support(FAKE, 1, 4, 0, None, None, None) == -1      # no result word
    assert lib.kvr_check_support(FAKE, 1, 4, 0, FAKE + 4, FAKE, None) == -1  # misaligned gpos
    assert lib.kvr_build_plan(FAKE, 4, 0, FAKE, FAKE, None) == -1
    assert lib.kvr_build_plan(FAKE, 0, 7, FAKE, FAKE, None) == 0
    assert lib.kvr_build_tile_map(FAKE, 5, 4, FAKE, None) == -1             # B > N
    assert lib.kvr_build_tile_map(FAKE, 0, 0, FAKE, None) == -1             # empty cache
    assert lib.kvr_build_tile_map(FAKE, 3, 40, None, None) == -1            # no output
    assert lib.kvr_build_tile_map(FAKE + 4, 3, 40, FAKE, None) == -1        # misaligned T


def test_build_runs_host_validation(kvr):
    lib = kvr.lib()
    out = kvr.kvr_repair_set(None, FAKE, FAKE, FAKE, 16)
    f = lambda T=FAKE, B=4, n=8, o=out: lib.kvr_build_runs(T, B, n, 0, C.byref(o), None, None)
    assert f(B=-1) == -1
    assert f(B=9) == -1                                    # B > N
    assert f(T=None) == -1
    assert f(T=FAKE + 4) == -1                             # misaligned
    assert f(B=17, n=40) == -1                             # cap < B
    no_counts = kvr.kvr_repair_set(None, FAKE, FAKE, None, 16)
    assert f(o=no_counts) == -1


def test_status_strings(kvr):
    for st, name in kvr.STATUS_NAMES.items():
        assert kvr.kvr_status_string(st) == name


def test_python_binding_has_the_c_names(kvr):
    for n in ("kvr_build_repair_set", "kvr_check_support", "kvr_build_plan",
              "kvr_workspace_bytes", "kvr_layer_repair", "kvr_stack_repair",
              "kvr_attention_workspace_bytes", "kvr_biased_attention", "kvr_shift_cache",
              "kvr_sur_scores", "kvr_sur_select", "kvr_build_runs", "kvr_build_tile_map",
              "kvr_status_string", "kvr_last_error", "kvr_timing_begin", "kvr_timing_end"):
        assert callable(getattr(kvr, n))


def _attn(kvr, cfg=None, B=4, n_tokens=512, q=FAKE, pos=FAKE, o=FAKE + 8192, ws_bytes=1 << 40,
          flags=FAKE, k=FAKE):
    lib = kvr.lib()
    cfg = cfg or _cfg(kvr)
    return lib.kvr_biased_attention(C.byref(cfg), kvr.kvr_kv(k, FAKE), flags, n_tokens, q, pos,
                                    B, o, FAKE, ws_bytes, None)


def test_biased_attention_host_validation(kvr):
    # only the attention fields of the config are read: a zero hidden size is fine
    assert _attn(kvr, cfg=_cfg(kvr, hidden=0, intermediate=0), ws_bytes=16) == -6
    assert _attn(kvr, cfg=_cfg(kvr, head_dim=96)) == -2
    assert _attn(kvr, cfg=_cfg(kvr, n_q_heads=6, n_kv_heads=4)) == -2
    assert _attn(kvr, cfg=_cfg(kvr, alpha=float("nan"))) == -1
    assert _attn(kvr, B=-1) == -1
    assert _attn(kvr, B=513) == -1
    assert _attn(kvr, q=None) == -1
    assert _attn(kvr, pos=FAKE + 4) == -1
    assert _attn(kvr, o=FAKE) == -1                        # o aliases q
    assert _attn(kvr, flags=None) == -1
    assert _attn(kvr, k=None) == -1
    assert _attn(kvr, ws_bytes=16) == -6
    assert _attn(kvr, B=0) == 0
    lib = kvr.lib()
    c = _cfg(kvr)
    a = lib.kvr_attention_workspace_bytes(C.byref(c), 1, 512)
    b = lib.kvr_attention_workspace_bytes(C.byref(c), 64, 512)
    assert 0 < a <= b
    assert lib.kvr_attention_workspace_bytes(C.byref(c), 600, 512) == 0


def _shift(kvr, cfg=None, n_layers=2, n_tokens=100, a=10, d=5, src=None, dst=None, fs=None,
           fd=None, bs=None, bd=None):
    lib = kvr.lib()
    cfg = cfg or _cfg(kvr)
    row = cfg.n_kv_heads * cfg.head_dim * 4              # float32 rows
    span = row * n_tokens
    src = src or [(FAKE + 2 * l * span, FAKE + (2 * l + 1) * span) for l in range(n_layers)]
    base = FAKE + 2 * n_layers * span + 4096
    dst = dst or [(base + 2 * l * span, base + (2 * l + 1) * span) for l in range(n_layers)]
    s_arr = (kvr.kvr_kv * n_layers)(*[kvr.kvr_kv(k, v) for k, v in src])
    d_arr = (kvr.kvr_kv * n_layers)(*[kvr.kvr_kv(k, v) for k, v in dst])
    return lib.kvr_shift_cache(C.byref(cfg), n_layers, s_arr, d_arr, fs, fd, bs, bd, n_tokens,
                               a, d, 0, None)


def test_shift_cache_host_validation(kvr):
    assert _shift(kvr, cfg=_cfg(kvr, head_dim=80)) == -2
    assert _shift(kvr, cfg=_cfg(kvr, rope_theta=-1.0)) == -1
    assert _shift(kvr, n_layers=0) == -1
    assert _shift(kvr, a=-1) == -1
    assert _shift(kvr, d=-1) == -1
    assert _shift(kvr, a=96, d=5) == -1                    # span past the end
    assert _shift(kvr, src=[(None, FAKE), (FAKE, FAKE)]) == -1
    assert _shift(kvr, fs=FAKE) == -1                      # flags src without dst
    assert _shift(kvr, bs=FAKE, bd=FAKE + 8) == -1         # misaligned block ids
    # in place (dst == src) and partial overlaps are refused
    src = [(FAKE, FAKE + (1 << 16)), (FAKE + (2 << 16), FAKE + (3 << 16))]
    assert _shift(kvr, src=src, dst=src) == -1
    dst = [(FAKE + (8 << 16), FAKE + (9 << 16)), (FAKE + (1 << 16) + 512, FAKE + (10 << 16))]
    assert _shift(kvr, src=src, dst=dst) == -1
    assert _shift(kvr, n_tokens=5, a=0, d=5) == 0          # nothing left: no device work


def test_sur_scores_host_validation(kvr):
    lib = kvr.lib()
    f = lambda dt=1, V=100, H=128, S=10, Q=4, E=FAKE, r=FAKE + 4096: lib.kvr_sur_scores(
        E, dt, V, H, FAKE, S, FAKE, Q, r, None)
    assert f(dt=5) == -1
    assert f(V=0) == -1
    assert f(S=-1) == -1
    assert f(Q=0) == -1
    assert f(Q=257) == -1
    assert f(H=100) == -2
    assert f(dt=0, H=8256) == -2                            # float32 rows > 8192
    assert f(E=None) == -1
    assert f(r=FAKE + 4) == -1
    assert f(S=0) == 0


def test_sur_select_host_validation(kvr):
    lib = kvr.lib()
    out = kvr.kvr_repair_set(FAKE, FAKE, FAKE, FAKE, 64)
    def f(S=100, U=5, B=10, pos0=0, ws_bytes=800, out=out, us=FAKE):
        return lib.kvr_sur_select(FAKE, S, us, U, B, pos0, FAKE, C.byref(out), FAKE, ws_bytes,
                                  None, None)
    assert f(S=0) == -1
    assert f(U=0) == -1
    assert f(U=101) == -1                                   # more units than tokens
    assert f(B=-1) == -1
    assert f(B=101) == -1
    assert f(pos0=-3) == -1
    assert f(us=None) == -1
    assert f(out=kvr.kvr_repair_set(FAKE, FAKE, FAKE, FAKE, 5)) == -1   # cap < budget
    assert f(ws_bytes=799) == -6
    assert f(S=10000, U=9000, B=10) == -2                   # too many units for the ranking
