"""The C ABI without a GPU: libgdn.so loads, exports every function that
include/gdn.h declares, and rejects invalid calls during host-side
validation (nothing is enqueued, no device memory is touched).

The validation cases pass placeholder addresses for device buffers; every
case is built to fail validation, and the tests that make such calls are
skipped whenever a GPU is visible so that a validation bug can never turn
into a launch on bogus pointers.
"""
import ctypes
import os
import subprocess
import threading

import numpy as np
import pytest
import torch

import gated_deltanet_linear_causal_amd as gdn

OK, EINVAL, EUNSUP, EWS = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return gdn.load_library()


def test_library_exports_every_header_function(lib):
    names = gdn.header_functions()
    assert set(names) == {"gdn_conv_update", "gdn_decode_step", "gdn_decode_multi",
                          "gdn_rewind", "gdn_prefill_workspace_bytes",
                          "gdn_prefill_chunked", "gdn_prefill_chunked_noalloc",
                          "gdn_mixer_workspace_bytes",
                          "gdn_mixer_prefill", "gdn_mixer_decode", "gdn_status_string",
                          "gdn_last_error"}
    dyn = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in dyn.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(names) == set(gdn._SIGNATURES)


def test_status_strings(lib):
    for code, name in gdn.STATUS.items():
        assert lib.gdn_status_string(code).decode() == name
    assert lib.gdn_status_string(99).decode() == "GDN_UNKNOWN"


def _cfg(**kw):
    base = dict(h_k=2, h_v=4, d_k=64, d_v=64, conv_k=4, act_dtype=0, out_dtype=1, gate=0,
                norm_eps=1e-6, l2_eps=1e-6, head_map=0, decay_mode=0)
    base.update(kw)
    return gdn._Config(**base)


def test_workspace_bytes(lib):
    c = _cfg()
    w0 = lib.gdn_prefill_workspace_bytes(ctypes.byref(c), 1, 0, 64)
    w1 = lib.gdn_prefill_workspace_bytes(ctypes.byref(c), 1, 100, 64)
    w2 = lib.gdn_prefill_workspace_bytes(ctypes.byref(c), 1, 200, 64)
    assert w0 == 0 and 0 < w1 < w2
    assert w1 % 256 == 0
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(c), 1, 100, 32) == 0
    bad = _cfg(h_v=3)
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(bad), 1, 100, 64) == 0
    assert lib.gdn_prefill_workspace_bytes(None, 1, 100, 64) == 0
    # one decay per key channel: q/k operands per value head, plus W's k operand
    kda = _cfg(decay_mode=1)
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(kda), 1, 100, 64) > w1


no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="placeholder device pointers are only passed where no GPU exists")

# distinct placeholder device addresses, far apart (never dereferenced)
_P = [ctypes.c_void_p(0x10000000000 * (i + 1)) for i in range(16)]


def _params():
    return gdn._Params(_P[10].value, _P[11].value, _P[12].value, _P[13].value, None)


def _decode(lib, cfg=None, params=None, batch=2, ptrs=None):
    p = _P[:7] if ptrs is None else ptrs
    c = cfg or _cfg()
    pr = params if params is not None else _params()
    return lib.gdn_decode_step(ctypes.byref(c), ctypes.byref(pr) if pr is not False else None,
                               batch, *p, None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(h_v=3), EINVAL), (dict(h_k=0), EINVAL), (dict(d_k=48), EUNSUP),
    (dict(d_v=256), EUNSUP), (dict(conv_k=5), EUNSUP), (dict(conv_k=0), EINVAL),
    (dict(act_dtype=7), EINVAL), (dict(gate=2), EINVAL), (dict(norm_eps=-1.0), EINVAL),
    (dict(l2_eps=float("nan")), EINVAL), (dict(head_map=2), EINVAL),
    (dict(decay_mode=2), EINVAL), (dict(state_cache=2), EINVAL), (dict(state_cache=-1), EINVAL)])
def test_decode_rejects_bad_config(lib, kw, code):
    assert _decode(lib, _cfg(**kw)) == code
    assert lib.gdn_last_error().decode() != ""


@no_gpu
def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, params=False) == EINVAL
    assert _decode(lib, params=gdn._Params(0, _P[11].value, _P[12].value, _P[13].value,
                                           None)) == EINVAL
    # exactly one of a_log and decay_coef
    assert _decode(lib, params=gdn._Params(_P[10].value, _P[11].value, _P[12].value,
                                           _P[13].value, _P[15].value)) == EINVAL
    assert "a_log" in lib.gdn_last_error().decode()
    assert _decode(lib, params=gdn._Params(_P[10].value, None, _P[12].value,
                                           _P[13].value, None)) == EINVAL
    # conv_w and norm_w are read in 16-byte rows
    assert _decode(lib, params=gdn._Params(_P[10].value + 4, _P[11].value, _P[12].value,
                                           _P[13].value, None)) == EINVAL
    assert "16-byte" in lib.gdn_last_error().decode()
    assert _decode(lib, params=gdn._Params(_P[10].value, _P[11].value, _P[12].value,
                                           _P[13].value + 8, None)) == EINVAL
    assert _decode(lib, batch=-1) == EINVAL
    assert _decode(lib, ptrs=[None] + _P[1:7]) == EINVAL
    # out aliasing the state
    assert _decode(lib, ptrs=_P[:5] + [_P[5], _P[5]]) == EINVAL
    # state overlapping qkv
    assert _decode(lib, ptrs=_P[:5] + [_P[0], _P[6]]) == EINVAL
    assert "overlap" in lib.gdn_last_error().decode()
    # batch 0 is accepted without touching anything
    assert _decode(lib, batch=0) == OK


def _multi(lib, cfg=None, batch=2, t_new=4, ptrs=None):
    # n_tok, qkv, z, a, b, conv_in, conv_out, state_in, state_out, ckpt, out
    p = [None] + _P[:4] + [_P[4], _P[5], _P[6], _P[7], None, _P[8]] if ptrs is None else ptrs
    c = cfg or _cfg()
    return lib.gdn_decode_multi(ctypes.byref(c), ctypes.byref(_params()), batch, t_new, *p, None)


def _rewind(lib, cfg=None, batch=2, t_rec=4, ptrs=None):
    # keep, qkv, a, b, state0, conv0, state, conv_state
    p = [None, _P[0], _P[2], _P[3], _P[6], _P[4], _P[7], _P[5]] if ptrs is None else ptrs
    c = cfg or _cfg()
    return lib.gdn_rewind(ctypes.byref(c), ctypes.byref(_params()), batch, t_rec, *p, None)


@no_gpu
def test_decode_multi_and_rewind_reject_bad_arguments(lib):
    assert _multi(lib, t_new=0) == EUNSUP
    assert _multi(lib, t_new=9) == EUNSUP
    assert "tokens per sequence" in lib.gdn_last_error().decode()
    # 8 tokens of a wide group do not fit the on-chip buffer
    assert _multi(lib, cfg=_cfg(h_k=1, h_v=16, d_k=128, d_v=128), t_new=8) == EUNSUP
    assert _multi(lib, batch=-1) == EINVAL
    assert _multi(lib, batch=0) == OK
    base = [None] + _P[:4] + [_P[4], _P[5], _P[6], _P[7], None, _P[8]]
    # qkv missing
    assert _multi(lib, ptrs=base[:1] + [None] + base[2:]) == EINVAL
    # z missing while out is requested
    assert _multi(lib, ptrs=base[:2] + [None] + base[3:]) == EINVAL
    # out aliasing state_out
    assert _multi(lib, ptrs=base[:10] + [_P[7]]) == EINVAL
    # checkpoints overlapping the input state
    assert _multi(lib, ptrs=base[:9] + [_P[6]] + base[10:]) == EINVAL
    # state_out partially overlapping state_in
    assert _multi(lib, ptrs=base[:8] + [ctypes.c_void_p(_P[6].value + 4)] + base[9:]) == EINVAL
    assert _rewind(lib, t_rec=9) == EUNSUP
    assert _rewind(lib, ptrs=[None, _P[0], _P[2], _P[3], None, _P[4], _P[7], _P[5]]) == EINVAL
    # the rewound state must not overlap the recorded inputs
    assert _rewind(lib, ptrs=[None, _P[0], _P[2], _P[3], _P[6], _P[4], _P[0], _P[5]]) == EINVAL
    assert _rewind(lib, batch=0) == OK


def _proj(hidden=64, **kw):
    base = dict(hidden=hidden, w_qkv=_P[10].value, w_z=_P[11].value, w_b=_P[12].value,
                w_a=_P[13].value, w_out=_P[15].value)
    base.update(kw)
    return gdn._Proj(**base)


@no_gpu
def test_mixer_rejects_bad_arguments(lib):
    c = _cfg()
    assert lib.gdn_mixer_workspace_bytes(ctypes.byref(c), 64, 1, 100) > \
        lib.gdn_prefill_workspace_bytes(ctypes.byref(c), 1, 100, 64)
    assert lib.gdn_mixer_workspace_bytes(ctypes.byref(c), 60, 1, 100) == 0

    def dec(cfg=None, proj=None, batch=2, ptrs=None, ws=(_P[9], 1 << 40)):
        p = ptrs or [_P[0], _P[4], _P[5], _P[6]]   # x, conv_state, state, y
        return lib.gdn_mixer_decode(ctypes.byref(cfg or c), ctypes.byref(_params()),
                                    ctypes.byref(proj or _proj()), batch, *p, ws[0], ws[1], None)
    assert dec(proj=_proj(hidden=60)) == EINVAL
    assert dec(proj=_proj(w_out=None)) == EINVAL
    assert dec(cfg=_cfg(act_dtype=1)) == EUNSUP
    assert dec(ws=(_P[9], 10)) == EWS
    assert dec(ptrs=[_P[0], _P[4], _P[5], _P[0]]) == EINVAL   # y aliasing x
    assert dec(batch=0) == OK
    cu = np.asarray([0, 10], dtype=np.int32)
    st = lib.gdn_mixer_prefill(ctypes.byref(c), ctypes.byref(_params()), ctypes.byref(_proj()),
                               1, 10, cu.ctypes.data_as(ctypes.c_void_p), _P[14], _P[0], _P[4],
                               _P[5], _P[6], _P[7], _P[0], _P[9], 1 << 40, None)
    assert st == EINVAL and "overlap" in lib.gdn_last_error().decode()


def _prefill(lib, cu, t_total, cfg=None, chunk=64, ws=(_P[9], 1 << 40), outs=None, qkv=_P[0],
             a=_P[2]):
    c = cfg or _cfg()
    cu_h = np.asarray(cu, dtype=np.int32)
    n = len(cu) - 1
    o = outs or dict(state_in=_P[4], state_out=_P[5], conv_in=_P[6], conv_out=_P[7], out=_P[8])
    return lib.gdn_prefill_chunked(
        ctypes.byref(c), ctypes.byref(_params()), chunk, n, t_total,
        cu_h.ctypes.data_as(ctypes.c_void_p), _P[14], qkv, _P[1], a, _P[3],
        o["state_in"], o["state_out"], o["conv_in"], o["conv_out"], o["out"], ws[0],
        ws[1], None)


@no_gpu
def test_prefill_rejects_bad_cu_seqlens(lib):
    assert _prefill(lib, [1, 5], 5) == EINVAL          # does not start at 0
    assert _prefill(lib, [0, 5, 3], 3) == EINVAL       # decreasing
    assert _prefill(lib, [0, 5, 9], 10) == EINVAL      # does not end at t_total
    assert "cu_seqlens" in lib.gdn_last_error().decode()


@no_gpu
def test_prefill_rejects_chunk_workspace_and_aliases(lib):
    assert _prefill(lib, [0, 10], 10, chunk=32) == EUNSUP
    assert _prefill(lib, [0, 10], 10, ws=(_P[9], 100)) == EWS
    assert _prefill(lib, [0, 10], 10, ws=(None, 1 << 40)) == EWS
    assert _prefill(lib, [0, 10], 10, ws=(ctypes.c_void_p(_P[9].value + 8), 1 << 40)) == EINVAL
    o = dict(state_in=_P[4], state_out=_P[5], conv_in=_P[6], conv_out=_P[7], out=_P[0])
    assert _prefill(lib, [0, 10], 10, outs=o) == EINVAL   # out overlaps qkv
    o = dict(state_in=_P[4], state_out=ctypes.c_void_p(_P[4].value + 4), conv_in=_P[6],
             conv_out=_P[7], out=_P[8])
    assert _prefill(lib, [0, 10], 10, outs=o) == EINVAL   # partial state overlap
    # activations are read in 16-byte pieces
    assert _prefill(lib, [0, 10], 10, qkv=ctypes.c_void_p(_P[0].value + 8)) == EINVAL
    assert "16-byte" in lib.gdn_last_error().decode()
    # with one decay per key channel a ([T][H_v*d_k]) is read in 16-byte rows too
    assert _prefill(lib, [0, 10], 10, cfg=_cfg(decay_mode=1), a=ctypes.c_void_p(_P[2].value + 2)) == EINVAL
    assert "16-byte" in lib.gdn_last_error().decode()


def _prefill_noalloc(lib, cu, t_total, cfg=None, chunk=64, outs=None, qkv=_P[0]):
    c = cfg or _cfg()
    cu_h = np.asarray(cu, dtype=np.int32)
    n = len(cu) - 1
    o = outs or dict(state_in=_P[4], state_out=_P[5], conv_in=_P[6], conv_out=_P[7], out=_P[8])
    return lib.gdn_prefill_chunked_noalloc(
        ctypes.byref(c), ctypes.byref(_params()), chunk, n, t_total,
        cu_h.ctypes.data_as(ctypes.c_void_p), _P[14], qkv, _P[1], _P[2], _P[3],
        o["state_in"], o["state_out"], o["conv_in"], o["conv_out"], o["out"], None)


@no_gpu
def test_prefill_noalloc_rejects_calls_beyond_its_scratch(lib):
    """The allocation-free prefill refuses, before anything is enqueued, a
    call whose workspace would not fit its static scratch, and validates
    like gdn_prefill_chunked otherwise."""
    big = _cfg(h_k=16, h_v=32, d_k=128, d_v=128)
    t = 4096
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(big), 1, t, 64) > gdn.PREFILL_NOALLOC_MAX_BYTES
    assert _prefill_noalloc(lib, [0, t], t, cfg=big) == EUNSUP
    assert "scratch" in lib.gdn_last_error().decode()
    assert _prefill_noalloc(lib, [0, 10], 10, chunk=32) == EUNSUP
    assert _prefill_noalloc(lib, [0, 5, 9], 10) == EINVAL
    o = dict(state_in=_P[4], state_out=_P[5], conv_in=_P[6], conv_out=_P[7], out=_P[0])
    assert _prefill_noalloc(lib, [0, 10], 10, outs=o) == EINVAL


@no_gpu
def test_shapes_beyond_the_launch_grids_are_rejected(lib):
    # (token, value head) rows and (sequence, key head) workgroups are counted in 32 bits
    t = (1 << 25) + 64
    assert _prefill(lib, [0, t], t, cfg=_cfg(h_k=16, h_v=32)) == EUNSUP
    assert "t_total * H_v" in lib.gdn_last_error().decode()
    wide = _cfg(h_k=32768, h_v=32768)
    assert _decode(lib, wide, batch=65535) == EUNSUP
    assert "batch * H_k" in lib.gdn_last_error().decode()
    assert _multi(lib, wide, batch=65535, t_new=1) == EUNSUP
    assert "batch * H_k" in lib.gdn_last_error().decode()


def test_last_error_is_thread_local(lib):
    c = _cfg(h_v=3)
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(c), 1, 10, 64) == 0
    seen = {}

    def worker():
        seen["msg"] = lib.gdn_last_error().decode()
    th = threading.Thread(target=worker)
    th.start()
    th.join()
    assert seen["msg"] == ""


def test_config_struct_layout_matches_header():
    """The binding's gdn_config mirrors include/gdn.h field for field (13
    four-byte fields, the cache hint last, zero meaning CACHED)."""
    names = [f[0] for f in gdn._Config._fields_]
    assert names[-1] == "state_cache" and len(names) == 13
    assert ctypes.sizeof(gdn._Config) == 13 * 4
    assert gdn.Config(2, 4, 64, 64).c_struct().state_cache == gdn.GDN_STATE_CACHED
    assert gdn.Config(2, 4, 64, 64, state_cache="streamed").c_struct().state_cache == \
        gdn.GDN_STATE_STREAMED
    with pytest.raises(ValueError):
        gdn.Config(2, 4, 64, 64, state_cache="warm").c_struct()
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "gdn.h")).read()
    body = hdr[hdr.index("typedef struct {\n    int32_t h_k, h_v;"):hdr.index("} gdn_config;")]
    assert "int32_t state_cache;" in body and body.rstrip().endswith("*/")


def test_traffic_counter_hash_covers_every_local_include():
    """The stored HBM traffic counters are keyed by a hash of the measured
    kernels' sources; every local header those kernels include must be part
    of it, or an edit there would leave stale counters in the bench line."""
    import re
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    hashed = {os.path.normpath(p) for p in bench.KERNEL_SOURCES}
    todo = [p for p in bench.KERNEL_SOURCES if p.endswith(".hip")]
    seen = set()
    while todo:
        rel = todo.pop()
        if rel in seen:
            continue
        seen.add(rel)
        with open(os.path.join(root, rel)) as f:
            for inc in re.findall(r'^#include "([^"]+)"', f.read(), re.M):
                dep = os.path.normpath(os.path.join(os.path.dirname(rel), inc))
                if dep.startswith("include" + os.sep):
                    continue  # the public C header: declarations only
                assert dep in hashed, f"{rel} includes {dep}, which the traffic hash does not cover"
                todo.append(dep)
