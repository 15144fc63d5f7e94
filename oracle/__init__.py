"""CPU oracle of the Gated DeltaNet mixer core (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It never serves the product path, and
it shares no code with the HIP library.

The arithmetic lives in ``gdn_oracle.c`` (plain C, IEEE double precision,
token by token, following "cherenkov qwen4_exp/cpu.rs" fn deltanet /
fn causal_conv and "oxinfer 0.0.5 src/qwen.rs" DeltaRule::run /
gdn_forward).  ``chunked.py`` holds the chunkwise (UT-transform) form of the
same recurrence in numpy, used only to cross-check the algebra the GPU
prefill is built on.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, library routines, brute force and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("conv_k", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("norm_eps", ctypes.c_double), ("l2_eps", ctypes.c_double),
                ("head_map", ctypes.c_int32), ("decay_mode", ctypes.c_int32)]


@dataclass(frozen=True)
class Shape:
    """Head geometry of one GDN layer."""
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_k: int = 4
    gate: str = "silu"          # "silu" or "sigmoid"
    norm_eps: float = 1e-6
    l2_eps: float = 1e-6
    head_map: str = "grouped"   # "grouped": hv // (H_v/H_k); "tiled": hv % H_k
    decay: str = "head"         # "head": one decay per value head; "channel": per key channel (KDA)

    @property
    def gate_width(self) -> int:
        """Values of `a` and dt_bias per value head."""
        return self.d_k if self.decay == "channel" else 1

    @property
    def conv_dim(self) -> int:
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v

    @property
    def value_dim(self) -> int:
        return self.h_v * self.d_v

    def c_struct(self) -> _Cfg:
        if self.gate not in ("silu", "sigmoid"):
            raise ValueError(f"unknown gate {self.gate!r}")
        if self.head_map not in ("grouped", "tiled"):
            raise ValueError(f"unknown head_map {self.head_map!r}")
        if self.decay not in ("head", "channel"):
            raise ValueError(f"unknown decay {self.decay!r}")
        return _Cfg(self.h_k, self.h_v, self.d_k, self.d_v, self.conv_k,
                    1 if self.gate == "sigmoid" else 0,
                    self.norm_eps, self.l2_eps,
                    1 if self.head_map == "tiled" else 0,
                    1 if self.decay == "channel" else 0)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or (
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_delta_core.restype = None
        lib.oracle_delta_core.argtypes = [ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32] + [dp] * 7
        lib.oracle_conv.restype = None
        lib.oracle_conv.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int32, ip,
                                    dp, dp, dp, dp]
        lib.oracle_mixer.restype = ctypes.c_int
        lib.oracle_mixer.argtypes = ([ctypes.POINTER(_Cfg), ctypes.c_int32, ip]
                                     + [dp] * 13
                                     + [ctypes.c_int32] * 3)
        _lib = lib
    return _lib


def _f64(x, shape=None):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        a = a.reshape(shape)
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def delta_core(q, k, v, g, beta, S0):
    """Gated delta rule on one head over L tokens.

    q, k: [L, d_k] already normalised; v: [L, d_v]; g, beta: [L];
    S0: [d_k, d_v].  Returns (o [L, d_v], S_L [d_k, d_v]).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    g, beta = _f64(g), _f64(beta)
    L, dk = q.shape
    dv = v.shape[1]
    S = _f64(S0).copy()
    o = np.zeros((L, dv))
    lib.oracle_delta_core(L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                          _ptr(beta), _ptr(S), _ptr(o))
    return o, S


def conv(shape: Shape, cu_seqlens, conv_w, x, conv0):
    """Standalone causal depthwise conv + SiLU with history carry.

    Returns (c [T, conv_dim], conv_state [N, K-1, conv_dim]).
    """
    lib = _load()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    n = cu.shape[0] - 1
    x = _f64(x)
    st = _f64(conv0).copy()
    c = np.zeros_like(x)
    cfg = shape.c_struct()
    lib.oracle_conv(ctypes.byref(cfg), n, _iptr(cu), _ptr(_f64(conv_w)),
                    _ptr(x), _ptr(st), _ptr(c))
    return c, st


def mixer(shape: Shape, cu_seqlens, params, qkv, z, a, b, S0, conv0,
          heads=None, nthreads=1, want_pre=False):
    """Run the full mixer core on packed sequences.

    params: dict with conv_w [conv_dim, K], dt_bias [H_v], norm_w [d_v] and
    exactly one of a_log [H_v] (coefficient -exp(a_log)) or decay_coef [H_v]
    (the coefficient itself).  S0: [N, H_v, d_k, d_v]; conv0: [N, K-1, conv_dim].
    heads: optional (begin, end) range of value heads to run (others leave
    their y / S entries untouched: y is zero there, S equals S0).
    Returns dict(y, S, conv, o_pre?) as float64 arrays.
    """
    lib = _load()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    n = cu.shape[0] - 1
    T = int(cu[-1])
    qkv = _f64(qkv, (T, shape.conv_dim))
    z = _f64(z, (T, shape.value_dim))
    a = _f64(a, (T, shape.h_v * shape.gate_width))
    b = _f64(b, (T, shape.h_v))
    S = _f64(S0).reshape(n, shape.h_v, shape.d_k, shape.d_v).copy()
    st = _f64(conv0).reshape(n, shape.conv_k - 1, shape.conv_dim).copy()
    y = np.zeros((T, shape.value_dim))
    o_pre = np.zeros((T, shape.value_dim)) if want_pre else None
    h0, h1 = (0, shape.h_v) if heads is None else heads
    cfg = shape.c_struct()
    a_log, coef = params.get("a_log"), params.get("decay_coef")
    if (a_log is None) == (coef is None):
        raise ValueError("give exactly one of a_log and decay_coef")
    a_log = None if a_log is None else _f64(a_log)
    coef = None if coef is None else _f64(coef)
    rc = lib.oracle_mixer(
        ctypes.byref(cfg), n, _iptr(cu),
        _ptr(_f64(params["conv_w"])), _ptr(a_log),
        _ptr(_f64(params["dt_bias"], (shape.h_v * shape.gate_width,))),
        _ptr(_f64(params["norm_w"])),
        _ptr(coef), _ptr(qkv), _ptr(z), _ptr(a), _ptr(b), _ptr(S), _ptr(st), _ptr(y),
        _ptr(o_pre), h0, h1, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_mixer rejected its arguments")
    out = {"y": y, "S": S, "conv": st}
    if want_pre:
        out["o_pre"] = o_pre
    return out


def mixer_layer(shape: Shape, cu_seqlens, params, proj, x, S0, conv0, nthreads=1):
    """The mixer with its projections ("oxinfer 0.0.5 src/qwen.rs", Gdn
    struct and gdn_forward): qkv, z, b, a = x W^T for the four in_proj
    weights (matrix products in float64 with numpy), the mixer core above,
    and out_proj y W_out^T.  proj: hidden and w_qkv [conv_dim, H],
    w_z [value_dim, H], w_b [H_v, H], w_a [H_v * gate_width, H],
    w_out [H, value_dim].  Returns dict(out, y, S, conv)."""
    x = _f64(x)
    qkv = x @ _f64(proj["w_qkv"]).T
    z = x @ _f64(proj["w_z"]).T
    b = x @ _f64(proj["w_b"]).T
    a = x @ _f64(proj["w_a"]).T
    r = mixer(shape, cu_seqlens, params, qkv, z, a, b, S0, conv0, nthreads=nthreads)
    r["out"] = r["y"] @ _f64(proj["w_out"]).T
    return r
