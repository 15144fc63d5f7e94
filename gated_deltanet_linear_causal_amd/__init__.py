"""Python binding of libgdn.so, the gfx950 Gated DeltaNet mixer-core library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gdn.h``.  PyTorch provides
device memory and the current stream.  If the library has not been built the
import of any entry point raises: there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "gdn.h")

GDN_BF16, GDN_F32 = 0, 1
GDN_GATE_SILU, GDN_GATE_SIGMOID = 0, 1
GDN_HEADS_GROUPED, GDN_HEADS_TILED = 0, 1
GDN_DECAY_HEAD, GDN_DECAY_CHANNEL = 0, 1
GDN_STATE_CACHED, GDN_STATE_STREAMED = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_EINVAL", 2: "GDN_EUNSUPPORTED",
          3: "GDN_EWORKSPACE", 4: "GDN_EHIP"}
CHUNK = 64


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("conv_k", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("l2_eps", ctypes.c_float),
                ("head_map", ctypes.c_int32), ("decay_mode", ctypes.c_int32),
                ("state_cache", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [("conv_w", ctypes.c_void_p), ("a_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("decay_coef", ctypes.c_void_p)]


class _Proj(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("w_qkv", ctypes.c_void_p), ("w_z", ctypes.c_void_p),
                ("w_b", ctypes.c_void_p), ("w_a", ctypes.c_void_p), ("w_out", ctypes.c_void_p)]


_VP, _I32 = ctypes.c_void_p, ctypes.c_int32
_SIGNATURES = {
    "gdn_conv_update": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                       _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "gdn_decode_step": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                       _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "gdn_decode_multi": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                        _I32, _I32] + [_VP] * 12),
    "gdn_rewind": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                  _I32, _I32] + [_VP] * 9),
    "gdn_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Config), _I32, _I32,
                                                      _I32]),
    "gdn_prefill_chunked": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                           _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP,
                                           _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                           _VP]),
    "gdn_prefill_chunked_noalloc": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                                   _I32, _I32, _I32] + [_VP] * 11 + [_VP]),
    "gdn_mixer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Config), _I32, _I32, _I32]),
    "gdn_mixer_prefill": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                         ctypes.POINTER(_Proj), _I32, _I32] + [_VP] * 9
                          + [ctypes.c_size_t, _VP]),
    "gdn_mixer_decode": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Params),
                                        ctypes.POINTER(_Proj), _I32] + [_VP] * 5
                         + [ctypes.c_size_t, _VP]),
    "gdn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdn_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load_library():
    """Load libgdn.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gated_deltanet_linear_causal_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions declared in include/gdn.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@dataclass(frozen=True)
class Config:
    """Geometry and dtypes of one GDN layer (mirrors gdn_config)."""
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_k: int = 4
    act_dtype: torch.dtype = torch.bfloat16
    out_dtype: torch.dtype = torch.bfloat16
    gate: str = "silu"
    norm_eps: float = 1e-6
    l2_eps: float = 1e-6
    head_map: str = "grouped"   # "grouped" (hv // group) or "tiled" (hv % h_k)
    decay: str = "head"         # "head" (one decay per value head) or "channel" (per key channel)
    # "cached" (the decode state is reread soon, from cache) or "streamed"
    # (evicted in between, e.g. many layers: loaded and stored non-temporally)
    state_cache: str = "cached"

    @property
    def gate_width(self):
        """Values of a and dt_bias per value head."""
        return self.d_k if self.decay == "channel" else 1

    @property
    def conv_dim(self):
        return 2 * self.h_k * self.d_k + self.h_v * self.d_v

    @property
    def value_dim(self):
        return self.h_v * self.d_v

    def c_struct(self) -> _Config:
        def code(dt):
            if dt == torch.bfloat16:
                return GDN_BF16
            if dt == torch.float32:
                return GDN_F32
            raise ValueError(f"unsupported dtype {dt}")
        if self.gate not in ("silu", "sigmoid"):
            raise ValueError(f"unknown gate {self.gate!r}")
        if self.head_map not in ("grouped", "tiled"):
            raise ValueError(f"unknown head_map {self.head_map!r}")
        if self.decay not in ("head", "channel"):
            raise ValueError(f"unknown decay {self.decay!r}")
        if self.state_cache not in ("cached", "streamed"):
            raise ValueError(f"unknown state_cache {self.state_cache!r}")
        return _Config(self.h_k, self.h_v, self.d_k, self.d_v, self.conv_k,
                       code(self.act_dtype), code(self.out_dtype),
                       GDN_GATE_SIGMOID if self.gate == "sigmoid" else GDN_GATE_SILU,
                       self.norm_eps, self.l2_eps,
                       GDN_HEADS_TILED if self.head_map == "tiled" else GDN_HEADS_GROUPED,
                       GDN_DECAY_CHANNEL if self.decay == "channel" else GDN_DECAY_HEAD,
                       GDN_STATE_STREAMED if self.state_cache == "streamed" else GDN_STATE_CACHED)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _params(cfg: Config, p: dict) -> _Params:
    """params: conv_w, dt_bias, norm_w and exactly one of a_log (g = -exp(a_log)
    softplus(...)) or decay_coef (g = decay_coef softplus(...))."""
    _check(p["conv_w"], "conv_w", (cfg.conv_dim, cfg.conv_k), torch.float32)
    a_log, coef = p.get("a_log"), p.get("decay_coef")
    if (a_log is None) == (coef is None):
        raise ValueError("give exactly one of a_log and decay_coef")
    if a_log is not None:
        _check(a_log, "a_log", (cfg.h_v,), torch.float32)
    else:
        _check(coef, "decay_coef", (cfg.h_v,), torch.float32)
    _check(p["dt_bias"], "dt_bias", (cfg.h_v * cfg.gate_width,), torch.float32)
    _check(p["norm_w"], "norm_w", (cfg.d_v,), torch.float32)
    return _Params(p["conv_w"].data_ptr(), None if a_log is None else a_log.data_ptr(),
                   p["dt_bias"].data_ptr(), p["norm_w"].data_ptr(),
                   None if coef is None else coef.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _alloc_on(stream):
    """Context in which the binding allocates its default outputs and
    temporary workspaces: the stream the kernels are enqueued on.  The caching
    allocator then ties each block to that stream, so a temporary dropped on
    return is reused only by work ordered after the kernels that use it."""
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _raise_on(status: int):
    if status != 0:
        raise GdnError(status, load_library().gdn_last_error().decode())


class SeqLens:
    """cu_seqlens held twice: on the host (validation, grid sizes) and on the
    device (kernels)."""

    def __init__(self, cu, device="cuda"):
        host = torch.as_tensor(cu, dtype=torch.int32).contiguous().cpu()
        self.host = host
        self.dev = host.to(device)
        self.n_seq = host.numel() - 1
        self.t_total = int(host[-1]) if host.numel() else 0


def conv_update(cfg: Config, params: dict, seqlens: SeqLens, x, conv_state, y=None,
                stream=None):
    """silu(causal conv) of packed raw inputs; conv_state updated in place.
    Returns y [T, conv_dim] fp32."""
    lib = load_library()
    with _alloc_on(stream):
        T, N = seqlens.t_total, seqlens.n_seq
        _check(x, "x", (T, cfg.conv_dim), cfg.act_dtype)
        _check(conv_state, "conv_state", (N, cfg.conv_k - 1, cfg.conv_dim), torch.float32)
        if y is None:
            y = torch.empty((T, cfg.conv_dim), dtype=torch.float32, device=x.device)
        _check(y, "y", (T, cfg.conv_dim), torch.float32)
        c, p = cfg.c_struct(), _params(cfg, params)
        _raise_on(lib.gdn_conv_update(ctypes.byref(c), ctypes.byref(p), N, T,
                                      ctypes.c_void_p(seqlens.host.data_ptr()), _ptr(seqlens.dev),
                                      _ptr(x), _ptr(conv_state), _ptr(y), _stream(stream)))
        return y


def decode_step(cfg: Config, params: dict, qkv, z, a, b, conv_state, state, out=None,
                stream=None):
    """One token per sequence; conv_state and state are updated in place.
    Returns out [B, H_v*d_v] (cfg.out_dtype)."""
    lib = load_library()
    with _alloc_on(stream):
        B = qkv.shape[0]
        _check(qkv, "qkv", (B, cfg.conv_dim), cfg.act_dtype)
        _check(z, "z", (B, cfg.value_dim), cfg.act_dtype)
        _check(a, "a", (B, cfg.h_v * cfg.gate_width), cfg.act_dtype)
        _check(b, "b", (B, cfg.h_v), cfg.act_dtype)
        _check(conv_state, "conv_state", (B, cfg.conv_k - 1, cfg.conv_dim), torch.float32)
        _check(state, "state", (B, cfg.h_v, cfg.d_k, cfg.d_v), torch.float32)
        if out is None:
            out = torch.empty((B, cfg.value_dim), dtype=cfg.out_dtype, device=qkv.device)
        _check(out, "out", (B, cfg.value_dim), cfg.out_dtype)
        c, p = cfg.c_struct(), _params(cfg, params)
        _raise_on(lib.gdn_decode_step(ctypes.byref(c), ctypes.byref(p), B, _ptr(qkv), _ptr(z),
                                      _ptr(a), _ptr(b), _ptr(conv_state), _ptr(state), _ptr(out),
                                      _stream(stream)))
        return out


    MAX_NEW_TOKENS = 8


def _check_counts(n, B, device):
    if n is None:
        return None
    if not isinstance(n, torch.Tensor):
        n = torch.as_tensor(n, dtype=torch.int32)
    n = n.to(device=device, dtype=torch.int32).contiguous()
    if tuple(n.shape) != (B,):
        raise ValueError(f"token counts have shape {tuple(n.shape)}, expected ({B},)")
    return n


def decode_multi(cfg: Config, params: dict, qkv, z, a, b, conv_state, state, out=None,
                 n_tok=None, conv_out=None, state_out=None, ckpt=None, want_out=True,
                 stream=None):
    """t_new tokens per sequence in one call.  qkv [B, t_new, conv_dim],
    z [B, t_new, value_dim], a, b [B, t_new, H_v].  The states are updated in
    place unless conv_out / state_out are given.  n_tok: optional [B] counts
    (first n_tok[i] tokens of sequence i).  ckpt: optional
    [B, t_new, H_v, d_k, d_v] fp32 per-token states.  Returns out
    [B, t_new, value_dim] (None when want_out is False)."""
    lib = load_library()
    with _alloc_on(stream):
        B, T = qkv.shape[0], qkv.shape[1]
        dev = qkv.device
        _check(qkv, "qkv", (B, T, cfg.conv_dim), cfg.act_dtype)
        _check(a, "a", (B, T, cfg.h_v * cfg.gate_width), cfg.act_dtype)
        _check(b, "b", (B, T, cfg.h_v), cfg.act_dtype)
        sshape = (B, cfg.h_v, cfg.d_k, cfg.d_v)
        cshape = (B, cfg.conv_k - 1, cfg.conv_dim)
        _check(conv_state, "conv_state", cshape, torch.float32)
        _check(state, "state", sshape, torch.float32)
        conv_out = conv_state if conv_out is None else conv_out
        state_out = state if state_out is None else state_out
        _check(conv_out, "conv_out", cshape, torch.float32)
        _check(state_out, "state_out", sshape, torch.float32)
        if ckpt is not None:
            _check(ckpt, "ckpt", (B, T, cfg.h_v, cfg.d_k, cfg.d_v), torch.float32)
        if want_out:
            _check(z, "z", (B, T, cfg.value_dim), cfg.act_dtype)
            if out is None:
                out = torch.empty((B, T, cfg.value_dim), dtype=cfg.out_dtype, device=dev)
            _check(out, "out", (B, T, cfg.value_dim), cfg.out_dtype)
        else:
            out = None
        n = _check_counts(n_tok, B, dev)
        c, p = cfg.c_struct(), _params(cfg, params)
        _raise_on(lib.gdn_decode_multi(ctypes.byref(c), ctypes.byref(p), B, T, _ptr(n), _ptr(qkv),
                                       _ptr(z) if want_out else None, _ptr(a), _ptr(b),
                                       _ptr(conv_state), _ptr(conv_out), _ptr(state),
                                       _ptr(state_out), _ptr(ckpt), _ptr(out), _stream(stream)))
        return out


def rewind(cfg: Config, params: dict, qkv_rec, a_rec, b_rec, state0, conv0, keep=None,
           state=None, conv_state=None, stream=None):
    """Rebuild each sequence's state from the saved state0 / conv0 by
    replaying its first keep[i] recorded tokens (all when keep is None).
    Returns (state, conv_state)."""
    lib = load_library()
    with _alloc_on(stream):
        B, T = qkv_rec.shape[0], qkv_rec.shape[1]
        dev = qkv_rec.device
        _check(qkv_rec, "qkv_rec", (B, T, cfg.conv_dim), cfg.act_dtype)
        _check(a_rec, "a_rec", (B, T, cfg.h_v * cfg.gate_width), cfg.act_dtype)
        _check(b_rec, "b_rec", (B, T, cfg.h_v), cfg.act_dtype)
        sshape = (B, cfg.h_v, cfg.d_k, cfg.d_v)
        cshape = (B, cfg.conv_k - 1, cfg.conv_dim)
        _check(state0, "state0", sshape, torch.float32)
        _check(conv0, "conv0", cshape, torch.float32)
        if state is None:
            state = torch.empty(sshape, dtype=torch.float32, device=dev)
        if conv_state is None:
            conv_state = torch.empty(cshape, dtype=torch.float32, device=dev)
        _check(state, "state", sshape, torch.float32)
        _check(conv_state, "conv_state", cshape, torch.float32)
        n = _check_counts(keep, B, dev)
        c, p = cfg.c_struct(), _params(cfg, params)
        _raise_on(lib.gdn_rewind(ctypes.byref(c), ctypes.byref(p), B, T, _ptr(n), _ptr(qkv_rec),
                                 _ptr(a_rec), _ptr(b_rec), _ptr(state0), _ptr(conv0), _ptr(state),
                                 _ptr(conv_state), _stream(stream)))
        return state, conv_state


def prefill_workspace_bytes(cfg: Config, n_seq: int, t_total: int, chunk: int = CHUNK) -> int:
    c = cfg.c_struct()
    return int(load_library().gdn_prefill_workspace_bytes(ctypes.byref(c), n_seq, t_total,
                                                          chunk))


def alloc_workspace(cfg: Config, n_seq: int, t_total: int, device="cuda", chunk=CHUNK):
    nbytes = max(prefill_workspace_bytes(cfg, n_seq, t_total, chunk), 256)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefill_chunked(cfg: Config, params: dict, seqlens: SeqLens, qkv, z, a, b,
                    state_in=None, state_out=None, conv_in=None, conv_out=None, out=None,
                    workspace=None, chunk: int = CHUNK, stream=None):
    """Chunked prefill over packed sequences.  Returns (out, state_out, conv_out)."""
    lib = load_library()
    with _alloc_on(stream):
        T, N = seqlens.t_total, seqlens.n_seq
        dev = qkv.device
        _check(qkv, "qkv", (T, cfg.conv_dim), cfg.act_dtype)
        _check(z, "z", (T, cfg.value_dim), cfg.act_dtype)
        _check(a, "a", (T, cfg.h_v * cfg.gate_width), cfg.act_dtype)
        _check(b, "b", (T, cfg.h_v), cfg.act_dtype)
        sshape = (N, cfg.h_v, cfg.d_k, cfg.d_v)
        cshape = (N, cfg.conv_k - 1, cfg.conv_dim)
        if state_in is not None:
            _check(state_in, "state_in", sshape, torch.float32)
        if conv_in is not None:
            _check(conv_in, "conv_in", cshape, torch.float32)
        if state_out is None:
            state_out = torch.empty(sshape, dtype=torch.float32, device=dev)
        if conv_out is None:
            conv_out = torch.empty(cshape, dtype=torch.float32, device=dev)
        if out is None:
            out = torch.empty((T, cfg.value_dim), dtype=cfg.out_dtype, device=dev)
        _check(state_out, "state_out", sshape, torch.float32)
        _check(conv_out, "conv_out", cshape, torch.float32)
        _check(out, "out", (T, cfg.value_dim), cfg.out_dtype)
        if workspace is None:
            workspace = alloc_workspace(cfg, N, T, dev, chunk)
        c, p = cfg.c_struct(), _params(cfg, params)
        _raise_on(lib.gdn_prefill_chunked(
            ctypes.byref(c), ctypes.byref(p), chunk, N, T,
            ctypes.c_void_p(seqlens.host.data_ptr()), _ptr(seqlens.dev),
            _ptr(qkv), _ptr(z), _ptr(a), _ptr(b), _ptr(state_in), _ptr(state_out),
            _ptr(conv_in), _ptr(conv_out), _ptr(out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)))
        return out, state_out, conv_out


PREFILL_NOALLOC_MAX_BYTES = 64 << 20   # GDN_PREFILL_NOALLOC_MAX_BYTES


def prefill_chunked_noalloc(cfg: Config, params: dict, seqlens: SeqLens, qkv, z, a, b,
                            state_in=None, state_out=None, conv_in=None, conv_out=None,
                            out=None, chunk: int = CHUNK, stream=None):
    """gdn_prefill_chunked_noalloc: the chunked prefill with its workspace in
    the library's static device scratch (no workspace argument; the C call
    allocates nothing).  Pass state_out, conv_out and out to keep this
    wrapper from allocating them.  Returns (out, state_out, conv_out)."""
    lib = load_library()
    with _alloc_on(stream):
        T, N = seqlens.t_total, seqlens.n_seq
        dev = qkv.device
        _check(qkv, "qkv", (T, cfg.conv_dim), cfg.act_dtype)
        _check(z, "z", (T, cfg.value_dim), cfg.act_dtype)
        _check(a, "a", (T, cfg.h_v * cfg.gate_width), cfg.act_dtype)
        _check(b, "b", (T, cfg.h_v), cfg.act_dtype)
        sshape = (N, cfg.h_v, cfg.d_k, cfg.d_v)
        cshape = (N, cfg.conv_k - 1, cfg.conv_dim)
        if state_in is not None:
            _check(state_in, "state_in", sshape, torch.float32)
        if conv_in is not None:
            _check(conv_in, "conv_in", cshape, torch.float32)
        if state_out is None:
            state_out = torch.empty(sshape, dtype=torch.float32, device=dev)
        if conv_out is None:
            conv_out = torch.empty(cshape, dtype=torch.float32, device=dev)
        if out is None:
            out = torch.empty((T, cfg.value_dim), dtype=cfg.out_dtype, device=dev)
        _check(state_out, "state_out", sshape, torch.float32)
        _check(conv_out, "conv_out", cshape, torch.float32)
        _check(out, "out", (T, cfg.value_dim), cfg.out_dtype)
        c, p = cfg.c_struct(), _params(cfg, params)
        _raise_on(lib.gdn_prefill_chunked_noalloc(
            ctypes.byref(c), ctypes.byref(p), chunk, N, T,
            ctypes.c_void_p(seqlens.host.data_ptr()), _ptr(seqlens.dev),
            _ptr(qkv), _ptr(z), _ptr(a), _ptr(b), _ptr(state_in), _ptr(state_out),
            _ptr(conv_in), _ptr(conv_out), _ptr(out), _stream(stream)))
        return out, state_out, conv_out


def _proj(cfg: Config, proj: dict) -> _Proj:
    """proj: hidden (int) and bf16 weights w_qkv [conv_dim, H], w_z [value_dim, H],
    w_b [H_v, H], w_a [H_v * gate_width, H], w_out [H, value_dim]."""
    H = int(proj["hidden"])
    bf = torch.bfloat16
    _check(proj["w_qkv"], "w_qkv", (cfg.conv_dim, H), bf)
    _check(proj["w_z"], "w_z", (cfg.value_dim, H), bf)
    _check(proj["w_b"], "w_b", (cfg.h_v, H), bf)
    _check(proj["w_a"], "w_a", (cfg.h_v * cfg.gate_width, H), bf)
    _check(proj["w_out"], "w_out", (H, cfg.value_dim), bf)
    return _Proj(H, *(proj[k].data_ptr() for k in ("w_qkv", "w_z", "w_b", "w_a", "w_out")))


def mixer_workspace_bytes(cfg: Config, hidden: int, n_seq: int, t_total: int) -> int:
    c = cfg.c_struct()
    return int(load_library().gdn_mixer_workspace_bytes(ctypes.byref(c), hidden, n_seq, t_total))


def mixer_prefill(cfg: Config, params: dict, proj: dict, seqlens: SeqLens, x, state_in=None,
                  state_out=None, conv_in=None, conv_out=None, y=None, workspace=None,
                  stream=None):
    """The mixer with its projections over packed sequences: x [T, H] bf16 ->
    y [T, H] (cfg.out_dtype).  Returns (y, state_out, conv_out)."""
    lib = load_library()
    with _alloc_on(stream):
        T, N, H = seqlens.t_total, seqlens.n_seq, int(proj["hidden"])
        dev = x.device
        _check(x, "x", (T, H), torch.bfloat16)
        sshape = (N, cfg.h_v, cfg.d_k, cfg.d_v)
        cshape = (N, cfg.conv_k - 1, cfg.conv_dim)
        if state_in is not None:
            _check(state_in, "state_in", sshape, torch.float32)
        if conv_in is not None:
            _check(conv_in, "conv_in", cshape, torch.float32)
        if state_out is None:
            state_out = torch.empty(sshape, dtype=torch.float32, device=dev)
        if conv_out is None:
            conv_out = torch.empty(cshape, dtype=torch.float32, device=dev)
        if y is None:
            y = torch.empty((T, H), dtype=cfg.out_dtype, device=dev)
        _check(y, "y", (T, H), cfg.out_dtype)
        if workspace is None:
            workspace = torch.empty(max(mixer_workspace_bytes(cfg, H, N, T), 256), dtype=torch.uint8,
                                    device=dev)
        c, p, pj = cfg.c_struct(), _params(cfg, params), _proj(cfg, proj)
        _raise_on(lib.gdn_mixer_prefill(
            ctypes.byref(c), ctypes.byref(p), ctypes.byref(pj), N, T,
            ctypes.c_void_p(seqlens.host.data_ptr()), _ptr(seqlens.dev), _ptr(x), _ptr(state_in),
            _ptr(state_out), _ptr(conv_in), _ptr(conv_out), _ptr(y), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)))
        return y, state_out, conv_out


def mixer_decode(cfg: Config, params: dict, proj: dict, x, conv_state, state, y=None,
                 workspace=None, stream=None):
    """One mixer decode step with projections: x [B, H] bf16 -> y [B, H];
    conv_state and state are updated in place."""
    lib = load_library()
    with _alloc_on(stream):
        B, H = x.shape[0], int(proj["hidden"])
        _check(x, "x", (B, H), torch.bfloat16)
        _check(conv_state, "conv_state", (B, cfg.conv_k - 1, cfg.conv_dim), torch.float32)
        _check(state, "state", (B, cfg.h_v, cfg.d_k, cfg.d_v), torch.float32)
        if y is None:
            y = torch.empty((B, H), dtype=cfg.out_dtype, device=x.device)
        _check(y, "y", (B, H), cfg.out_dtype)
        if workspace is None:
            workspace = torch.empty(max(mixer_workspace_bytes(cfg, H, B, B), 256), dtype=torch.uint8,
                                    device=x.device)
        c, p, pj = cfg.c_struct(), _params(cfg, params), _proj(cfg, proj)
        _raise_on(lib.gdn_mixer_decode(ctypes.byref(c), ctypes.byref(p), ctypes.byref(pj), B, _ptr(x),
                                       _ptr(conv_state), _ptr(state), _ptr(y), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))
        return y


    __all__ = ["Config", "SeqLens", "GdnError", "load_library", "header_functions",
               "conv_update", "decode_step", "decode_multi", "rewind", "prefill_workspace_bytes",
               "alloc_workspace", "prefill_chunked", "prefill_chunked_noalloc",
           "PREFILL_NOALLOC_MAX_BYTES", "mixer_workspace_bytes", "mixer_prefill",
               "mixer_decode", "LIB_PATH", "CHUNK", "MAX_NEW_TOKENS"]
