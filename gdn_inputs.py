"""Seeded synthetic inputs for the Gated DeltaNet mixer core.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the oracle side (tests, CPU baseline) and the GPU side
(binding, bench) consume the very same host tensors, so neither side ever
sees a value the other produced.

Recipe (the pages measure no dataset for this path; every input is
synthetic):
  * a torch CPU Generator seeded per case; draw order is lengths, then
    parameters, then states, then activations;
  * "N(0, s)" means standard deviation s;
  * conv weights ~ N(0, 1/K); A_log = log U[1, 16] (strong decay) or
    log U[0.001, 0.01] (weak decay, exercises long memory); dt_bias ~ N(0, 1);
    gated-norm weight 1 + N(0, 0.1);
  * states S ~ N(0, s0_std), conv history ~ N(0, conv0_std) (zero if std 0);
  * activations q/k/v (fused), z, a, b ~ N(0, 1); rounded to bfloat16 (round
    to nearest even) when the case's activation dtype is bf16, and kept as
    float32 tensors holding those exact values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Dims:
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    conv_k: int = 4
    gate: str = "silu"
    head_map: str = "grouped"      # key head of value head hv: hv // group or hv % h_k
    decay: str = "head"            # one decay per value head, or per key channel ("channel")

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


@dataclass
class Case:
    dims: Dims
    act_dtype: str                 # "bf16" or "f32"
    cu_seqlens: list               # [N+1] python ints
    params: dict                   # conv_w, a_log, dt_bias, norm_w (fp32)
    S0: torch.Tensor               # [N, H_v, d_k, d_v] fp32
    conv0: torch.Tensor            # [N, K-1, conv_dim] fp32
    qkv: torch.Tensor              # [T, conv_dim]
    z: torch.Tensor                # [T, value_dim]
    a: torch.Tensor                # [T, H_v] ([T, H_v * d_k] with per-channel decay)
    b: torch.Tensor                # [T, H_v]
    # decode continuation: [steps, N, ...] per-step single-token inputs
    dec: dict = field(default_factory=dict)
    name: str = ""

    @property
    def n_seq(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def t_total(self) -> int:
        return int(self.cu_seqlens[-1])


def _normal(gen, shape, std):
    if std == 0:
        return torch.zeros(shape, dtype=torch.float32)
    return torch.randn(shape, generator=gen, dtype=torch.float32) * std


def _uniform(gen, shape, lo, hi):
    return torch.rand(shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo


def _act(gen, shape, act_dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if act_dtype == "bf16":
        x = x.to(torch.bfloat16).to(torch.float32)
    return x


def make_params(gen, dims: Dims, decay: str = "strong") -> dict:
    K = dims.conv_k
    conv_w = _normal(gen, (dims.conv_dim, K), 1.0 / K)
    if decay == "strong":
        a_log = torch.log(_uniform(gen, (dims.h_v,), 1.0, 16.0))
    elif decay == "weak":
        a_log = torch.log(_uniform(gen, (dims.h_v,), 0.001, 0.01))
    else:
        raise ValueError(decay)
    dt_bias = _normal(gen, (dims.h_v * dims.gate_width,), 1.0)
    norm_w = 1.0 + _normal(gen, (dims.d_v,), 0.1)
    return {"conv_w": conv_w, "a_log": a_log, "dt_bias": dt_bias,
            "norm_w": norm_w}


def with_decay_coef(params: dict) -> dict:
    """The same parameters with the decay given as the coefficient
    -exp(A_log) itself (rounded once to float32) instead of A_log."""
    out = {k: v for k, v in params.items() if k != "a_log"}
    out["decay_coef"] = (-torch.exp(params["a_log"].double())).float()
    return out


def make_case(dims: Dims, lengths, act_dtype="bf16", seed=0, decay="strong",
              s0_std=0.0, conv0_std=0.0, decode_steps=0, name="") -> Case:
    """Draw one packed varlen case.  ``lengths`` may be a list of ints or a
    callable gen -> list (drawn first, so it is part of the seeded stream)."""
    gen = torch.Generator().manual_seed(seed)
    if callable(lengths):
        lengths = lengths(gen)
    lengths = [int(x) for x in lengths]
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    n, T = len(lengths), cu[-1]
    params = make_params(gen, dims, decay)
    S0 = _normal(gen, (n, dims.h_v, dims.d_k, dims.d_v), s0_std)
    conv0 = _normal(gen, (n, dims.conv_k - 1, dims.conv_dim), conv0_std)
    qkv = _act(gen, (T, dims.conv_dim), act_dtype)
    z = _act(gen, (T, dims.value_dim), act_dtype)
    a = _act(gen, (T, dims.h_v * dims.gate_width), act_dtype)
    b = _act(gen, (T, dims.h_v), act_dtype)
    dec = {}
    if decode_steps:
        dec = {
            "qkv": _act(gen, (decode_steps, n, dims.conv_dim), act_dtype),
            "z": _act(gen, (decode_steps, n, dims.value_dim), act_dtype),
            "a": _act(gen, (decode_steps, n, dims.h_v * dims.gate_width), act_dtype),
            "b": _act(gen, (decode_steps, n, dims.h_v), act_dtype),
        }
    return Case(dims, act_dtype, cu, params, S0, conv0, qkv, z, a, b, dec,
                name)


def make_projections(dims: Dims, hidden: int, seed: int) -> dict:
    """Random projection weights of the mixer (bf16 values held in float32):
    N(0, 1/sqrt(H)) for in_proj, so the projected activations are about
    N(0, 1), and N(0, 1/sqrt(value_dim)) for out_proj."""
    gen = torch.Generator().manual_seed(seed)

    def w(rows, cols):
        x = torch.randn((rows, cols), generator=gen, dtype=torch.float32) / cols ** 0.5
        return x.to(torch.bfloat16).to(torch.float32)
    return {"hidden": hidden,
            "w_qkv": w(dims.conv_dim, hidden), "w_z": w(dims.value_dim, hidden),
            "w_b": w(dims.h_v, hidden), "w_a": w(dims.h_v * dims.gate_width, hidden),
            "w_out": w(hidden, dims.value_dim)}


def make_hidden(rows: int, hidden: int, seed: int) -> torch.Tensor:
    """Model hidden states ~ N(0, 1), rounded to bf16 (held in float32)."""
    gen = torch.Generator().manual_seed(seed)
    return torch.randn((rows, hidden), generator=gen, dtype=torch.float32).to(
        torch.bfloat16).to(torch.float32)


# --- the five named workloads ---------------------------------------------

BIG = Dims(h_k=16, h_v=32, d_k=128, d_v=128, conv_k=4)


def tiny_recurrent() -> Case:
    """1 sequence, 64 tokens fed one at a time, H_k=H_v=2, d=32, K=4, fp32,
    zero initial state, SiLU gate, seed 0."""
    dims = Dims(h_k=2, h_v=2, d_k=32, d_v=32, conv_k=4)
    return make_case(dims, [0], act_dtype="f32", seed=0, decode_steps=64,
                     name="tiny_recurrent")


def decode_batch(steps=100, batch=64) -> Case:
    """B=64 sequences, one token each per step, bf16 activations, fp32
    states S ~ N(0, 0.02) and conv history ~ N(0, 1)."""
    return make_case(BIG, [0] * batch, act_dtype="bf16", seed=1,
                     s0_std=0.02, conv0_std=1.0, decode_steps=steps,
                     name="decode_b64")


def chunked_prefill(T=4096) -> Case:
    """B=1, T=4096, bf16 activations, zero initial state."""
    return make_case(BIG, [T], act_dtype="bf16", seed=2, name="prefill_t4096")


def varlen_prefill(n=8, lo=512, hi=8192) -> Case:
    """8 sequences with lengths ~ U{512..8192}, random initial states."""
    def lengths(gen):
        return torch.randint(lo, hi + 1, (n,), generator=gen).tolist()
    return make_case(BIG, lengths, act_dtype="bf16", seed=3, s0_std=0.02,
                     conv0_std=1.0, name="varlen_8")


def long_handoff(T=65536, steps=256) -> Case:
    """B=1 prefill of T=65536 then 256 decode steps, sigmoid output gate."""
    dims = Dims(h_k=16, h_v=32, d_k=128, d_v=128, conv_k=4, gate="sigmoid")
    return make_case(dims, [T], act_dtype="bf16", seed=4, decode_steps=steps,
                     name="long_handoff")
