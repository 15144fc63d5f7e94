"""Shared helpers of the parity tests: move a seeded case to the device, run
the oracle on the same host tensors, and compare under the stated bars.

Tolerance (floating point): max |y_gpu - y_oracle| <= 2e-3 * rms(y_oracle)
over the compared outputs, and ||S_gpu - S_oracle||_F / ||S_oracle||_F <=
1e-3 on final states.  Conv histories are raw inputs copied, so they must
match exactly.  Outputs are compared in fp32: rounding the output to bf16
alone costs more than the bar (the outputs are heavy tailed).
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from gdn_inputs import Case, Dims

Y_TOL = 2e-3        # max abs error / rms of the reference output
S_TOL = 1e-3        # relative Frobenius error of the final state


def n_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def oracle_shape(d: Dims) -> oracle.Shape:
    return oracle.Shape(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k, d.gate, head_map=d.head_map,
                        decay=d.decay)


def gpu_config(d: Dims, act_dtype: str, out_dtype=torch.float32):
    import gated_deltanet_linear_causal_amd as gdn
    return gdn.Config(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k,
                      torch.bfloat16 if act_dtype == "bf16" else torch.float32,
                      out_dtype, d.gate, head_map=d.head_map, decay=d.decay)


def to_dev(t: torch.Tensor, act_dtype: str | None = None, device="cuda"):
    """Host fp32 tensor -> device tensor (bf16 if the case is bf16: exact,
    the host values are already bf16-representable)."""
    if act_dtype == "bf16":
        return t.to(torch.bfloat16).contiguous().to(device)
    return t.contiguous().to(device)


def dev_params(case: Case, device="cuda"):
    return {k: v.contiguous().to(device) for k, v in case.params.items()}


def subcase(case: Case, hk: int) -> Case:
    """The same case restricted to key head hk and its value-head group: a
    layer with H_k = 1, H_v = group whose channels are gathered from the
    full layer.  Sequences and heads are independent, so running the
    oracle on it gives exactly the full layer's results for those heads."""
    d = case.dims
    assert d.head_map == "grouped" and d.decay == "head" and "a_log" in case.params
    grp = d.h_v // d.h_k
    HK, DK, DV = d.h_k, d.d_k, d.d_v
    qc = list(range(hk * DK, (hk + 1) * DK))
    kc = list(range(HK * DK + hk * DK, HK * DK + (hk + 1) * DK))
    vc = list(range(2 * HK * DK + hk * grp * DV, 2 * HK * DK + (hk + 1) * grp * DV))
    ch = torch.tensor(qc + kc + vc)
    hv = torch.arange(hk * grp, (hk + 1) * grp)
    zc = torch.arange(hk * grp * DV, (hk + 1) * grp * DV)
    sd = Dims(1, grp, DK, DV, d.conv_k, d.gate)
    params = {"conv_w": case.params["conv_w"][ch], "a_log": case.params["a_log"][hv],
              "dt_bias": case.params["dt_bias"][hv], "norm_w": case.params["norm_w"]}
    dec = {}
    if case.dec:
        dec = {"qkv": case.dec["qkv"][..., ch], "z": case.dec["z"][..., zc],
               "a": case.dec["a"][..., hv], "b": case.dec["b"][..., hv]}
    return Case(sd, case.act_dtype, list(case.cu_seqlens), params, case.S0[:, hv],
                case.conv0[:, :, ch], case.qkv[:, ch], case.z[:, zc], case.a[:, hv],
                case.b[:, hv], dec, case.name + f"[hk={hk}]")


def run_oracle(case: Case, heads=None, S0=None, conv0=None, want_pre=False):
    return oracle.mixer(oracle_shape(case.dims), case.cu_seqlens, case.params,
                        case.qkv, case.z, case.a, case.b,
                        case.S0 if S0 is None else S0,
                        case.conv0 if conv0 is None else conv0,
                        heads=heads, nthreads=n_threads(), want_pre=want_pre)


def decode_as_sequences(case: Case, steps: int | None = None):
    """Decode inputs [steps][B][...] regrouped as B packed sequences of
    `steps` tokens, for the oracle."""
    st = case.dec["qkv"].shape[0] if steps is None else steps
    B = case.dec["qkv"].shape[1]

    def pack(x):
        return x[:st].transpose(0, 1).reshape(B * st, -1)
    cu = [i * st for i in range(B + 1)]
    return cu, pack(case.dec["qkv"]), pack(case.dec["z"]), pack(case.dec["a"]), pack(case.dec["b"])


def assert_y_close(y_gpu, y_ref, what="out"):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(y_ref * y_ref)))
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    assert err <= Y_TOL * rms, f"{what}: max|err| {err:.3e} > {Y_TOL} * rms {rms:.3e} (ratio {err / max(rms, 1e-300):.2e})"
    return err / max(rms, 1e-300)


def assert_state_close(S_gpu, S_ref, what="state"):
    S_gpu = np.asarray(S_gpu, np.float64)
    S_ref = np.asarray(S_ref, np.float64)
    assert np.isfinite(S_gpu).all(), f"{what}: non-finite values"
    den = float(np.linalg.norm(S_ref))
    rel = float(np.linalg.norm(S_gpu - S_ref)) / max(den, 1e-300)
    if den == 0.0:
        assert float(np.abs(S_gpu).max()) == 0.0, f"{what}: expected zeros"
        return 0.0
    assert rel <= S_TOL, f"{what}: relative Frobenius error {rel:.3e} > {S_TOL}"
    return rel
