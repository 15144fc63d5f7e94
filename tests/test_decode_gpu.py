"""Parity of gdn_decode_step (one fused kernel per step) with the oracle.

The oracle runs the same tokens as packed sequences (one sequence per batch
row), which its split/resume pin shows equals stepping one token at a time.
"""
import numpy as np
import pytest
import torch

import gdn_parity as P
import oracle
from gdn_inputs import Dims, decode_batch, make_case, tiny_recurrent, with_decay_coef

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_linear_causal_amd as g
    g.load_library()
    return g


def run_decode(gdn, case, steps, out_dtype=torch.float32, S=None, conv=None):
    cfg = P.gpu_config(case.dims, case.act_dtype, out_dtype)
    params = P.dev_params(case)
    S = (case.S0 if S is None else S).clone().cuda()
    conv = (case.conv0 if conv is None else conv).clone().cuda()
    dq = P.to_dev(case.dec["qkv"][:steps], case.act_dtype)
    dz = P.to_dev(case.dec["z"][:steps], case.act_dtype)
    da = P.to_dev(case.dec["a"][:steps], case.act_dtype)
    db = P.to_dev(case.dec["b"][:steps], case.act_dtype)
    outs = []
    for s in range(steps):
        outs.append(gdn.decode_step(cfg, params, dq[s], dz[s], da[s], db[s], conv, S))
    torch.cuda.synchronize()
    return torch.stack(outs).float().cpu(), S.cpu(), conv.cpu()


def oracle_decode(case, steps, S0=None, conv0=None):
    cu, qkv, z, a, b = P.decode_as_sequences(case, steps)
    r = oracle.mixer(P.oracle_shape(case.dims), cu, case.params, qkv, z, a, b,
                     case.S0 if S0 is None else S0, case.conv0 if conv0 is None else conv0,
                     nthreads=P.n_threads())
    B = len(cu) - 1
    y = r["y"].reshape(B, steps, -1).transpose(1, 0, 2)
    return y, r["S"], r["conv"]


def test_tiny_recurrent_64_steps(gdn):
    """1 sequence, 64 tokens one at a time, H_k=H_v=2, d=32, K=4, fp32, SiLU."""
    case = tiny_recurrent()
    y, S, conv = run_decode(gdn, case, 64)
    y_ref, S_ref, conv_ref = oracle_decode(case, 64)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


def test_decode_batch_64x100_steps(gdn):
    """B=64, H_k=16, H_v=32, d=128, K=4, bf16 inputs, prefilled states, 100
    consecutive steps; every output and the final states are compared."""
    case = decode_batch(steps=100)
    y, S, conv = run_decode(gdn, case, 100)
    y_ref, S_ref, conv_ref = oracle_decode(case, 100)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


def test_decode_batch_64x100_steps_weak_decay(gdn):
    """The B=64 decode batch with a weak decay (A_log = log U[0.001, 0.01]),
    so the prefilled states and every step's writes carry through all 100
    steps; every output and the final states are compared."""
    base = decode_batch(steps=100)
    case = make_case(base.dims, [0] * 64, act_dtype="bf16", seed=11, decay="weak",
                     s0_std=0.02, conv0_std=1.0, decode_steps=100)
    y, S, conv = run_decode(gdn, case, 100)
    y_ref, S_ref, conv_ref = oracle_decode(case, 100)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


@pytest.mark.parametrize("decay", ["head", "channel"])
def test_decode_gate_edge_inputs(gdn, decay):
    """Gate inputs on the gates' edges: a + dt_bias straddling the softplus
    threshold (20) and b = +-30, over 8 steps for 3 sequences."""
    d = Dims(2, 4, 64, 64, 4, "silu" if decay == "head" else "sigmoid", decay=decay)
    case = make_case(d, [0, 0, 0], act_dtype="bf16", seed=12, decay="weak", s0_std=0.3,
                     conv0_std=1.0, decode_steps=8)
    a_vals = torch.tensor([19.875, 20.0, 20.125, 24.0, -30.0, 30.0, 0.5])
    b_vals = torch.tensor([30.0, -30.0, 0.0, 5.0, -30.0])
    sa = case.dec["a"].shape
    sb = case.dec["b"].shape
    case.dec["a"] = a_vals[torch.arange(sa.numel()).view(sa) % len(a_vals)].clone()
    case.dec["b"] = b_vals[torch.arange(sb.numel()).view(sb) % len(b_vals)].clone()
    dtb = case.params["dt_bias"].clone()
    dtb[: dtb.numel() // 2] = 0.0
    dtb[dtb.numel() // 2:] = 0.0625
    case.params["dt_bias"] = dtb
    y, S, conv = run_decode(gdn, case, 8)
    y_ref, S_ref, conv_ref = oracle_decode(case, 8)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


VARIANTS = [
    # h_k, h_v, d_k, d_v, K, gate, decay
    (2, 2, 32, 32, 4, "silu", "weak"),
    (2, 4, 64, 64, 4, "sigmoid", "weak"),
    (1, 4, 128, 128, 3, "silu", "weak"),
    (2, 4, 32, 128, 2, "sigmoid", "strong"),
    (2, 2, 128, 64, 4, "silu", "weak"),
    (1, 3, 64, 32, 1, "silu", "weak"),
    (1, 8, 64, 64, 4, "silu", "weak"),
    # a group too wide for the per-key-head buffer: the persistent kernel
    (1, 64, 128, 128, 4, "silu", "weak"),
]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: "hk%d_hv%d_dk%d_dv%d_K%d_%s_%s" % v)
def test_decode_variants(gdn, v, act):
    hk, hv, dk, dv, K, gate, decay = v
    d = Dims(hk, hv, dk, dv, K, gate)
    case = make_case(d, [0, 0, 0], act_dtype=act, seed=hk * 100 + hv + dk + K,
                     decay=decay, s0_std=0.3, conv0_std=1.0, decode_steps=9)
    y, S, conv = run_decode(gdn, case, 9)
    y_ref, S_ref, conv_ref = oracle_decode(case, 9)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


LAYOUTS = [
    # h_k, h_v, d, head_map, decay form
    (2, 6, 64, "tiled", "decay_coef"),
    (4, 8, 128, "tiled", "a_log"),
    (2, 6, 32, "grouped", "decay_coef"),
    (3, 3, 64, "tiled", "a_log"),
]


@pytest.mark.parametrize("v", LAYOUTS, ids=lambda v: "hk%d_hv%d_d%d_%s_%s" % v)
def test_decode_head_map_and_decay_coef(gdn, v):
    """Tiled key-head order (hv % H_k) and the decay coefficient given
    directly ("oxinfer 0.0.5 src/qwen.rs", DeltaRule::run and weight
    loading)."""
    hk, hv, dd, head_map, form = v
    d = Dims(hk, hv, dd, dd, 4, "silu", head_map)
    case = make_case(d, [0, 0, 0], act_dtype="bf16", seed=300 + hk + hv + dd,
                     decay="weak", s0_std=0.3, conv0_std=1.0, decode_steps=7)
    if form == "decay_coef":
        case.params = with_decay_coef(case.params)
    y, S, conv = run_decode(gdn, case, 7)
    y_ref, S_ref, conv_ref = oracle_decode(case, 7)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


KDA = [
    # h_k, h_v, d_k, d_v, K, act, gate, head_map
    (2, 4, 128, 128, 4, "bf16", "sigmoid", "grouped"),
    (2, 2, 64, 32, 3, "f32", "sigmoid", "tiled"),
    (1, 3, 32, 64, 4, "bf16", "silu", "grouped"),
]


@pytest.mark.parametrize("v", KDA, ids=lambda v: "hk%d_hv%d_dk%d_dv%d_K%d_%s_%s_%s" % v)
def test_decode_per_channel_decay(gdn, v):
    """One decay per key channel (Kimi Delta Attention, "cortiq-engine
    0.8.76 pipeline.rs", AttnKind::Kda), consecutive single-token steps."""
    hk, hv, dk, dv, K, act, gate, head_map = v
    d = Dims(hk, hv, dk, dv, K, gate, head_map, decay="channel")
    case = make_case(d, [0, 0, 0], act_dtype=act, seed=600 + hk + hv + dk + dv, decay="weak",
                     s0_std=0.3, conv0_std=1.0, decode_steps=8)
    y, S, conv = run_decode(gdn, case, 8)
    y_ref, S_ref, conv_ref = oracle_decode(case, 8)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


def test_decode_per_channel_decay_b64(gdn):
    """The full layer with one decay per key channel at B=64, three
    consecutive steps."""
    d = Dims(16, 32, 128, 128, 4, "sigmoid", decay="channel")
    case = make_case(d, [0] * 64, act_dtype="bf16", seed=610, decay="weak", s0_std=0.02,
                     conv0_std=1.0, decode_steps=3)
    y, S, conv = run_decode(gdn, case, 3)
    y_ref, S_ref, conv_ref = oracle_decode(case, 3)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


def test_decode_bf16_out_is_rne_of_fp32_out(gdn):
    case = make_case(Dims(2, 4, 128, 128), [0] * 5, act_dtype="bf16", seed=7,
                     s0_std=0.02, conv0_std=1.0, decode_steps=3)
    y32, S32, c32 = run_decode(gdn, case, 3, torch.float32)
    y16, S16, c16 = run_decode(gdn, case, 3, torch.bfloat16)
    assert torch.equal(y32.to(torch.bfloat16).float(), y16)
    assert torch.equal(S32, S16) and torch.equal(c32, c16)


def test_decode_deterministic(gdn):
    case = make_case(Dims(2, 4, 64, 64), [0] * 4, act_dtype="bf16", seed=8,
                     s0_std=0.02, conv0_std=1.0, decode_steps=5)
    a = run_decode(gdn, case, 5)
    b = run_decode(gdn, case, 5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_decode_batch_zero_is_noop(gdn):
    d = Dims(2, 4, 64, 64)
    cfg = P.gpu_config(d, "bf16")
    case = make_case(d, [0], act_dtype="bf16", seed=9)
    params = P.dev_params(case)
    e = torch.empty((0, d.conv_dim), dtype=torch.bfloat16, device="cuda")
    out = gdn.decode_step(cfg, params, e, torch.empty((0, d.value_dim), dtype=torch.bfloat16, device="cuda"),
                          torch.empty((0, d.h_v), dtype=torch.bfloat16, device="cuda"),
                          torch.empty((0, d.h_v), dtype=torch.bfloat16, device="cuda"),
                          torch.empty((0, 3, d.conv_dim), device="cuda"),
                          torch.empty((0, d.h_v, 64, 64), device="cuda"))
    assert out.shape == (0, d.value_dim)


def test_decode_steps_replayed_as_a_graph_match_eager(gdn):
    """The decode steps captured in a HIP graph (as the bench times the
    launch-bound workloads) give, replay after replay with eager work in
    between, the states and outputs of the same steps run eagerly."""
    case = tiny_recurrent()
    steps = 8
    cfg = P.gpu_config(case.dims, case.act_dtype)
    params = P.dev_params(case)
    x = [P.to_dev(case.dec[k][:steps], case.act_dtype) for k in ("qkv", "z", "a", "b")]
    S, C = case.S0.clone().cuda(), case.conv0.clone().cuda()
    outs = torch.zeros((steps, 1, case.dims.value_dim), device="cuda")

    def run():
        for j in range(steps):
            gdn.decode_step(cfg, params, x[0][j], x[1][j], x[2][j], x[3][j], C, S, out=outs[j])

    S0, C0 = S.clone(), C.clone()
    run()
    torch.cuda.synchronize()
    ref = (outs.clone(), S.clone(), C.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.copy_(S0)
        C.copy_(C0)
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(3):
        S.copy_(S0)
        C.copy_(C0)
        outs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref[0]) and torch.equal(S, ref[1]) and torch.equal(C, ref[2])


@pytest.mark.parametrize("batch,t_new", [(64, 1), (64, 4), (8, 1), (2, 3), (64, 8), (4, 8)])
def test_state_cache_hint_changes_nothing_but_speed(gdn, batch, t_new):
    """The streamed state hint (non-temporal state loads and stores) gives
    the cached path's outputs, states and conv histories bit for bit, for
    single steps and multi-token calls (stepped, and at 8 tokens in the
    in-call UT form), one head per pass and two side by side."""
    import dataclasses
    case = decode_batch(steps=2 * t_new, batch=batch)
    cfg = P.gpu_config(case.dims, case.act_dtype)
    params = P.dev_params(case)
    x = [P.to_dev(case.dec[k], case.act_dtype) for k in ("qkv", "z", "a", "b")]
    res = []
    for c in (cfg, dataclasses.replace(cfg, state_cache="streamed")):
        S, C = case.S0.clone().cuda(), case.conv0.clone().cuda()
        ys = []
        for call in range(2):
            xs = [v[call * t_new:(call + 1) * t_new] for v in x]
            if t_new == 1:
                ys.append(gdn.decode_step(c, params, *(v[0] for v in xs), C, S))
            else:
                xm = [v.transpose(0, 1).contiguous() for v in xs]
                ys.append(gdn.decode_multi(c, params, *xm, C, S))
        torch.cuda.synchronize()
        res.append((torch.stack(ys).cpu(), S.cpu(), C.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)
