"""Parity of gdn_prefill_chunked with the token-by-token oracle.

Small cases compare every output; the full-size workloads compare all
outputs where the oracle finishes in seconds (T=4096) and otherwise sampled
key heads, which the oracle computes exactly because heads are independent.
"""
import numpy as np
import pytest
import torch

import gdn_parity as P
from gdn_inputs import (Dims, chunked_prefill, long_handoff, make_case,
                        varlen_prefill, with_decay_coef)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_linear_causal_amd as g
    g.load_library()
    return g


def run_prefill(gdn, case, out_dtype=torch.float32, state_in=True, conv_in=True,
                inplace=False):
    cfg = P.gpu_config(case.dims, case.act_dtype, out_dtype)
    sl = gdn.SeqLens(case.cu_seqlens)
    S_in = case.S0.clone().cuda() if state_in else None
    c_in = case.conv0.clone().cuda() if conv_in else None
    kw = {}
    if inplace:
        kw = {"state_out": S_in, "conv_out": c_in}
    out, S, conv = gdn.prefill_chunked(cfg, P.dev_params(case), sl,
                                       P.to_dev(case.qkv, case.act_dtype),
                                       P.to_dev(case.z, case.act_dtype),
                                       P.to_dev(case.a, case.act_dtype),
                                       P.to_dev(case.b, case.act_dtype),
                                       state_in=S_in, conv_in=c_in, **kw)
    torch.cuda.synchronize()
    return out.float().cpu(), S.cpu(), conv.cpu()


SMALL = [
    # h_k, h_v, d_k, d_v, K, gate, decay, lengths
    (2, 4, 64, 64, 4, "silu", "weak", [1, 63, 65, 130]),
    (2, 4, 64, 64, 4, "sigmoid", "strong", [130, 64, 7]),
    (1, 2, 128, 128, 4, "silu", "weak", [200]),
    (2, 2, 32, 32, 4, "silu", "weak", [64, 129, 0, 2]),
    (1, 2, 128, 32, 3, "sigmoid", "weak", [100, 31]),
    (2, 2, 32, 128, 2, "silu", "weak", [77]),
    (1, 3, 64, 64, 1, "silu", "weak", [70, 5]),
]


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("v", SMALL, ids=lambda v: "hk%d_hv%d_dk%d_dv%d_K%d_%s_%s_%s" % (
    *v[:7], "-".join(map(str, v[7]))))
def test_prefill_small(gdn, v, act):
    hk, hv, dk, dv, K, gate, decay, lengths = v
    d = Dims(hk, hv, dk, dv, K, gate)
    case = make_case(d, lengths, act_dtype=act, seed=sum(lengths) + K, decay=decay,
                     s0_std=0.3, conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


# Enough sequences that the scan widens its column slices: with 256 compute
# units and 4 value heads per sequence, d_v = 64 takes two 16-column tiles
# per workgroup from 32 sequences and four (the whole head) from 64; d_v =
# 128 takes two from 16 sequences and four from 32.  The scan takes the
# first 64 sequences longest first and any later ones in their own order
# (80 sequences: both).
MANY = [
    # h_k, h_v, d_k, d_v, decay mode, n_seq
    (2, 4, 64, 64, "head", 32),
    (2, 4, 64, 64, "head", 64),
    (2, 4, 64, 64, "head", 80),
    (1, 4, 128, 128, "head", 16),
    (1, 4, 128, 128, "head", 32),
    (2, 4, 32, 64, "channel", 64),
]


@pytest.mark.parametrize("v", MANY, ids=lambda v: "hk%d_hv%d_dk%d_dv%d_%s_n%d" % v)
def test_prefill_many_sequences_wide_slices(gdn, v):
    hk, hv, dk, dv, mode, n = v
    d = Dims(hk, hv, dk, dv, 4, "silu" if mode == "head" else "sigmoid", decay=mode)
    lens = [(37 * i + 11) % 150 for i in range(n)]
    lens[3], lens[5] = 0, 1
    case = make_case(d, lens, act_dtype="bf16", seed=500 + n + dk + dv, decay="weak",
                     s0_std=0.3, conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


LAYOUTS = [
    # h_k, h_v, d, head_map, decay form
    (2, 6, 64, "tiled", "decay_coef"),
    (2, 4, 128, "tiled", "a_log"),
    (2, 6, 32, "grouped", "decay_coef"),
]


@pytest.mark.parametrize("v", LAYOUTS, ids=lambda v: "hk%d_hv%d_d%d_%s_%s" % v)
def test_prefill_head_map_and_decay_coef(gdn, v):
    """Tiled key-head order (hv % H_k) and the decay coefficient given
    directly ("oxinfer 0.0.5 src/qwen.rs", DeltaRule::run and weight
    loading), over ragged chunks."""
    hk, hv, dd, head_map, form = v
    d = Dims(hk, hv, dd, dd, 4, "silu", head_map)
    case = make_case(d, [1, 63, 65, 130], act_dtype="bf16", seed=400 + hk + hv + dd,
                     decay="weak", s0_std=0.3, conv0_std=1.0)
    if form == "decay_coef":
        case.params = with_decay_coef(case.params)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


KDA_SMALL = [
    # h_k, h_v, d_k, d_v, K, decay, head_map, act, lengths
    (2, 4, 64, 64, 4, "weak", "grouped", "bf16", [1, 63, 65, 130]),
    (2, 4, 64, 64, 4, "strong", "tiled", "f32", [130, 64, 7]),
    (1, 2, 128, 128, 4, "weak", "grouped", "bf16", [200]),
    (2, 2, 32, 32, 3, "weak", "grouped", "f32", [64, 129, 0, 2]),
    (1, 2, 128, 32, 2, "strong", "grouped", "bf16", [100, 31]),
    (2, 2, 32, 128, 4, "weak", "tiled", "bf16", [77]),
]


@pytest.mark.parametrize("v", KDA_SMALL, ids=lambda v: "hk%d_hv%d_dk%d_dv%d_K%d_%s_%s_%s_%s" % (
    *v[:8], "-".join(map(str, v[8]))))
def test_prefill_per_channel_decay(gdn, v):
    """One decay per key channel (Kimi Delta Attention, "cortiq-engine
    0.8.76 pipeline.rs", AttnKind::Kda), sigmoid output gate, non-zero
    initial states, ragged chunks."""
    hk, hv, dk, dv, K, decay, head_map, act, lengths = v
    d = Dims(hk, hv, dk, dv, K, "sigmoid", head_map, decay="channel")
    case = make_case(d, lengths, act_dtype=act, seed=700 + sum(lengths) + dk, decay=decay,
                     s0_std=0.3, conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


def test_prefill_per_channel_decay_t1024_all_heads(gdn):
    """The full layer (H_k=16, H_v=32, d=128, K=4, bf16) over T=1024 with one
    decay per key channel and a weak decay, so that the state carries across
    all 16 chunks."""
    d = Dims(16, 32, 128, 128, 4, "sigmoid", decay="channel")
    case = make_case(d, [1024], act_dtype="bf16", seed=701, decay="weak", s0_std=0.02,
                     conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


KDA_WALK = [
    # h_k, h_v, d, act, lengths: enough (chunk, value head) pairs that each
    # kda_intra workgroup walks two or three chunks of its head (on 256 CUs),
    # with partial last chunks and several sequences
    (4, 8, 128, "bf16", [1500, 1409, 700]),
    (4, 8, 64, "f32", [2000, 1000, 33]),
]


@pytest.mark.parametrize("v", KDA_WALK, ids=lambda v: "hk%d_hv%d_d%d_%s_%s" % (*v[:4], "-".join(map(str, v[4]))))
def test_prefill_per_channel_decay_chunk_walk(gdn, v):
    """Per-channel decay with workgroups that process several consecutive
    chunks of a head (the next chunk's inputs loaded during the current
    one), weak decay so that every chunk's operands reach the output."""
    hk, hv, dd, act, lengths = v
    d = Dims(hk, hv, dd, dd, 4, "sigmoid", decay="channel")
    case = make_case(d, lengths, act_dtype=act, seed=702 + dd, decay="weak", s0_std=0.1,
                     conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


def test_prefill_zero_state_pointers_and_empty_sequences(gdn):
    """NULL state_in / conv_in mean zeros; empty sequences pass their state
    through unchanged."""
    d = Dims(2, 4, 64, 64)
    case = make_case(d, [0, 90, 0, 3], act_dtype="bf16", seed=21)
    y, S, conv = run_prefill(gdn, case, state_in=False, conv_in=False)
    r = P.run_oracle(case)  # the case's S0 / conv0 are zeros
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])
    case2 = make_case(d, [0, 5, 0], act_dtype="bf16", seed=22, s0_std=0.5, conv0_std=1.0)
    y2, S2, c2 = run_prefill(gdn, case2)
    assert torch.equal(S2[0], case2.S0[0]) and torch.equal(S2[2], case2.S0[2])
    assert torch.equal(c2[0], case2.conv0[0]) and torch.equal(c2[2], case2.conv0[2])


def test_prefill_in_place_states(gdn):
    d = Dims(2, 4, 64, 64)
    case = make_case(d, [70, 1, 150], act_dtype="bf16", seed=23, decay="weak",
                     s0_std=0.3, conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case, inplace=True)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


def test_prefill_bf16_out_is_rne_of_fp32_out_and_deterministic(gdn):
    d = Dims(2, 4, 128, 128)
    case = make_case(d, [300, 45], act_dtype="bf16", seed=24, s0_std=0.02, conv0_std=1.0)
    y32, S32, c32 = run_prefill(gdn, case, torch.float32)
    y16, S16, c16 = run_prefill(gdn, case, torch.bfloat16)
    assert torch.equal(y32.to(torch.bfloat16).float(), y16)
    assert torch.equal(S32, S16) and torch.equal(c32, c16)
    y32b, S32b, _ = run_prefill(gdn, case, torch.float32)
    assert torch.equal(y32, y32b) and torch.equal(S32, S32b)


def test_prefill_split_resume_matches_oracle(gdn):
    """Prefill [0,T1) then [T1,T) from the returned (S, conv) agrees with the
    oracle over [0,T)."""
    d = Dims(2, 4, 64, 64)
    case = make_case(d, [333], act_dtype="bf16", seed=25, decay="weak", s0_std=0.1,
                     conv0_std=1.0)
    cfg = P.gpu_config(d, "bf16")
    params = P.dev_params(case)
    x = {k: P.to_dev(getattr(case, k), "bf16") for k in ("qkv", "z", "a", "b")}
    T1 = 100
    y1, S1, c1 = gdn.prefill_chunked(cfg, params, gdn.SeqLens([0, T1]),
                                     *(x[k][:T1].contiguous() for k in ("qkv", "z", "a", "b")),
                                     state_in=case.S0.cuda(), conv_in=case.conv0.cuda())
    y2, S2, c2 = gdn.prefill_chunked(cfg, params, gdn.SeqLens([0, 333 - T1]),
                                     *(x[k][T1:].contiguous() for k in ("qkv", "z", "a", "b")),
                                     state_in=S1, conv_in=c1)
    torch.cuda.synchronize()
    r = P.run_oracle(case)
    P.assert_y_close(torch.cat([y1, y2]).cpu(), r["y"])
    P.assert_state_close(S2.cpu(), r["S"])
    np.testing.assert_array_equal(c2.cpu().numpy(), r["conv"])


@pytest.mark.slow
def test_prefill_t4096_all_heads(gdn):
    """B=1, T=4096, H_k=16, H_v=32, d=128, C=64, bf16 inputs, zero state."""
    case = chunked_prefill()
    y, S, conv = run_prefill(gdn, case, state_in=False, conv_in=False)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


@pytest.mark.slow
def test_prefill_t4096_weak_decay_all_heads(gdn):
    """The T=4096 layer with a weak decay (A_log = log U[0.001, 0.01]) and a
    non-zero initial state and history, so that the carried state matters
    across all 64 chunks; every output and head is compared."""
    d = chunked_prefill().dims
    case = make_case(d, [4096], act_dtype="bf16", seed=26, decay="weak", s0_std=0.02,
                     conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


@pytest.mark.slow
def test_prefill_varlen_8_all_heads(gdn):
    """8 sequences of U{512..8192} tokens packed via cu_seqlens, random
    initial states and histories; every output, state and head is compared
    with the oracle over the packed batch."""
    case = varlen_prefill()
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


@pytest.mark.slow
def test_prefill_varlen_8_weak_decay_all_heads(gdn):
    """The packed varlen batch again with a weak decay, so each sequence's
    initial state reaches its last tokens."""
    base = varlen_prefill()
    lens = [base.cu_seqlens[i + 1] - base.cu_seqlens[i] for i in range(base.n_seq)]
    case = make_case(base.dims, lens, act_dtype="bf16", seed=27, decay="weak", s0_std=0.02,
                     conv0_std=1.0)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


@pytest.mark.slow
def test_long_handoff_prefill_then_decode_all_heads(gdn):
    """B=1 prefill of T=65536 (sigmoid gate), then 256 decode steps from the
    returned state and history; every head, output and state is compared
    with the oracle run over all 65536 + 256 tokens."""
    case = long_handoff()
    cfg = P.gpu_config(case.dims, "bf16")
    params = P.dev_params(case)
    y, S, conv = gdn.prefill_chunked(cfg, params, gdn.SeqLens(case.cu_seqlens),
                                     *(P.to_dev(getattr(case, k), "bf16") for k in ("qkv", "z", "a", "b")))
    torch.cuda.synchronize()
    S_pf, c_pf = S.cpu(), conv.cpu()
    ys = []
    for s in range(case.dec["qkv"].shape[0]):
        ys.append(gdn.decode_step(cfg, params, *(P.to_dev(case.dec[k][s], "bf16") for k in ("qkv", "z", "a", "b")),
                                  conv, S))
    torch.cuda.synchronize()
    r = P.run_oracle(case)
    P.assert_y_close(y.float().cpu(), r["y"], "prefill out")
    P.assert_state_close(S_pf, r["S"], "state after the prefill")
    np.testing.assert_array_equal(c_pf.numpy(), r["conv"])
    steps = case.dec["qkv"].shape[0]
    cu, qkv, z, a, b = P.decode_as_sequences(case, steps)
    import oracle
    r2 = oracle.mixer(P.oracle_shape(case.dims), cu, case.params, qkv, z, a, b, r["S"], r["conv"],
                      nthreads=P.n_threads())
    yd = torch.stack(ys).float().cpu()[:, 0]
    P.assert_y_close(yd, r2["y"], "decode out")
    P.assert_state_close(S.cpu(), r2["S"], "final state")
    np.testing.assert_array_equal(conv.cpu().numpy(), r2["conv"])


def gate_edge_case(d, lengths, act, seed):
    """A weak-decay case whose gate inputs sit on the edges of the gates:
    a + dt_bias straddles the softplus threshold (20) and b = +-30 (beta
    within 1e-13 of 1 and of 0), mixed with ordinary values."""
    case = make_case(d, lengths, act_dtype=act, seed=seed, decay="weak", s0_std=0.3,
                     conv0_std=1.0)
    T, W = case.a.shape
    a_vals = torch.tensor([19.875, 20.0, 20.125, 24.0, -30.0, 30.0, 0.5])
    b_vals = torch.tensor([30.0, -30.0, 0.0, 5.0, -30.0])
    idx = torch.arange(T * W).view(T, W)
    case.a = a_vals[idx % len(a_vals)].clone()
    case.b = b_vals[torch.arange(T * d.h_v).view(T, d.h_v) % len(b_vals)].clone()
    dtb = case.params["dt_bias"].clone()
    dtb[: dtb.numel() // 2] = 0.0
    dtb[dtb.numel() // 2:] = 0.0625
    case.params["dt_bias"] = dtb
    return case


@pytest.mark.parametrize("decay", ["head", "channel"])
def test_prefill_gate_edge_inputs(gdn, decay):
    d = Dims(2, 4, 64, 64, 4, "silu" if decay == "head" else "sigmoid", decay=decay)
    case = gate_edge_case(d, [70, 130, 1], "bf16", 28)
    y, S, conv = run_prefill(gdn, case)
    r = P.run_oracle(case)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(conv.numpy(), r["conv"])


def test_prefill_all_sequences_empty(gdn):
    """t_total = 0 with several sequences: no chunk exists, the call reads no
    workspace (NULL here, through the C ABI) and each sequence's state and
    history pass through (zeros when none is given)."""
    import ctypes
    d = Dims(2, 4, 64, 64)
    case = make_case(d, [0, 0, 0], act_dtype="bf16", seed=29, s0_std=0.5, conv0_std=1.0)
    cfg = P.gpu_config(d, "bf16")
    assert gdn.prefill_workspace_bytes(cfg, 3, 0) == 0
    lib = gdn.load_library()
    sl = gdn.SeqLens(case.cu_seqlens)
    S_in, c_in = case.S0.cuda(), case.conv0.cuda()
    for with_in in (True, False):
        S_out = torch.full_like(S_in, 7.0)
        c_out = torch.full_like(c_in, 7.0)
        c, p = cfg.c_struct(), gdn._params(cfg, P.dev_params(case))
        st = lib.gdn_prefill_chunked(
            ctypes.byref(c), ctypes.byref(p), 64, 3, 0, ctypes.c_void_p(sl.host.data_ptr()),
            ctypes.c_void_p(sl.dev.data_ptr()), None, None, None, None,
            ctypes.c_void_p(S_in.data_ptr()) if with_in else None, ctypes.c_void_p(S_out.data_ptr()),
            ctypes.c_void_p(c_in.data_ptr()) if with_in else None, ctypes.c_void_p(c_out.data_ptr()),
            None, None, 0, None)
        assert st == 0, lib.gdn_last_error()
        torch.cuda.synchronize()
        if with_in:
            assert torch.equal(S_out, S_in) and torch.equal(c_out, c_in)
        else:
            assert not S_out.any() and not c_out.any()
    # in place, through the binding
    S_io, c_io = S_in.clone(), c_in.clone()
    out, S2, c2 = gdn.prefill_chunked(cfg, P.dev_params(case), sl,
                                      *(P.to_dev(getattr(case, k), "bf16") for k in ("qkv", "z", "a", "b")),
                                      state_in=S_io, conv_in=c_io, state_out=S_io, conv_out=c_io)
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(S2, S_in) and torch.equal(c2, c_in)


def test_prefill_on_side_stream_then_allocations_on_current(gdn):
    """The binding allocates its default outputs and its temporary workspace
    on the stream it enqueues the kernels on: a call on a side stream,
    followed at once by allocations written on the current stream, gives
    the same bits as a call on the current stream."""
    d = Dims(2, 4, 64, 64)
    case = make_case(d, [300, 77], act_dtype="bf16", seed=30, decay="weak", s0_std=0.1,
                     conv0_std=1.0)
    y_ref, S_ref, c_ref = run_prefill(gdn, case)
    cfg = P.gpu_config(d, "bf16")
    params = P.dev_params(case)
    x = [P.to_dev(getattr(case, k), "bf16") for k in ("qkv", "z", "a", "b")]
    sl = gdn.SeqLens(case.cu_seqlens)
    S_in, c_in = case.S0.cuda(), case.conv0.cuda()
    nbytes = gdn.prefill_workspace_bytes(cfg, case.n_seq, case.t_total)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y, S, c = gdn.prefill_chunked(cfg, params, sl, *x, state_in=S_in, conv_in=c_in, stream=side)
    junk = [torch.full((nbytes // 4 + 1024,), float("nan"), device="cuda") for _ in range(3)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    assert torch.equal(y.float().cpu(), y_ref)
    assert torch.equal(S.cpu(), S_ref) and torch.equal(c.cpu(), c_ref)
