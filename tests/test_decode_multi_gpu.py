"""Parity of gdn_decode_multi (several new tokens per sequence in one call)
and gdn_rewind (replay from a saved state) with the oracle.

The oracle runs each sequence's tokens as one packed sequence, which its
split/resume pin shows equals stepping one token at a time.  The rewind is
checked as the pages define it ("oxinfer 0.0.5 src/qwen.rs",
QwenSession::rewind): the state before the span, replayed over the kept
tokens, must equal what the forward reached after them -- bit for bit when
all recorded tokens are kept, since it is the same arithmetic.
"""
import numpy as np
import pytest
import torch

import gdn_parity as P
import oracle
from gdn_inputs import BIG, Dims, make_case, with_decay_coef

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_linear_causal_amd as g
    g.load_library()
    return g


def spec_case(d, B, T, act, seed, decay="weak", coef=False):
    """B sequences with prefilled states and T new tokens each; the decode
    inputs are [T][B][...], regrouped here as [B][T][...]."""
    case = make_case(d, [0] * B, act_dtype=act, seed=seed, decay=decay, s0_std=0.3,
                     conv0_std=1.0, decode_steps=T)
    if coef:
        case.params = with_decay_coef(case.params)
    return case


def bt(case, key):
    return case.dec[key].transpose(0, 1).contiguous()


def oracle_prefix(case, counts):
    """Oracle over the first counts[i] new tokens of each sequence.
    Returns (y [B][T][value_dim] with zeros past each count, S, conv)."""
    B, T = len(counts), case.dec["qkv"].shape[0]
    cu = [0]
    for n in counts:
        cu.append(cu[-1] + n)

    def pack(key):
        x = bt(case, key)
        return torch.cat([x[i, :counts[i]] for i in range(B)]) if cu[-1] else x[:0, 0]
    r = oracle.mixer(P.oracle_shape(case.dims), cu, case.params, pack("qkv"), pack("z"),
                     pack("a"), pack("b"), case.S0, case.conv0, nthreads=P.n_threads())
    y = np.zeros((B, T, case.dims.value_dim))
    for i in range(B):
        y[i, :counts[i]] = r["y"][cu[i]:cu[i + 1]]
    return y, r["S"], r["conv"]


def run_multi(gdn, case, counts=None, ckpt=False, out_dtype=torch.float32, want_out=True):
    cfg = P.gpu_config(case.dims, case.act_dtype, out_dtype)
    S = case.S0.clone().cuda()
    conv = case.conv0.clone().cuda()
    B, T = case.S0.shape[0], case.dec["qkv"].shape[0]
    d = case.dims
    ck = torch.full((B, T, d.h_v, d.d_k, d.d_v), float("nan"), device="cuda") if ckpt else None
    n = None if counts is None else torch.tensor(counts, dtype=torch.int32)
    out = None
    if want_out:
        out = torch.full((B, T, d.value_dim), float("nan"), dtype=out_dtype, device="cuda")
    out = gdn.decode_multi(cfg, P.dev_params(case), P.to_dev(bt(case, "qkv"), case.act_dtype),
                           P.to_dev(bt(case, "z"), case.act_dtype),
                           P.to_dev(bt(case, "a"), case.act_dtype),
                           P.to_dev(bt(case, "b"), case.act_dtype), conv, S, out=out, n_tok=n,
                           ckpt=ck, want_out=want_out)
    torch.cuda.synchronize()
    return (None if out is None else out.float().cpu(), S.cpu(), conv.cpu(),
            None if ck is None else ck.cpu())


VARIANTS = [
    # h_k, h_v, d_k, d_v, K, act, T, head_map, decay_coef
    (2, 4, 128, 128, 4, "bf16", 5, "grouped", False),
    (1, 3, 64, 64, 3, "f32", 8, "grouped", False),
    (2, 2, 32, 32, 2, "bf16", 3, "grouped", True),
    (2, 6, 64, 64, 4, "bf16", 4, "tiled", False),
    (2, 4, 32, 128, 1, "f32", 6, "tiled", True),
    (1, 2, 128, 64, 4, "bf16", 7, "grouped", False),
    # one decay per key channel (Kimi Delta Attention)
    (2, 4, 128, 128, 4, "bf16", 6, "grouped", "channel"),
    (2, 2, 64, 64, 2, "f32", 8, "tiled", "channel"),
]


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: "hk%d_hv%d_dk%d_dv%d_K%d_%s_T%d_%s_%s" % v)
def test_decode_multi_ragged_counts_and_checkpoints(gdn, v):
    """Per-sequence token counts (0, T and in between), outputs, final
    states, histories and every per-token checkpoint against the oracle."""
    hk, hv, dk, dv, K, act, T, head_map, coef = v
    chan = coef == "channel"
    d = Dims(hk, hv, dk, dv, K, "sigmoid" if chan else "silu", head_map,
             decay="channel" if chan else "head")
    B = 5
    case = spec_case(d, B, T, act, seed=500 + hk * 10 + hv + dk + T, coef=coef is True)
    counts = [T, 0, 1, T - 1, max(T // 2, 1)]
    y, S, conv, ck = run_multi(gdn, case, counts, ckpt=True)
    y_ref, S_ref, conv_ref = oracle_prefix(case, counts)
    live = np.zeros(y.shape[:2], bool)
    for i, c in enumerate(counts):
        live[i, :c] = True
    assert torch.isnan(y[~torch.from_numpy(live)]).all(), "output written past the count"
    P.assert_y_close(y.numpy()[live], y_ref[live])
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)
    for t in range(T):
        pre = [min(c, t + 1) for c in counts]
        _, S_t, _ = oracle_prefix(case, pre)
        for i in range(B):
            if t < counts[i]:
                P.assert_state_close(ck[i, t], S_t[i], what=f"checkpoint seq {i} token {t}")
            else:
                assert torch.isnan(ck[i, t]).all(), "checkpoint written past the count"


LONG_VARIANTS = [
    # calls of 7 (stepped) or 8 tokens (in the in-call UT form) without
    # per-token states
    (2, 4, 128, 128, 4, "bf16", 8, "grouped", False),
    (1, 3, 64, 64, 3, "f32", 8, "grouped", False),
    (2, 4, 32, 128, 1, "f32", 7, "tiled", True),
    (1, 2, 128, 64, 4, "bf16", 7, "grouped", False),
    (2, 2, 32, 32, 2, "bf16", 8, "grouped", True),
]


@pytest.mark.parametrize("v", LONG_VARIANTS, ids=lambda v: "hk%d_hv%d_dk%d_dv%d_K%d_%s_T%d_%s_%s" % v)
def test_decode_multi_ragged_counts_without_checkpoints(gdn, v):
    """Calls of 7 or 8 tokens without per-token states (8: the tokens
    combined in the in-call UT form on the matrix cores): per-sequence
    counts, outputs, final states and histories against the oracle, nothing
    written past a count."""
    hk, hv, dk, dv, K, act, T, head_map, coef = v
    d = Dims(hk, hv, dk, dv, K, "silu", head_map)
    B = 5
    case = spec_case(d, B, T, act, seed=540 + hk * 10 + hv + dk + T, coef=coef is True)
    counts = [T, 0, 1, T - 1, max(T // 2, 1)]
    y, S, conv, _ = run_multi(gdn, case, counts)
    y_ref, S_ref, conv_ref = oracle_prefix(case, counts)
    live = np.zeros(y.shape[:2], bool)
    for i, c in enumerate(counts):
        live[i, :c] = True
    assert torch.isnan(y[~torch.from_numpy(live)]).all(), "output written past the count"
    P.assert_y_close(y.numpy()[live], y_ref[live])
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


@pytest.mark.parametrize("T", [4, 8])
def test_decode_multi_b64_full_size_weak_decay(gdn, T):
    """B=64 sequences of the full layer with a weak decay and random states
    (so that the state and every token's update reach the outputs), 4
    drafted tokens (stepped) and 8 (in-call UT form) at the benched shape."""
    case = spec_case(BIG, 64, T, "bf16", seed=12 + T, decay="weak")
    case.S0 = case.S0 * (0.1 / 0.3)
    y, S, conv, _ = run_multi(gdn, case)
    y_ref, S_ref, conv_ref = oracle_prefix(case, [T] * 64)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_multi_b64_full_size_per_channel_decay(gdn, T):
    """B=64 sequences of the full layer with one decay per key channel
    ("cortiq-engine 0.8.76 pipeline.rs", AttnKind::Kda; sigmoid output gate),
    weak decay and random states, 1, 4 and 8 tokens: the benched shapes of the
    per-channel-decay decode."""
    d = Dims(BIG.h_k, BIG.h_v, BIG.d_k, BIG.d_v, BIG.conv_k, "sigmoid", decay="channel")
    case = spec_case(d, 64, T, "bf16", seed=31 + T, decay="weak")
    case.S0 = case.S0 * (0.1 / 0.3)
    y, S, conv, _ = run_multi(gdn, case)
    y_ref, S_ref, conv_ref = oracle_prefix(case, [T] * 64)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


def test_decode_multi_b64_t4_full_size(gdn):
    """B=64 sequences of the full layer (H_k=16, H_v=32, d=128, K=4, bf16),
    4 drafted tokens each: every output, state and history."""
    case = spec_case(BIG, 64, 4, "bf16", seed=11, decay="strong")
    case.S0 = case.S0 * (0.02 / 0.3)
    y, S, conv, _ = run_multi(gdn, case)
    y_ref, S_ref, conv_ref = oracle_prefix(case, [4] * 64)
    P.assert_y_close(y, y_ref)
    P.assert_state_close(S, S_ref)
    np.testing.assert_array_equal(conv.numpy(), conv_ref)


def test_verify_then_rewind(gdn):
    """Verify T drafted tokens, then rewind each sequence to a kept prefix:
    keeping all of them reproduces the verified state bit for bit; keeping
    fewer equals a forward over that prefix bit for bit and the oracle
    within the bar."""
    d = Dims(2, 4, 128, 128, 4)
    B, T = 4, 6
    case = spec_case(d, B, T, "bf16", seed=21)
    cfg = P.gpu_config(d, "bf16")
    prm = P.dev_params(case)
    qkv, a, b = (P.to_dev(bt(case, k), "bf16") for k in ("qkv", "a", "b"))
    z = P.to_dev(bt(case, "z"), "bf16")
    S0, C0 = case.S0.clone().cuda(), case.conv0.clone().cuda()
    S, C = S0.clone(), C0.clone()
    gdn.decode_multi(cfg, prm, qkv, z, a, b, C, S)
    S_all, C_all = gdn.rewind(cfg, prm, qkv, a, b, S0, C0)
    torch.cuda.synchronize()
    assert torch.equal(S_all, S) and torch.equal(C_all, C)

    keep = [0, 2, 5, 6]
    S_k, C_k = gdn.rewind(cfg, prm, qkv, a, b, S0, C0, keep=keep)
    S_f, C_f = S0.clone(), C0.clone()
    gdn.decode_multi(cfg, prm, qkv, z, a, b, C_f, S_f, n_tok=keep, want_out=False)
    torch.cuda.synchronize()
    assert torch.equal(S_k, S_f) and torch.equal(C_k, C_f)
    _, S_ref, C_ref = oracle_prefix(case, keep)
    P.assert_state_close(S_k.cpu(), S_ref)
    np.testing.assert_array_equal(C_k.cpu().numpy(), C_ref)
    # the saved state is untouched, and rewinding in place works too
    assert torch.equal(S0.cpu(), case.S0) and torch.equal(C0.cpu(), case.conv0)
    gdn.rewind(cfg, prm, qkv, a, b, S0, C0, keep=keep, state=S0, conv_state=C0)
    torch.cuda.synchronize()
    assert torch.equal(S0, S_k) and torch.equal(C0, C_k)


def test_verify_then_rewind_eight_tokens(gdn):
    """The rewind contract for 8 recorded tokens, where verification and
    replay run in the in-call UT form: keeping all tokens reproduces the
    verified state bit for bit, keeping fewer equals a forward over the
    prefix bit for bit and the oracle within the bar."""
    d = Dims(2, 4, 128, 128, 4)
    B, T = 4, 8
    case = spec_case(d, B, T, "bf16", seed=23)
    cfg = P.gpu_config(d, "bf16")
    prm = P.dev_params(case)
    qkv, a, b = (P.to_dev(bt(case, k), "bf16") for k in ("qkv", "a", "b"))
    z = P.to_dev(bt(case, "z"), "bf16")
    S0, C0 = case.S0.clone().cuda(), case.conv0.clone().cuda()
    S, C = S0.clone(), C0.clone()
    gdn.decode_multi(cfg, prm, qkv, z, a, b, C, S)
    S_all, C_all = gdn.rewind(cfg, prm, qkv, a, b, S0, C0)
    torch.cuda.synchronize()
    assert torch.equal(S_all, S) and torch.equal(C_all, C)
    keep = [0, 3, 7, 8]
    S_k, C_k = gdn.rewind(cfg, prm, qkv, a, b, S0, C0, keep=keep)
    S_f, C_f = S0.clone(), C0.clone()
    gdn.decode_multi(cfg, prm, qkv, z, a, b, C_f, S_f, n_tok=keep, want_out=False)
    torch.cuda.synchronize()
    assert torch.equal(S_k, S_f) and torch.equal(C_k, C_f)
    _, S_ref, C_ref = oracle_prefix(case, keep)
    P.assert_state_close(S_k.cpu(), S_ref)
    np.testing.assert_array_equal(C_k.cpu().numpy(), C_ref)


def test_verify_then_rewind_per_channel_decay(gdn):
    """The rewind contract with one decay per key channel."""
    d = Dims(2, 4, 64, 64, 4, "sigmoid", decay="channel")
    B, T = 3, 5
    case = spec_case(d, B, T, "bf16", seed=22)
    cfg = P.gpu_config(d, "bf16")
    prm = P.dev_params(case)
    qkv, a, b = (P.to_dev(bt(case, k), "bf16") for k in ("qkv", "a", "b"))
    z = P.to_dev(bt(case, "z"), "bf16")
    S0, C0 = case.S0.clone().cuda(), case.conv0.clone().cuda()
    S, C = S0.clone(), C0.clone()
    gdn.decode_multi(cfg, prm, qkv, z, a, b, C, S)
    S_all, C_all = gdn.rewind(cfg, prm, qkv, a, b, S0, C0)
    keep = [1, 3, 5]
    S_k, C_k = gdn.rewind(cfg, prm, qkv, a, b, S0, C0, keep=keep)
    torch.cuda.synchronize()
    assert torch.equal(S_all, S) and torch.equal(C_all, C)
    _, S_ref, C_ref = oracle_prefix(case, keep)
    P.assert_state_close(S_k.cpu(), S_ref)
    np.testing.assert_array_equal(C_k.cpu().numpy(), C_ref)


def test_decode_multi_one_token_matches_decode_step(gdn):
    d = Dims(2, 4, 64, 64)
    case = spec_case(d, 3, 1, "bf16", seed=31)
    y, S, conv, _ = run_multi(gdn, case)
    cfg = P.gpu_config(d, "bf16")
    S1, C1 = case.S0.clone().cuda(), case.conv0.clone().cuda()
    y1 = gdn.decode_step(cfg, P.dev_params(case), P.to_dev(case.dec["qkv"][0], "bf16"),
                         P.to_dev(case.dec["z"][0], "bf16"), P.to_dev(case.dec["a"][0], "bf16"),
                         P.to_dev(case.dec["b"][0], "bf16"), C1, S1)
    torch.cuda.synchronize()
    P.assert_y_close(y[:, 0], y1.float().cpu().numpy(), what="one-token multi vs step")
    P.assert_state_close(S, S1.cpu(), what="one-token multi vs step")
    assert torch.equal(conv, C1.cpu())


def test_decode_multi_bf16_out_in_place_and_deterministic(gdn):
    d = Dims(2, 4, 128, 128)
    case = spec_case(d, 3, 4, "bf16", seed=41)
    y32, S32, c32, _ = run_multi(gdn, case)
    y16, S16, c16, _ = run_multi(gdn, case, out_dtype=torch.bfloat16)
    assert torch.equal(y32.to(torch.bfloat16).float(), y16)
    assert torch.equal(S32, S16) and torch.equal(c32, c16)
    # out of place gives the same bits and leaves the inputs alone
    cfg = P.gpu_config(d, "bf16")
    S_in, C_in = case.S0.clone().cuda(), case.conv0.clone().cuda()
    S_out, C_out = torch.empty_like(S_in), torch.empty_like(C_in)
    y = gdn.decode_multi(cfg, P.dev_params(case), P.to_dev(bt(case, "qkv"), "bf16"),
                         P.to_dev(bt(case, "z"), "bf16"), P.to_dev(bt(case, "a"), "bf16"),
                         P.to_dev(bt(case, "b"), "bf16"), C_in, S_in, conv_out=C_out,
                         state_out=S_out)
    torch.cuda.synchronize()
    assert torch.equal(y.float().cpu(), y32)
    assert torch.equal(S_out.cpu(), S32) and torch.equal(C_out.cpu(), c32)
    assert torch.equal(S_in.cpu(), case.S0) and torch.equal(C_in.cpu(), case.conv0)
