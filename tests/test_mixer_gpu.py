"""Parity of the mixer with its projections (gdn_mixer_prefill and
gdn_mixer_decode: in_proj GEMMs, the core, out_proj GEMM) with the oracle
("oxinfer 0.0.5 src/qwen.rs", Gdn struct and gdn_forward).

The oracle projects in float64 from the same bf16 weights and hidden states;
the GPU accumulates the projections in fp32 and keeps the projected
activations in fp32, so the conv histories (raw projected inputs) agree to
fp32 rounding, not bit for bit.  Outputs and states use the core's bars.
"""
import numpy as np
import pytest
import torch

import gdn_parity as P
import oracle
from gdn_inputs import BIG, Dims, make_case, make_hidden, make_projections

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_linear_causal_amd as g
    g.load_library()
    return g


def dev_proj(proj):
    return {k: (v if k == "hidden" else v.to(torch.bfloat16).contiguous().cuda())
            for k, v in proj.items()}


def conv_close(conv_gpu, conv_ref):
    np.testing.assert_allclose(np.asarray(conv_gpu, np.float64), conv_ref, rtol=1e-5, atol=1e-5)


LAYERS = [
    # h_k, h_v, d, hidden, decay, lengths
    (2, 4, 64, 256, "head", [1, 63, 65, 130]),
    (2, 4, 64, 128, "channel", [100, 7]),
    (1, 2, 128, 512, "head", [200]),
]


@pytest.mark.parametrize("v", LAYERS, ids=lambda v: "hk%d_hv%d_d%d_H%d_%s_%s" % (
    *v[:5], "-".join(map(str, v[5]))))
def test_mixer_prefill(gdn, v):
    hk, hv, dd, H, decay, lengths = v
    d = Dims(hk, hv, dd, dd, 4, "sigmoid" if decay == "channel" else "silu", decay=decay)
    case = make_case(d, lengths, act_dtype="bf16", seed=800 + H + dd, decay="weak", s0_std=0.3,
                     conv0_std=1.0)
    proj = make_projections(d, H, seed=801 + H)
    x = make_hidden(case.t_total, H, seed=802 + H)
    cfg = P.gpu_config(d, "bf16", torch.float32)
    out, S, conv = gdn.mixer_prefill(cfg, P.dev_params(case), dev_proj(proj),
                                     gdn.SeqLens(case.cu_seqlens),
                                     x.to(torch.bfloat16).cuda(), state_in=case.S0.cuda(),
                                     conv_in=case.conv0.cuda())
    torch.cuda.synchronize()
    r = oracle.mixer_layer(P.oracle_shape(d), case.cu_seqlens, case.params, proj, x, case.S0,
                           case.conv0, nthreads=P.n_threads())
    P.assert_y_close(out.cpu(), r["out"], "mixer out")
    P.assert_state_close(S.cpu(), r["S"])
    conv_close(conv.cpu(), r["conv"])


def test_mixer_decode_steps(gdn):
    """Six consecutive mixer decode steps for five sequences."""
    d = Dims(2, 4, 64, 64)
    H, B, steps = 256, 5, 6
    case = make_case(d, [0] * B, act_dtype="bf16", seed=810, decay="weak", s0_std=0.3,
                     conv0_std=1.0)
    proj = make_projections(d, H, seed=811)
    xs = make_hidden(steps * B, H, seed=812).view(steps, B, H)
    cfg = P.gpu_config(d, "bf16", torch.float32)
    prm, pj = P.dev_params(case), dev_proj(proj)
    S, C = case.S0.clone().cuda(), case.conv0.clone().cuda()
    outs = [gdn.mixer_decode(cfg, prm, pj, xs[s].to(torch.bfloat16).cuda(), C, S)
            for s in range(steps)]
    torch.cuda.synchronize()
    y = torch.stack(outs).float().cpu()                       # [steps, B, H]
    x_seq = xs.transpose(0, 1).reshape(B * steps, H)          # sequence-major
    r = oracle.mixer_layer(P.oracle_shape(d), [i * steps for i in range(B + 1)], case.params,
                           proj, x_seq, case.S0, case.conv0, nthreads=P.n_threads())
    P.assert_y_close(y.transpose(0, 1).reshape(B * steps, H), r["out"], "mixer decode out")
    P.assert_state_close(S.cpu(), r["S"])
    conv_close(C.cpu(), r["conv"])


DECODE_LAYERS = [
    # h_k, h_v, d, hidden, decay mode, K, batch.  The decode step projects on
    # the matrix cores (conv in the in_proj epilogue) when hidden and
    # value_dim are multiples of 256, H_v of 4 and batch <= 64 (hidden 4096:
    # four contraction slices and a separate epilogue; hidden 2048 with
    # d = 128 above 8 sequences: two slices that the recurrence kernel sums
    # while it loads them); the last three cases take the library GEMMs
    # (hidden, batch, H_v).
    (2, 4, 64, 256, "head", 4, 5),
    (2, 4, 64, 256, "channel", 3, 7),
    (1, 4, 128, 512, "head", 1, 33),
    (4, 8, 32, 1024, "head", 2, 64),
    (2, 4, 64, 4096, "head", 4, 3),
    (1, 4, 128, 2048, "head", 4, 20),
    (2, 4, 128, 2048, "head", 2, 9),
    # the one-slice product with the conv in its epilogue at K = 2 and K = 1
    (2, 4, 64, 256, "head", 2, 6),
    (2, 4, 64, 512, "head", 1, 8),
    (2, 4, 32, 200, "head", 4, 3),
    (2, 4, 64, 256, "head", 4, 70),
    (1, 2, 128, 256, "head", 4, 4),
]


@pytest.mark.parametrize("v", DECODE_LAYERS, ids=lambda v: "hk%d_hv%d_d%d_H%d_%s_K%d_B%d" % v)
def test_mixer_decode_layers(gdn, v):
    """Four consecutive mixer decode steps against the oracle's layer run
    over the same tokens ("oxinfer 0.0.5 src/qwen.rs", gdn_forward)."""
    hk, hv, dd, H, mode, K, B = v
    d = Dims(hk, hv, dd, dd, K, "sigmoid" if mode == "channel" else "silu", decay=mode)
    steps = 4
    case = make_case(d, [0] * B, act_dtype="bf16", seed=850 + H + B + K, decay="weak",
                     s0_std=0.3, conv0_std=1.0)
    proj = make_projections(d, H, seed=851 + H)
    xs = make_hidden(steps * B, H, seed=852 + B).view(steps, B, H)
    cfg = P.gpu_config(d, "bf16", torch.float32)
    prm, pj = P.dev_params(case), dev_proj(proj)
    S, C = case.S0.clone().cuda(), case.conv0.clone().cuda()
    outs = [gdn.mixer_decode(cfg, prm, pj, xs[t].to(torch.bfloat16).cuda(), C, S)
            for t in range(steps)]
    torch.cuda.synchronize()
    y = torch.stack(outs).float().cpu()
    x_seq = xs.transpose(0, 1).reshape(B * steps, H)
    r = oracle.mixer_layer(P.oracle_shape(d), [i * steps for i in range(B + 1)], case.params,
                           proj, x_seq, case.S0, case.conv0, nthreads=P.n_threads())
    P.assert_y_close(y.transpose(0, 1).reshape(B * steps, H), r["out"], "mixer decode out")
    P.assert_state_close(S.cpu(), r["S"])
    conv_close(C.cpu(), r["conv"])


@pytest.mark.parametrize("B", [1, 8, 64])
def test_mixer_decode_full_layer(gdn, B):
    """The full layer (hidden 2048, H_k=16, H_v=32, d=128), one step at the
    benched batch sizes (B = 1 and 8: the one-slice product with the conv in
    its epilogue; B = 64: two slices summed by the core), bf16 output = RNE
    of the fp32 output."""
    H = 2048
    case = make_case(BIG, [0] * B, act_dtype="bf16", seed=820 + B, s0_std=0.02, conv0_std=1.0)
    proj = make_projections(BIG, H, seed=821)
    x = make_hidden(B, H, seed=822)
    prm, pj = P.dev_params(case), dev_proj(proj)
    res = {}
    for dt in (torch.float32, torch.bfloat16):
        cfg = P.gpu_config(BIG, "bf16", dt)
        S, C = case.S0.clone().cuda(), case.conv0.clone().cuda()
        res[dt] = (gdn.mixer_decode(cfg, prm, pj, x.to(torch.bfloat16).cuda(), C, S), S, C)
    torch.cuda.synchronize()
    y32, S, C = (t.cpu() for t in res[torch.float32])
    assert torch.equal(y32.to(torch.bfloat16), res[torch.bfloat16][0].cpu())
    r = oracle.mixer_layer(P.oracle_shape(BIG), list(range(B + 1)), case.params, proj, x,
                           case.S0, case.conv0, nthreads=P.n_threads())
    P.assert_y_close(y32.float(), r["out"], "mixer out")
    P.assert_state_close(S, r["S"])
    conv_close(C, r["conv"])


@pytest.mark.slow
def test_mixer_prefill_full_layer_hidden_2048(gdn):
    """The full layer (hidden 2048, H_k=16, H_v=32, d=128, K=4) over two
    sequences (1024 and 300 tokens) with a weak decay and random initial
    states: the GEMM shapes hipBLASLt plans at full size, every output and
    head compared."""
    H = 2048
    case = make_case(BIG, [1024, 300], act_dtype="bf16", seed=830, decay="weak", s0_std=0.02,
                     conv0_std=1.0)
    proj = make_projections(BIG, H, seed=831)
    x = make_hidden(case.t_total, H, seed=832)
    cfg = P.gpu_config(BIG, "bf16", torch.float32)
    out, S, conv = gdn.mixer_prefill(cfg, P.dev_params(case), dev_proj(proj),
                                     gdn.SeqLens(case.cu_seqlens),
                                     x.to(torch.bfloat16).cuda(), state_in=case.S0.cuda(),
                                     conv_in=case.conv0.cuda())
    torch.cuda.synchronize()
    r = oracle.mixer_layer(P.oracle_shape(BIG), case.cu_seqlens, case.params, proj, x, case.S0,
                           case.conv0, nthreads=P.n_threads())
    P.assert_y_close(out.cpu(), r["out"], "mixer out")
    P.assert_state_close(S.cpu(), r["S"])
    conv_close(conv.cpu(), r["conv"])


def test_mixer_prefill_all_sequences_empty(gdn):
    """t_total = 0 with three sequences: states and histories pass through."""
    d = Dims(2, 4, 64, 64)
    H = 128
    case = make_case(d, [0, 0, 0], act_dtype="bf16", seed=840, s0_std=0.5, conv0_std=1.0)
    proj = make_projections(d, H, seed=841)
    cfg = P.gpu_config(d, "bf16", torch.float32)
    x = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    out, S, conv = gdn.mixer_prefill(cfg, P.dev_params(case), dev_proj(proj),
                                     gdn.SeqLens(case.cu_seqlens), x, state_in=case.S0.cuda(),
                                     conv_in=case.conv0.cuda())
    torch.cuda.synchronize()
    assert out.numel() == 0
    assert torch.equal(S.cpu(), case.S0) and torch.equal(conv.cpu(), case.conv0)
