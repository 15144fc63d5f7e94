"""Parity of gdn_conv_update (causal depthwise conv + SiLU with history
carry over packed sequences) with the oracle's conv."""
import numpy as np
import pytest
import torch

import gdn_parity as P
import oracle
from gdn_inputs import Dims, make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_linear_causal_amd as g
    g.load_library()
    return g


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_conv_update_varlen(gdn, K, act):
    d = Dims(2, 4, 32, 64, conv_k=K)
    lengths = [0, 1, 2, 5, 64, 65, 130, 3]
    case = make_case(d, lengths, act_dtype=act, seed=K, conv0_std=1.0)
    cfg = P.gpu_config(d, act)
    sl = gdn.SeqLens(case.cu_seqlens)
    conv = case.conv0.clone().cuda()
    y = gdn.conv_update(cfg, P.dev_params(case), sl, P.to_dev(case.qkv, act), conv)
    torch.cuda.synchronize()
    y_ref, st_ref = oracle.conv(P.oracle_shape(d), case.cu_seqlens, case.params["conv_w"],
                                case.qkv, case.conv0)
    P.assert_y_close(y.cpu(), y_ref, "conv out")
    np.testing.assert_allclose(y.cpu().numpy(), y_ref, rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(conv.cpu().numpy(), st_ref)


def test_conv_update_split_resume(gdn):
    """Two calls with the carried history equal one call over the whole
    sequence (same fp32 arithmetic per token: bit-exact)."""
    d = Dims(2, 2, 64, 64, conv_k=4)
    case = make_case(d, [200], act_dtype="bf16", seed=5, conv0_std=1.0)
    cfg = P.gpu_config(d, "bf16")
    params = P.dev_params(case)
    x = P.to_dev(case.qkv, "bf16")
    c_all = case.conv0.clone().cuda()
    y_all = gdn.conv_update(cfg, params, gdn.SeqLens([0, 200]), x, c_all)
    c_sp = case.conv0.clone().cuda()
    y1 = gdn.conv_update(cfg, params, gdn.SeqLens([0, 77]), x[:77].contiguous(), c_sp)
    y2 = gdn.conv_update(cfg, params, gdn.SeqLens([0, 123]), x[77:].contiguous(), c_sp)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2]), y_all)
    assert torch.equal(c_sp, c_all)
