"""gdn_prefill_chunked_noalloc, the allocation-free prefill (its workspace is
the library's static device scratch), against gdn_prefill_chunked with a
caller workspace: both run the same kernels, so outputs, states and
histories must agree bit for bit.  Two calls in a row, the second smaller,
so the second runs over what the first left in the shared scratch."""
import ctypes

import numpy as np
import pytest
import torch

import gdn_parity as P
from gdn_inputs import BIG, Dims, make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_linear_causal_amd as g
    g.load_library()
    return g


def both(gdn, case, out_dtype=torch.float32):
    cfg = P.gpu_config(case.dims, case.act_dtype, out_dtype)
    assert gdn.prefill_workspace_bytes(cfg, case.n_seq, case.t_total) <= gdn.PREFILL_NOALLOC_MAX_BYTES
    params = P.dev_params(case)
    sl = gdn.SeqLens(case.cu_seqlens)
    x = [P.to_dev(getattr(case, k), case.act_dtype) for k in ("qkv", "z", "a", "b")]
    S_in, c_in = case.S0.cuda(), case.conv0.cuda()
    res = []
    for fn in (gdn.prefill_chunked, gdn.prefill_chunked_noalloc):
        out = torch.full((case.t_total, case.dims.value_dim), float("nan"), dtype=out_dtype,
                         device="cuda")
        S = torch.full_like(S_in, float("nan"))
        C = torch.full_like(c_in, float("nan"))
        fn(cfg, params, sl, *x, state_in=S_in, conv_in=c_in, state_out=S, conv_out=C, out=out)
        torch.cuda.synchronize()
        res.append((out.float().cpu(), S.cpu(), C.cpu()))
    (y0, S0, C0), (y1, S1, C1) = res
    assert torch.equal(y0, y1), "out differs"
    assert torch.equal(S0, S1), "state differs"
    assert torch.equal(C0, C1), "conv history differs"
    return y1, S1, C1


def test_noalloc_two_calls_match_the_workspace_entry_point(gdn):
    # 1: the full layer (H_k=16, H_v=32, d=128), two sequences, weak decay
    case1 = make_case(BIG, [300, 150], act_dtype="bf16", seed=950, decay="weak", s0_std=0.02,
                      conv0_std=1.0)
    y, S, C = both(gdn, case1)
    r = P.run_oracle(case1)
    P.assert_y_close(y, r["y"])
    P.assert_state_close(S, r["S"])
    np.testing.assert_array_equal(C.numpy(), r["conv"])
    # 2: a smaller call right after, on what the first left in the scratch
    case2 = make_case(Dims(2, 4, 64, 64), [1, 63, 65, 0, 7], act_dtype="bf16", seed=951,
                      decay="weak", s0_std=0.3, conv0_std=1.0)
    y2, S2, C2 = both(gdn, case2, torch.bfloat16)
    case2b = make_case(Dims(2, 4, 64, 64), [100], act_dtype="f32", seed=952, s0_std=0.3,
                       conv0_std=1.0)
    both(gdn, case2b)


def test_noalloc_rejects_calls_beyond_its_scratch(gdn):
    """A call whose workspace would exceed the static scratch is refused
    before anything is enqueued: its outputs keep their contents."""
    T = 4096
    cfg = P.gpu_config(BIG, "bf16")
    assert gdn.prefill_workspace_bytes(cfg, 1, T) > gdn.PREFILL_NOALLOC_MAX_BYTES
    case = make_case(BIG, [T], act_dtype="bf16", seed=953)
    x = [P.to_dev(getattr(case, k), "bf16") for k in ("qkv", "z", "a", "b")]
    S = torch.full((1, BIG.h_v, BIG.d_k, BIG.d_v), 3.0, device="cuda")
    C = torch.full((1, BIG.conv_k - 1, BIG.conv_dim), 3.0, device="cuda")
    out = torch.full((T, BIG.value_dim), 3.0, device="cuda")
    with pytest.raises(gdn.GdnError) as ei:
        gdn.prefill_chunked_noalloc(cfg, P.dev_params(case), gdn.SeqLens([0, T]), *x,
                                    state_out=S, conv_out=C, out=out)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    assert bool((S == 3.0).all()) and bool((C == 3.0).all()) and bool((out == 3.0).all())
