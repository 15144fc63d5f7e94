"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one part of the oracle to something fixed independently of
its code: a closed form reached by hand, a textbook library routine, a
brute-force transition-matrix formulation, or an invariant of the method.
A dropped term, flipped sign, wrong index or transposed operand anywhere in
the oracle breaks at least one of them.

Sources of the method: "cherenkov qwen4_exp/cpu.rs" (fn deltanet,
fn causal_conv), "oxinfer 0.0.5 src/qwen.rs" (DeltaRule::run, gdn_forward,
GdnState), "cortiq-engine 0.6.5 src/qwen4_exp.rs" (fn sigmoid, fn silu).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.signal import lfilter

import oracle
from oracle.chunked import chunked_core
from gdn_inputs import Dims, make_case

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _shape(d: Dims, **kw):
    return oracle.Shape(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k,
                        kw.get("gate", d.gate))


def _t(x):
    return torch.as_tensor(np.asarray(x, np.float64))


def _rand_unit_rows(rng, L, d):
    x = rng.standard_normal((L, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


# --------------------------------------------------------------------------
# causal conv + SiLU  (cpu.rs fn causal_conv; qwen.rs gdn_forward)
# --------------------------------------------------------------------------

def test_conv_current_tap_only_is_silu():
    """W = e_{K-1}: the conv is the identity, leaving torch's SiLU."""
    d = Dims(1, 1, 4, 4, conv_k=4)
    rng = np.random.default_rng(0)
    L = 9
    x = rng.standard_normal((L, d.conv_dim)) * 3
    w = np.zeros((d.conv_dim, 4))
    w[:, 3] = 1.0
    h0 = rng.standard_normal((1, 3, d.conv_dim))
    c, _ = oracle.conv(_shape(d), [0, L], w, x, h0)
    np.testing.assert_allclose(c, F.silu(_t(x)).numpy(), rtol=1e-15, atol=0)


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_is_textbook_fir_filter(K):
    """With a history, each channel equals scipy's causal FIR filter run over
    [history, x] (taps reversed: the newest input meets w[K-1]).  K = 1 is a
    per-channel scale with an empty history."""
    d = Dims(1, 2, 3, 5, conv_k=K)
    rng = np.random.default_rng(K)
    L = 11
    x = rng.standard_normal((L, d.conv_dim))
    w = rng.standard_normal((d.conv_dim, K))
    hist = rng.standard_normal((1, K - 1, d.conv_dim))
    c, st = oracle.conv(_shape(d), [0, L], w, x, hist)
    full = np.concatenate([hist[0], x], axis=0)
    for ch in range(d.conv_dim):
        h = lfilter(w[ch, ::-1], [1.0], full[:, ch])[K - 1:]
        ref = F.silu(_t(h)).numpy()
        np.testing.assert_allclose(c[:, ch], ref, rtol=1e-13, atol=1e-15)
    # new history: last K-1 raw inputs, oldest first (none when K = 1)
    assert st.shape == (1, K - 1, d.conv_dim)
    if K > 1:
        np.testing.assert_array_equal(st[0], full[-(K - 1):])


@pytest.mark.parametrize("L", [0, 1, 2, 3, 5])
def test_conv_history_short_sequences(L):
    """L < K-1 keeps the tail of the old history ahead of the new inputs;
    L = 0 passes the history through untouched."""
    d = Dims(1, 1, 2, 2, conv_k=4)
    rng = np.random.default_rng(L)
    x = rng.standard_normal((L, d.conv_dim))
    hist = rng.standard_normal((1, 3, d.conv_dim))
    _, st = oracle.conv(_shape(d), [0, L], rng.standard_normal((d.conv_dim, 4)),
                        x, hist)
    full = np.concatenate([hist[0], x], axis=0)
    np.testing.assert_array_equal(st[0], full[-3:])


def test_conv_split_resume_bit_exact():
    d = Dims(1, 2, 4, 4, conv_k=4)
    rng = np.random.default_rng(3)
    L, L1 = 20, 7
    x = rng.standard_normal((L, d.conv_dim))
    w = rng.standard_normal((d.conv_dim, 4))
    h0 = rng.standard_normal((1, 3, d.conv_dim))
    c, st = oracle.conv(_shape(d), [0, L], w, x, h0)
    c1, st1 = oracle.conv(_shape(d), [0, L1], w, x[:L1], h0)
    c2, st2 = oracle.conv(_shape(d), [0, L - L1], w, x[L1:], st1)
    np.testing.assert_array_equal(np.concatenate([c1, c2]), c)
    np.testing.assert_array_equal(st2, st)


# --------------------------------------------------------------------------
# delta-rule core  (cpu.rs fn deltanet; qwen.rs DeltaRule::run)
# --------------------------------------------------------------------------

def test_core_beta_zero_only_decays():
    """beta = 0: nothing is written, S_L = exp(sum g) S_0 and every readout
    comes from the decayed initial state."""
    rng = np.random.default_rng(1)
    L, dk, dv = 13, 6, 5
    q = rng.standard_normal((L, dk))
    k = _rand_unit_rows(rng, L, dk)
    v = rng.standard_normal((L, dv))
    g = -rng.uniform(0.0, 0.5, L)
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.delta_core(q, k, v, g, np.zeros(L), S0)
    G = np.cumsum(g)
    np.testing.assert_allclose(S, np.exp(G[-1]) * S0, rtol=1e-13)
    np.testing.assert_allclose(o, np.exp(G)[:, None] * (q @ S0), rtol=1e-12,
                               atol=1e-14)


def test_core_store_and_retrieve_orthonormal_keys():
    """g = 0, beta = 1, keys = distinct basis vectors, S_0 = 0: the state is
    sum e_i v_i^T exactly and S^T e_j returns v_j bit for bit."""
    rng = np.random.default_rng(2)
    dk, dv = 8, 7
    perm = rng.permutation(dk)
    k = np.eye(dk)[perm]
    v = rng.standard_normal((dk, dv))
    q = np.eye(dk)[perm]
    o, S = oracle.delta_core(q, k, v, np.zeros(dk), np.ones(dk),
                             np.zeros((dk, dv)))
    expect = np.zeros((dk, dv))
    expect[perm] = v
    np.testing.assert_array_equal(S, expect)
    np.testing.assert_array_equal(o, v)          # read back what was stored
    for j in range(dk):
        np.testing.assert_array_equal(S.T @ np.eye(dk)[perm[j]], v[j])


def test_core_same_key_overwrites():
    """Writing the same unit key twice with beta = 1, g = 0 leaves the latest
    value under that key, to rounding (s + (v - s) is v within an ulp): the
    delta rule replaces, it does not accumulate."""
    rng = np.random.default_rng(5)
    dk, dv = 4, 3
    key = np.eye(dk)[2]
    k = np.stack([key, key])
    v = rng.standard_normal((2, dv))
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.delta_core(k, k, v, np.zeros(2), np.ones(2), S0)
    np.testing.assert_allclose(S.T @ key, v[1], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(o[1], v[1], rtol=1e-15, atol=1e-16)
    # other keys' rows are untouched
    np.testing.assert_array_equal(np.delete(S, 2, axis=0),
                                  np.delete(S0, 2, axis=0))


def _brute_force_core(q, k, v, g, beta, S0):
    """Transition-matrix form: S_t = a_t (I - b_t k k^T) S_{t-1} + b_t k v^T,
    o_t = S_t^T q_t, with explicit d_k x d_k matrices."""
    S = S0.copy()
    dk = S.shape[0]
    out = []
    for t in range(len(g)):
        kk = k[t][:, None]
        Tm = np.exp(g[t]) * (np.eye(dk) - beta[t] * (kk @ kk.T))
        S = Tm @ S + beta[t] * (kk @ v[t][None, :])
        out.append(S.T @ q[t])
    return np.array(out), S


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_core_matches_transition_matrix_brute_force(seed):
    rng = np.random.default_rng(seed)
    L, dk, dv = 17, 5, 4
    q = rng.standard_normal((L, dk)) * 0.4
    k = _rand_unit_rows(rng, L, dk)
    v = rng.standard_normal((L, dv))
    g = -rng.uniform(0.0, 1.0, L)
    beta = rng.uniform(0.0, 1.0, L)
    S0 = rng.standard_normal((dk, dv)) * 0.3
    o, S = oracle.delta_core(q, k, v, g, beta, S0)
    o_ref, S_ref = _brute_force_core(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 64])
@pytest.mark.parametrize("decay", ["strong", "weak"])
def test_chunked_form_matches_recurrence(chunk, decay):
    """The chunkwise UT-transform form agrees with the token recurrence in
    float64, for lengths that are not multiples of the chunk."""
    rng = np.random.default_rng(chunk)
    L, dk, dv = 130, 8, 6
    q = rng.standard_normal((L, dk)) / np.sqrt(dk)
    k = _rand_unit_rows(rng, L, dk)
    v = rng.standard_normal((L, dv))
    g = -(rng.uniform(1, 16, L) if decay == "strong"
          else rng.uniform(0.001, 0.01, L))
    beta = rng.uniform(0, 1, L)
    S0 = rng.standard_normal((dk, dv)) * 0.02
    o, S = oracle.delta_core(q, k, v, g, beta, S0)
    oc, Sc = chunked_core(q, k, v, g, beta, S0, chunk)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-14)


def test_core_linear_in_state_and_values():
    """(S_0, v) -> (c S_0, c v) scales every readout and the final state by c
    (beta, g and the keys fix a linear map)."""
    rng = np.random.default_rng(9)
    L, dk, dv = 12, 6, 6
    q = rng.standard_normal((L, dk))
    k = _rand_unit_rows(rng, L, dk)
    v = rng.standard_normal((L, dv))
    g = -rng.uniform(0, 1, L)
    beta = rng.uniform(0, 1, L)
    S0 = rng.standard_normal((dk, dv))
    o1, S1 = oracle.delta_core(q, k, v, g, beta, S0)
    o2, S2 = oracle.delta_core(q, k, 2.5 * v, g, beta, 2.5 * S0)
    np.testing.assert_allclose(o2, 2.5 * o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, 2.5 * S1, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# full mixer  (cpu.rs fn deltanet; qwen.rs gdn_forward)
# --------------------------------------------------------------------------

def _case(d, lengths, seed=0, **kw):
    kw.setdefault("act_dtype", "f32")
    return make_case(d, lengths, seed=seed, **kw)


def _run(c, d=None, **kw):
    d = d or c.dims
    return oracle.mixer(_shape(d, **{k: v for k, v in kw.items() if k == "gate"}),
                        c.cu_seqlens, c.params, c.qkv, c.z, c.a, c.b, c.S0,
                        c.conv0, **{k: v for k, v in kw.items() if k != "gate"})


@pytest.mark.parametrize("gate", ["silu", "sigmoid"])
def test_mixer_single_token_closed_form(gate):
    """From S_0 = 0 and a zero history, one token gives
    o = beta (q^.k^) v, hence y = rms_norm(o) * w * gate(z), built here from
    torch's normalize / rms_norm / sigmoid / silu routines."""
    d = Dims(2, 4, 16, 8, conv_k=4, gate=gate)
    c = _case(d, [1], seed=11)
    c.qkv *= 3.0   # keep |q|^2, |k|^2 >> the 1e-6 inside the norm
    out = _run(c, gate=gate)
    x = _t(c.qkv[0])
    h = _t(c.params["conv_w"][:, -1]) * x          # only the current tap
    cact = F.silu(h)
    HK, HV, DK, DV = d.h_k, d.h_v, d.d_k, d.d_v
    qh = F.normalize(cact[:HK * DK].view(HK, DK), dim=1) / np.sqrt(DK)
    kh = F.normalize(cact[HK * DK:2 * HK * DK].view(HK, DK), dim=1)
    vv = cact[2 * HK * DK:].view(HV, DV)
    beta = torch.sigmoid(_t(c.b[0]))
    grp = HV // HK
    qk = (qh * kh).sum(1).repeat_interleave(grp)
    o = (beta * qk)[:, None] * vv
    gz = (torch.sigmoid if gate == "sigmoid" else F.silu)(_t(c.z[0]).view(HV, DV))
    y = F.rms_norm(o, (DV,), _t(c.params["norm_w"]), eps=1e-6) * gz
    np.testing.assert_allclose(out["y"][0], y.reshape(-1).numpy(),
                               rtol=1e-5, atol=1e-9)
    # the state is the single rank-one write k^ (beta v)^T
    S_ref = kh.repeat_interleave(grp, 0)[:, :, None] * (beta[:, None] * vv)[:, None, :]
    np.testing.assert_allclose(out["S"][0], S_ref.numpy(), rtol=1e-5, atol=1e-12)


def test_mixer_gates_via_beta_zero_decay():
    """b = -inf makes beta = 0, so S_L = exp(sum_t g_t) S_0 with
    g = -exp(A_log) softplus(a + dt_bias) from torch's softplus (threshold
    20); the a values straddle the threshold."""
    d = Dims(1, 2, 4, 3, conv_k=3)
    L = 6
    c = _case(d, [L], seed=12, s0_std=1.0, conv0_std=1.0)
    c.b[:] = -float("inf")
    c.a[:] = torch.tensor([[-3.0, 19.5], [0.5, 20.5], [2.0, 25.0],
                           [-1.0, 19.9], [21.0, 1.0], [0.0, 30.0]])
    c.params["dt_bias"][:] = torch.tensor([0.25, 0.3])
    c.params["a_log"][:] = torch.tensor([-2.0, -3.5])
    out = _run(c)
    sp = F.softplus(_t(c.a) + _t(c.params["dt_bias"]), beta=1, threshold=20)
    g = -torch.exp(_t(c.params["a_log"])) * sp
    decay = torch.exp(g.sum(0)).numpy()
    np.testing.assert_allclose(out["S"][0], decay[:, None, None] * c.S0[0].numpy(),
                               rtol=1e-13)


@pytest.mark.parametrize("gate", ["silu", "sigmoid"])
def test_mixer_gated_norm_is_torch_rms_norm(gate):
    d = Dims(2, 4, 8, 16, conv_k=4, gate=gate)
    c = _case(d, [5, 9], seed=13, s0_std=0.3, conv0_std=1.0)
    out = _run(c, gate=gate, want_pre=True)
    o = _t(out["o_pre"]).view(-1, d.h_v, d.d_v)
    zz = _t(c.z).view(-1, d.h_v, d.d_v)
    gz = torch.sigmoid(zz) if gate == "sigmoid" else F.silu(zz)
    y = F.rms_norm(o, (d.d_v,), _t(c.params["norm_w"]), eps=1e-6) * gz
    np.testing.assert_allclose(out["y"], y.reshape(out["y"].shape).numpy(),
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("head_map,decay_form", [("grouped", "a_log"), ("tiled", "a_log"),
                                                  ("grouped", "decay_coef"),
                                                  ("tiled", "decay_coef")])
def test_mixer_matches_independent_formulation(head_map, decay_form):
    """Whole mixer vs. a second formulation: scipy FIR conv, torch SiLU /
    sigmoid / softplus / rms_norm, explicit L2 scaling, transition-matrix
    recurrence; several tokens, grouped heads, non-zero states.  Both key-head
    orders ("oxinfer 0.0.5 src/qwen.rs", DeltaRule::run: contiguous groups
    hv // (H_v/H_k), or tiled hv % H_k) and both forms of the decay
    coefficient (-exp(A_log), or the coefficient given directly as GGUF's
    ssm_a stores it).  H_v/H_k = 3 and H_k = 2, so that neither order can
    pass for the other or for hv % group."""
    d = Dims(2, 6, 6, 5, conv_k=4)
    L = 10
    c = _case(d, [L], seed=14, s0_std=0.3, conv0_std=1.0, decay="weak")
    if decay_form == "decay_coef":
        c.params["decay_coef"] = -torch.exp(c.params.pop("a_log").double()).float()
    out = oracle.mixer(oracle.Shape(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k, d.gate,
                                    head_map=head_map),
                       c.cu_seqlens, c.params, c.qkv, c.z, c.a, c.b, c.S0, c.conv0,
                       want_pre=True)
    HK, HV, DK, DV, K = d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k
    x = np.asarray(c.qkv, np.float64)
    full = np.concatenate([np.asarray(c.conv0[0], np.float64), x])
    w = np.asarray(c.params["conv_w"], np.float64)
    h = np.stack([lfilter(w[ch, ::-1], [1.0], full[:, ch])[K - 1:]
                  for ch in range(d.conv_dim)], axis=1)
    act = F.silu(_t(h)).numpy()
    sp = F.softplus(_t(c.a) + _t(c.params["dt_bias"]), threshold=20).numpy()
    if decay_form == "decay_coef":
        g = np.asarray(c.params["decay_coef"], np.float64) * sp
    else:
        g = -np.exp(np.asarray(c.params["a_log"], np.float64)) * sp
    beta = torch.sigmoid(_t(c.b)).numpy()
    for hv in range(HV):
        hk = hv % HK if head_map == "tiled" else hv // (HV // HK)
        q = act[:, hk * DK:(hk + 1) * DK]
        k = act[:, HK * DK + hk * DK:HK * DK + (hk + 1) * DK]
        v = act[:, 2 * HK * DK + hv * DV:2 * HK * DK + (hv + 1) * DV]
        qn = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6) / np.sqrt(DK)
        kn = k / np.sqrt((k * k).sum(1, keepdims=True) + 1e-6)
        o_ref, S_ref = _brute_force_core(qn, kn, v, g[:, hv], beta[:, hv],
                                         np.asarray(c.S0[0, hv], np.float64))
        np.testing.assert_allclose(out["o_pre"][:, hv * DV:(hv + 1) * DV], o_ref,
                                   rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(out["S"][0, hv], S_ref, rtol=1e-11,
                                   atol=1e-13)
    np.testing.assert_array_equal(out["conv"][0], full[-(K - 1):])


def test_mixer_grouped_heads_equal_duplicated_key_heads():
    """Value head hv reads key head hv // (H_v / H_k): the grouped layer
    equals an ungrouped one whose q/k channels (weights and history) are
    each key head repeated for its contiguous group."""
    dg = Dims(2, 6, 4, 3, conv_k=4)
    c = _case(dg, [7, 4], seed=15, s0_std=0.2, conv0_std=1.0)
    out = _run(c)
    grp = 3
    du = Dims(6, 6, 4, 3, conv_k=4)
    HK, DK = dg.h_k, dg.d_k

    def expand(arr, axis):
        arr = np.asarray(arr, np.float64)
        q = np.take(arr, range(0, HK * DK), axis=axis)
        k = np.take(arr, range(HK * DK, 2 * HK * DK), axis=axis)
        v = np.take(arr, range(2 * HK * DK, arr.shape[axis]), axis=axis)

        def rep(part):
            sh = list(part.shape)
            sh[axis:axis + 1] = [HK, DK]
            part = np.repeat(part.reshape(sh), grp, axis=axis)
            sh2 = list(part.shape)
            sh2[axis:axis + 2] = [HK * grp * DK]
            return part.reshape(sh2)
        return np.concatenate([rep(q), rep(k), v], axis=axis)

    params = dict(c.params)
    params["conv_w"] = expand(c.params["conv_w"], 0)
    ref = oracle.mixer(_shape(du), c.cu_seqlens, params, expand(c.qkv, 1), c.z,
                       c.a, c.b, c.S0, expand(c.conv0, 2))
    np.testing.assert_array_equal(out["y"], ref["y"])
    np.testing.assert_array_equal(out["S"], ref["S"])


def test_mixer_split_resume_and_varlen_bit_exact():
    """Carrying (S, conv history) across a split, and packing sequences via
    cu_seqlens, give bit-identical results to one long call / separate
    calls."""
    d = Dims(2, 4, 8, 8, conv_k=4)
    c = _case(d, [23, 0, 2, 17], seed=16, s0_std=0.1, conv0_std=1.0)
    packed = _run(c)
    cu = c.cu_seqlens
    for n in range(4):
        s, e = cu[n], cu[n + 1]
        sub = oracle.mixer(_shape(d), [0, e - s], c.params, c.qkv[s:e],
                           c.z[s:e], c.a[s:e], c.b[s:e], c.S0[n:n + 1],
                           c.conv0[n:n + 1])
        np.testing.assert_array_equal(packed["y"][s:e], sub["y"])
        np.testing.assert_array_equal(packed["S"][n], sub["S"][0])
        np.testing.assert_array_equal(packed["conv"][n], sub["conv"][0])
    # split the first sequence at 9 and resume
    s, e, m = cu[0], cu[1], 9
    p1 = oracle.mixer(_shape(d), [0, m], c.params, c.qkv[s:m], c.z[s:m],
                      c.a[s:m], c.b[s:m], c.S0[:1], c.conv0[:1])
    p2 = oracle.mixer(_shape(d), [0, e - m], c.params, c.qkv[m:e], c.z[m:e],
                      c.a[m:e], c.b[m:e], p1["S"], p1["conv"])
    np.testing.assert_array_equal(np.concatenate([p1["y"], p2["y"]]),
                                  packed["y"][s:e])
    np.testing.assert_array_equal(p2["S"][0], packed["S"][0])
    np.testing.assert_array_equal(p2["conv"][0], packed["conv"][0])
    # an empty sequence passes its state and history through
    np.testing.assert_array_equal(packed["S"][1], c.S0[1].numpy())
    np.testing.assert_array_equal(packed["conv"][1], c.conv0[1].numpy())


def test_mixer_head_subset_and_threads_bit_exact():
    d = Dims(2, 4, 8, 8, conv_k=4)
    c = _case(d, [12, 5], seed=17, s0_std=0.1, conv0_std=1.0)
    full = _run(c, nthreads=1)
    thr = _run(c, nthreads=4)
    sub = _run(c, heads=(1, 3))
    np.testing.assert_array_equal(full["y"], thr["y"])
    np.testing.assert_array_equal(full["S"], thr["S"])
    sl = slice(1 * 8, 3 * 8)
    np.testing.assert_array_equal(sub["y"][:, sl], full["y"][:, sl])
    np.testing.assert_array_equal(sub["S"][:, 1:3], full["S"][:, 1:3])
    np.testing.assert_array_equal(sub["S"][:, 0], c.S0[:, 0].numpy())
    np.testing.assert_array_equal(sub["conv"], full["conv"])


def test_mixer_rejects_both_or_neither_decay_form():
    d = Dims(1, 1, 4, 4, conv_k=2)
    c = _case(d, [3], seed=18)
    both = dict(c.params, decay_coef=-torch.exp(c.params["a_log"]))
    with pytest.raises(ValueError):
        _run(c.__class__(**{**c.__dict__, "params": both}))
    neither = {k: v for k, v in c.params.items() if k != "a_log"}
    with pytest.raises(ValueError):
        _run(c.__class__(**{**c.__dict__, "params": neither}))


# --------------------------------------------------------------------------
# per-channel decay (Kimi Delta Attention; "cortiq-engine 0.8.76
# pipeline.rs", AttnKind::Kda)
# --------------------------------------------------------------------------

def _kda_shape(d, **kw):
    return oracle.Shape(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k, d.gate, decay="channel", **kw)


def test_kda_equal_channels_is_the_scalar_rule():
    """Per-channel gate inputs that are equal across the channels of a head
    give the scalar-decay rule bit for bit."""
    d = Dims(2, 4, 8, 6, conv_k=4)
    c = _case(d, [9, 3], seed=31, s0_std=0.3, conv0_std=1.0, decay="weak")
    ref = _run(c)
    a_ch = np.repeat(np.asarray(c.a, np.float64), d.d_k, axis=1)
    params = dict(c.params, dt_bias=np.repeat(np.asarray(c.params["dt_bias"], np.float64), d.d_k))
    out = oracle.mixer(_kda_shape(d), c.cu_seqlens, params, c.qkv, c.z, a_ch, c.b, c.S0, c.conv0)
    np.testing.assert_array_equal(out["y"], ref["y"])
    np.testing.assert_array_equal(out["S"], ref["S"])


def test_kda_beta_zero_decays_each_key_row():
    """b = -inf makes beta = 0, so S_L = diag(exp(sum_t g_t)) S_0 with
    g_t[i] = -exp(A_log) softplus(a_t[i] + dt_bias[i]) from torch."""
    d = Dims(1, 2, 4, 3, conv_k=2, decay="channel")
    L = 5
    c = _case(d, [L], seed=32, s0_std=1.0, conv0_std=1.0, decay="weak")
    c.b[:] = -float("inf")
    c.a[:] = torch.linspace(-3.0, 25.0, L * 8).reshape(L, 8)
    out = oracle.mixer(_kda_shape(d), c.cu_seqlens, c.params, c.qkv, c.z, c.a, c.b, c.S0,
                       c.conv0)
    sp = F.softplus(_t(c.a) + _t(c.params["dt_bias"]), threshold=20)   # [L, H_v*d_k]
    g = -torch.exp(_t(c.params["a_log"])).repeat_interleave(d.d_k) * sp
    decay = torch.exp(g.sum(0)).view(d.h_v, d.d_k).numpy()
    np.testing.assert_allclose(out["S"][0], decay[:, :, None] * c.S0[0].numpy(), rtol=1e-13)


def _brute_force_channel_core(q, k, v, g, beta, S0):
    """Transition-matrix form with a diagonal decay:
    S_t = (I - b_t k k^T) diag(exp(g_t)) S_{t-1} + b_t k v^T, o_t = S_t^T q_t."""
    S = S0.copy()
    dk = S.shape[0]
    out = []
    for t in range(len(beta)):
        kk = k[t][:, None]
        Tm = (np.eye(dk) - beta[t] * (kk @ kk.T)) @ np.diag(np.exp(g[t]))
        S = Tm @ S + beta[t] * (kk @ v[t][None, :])
        out.append(S.T @ q[t])
    return np.array(out), S


@pytest.mark.parametrize("head_map", ["grouped", "tiled"])
def test_kda_matches_independent_formulation(head_map):
    """Per-channel decay vs a second formulation: scipy FIR conv, torch
    nonlinearities, explicit L2 scaling and diagonal-decay transition
    matrices."""
    d = Dims(2, 4, 6, 5, conv_k=4, decay="channel", head_map=head_map)
    L = 9
    c = _case(d, [L], seed=33, s0_std=0.3, conv0_std=1.0, decay="weak")
    out = oracle.mixer(_kda_shape(d, head_map=head_map), c.cu_seqlens, c.params, c.qkv, c.z,
                       c.a, c.b, c.S0, c.conv0, want_pre=True)
    HK, HV, DK, DV, K = d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k
    x = np.asarray(c.qkv, np.float64)
    full = np.concatenate([np.asarray(c.conv0[0], np.float64), x])
    w = np.asarray(c.params["conv_w"], np.float64)
    h = np.stack([lfilter(w[ch, ::-1], [1.0], full[:, ch])[K - 1:]
                  for ch in range(d.conv_dim)], axis=1)
    act = F.silu(_t(h)).numpy()
    sp = F.softplus(_t(c.a) + _t(c.params["dt_bias"]), threshold=20).numpy()
    coef = -np.exp(np.asarray(c.params["a_log"], np.float64))
    beta = torch.sigmoid(_t(c.b)).numpy()
    for hv in range(HV):
        hk = hv % HK if head_map == "tiled" else hv // (HV // HK)
        q = act[:, hk * DK:(hk + 1) * DK]
        k = act[:, HK * DK + hk * DK:HK * DK + (hk + 1) * DK]
        v = act[:, 2 * HK * DK + hv * DV:2 * HK * DK + (hv + 1) * DV]
        qn = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6) / np.sqrt(DK)
        kn = k / np.sqrt((k * k).sum(1, keepdims=True) + 1e-6)
        g = coef[hv] * sp[:, hv * DK:(hv + 1) * DK]
        o_ref, S_ref = _brute_force_channel_core(qn, kn, v, g, beta[:, hv],
                                                 np.asarray(c.S0[0, hv], np.float64))
        np.testing.assert_allclose(out["o_pre"][:, hv * DV:(hv + 1) * DV], o_ref,
                                   rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(out["S"][0, hv], S_ref, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# the mixer with its projections ("oxinfer 0.0.5 src/qwen.rs", Gdn struct,
# gdn_forward)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("decay", ["head", "channel"])
def test_mixer_layer_with_selection_weights_is_the_core(decay):
    """With in_proj weights that select consecutive slices of x (identity
    blocks) the layer's core runs on those slices: a wrong weight for any of
    qkv, z, b or a fails.  out_proj is a rectangular, non-symmetric
    selection ([value_dim + 1][value_dim]: output column r is core column
    r + 1 cyclically, the extra column 2 y_0 - y_1), so the orientation of
    the output weight is fixed too: applying it transposed fails."""
    d = Dims(2, 4, 4, 3, conv_k=3, decay=decay)
    c = _case(d, [6, 4], seed=41, s0_std=0.3, conv0_std=1.0, decay="weak")
    widths = [d.conv_dim, d.value_dim, d.h_v, d.h_v * d.gate_width]
    H = sum(widths)
    x = np.concatenate([np.asarray(c.qkv, np.float64), np.asarray(c.z, np.float64),
                        np.asarray(c.b, np.float64), np.asarray(c.a, np.float64)], axis=1)
    eye = np.eye(H)
    off = np.cumsum([0] + widths)
    V = d.value_dim
    w_out = np.zeros((V + 1, V))
    for r in range(V):
        w_out[r, (r + 1) % V] = 1.0
    w_out[V, 0], w_out[V, 1] = 2.0, -1.0
    proj = {"hidden": H, "w_qkv": eye[off[0]:off[1]], "w_z": eye[off[1]:off[2]],
            "w_b": eye[off[2]:off[3]], "w_a": eye[off[3]:off[4]], "w_out": w_out}
    shape = oracle.Shape(d.h_k, d.h_v, d.d_k, d.d_v, d.conv_k, d.gate, decay=decay)
    layer = oracle.mixer_layer(shape, c.cu_seqlens, c.params, proj, x, c.S0, c.conv0)
    core = oracle.mixer(shape, c.cu_seqlens, c.params, c.qkv, c.z, c.a, c.b, c.S0, c.conv0)
    np.testing.assert_array_equal(layer["y"], core["y"])
    y = core["y"]
    assert layer["out"].shape == (y.shape[0], V + 1)
    np.testing.assert_array_equal(layer["out"][:, :V], np.roll(y, -1, axis=1))
    np.testing.assert_array_equal(layer["out"][:, V], 2.0 * y[:, 0] - y[:, 1])
    np.testing.assert_array_equal(layer["S"], core["S"])
