// C ABI of the GDN library: host-side validation and dispatch.  Nothing is
// enqueued until every argument has been checked, so a call that fails
// writes nothing (the pages' engines likewise refuse a bad tensor shape
// before using it: "oxinfer 0.0.5 src/qwen.rs" Loader::getf).

#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace {

thread_local char g_err[512];

gdn_status fail(gdn_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

gdn_status ok()
{
    g_err[0] = '\0';
    return GDN_OK;
}

bool dim_supported(int d) { return d == 32 || d == 64 || d == 128; }

// Checks the configuration and fills the internal dims.
gdn_status check_config(const gdn_config *cfg, gdn::Dims &d)
{
    if (!cfg) return fail(GDN_EINVAL, "cfg is NULL");
    if (cfg->h_k <= 0 || cfg->h_v <= 0 || cfg->d_k <= 0 || cfg->d_v <= 0)
        return fail(GDN_EINVAL, "head counts and head dims must be positive (h_k=%d h_v=%d d_k=%d d_v=%d)",
                    cfg->h_k, cfg->h_v, cfg->d_k, cfg->d_v);
    if (cfg->h_v % cfg->h_k != 0)
        return fail(GDN_EINVAL, "h_v (%d) must be a multiple of h_k (%d)", cfg->h_v, cfg->h_k);
    if (cfg->conv_k < 1)
        return fail(GDN_EINVAL, "conv_k must be >= 1 (got %d)", cfg->conv_k);
    if (cfg->act_dtype != GDN_BF16 && cfg->act_dtype != GDN_F32)
        return fail(GDN_EINVAL, "act_dtype %d is not a gdn_dtype", cfg->act_dtype);
    if (cfg->out_dtype != GDN_BF16 && cfg->out_dtype != GDN_F32)
        return fail(GDN_EINVAL, "out_dtype %d is not a gdn_dtype", cfg->out_dtype);
    if (cfg->gate != GDN_GATE_SILU && cfg->gate != GDN_GATE_SIGMOID)
        return fail(GDN_EINVAL, "gate %d is not a gdn_gate", cfg->gate);
    if (cfg->head_map != GDN_HEADS_GROUPED && cfg->head_map != GDN_HEADS_TILED)
        return fail(GDN_EINVAL, "head_map %d is not a gdn_head_map", cfg->head_map);
    if (cfg->decay_mode != GDN_DECAY_HEAD && cfg->decay_mode != GDN_DECAY_CHANNEL)
        return fail(GDN_EINVAL, "decay_mode %d is not a gdn_decay_mode", cfg->decay_mode);
    if (cfg->state_cache != GDN_STATE_CACHED && cfg->state_cache != GDN_STATE_STREAMED)
        return fail(GDN_EINVAL, "state_cache %d is not a gdn_state_cache", cfg->state_cache);
    if (!(cfg->norm_eps >= 0.0f) || !std::isfinite(cfg->norm_eps) || !(cfg->l2_eps >= 0.0f) ||
        !std::isfinite(cfg->l2_eps))
        return fail(GDN_EINVAL, "norm_eps and l2_eps must be finite and >= 0");
    if (!dim_supported(cfg->d_k) || !dim_supported(cfg->d_v))
        return fail(GDN_EUNSUPPORTED, "d_k and d_v must be 32, 64 or 128 (got %d, %d)", cfg->d_k,
                    cfg->d_v);
    if (cfg->conv_k > 4)
        return fail(GDN_EUNSUPPORTED, "conv_k must be <= 4 (got %d)", cfg->conv_k);
    const long long cd = 2LL * cfg->h_k * cfg->d_k + (long long)cfg->h_v * cfg->d_v;
    if (cd > (1LL << 30) || cfg->h_k > 65535)
        return fail(GDN_EUNSUPPORTED, "layer too wide (conv_dim %lld)", cd);
    d.h_k = cfg->h_k;
    d.h_v = cfg->h_v;
    d.d_k = cfg->d_k;
    d.d_v = cfg->d_v;
    d.conv_k = cfg->conv_k;
    d.group = cfg->h_v / cfg->h_k;
    d.conv_dim = (int)cd;
    d.value_dim = cfg->h_v * cfg->d_v;
    d.act_bf16 = cfg->act_dtype == GDN_BF16;
    d.out_bf16 = cfg->out_dtype == GDN_BF16;
    d.out_split = 0;
    d.preconv = 0;
    d.in_split = 1;
    d.in_ld = 0;
    d.in_split_stride = 0;
    d.gate = cfg->gate;
    d.tiled = cfg->head_map == GDN_HEADS_TILED;
    d.chan_decay = cfg->decay_mode == GDN_DECAY_CHANNEL;
    d.nt_state = cfg->state_cache == GDN_STATE_STREAMED;
    d.norm_eps = cfg->norm_eps;
    d.l2_eps = cfg->l2_eps;
    return GDN_OK;
}

gdn_status check_params(const gdn_params *p, gdn::Params &out)
{
    if (!p) return fail(GDN_EINVAL, "params is NULL");
    if (!p->conv_w || !p->dt_bias || !p->norm_w)
        return fail(GDN_EINVAL, "conv_w, dt_bias and norm_w must be non-NULL");
    if ((p->a_log == nullptr) == (p->decay_coef == nullptr))
        return fail(GDN_EINVAL, "exactly one of a_log and decay_coef must be given");
    if ((reinterpret_cast<uintptr_t>(p->conv_w) | reinterpret_cast<uintptr_t>(p->norm_w)) & 15)
        return fail(GDN_EINVAL, "conv_w and norm_w must be 16-byte aligned");
    out.conv_w = p->conv_w;
    out.a_log = p->a_log;
    out.decay_coef = p->decay_coef;
    out.dt_bias = p->dt_bias;
    out.norm_w = p->norm_w;
    return GDN_OK;
}

// cu_seqlens: [n+1], starts at 0, non-decreasing, ends at t_total.
gdn_status check_cu(int n_seq, int t_total, const int32_t *cu_host, const int32_t *cu_dev,
                    int &max_len)
{
    if (n_seq < 0 || t_total < 0)
        return fail(GDN_EINVAL, "n_seq (%d) and t_total (%d) must be >= 0", n_seq, t_total);
    if (n_seq > 65535) return fail(GDN_EUNSUPPORTED, "n_seq must be <= 65535 (got %d)", n_seq);
    if (!cu_host || !cu_dev) return fail(GDN_EINVAL, "cu_seqlens_host and cu_seqlens_dev are required");
    if (cu_host[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0] must be 0 (got %d)", cu_host[0]);
    max_len = 0;
    for (int i = 0; i < n_seq; ++i) {
        if (cu_host[i + 1] < cu_host[i])
            return fail(GDN_EINVAL, "cu_seqlens must be non-decreasing (cu[%d]=%d > cu[%d]=%d)", i,
                        cu_host[i], i + 1, cu_host[i + 1]);
        const int L = cu_host[i + 1] - cu_host[i];
        if (L > max_len) max_len = L;
    }
    if (cu_host[n_seq] != t_total)
        return fail(GDN_EINVAL, "cu_seqlens[n_seq] (%d) must equal t_total (%d)", cu_host[n_seq],
                    t_total);
    return GDN_OK;
}

struct Range {
    const void *p;
    size_t bytes;
};

bool overlap(Range a, Range b)
{
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const auto x0 = reinterpret_cast<uintptr_t>(a.p), y0 = reinterpret_cast<uintptr_t>(b.p);
    return x0 < y0 + b.bytes && y0 < x0 + a.bytes;
}

gdn_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(GDN_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

} // namespace

extern "C" {

gdn_status gdn_conv_update(const gdn_config *cfg, const gdn_params *params, int32_t n_seq,
                           int32_t t_total, const int32_t *cu_seqlens_host,
                           const int32_t *cu_seqlens_dev, const void *x, float *conv_state,
                           float *y, void *stream)
{
    gdn::Dims d;
    gdn::Params p;
    gdn_status st;
    if ((st = check_config(cfg, d)) != GDN_OK) return st;
    if ((st = check_params(params, p)) != GDN_OK) return st;
    int max_len = 0;
    if ((st = check_cu(n_seq, t_total, cu_seqlens_host, cu_seqlens_dev, max_len)) != GDN_OK) return st;
    if ((long long)t_total * d.h_v > (1LL << 30)) // (token, value head) rows are counted in int
        return fail(GDN_EUNSUPPORTED, "t_total * H_v must be <= 2^30 (got %lld)", (long long)t_total * d.h_v);
    if (t_total > 0 && (!x || !y)) return fail(GDN_EINVAL, "x and y are required when t_total > 0");
    if (n_seq > 0 && d.conv_k > 1 && !conv_state) return fail(GDN_EINVAL, "conv_state is required");
    const size_t esz = d.act_bf16 ? 2 : 4;
    const Range rx{x, (size_t)t_total * d.conv_dim * esz};
    const Range ry{y, (size_t)t_total * d.conv_dim * 4};
    const Range rc{conv_state, (size_t)n_seq * (d.conv_k - 1) * d.conv_dim * 4};
    if (overlap(ry, rx) || overlap(ry, rc) || overlap(rx, rc))
        return fail(GDN_EINVAL, "y, x and conv_state must not overlap");
    if (max_len > 65535 * 64) return fail(GDN_EUNSUPPORTED, "sequence longer than %d", 65535 * 64);
    return hip_status(gdn::launch_conv_update(d, p, n_seq, max_len, cu_seqlens_dev, x, conv_state,
                                              y, static_cast<hipStream_t>(stream)),
                      "gdn_conv_update launch");
}

gdn_status gdn_decode_step(const gdn_config *cfg, const gdn_params *params, int32_t batch,
                           const void *qkv, const void *z, const void *a, const void *b,
                           float *conv_state, float *state, void *out, void *stream)
{
    gdn::Dims d;
    gdn::Params p;
    gdn_status st;
    if ((st = check_config(cfg, d)) != GDN_OK) return st;
    if ((st = check_params(params, p)) != GDN_OK) return st;
    if (batch < 0) return fail(GDN_EINVAL, "batch must be >= 0 (got %d)", batch);
    if (batch > 65535) return fail(GDN_EUNSUPPORTED, "batch must be <= 65535 (got %d)", batch);
    if ((long long)batch * d.h_k > (1LL << 30)) // one workgroup per (sequence, key head)
        return fail(GDN_EUNSUPPORTED, "batch * H_k must be <= 2^30 (got %lld)", (long long)batch * d.h_k);
    if (batch == 0) return ok();
    if (!qkv || !z || !a || !b || !state || !out || (d.conv_k > 1 && !conv_state))
        return fail(GDN_EINVAL, "qkv, z, a, b, state, out (and conv_state when K > 1) are required");
    const size_t esz = d.act_bf16 ? 2 : 4, osz = d.out_bf16 ? 2 : 4;
    const Range rs{state, (size_t)batch * d.h_v * d.d_k * d.d_v * 4};
    const Range rc{conv_state, (size_t)batch * (d.conv_k - 1) * d.conv_dim * 4};
    const Range ro{out, (size_t)batch * d.value_dim * osz};
    const Range ins[] = {{qkv, (size_t)batch * d.conv_dim * esz},
                         {z, (size_t)batch * d.value_dim * esz},
                         {a, (size_t)batch * d.h_v * (d.chan_decay ? d.d_k : 1) * esz},
                         {b, (size_t)batch * d.h_v * esz}};
    for (const Range &r : ins)
        if (overlap(ro, r) || overlap(rs, r) || overlap(rc, r))
            return fail(GDN_EINVAL, "outputs and states must not overlap the inputs");
    if (overlap(ro, rs) || overlap(ro, rc) || overlap(rs, rc))
        return fail(GDN_EINVAL, "out, state and conv_state must not overlap each other");
    // One token is the multi-token kernel with t_new = 1 whenever its
    // per-key-head buffer fits; very wide groups use the persistent
    // single-token kernel, which needs no per-token buffer (and has no
    // per-channel decay).
    const bool fits = gdn::decode_multi_lds_bytes(d, 1) <= gdn::kDecodeMultiMaxLds;
    if (!fits && d.chan_decay)
        return fail(GDN_EUNSUPPORTED,
                    "per-channel decay needs %d conv channels per key head to fit the on-chip "
                    "buffer", 2 * d.d_k + d.group * d.d_v);
    if (fits)
        return hip_status(gdn::launch_decode_multi(d, p, batch, 1, nullptr, qkv, z, a, b,
                                                   conv_state, conv_state, state, state, nullptr,
                                                   out, static_cast<hipStream_t>(stream)),
                          "gdn_decode_step launch");
    return hip_status(gdn::launch_decode(d, p, batch, qkv, z, a, b, conv_state, state, out,
                                         static_cast<hipStream_t>(stream)),
                      "gdn_decode_step launch");
}

} // extern "C"

namespace {

// Shared checks of the multi-token entry points; fills the ranges used for
// the overlap tests.
gdn_status check_multi(const gdn::Dims &d, int32_t batch, int32_t t_new, const void *qkv,
                       const void *a, const void *b, const float *conv_in,
                       const float *conv_out, const float *state_in, const float *state_out)
{
    if (batch < 0) return fail(GDN_EINVAL, "batch must be >= 0 (got %d)", batch);
    if (batch > 65535) return fail(GDN_EUNSUPPORTED, "batch must be <= 65535 (got %d)", batch);
    if ((long long)batch * d.h_k > (1LL << 30)) // one workgroup per (sequence, key head)
        return fail(GDN_EUNSUPPORTED, "batch * H_k must be <= 2^30 (got %lld)", (long long)batch * d.h_k);
    if (t_new < 1 || t_new > gdn::kDecodeMultiMaxTokens)
        return fail(GDN_EUNSUPPORTED, "tokens per sequence must be in [1, %d] (got %d)",
                    gdn::kDecodeMultiMaxTokens, t_new);
    if (gdn::decode_multi_lds_bytes(d, t_new) > gdn::kDecodeMultiMaxLds)
        return fail(GDN_EUNSUPPORTED,
                    "%d tokens of %d conv channels per key head exceed the on-chip buffer",
                    t_new, 2 * d.d_k + d.group * d.d_v);
    if (batch == 0) return GDN_OK;
    if (!qkv || !a || !b || !state_in || !state_out ||
        (d.conv_k > 1 && (!conv_in || !conv_out)))
        return fail(GDN_EINVAL,
                    "qkv, a, b, the states (and the conv histories when K > 1) are required");
    return GDN_OK;
}

gdn_status launch_multi_checked(const gdn::Dims &d, const gdn::Params &p, int32_t batch,
                                int32_t t_new, const int32_t *n_tok, const void *qkv,
                                const void *z, const void *a, const void *b,
                                const float *conv_in, float *conv_out, const float *state_in,
                                float *state_out, float *ckpt, void *out, void *stream,
                                const char *what)
{
    const size_t esz = d.act_bf16 ? 2 : 4, osz = d.out_bf16 ? 2 : 4;
    const size_t tok = (size_t)batch * t_new;
    const size_t sbytes = (size_t)batch * d.h_v * d.d_k * d.d_v * 4;
    const size_t cbytes = (size_t)batch * (d.conv_k - 1) * d.conv_dim * 4;
    const Range ins[] = {{qkv, tok * d.conv_dim * esz},
                         {z, tok * d.value_dim * esz},
                         {a, tok * d.h_v * (d.chan_decay ? d.d_k : 1) * esz},
                         {b, tok * d.h_v * esz},
                         {n_tok, (size_t)batch * 4}};
    const Range rsi{state_in, sbytes}, rso{state_out, sbytes};
    const Range rci{conv_in, cbytes}, rco{conv_out, cbytes};
    const Range rck{ckpt, tok * d.h_v * d.d_k * d.d_v * 4};
    const Range ro{out, tok * d.value_dim * osz};
    const Range outs[] = {rso, rco, rck, ro};
    for (const Range &o : outs)
        for (const Range &r : ins)
            if (overlap(o, r)) return fail(GDN_EINVAL, "outputs and states must not overlap the inputs");
    if (overlap(rso, rco) || overlap(rso, rck) || overlap(rso, ro) || overlap(rco, rck) ||
        overlap(rco, ro) || overlap(rck, ro) || overlap(rck, rsi) || overlap(rck, rci) ||
        overlap(ro, rsi) || overlap(ro, rci) || overlap(rso, rci) || overlap(rco, rsi))
        return fail(GDN_EINVAL, "out, checkpoints, state_out and conv_out must be disjoint buffers");
    if (overlap(rsi, rso) && state_in != state_out)
        return fail(GDN_EINVAL, "state_out may equal state_in but must not partially overlap it");
    if (overlap(rci, rco) && conv_in != conv_out)
        return fail(GDN_EINVAL, "conv_out may equal conv_in but must not partially overlap it");
    return hip_status(gdn::launch_decode_multi(d, p, batch, t_new, n_tok, qkv, z, a, b, conv_in,
                                               conv_out, state_in, state_out, ckpt, out,
                                               static_cast<hipStream_t>(stream)),
                      what);
}

} // namespace

extern "C" {

gdn_status gdn_decode_multi(const gdn_config *cfg, const gdn_params *params, int32_t batch,
                            int32_t t_new, const int32_t *n_tok_dev, const void *qkv,
                            const void *z, const void *a, const void *b, const float *conv_in,
                            float *conv_out, const float *state_in, float *state_out,
                            float *state_ckpt, void *out, void *stream)
{
    gdn::Dims d;
    gdn::Params p;
    gdn_status st;
    if ((st = check_config(cfg, d)) != GDN_OK) return st;
    if ((st = check_params(params, p)) != GDN_OK) return st;
    if ((st = check_multi(d, batch, t_new, qkv, a, b, conv_in, conv_out, state_in, state_out)) !=
        GDN_OK)
        return st;
    if (batch == 0) return ok();
    if (out && !z) return fail(GDN_EINVAL, "z is required when out is given");
    return launch_multi_checked(d, p, batch, t_new, n_tok_dev, qkv, out ? z : nullptr, a, b,
                                conv_in, conv_out, state_in, state_out, state_ckpt, out, stream,
                                "gdn_decode_multi launch");
}

gdn_status gdn_rewind(const gdn_config *cfg, const gdn_params *params, int32_t batch,
                      int32_t t_rec, const int32_t *keep_dev, const void *qkv_rec,
                      const void *a_rec, const void *b_rec, const float *state0,
                      const float *conv0, float *state, float *conv_state, void *stream)
{
    gdn::Dims d;
    gdn::Params p;
    gdn_status st;
    if ((st = check_config(cfg, d)) != GDN_OK) return st;
    if ((st = check_params(params, p)) != GDN_OK) return st;
    if ((st = check_multi(d, batch, t_rec, qkv_rec, a_rec, b_rec, conv0, conv_state, state0,
                          state)) != GDN_OK)
        return st;
    if (batch == 0) return ok();
    return launch_multi_checked(d, p, batch, t_rec, keep_dev, qkv_rec, nullptr, a_rec, b_rec,
                                conv0, conv_state, state0, state, nullptr, nullptr, stream,
                                "gdn_rewind launch");
}

} // extern "C"

extern "C" {

size_t gdn_prefill_workspace_bytes(const gdn_config *cfg, int32_t n_seq, int32_t t_total,
                                   int32_t chunk)
{
    gdn::Dims d;
    if (check_config(cfg, d) != GDN_OK || n_seq < 0 || t_total < 0 || chunk != 64) return 0;
    return gdn::prefill_workspace_bytes(d, n_seq, t_total);
}

} // extern "C"

namespace {

// The chunked prefill with its workspace either given by the caller
// (static_ws false) or taken from the library's static scratch.
gdn_status prefill_common(const gdn_config *cfg, const gdn_params *params, int32_t chunk,
                          int32_t n_seq, int32_t t_total, const int32_t *cu_seqlens_host,
                          const int32_t *cu_seqlens_dev, const void *qkv, const void *z,
                          const void *a, const void *b, const float *state_in, float *state_out,
                          const float *conv_in, float *conv_out, void *out, void *workspace,
                          size_t ws_bytes, bool static_ws, void *stream)
{
    gdn::Dims d;
    gdn::Params p;
    gdn_status st;
    if ((st = check_config(cfg, d)) != GDN_OK) return st;
    if ((st = check_params(params, p)) != GDN_OK) return st;
    if (chunk != 64) return fail(GDN_EUNSUPPORTED, "chunk must be 64 (got %d)", chunk);
    int max_len = 0;
    if ((st = check_cu(n_seq, t_total, cu_seqlens_host, cu_seqlens_dev, max_len)) != GDN_OK) return st;
    if ((long long)t_total * d.h_v > (1LL << 30)) // (token, value head) rows are counted in int
        return fail(GDN_EUNSUPPORTED, "t_total * H_v must be <= 2^30 (got %lld)", (long long)t_total * d.h_v);
    if (max_len > 65535 * 64) return fail(GDN_EUNSUPPORTED, "sequence longer than %d", 65535 * 64);
    if (t_total > 0 && (!qkv || !z || !a || !b || !out))
        return fail(GDN_EINVAL, "qkv, z, a, b and out are required when t_total > 0");
    if (t_total > 0 && ((reinterpret_cast<uintptr_t>(qkv) | reinterpret_cast<uintptr_t>(z) |
                         reinterpret_cast<uintptr_t>(out)) & 15))
        return fail(GDN_EINVAL, "qkv, z and out must be 16-byte aligned");
    if (t_total > 0 && d.chan_decay && (reinterpret_cast<uintptr_t>(a) & 15))
        return fail(GDN_EINVAL, "a must be 16-byte aligned with per-channel decay");
    if (n_seq > 0 && (!state_out || (d.conv_k > 1 && !conv_out)))
        return fail(GDN_EINVAL, "state_out (and conv_out when K > 1) are required");
    const size_t need = gdn::prefill_workspace_bytes(d, n_seq, t_total);
    if (static_ws) {
        if (need > gdn::kStaticScratchBytes)
            return fail(GDN_EUNSUPPORTED,
                        "this call needs %zu bytes of scratch; the allocation-free prefill holds "
                        "%zu (use gdn_prefill_chunked with a workspace)",
                        need, gdn::kStaticScratchBytes);
    } else {
        if (need > 0 && (!workspace || ws_bytes < need))
            return fail(GDN_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                        workspace ? ws_bytes : (size_t)0);
        if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255))
            return fail(GDN_EINVAL, "workspace must be 256-byte aligned");
    }
    const size_t esz = d.act_bf16 ? 2 : 4, osz = d.out_bf16 ? 2 : 4;
    const size_t sbytes = (size_t)n_seq * d.h_v * d.d_k * d.d_v * 4;
    const size_t cbytes = (size_t)n_seq * (d.conv_k - 1) * d.conv_dim * 4;
    const Range ins[] = {{qkv, (size_t)t_total * d.conv_dim * esz},
                         {z, (size_t)t_total * d.value_dim * esz},
                         {a, (size_t)t_total * d.h_v * (d.chan_decay ? d.d_k : 1) * esz},
                         {b, (size_t)t_total * d.h_v * esz}};
    const Range ro{out, (size_t)t_total * d.value_dim * osz};
    const Range rsi{state_in, sbytes}, rso{state_out, sbytes};
    const Range rci{conv_in, cbytes}, rco{conv_out, cbytes};
    const Range rws{static_ws ? nullptr : workspace, need};
    const Range outs[] = {ro, rso, rco, rws};
    for (const Range &o : outs)
        for (const Range &r : ins)
            if (overlap(o, r)) return fail(GDN_EINVAL, "outputs and workspace must not overlap the inputs");
    if (overlap(ro, rso) || overlap(ro, rco) || overlap(ro, rws) || overlap(rso, rco) ||
        overlap(rso, rws) || overlap(rco, rws) || overlap(ro, rsi) || overlap(ro, rci) ||
        overlap(rws, rsi) || overlap(rws, rci) || overlap(rso, rci) || overlap(rco, rsi))
        return fail(GDN_EINVAL, "out, state_out, conv_out and workspace must be disjoint buffers");
    if (overlap(rsi, rso) && state_in != state_out)
        return fail(GDN_EINVAL, "state_out may equal state_in but must not partially overlap it");
    if (overlap(rci, rco) && conv_in != conv_out)
        return fail(GDN_EINVAL, "conv_out may equal conv_in but must not partially overlap it");
    if (static_ws) {
        hipError_t e = gdn::static_scratch(&workspace);
        if (e != hipSuccess) return hip_status(e, "static scratch address");
    }
    return hip_status(gdn::launch_prefill(d, p, n_seq, t_total, max_len, cu_seqlens_host,
                                          cu_seqlens_dev, qkv, z, a,
                                          b, state_in, state_out, conv_in, conv_out, out, workspace,
                                          static_cast<hipStream_t>(stream)),
                      static_ws ? "gdn_prefill_chunked_noalloc launch" : "gdn_prefill_chunked launch");
}

} // namespace

extern "C" {

gdn_status gdn_prefill_chunked(const gdn_config *cfg, const gdn_params *params, int32_t chunk,
                               int32_t n_seq, int32_t t_total, const int32_t *cu_seqlens_host,
                               const int32_t *cu_seqlens_dev, const void *qkv, const void *z,
                               const void *a, const void *b, const float *state_in,
                               float *state_out, const float *conv_in, float *conv_out, void *out,
                               void *workspace, size_t ws_bytes, void *stream)
{
    return prefill_common(cfg, params, chunk, n_seq, t_total, cu_seqlens_host, cu_seqlens_dev, qkv,
                          z, a, b, state_in, state_out, conv_in, conv_out, out, workspace, ws_bytes,
                          false, stream);
}

static_assert(GDN_PREFILL_NOALLOC_MAX_BYTES == gdn::kStaticScratchBytes,
              "the header states the static scratch size");

gdn_status gdn_prefill_chunked_noalloc(const gdn_config *cfg, const gdn_params *params,
                                       int32_t chunk, int32_t n_seq, int32_t t_total,
                                       const int32_t *cu_seqlens_host,
                                       const int32_t *cu_seqlens_dev, const void *qkv,
                                       const void *z, const void *a, const void *b,
                                       const float *state_in, float *state_out,
                                       const float *conv_in, float *conv_out, void *out,
                                       void *stream)
{
    return prefill_common(cfg, params, chunk, n_seq, t_total, cu_seqlens_host, cu_seqlens_dev, qkv,
                          z, a, b, state_in, state_out, conv_in, conv_out, out, nullptr, 0, true,
                          stream);
}

} // extern "C"

namespace {

gdn_status check_proj(const gdn::Dims &d, const gdn_config *cfg, const gdn_proj *proj,
                      gdn::Proj &out)
{
    if (!proj) return fail(GDN_EINVAL, "proj is NULL");
    if (proj->hidden <= 0 || proj->hidden % 8 != 0 || proj->hidden > (1 << 20))
        return fail(GDN_EINVAL, "hidden must be a positive multiple of 8 (got %d)", proj->hidden);
    if (!proj->w_qkv || !proj->w_z || !proj->w_b || !proj->w_a || !proj->w_out)
        return fail(GDN_EINVAL, "every projection weight must be non-NULL");
    if (cfg->act_dtype != GDN_BF16)
        return fail(GDN_EUNSUPPORTED, "the mixer takes bf16 hidden states (act_dtype GDN_BF16)");
    (void)d;
    out.hidden = proj->hidden;
    out.w_qkv = proj->w_qkv;
    out.w_z = proj->w_z;
    out.w_b = proj->w_b;
    out.w_a = proj->w_a;
    out.w_out = proj->w_out;
    return GDN_OK;
}

gdn_status check_workspace(void *workspace, size_t ws_bytes, size_t need)
{
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(GDN_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                    workspace ? ws_bytes : (size_t)0);
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255))
        return fail(GDN_EINVAL, "workspace must be 256-byte aligned");
    return GDN_OK;
}

} // namespace

extern "C" {

size_t gdn_mixer_workspace_bytes(const gdn_config *cfg, int32_t hidden, int32_t n_seq,
                                 int32_t t_total)
{
    gdn::Dims d;
    if (check_config(cfg, d) != GDN_OK || hidden <= 0 || hidden % 8 != 0 || n_seq < 0 ||
        t_total < 0)
        return 0;
    return gdn::mixer_workspace_bytes(d, hidden, n_seq, t_total, true);
}

gdn_status gdn_mixer_prefill(const gdn_config *cfg, const gdn_params *params,
                             const gdn_proj *proj, int32_t n_seq, int32_t t_total,
                             const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                             const void *x, const float *state_in, float *state_out,
                             const float *conv_in, float *conv_out, void *y, void *workspace,
                             size_t ws_bytes, void *stream)
{
    gdn::Dims d;
    gdn::Params p;
    gdn::Proj pj;
    gdn_status st;
    if ((st = check_config(cfg, d)) != GDN_OK) return st;
    if ((st = check_params(params, p)) != GDN_OK) return st;
    if ((st = check_proj(d, cfg, proj, pj)) != GDN_OK) return st;
    int max_len = 0;
    if ((st = check_cu(n_seq, t_total, cu_seqlens_host, cu_seqlens_dev, max_len)) != GDN_OK) return st;
    if ((long long)t_total * d.h_v > (1LL << 30)) // (token, value head) rows are counted in int
        return fail(GDN_EUNSUPPORTED, "t_total * H_v must be <= 2^30 (got %lld)", (long long)t_total * d.h_v);
    if (max_len > 65535 * 64) return fail(GDN_EUNSUPPORTED, "sequence longer than %d", 65535 * 64);
    if (t_total > 0 && (!x || !y)) return fail(GDN_EINVAL, "x and y are required when t_total > 0");
    if (n_seq > 0 && (!state_out || (d.conv_k > 1 && !conv_out)))
        return fail(GDN_EINVAL, "state_out (and conv_out when K > 1) are required");
    const size_t need = gdn::mixer_workspace_bytes(d, pj.hidden, n_seq, t_total, true);
    if ((st = check_workspace(workspace, ws_bytes, need)) != GDN_OK) return st;
    const size_t osz = d.out_bf16 ? 2 : 4;
    const size_t sbytes = (size_t)n_seq * d.h_v * d.d_k * d.d_v * 4;
    const size_t cbytes = (size_t)n_seq * (d.conv_k - 1) * d.conv_dim * 4;
    const Range rx{x, (size_t)t_total * pj.hidden * 2}, ry{y, (size_t)t_total * pj.hidden * osz};
    const Range rsi{state_in, sbytes}, rso{state_out, sbytes}, rci{conv_in, cbytes},
        rco{conv_out, cbytes}, rws{workspace, need};
    const Range outs[] = {ry, rso, rco, rws};
    for (const Range &o : outs)
        if (overlap(o, rx)) return fail(GDN_EINVAL, "outputs and workspace must not overlap x");
    if (overlap(ry, rso) || overlap(ry, rco) || overlap(ry, rws) || overlap(rso, rco) ||
        overlap(rso, rws) || overlap(rco, rws) || overlap(ry, rsi) || overlap(ry, rci) ||
        overlap(rws, rsi) || overlap(rws, rci) || overlap(rso, rci) || overlap(rco, rsi))
        return fail(GDN_EINVAL, "y, state_out, conv_out and workspace must be disjoint buffers");
    if (overlap(rsi, rso) && state_in != state_out)
        return fail(GDN_EINVAL, "state_out may equal state_in but must not partially overlap it");
    if (overlap(rci, rco) && conv_in != conv_out)
        return fail(GDN_EINVAL, "conv_out may equal conv_in but must not partially overlap it");
    return hip_status(gdn::launch_mixer_prefill(d, p, pj, n_seq, t_total, max_len, cu_seqlens_host,
                                                cu_seqlens_dev,
                                                x, state_in, state_out, conv_in, conv_out, y,
                                                workspace, static_cast<hipStream_t>(stream)),
                      "gdn_mixer_prefill launch");
}

gdn_status gdn_mixer_decode(const gdn_config *cfg, const gdn_params *params,
                            const gdn_proj *proj, int32_t batch, const void *x,
                            float *conv_state, float *state, void *y, void *workspace,
                            size_t ws_bytes, void *stream)
{
    gdn::Dims d;
    gdn::Params p;
    gdn::Proj pj;
    gdn_status st;
    if ((st = check_config(cfg, d)) != GDN_OK) return st;
    if ((st = check_params(params, p)) != GDN_OK) return st;
    if ((st = check_proj(d, cfg, proj, pj)) != GDN_OK) return st;
    if (batch < 0) return fail(GDN_EINVAL, "batch must be >= 0 (got %d)", batch);
    if (batch > 65535) return fail(GDN_EUNSUPPORTED, "batch must be <= 65535 (got %d)", batch);
    if ((long long)batch * d.h_k > (1LL << 30)) // one workgroup per (sequence, key head)
        return fail(GDN_EUNSUPPORTED, "batch * H_k must be <= 2^30 (got %lld)", (long long)batch * d.h_k);
    if (batch == 0) return ok();
    if (!x || !y || !state || (d.conv_k > 1 && !conv_state))
        return fail(GDN_EINVAL, "x, y, state (and conv_state when K > 1) are required");
    if (d.chan_decay && gdn::decode_multi_lds_bytes(d, 1) > gdn::kDecodeMultiMaxLds)
        return fail(GDN_EUNSUPPORTED,
                    "per-channel decay needs %d conv channels per key head to fit the on-chip "
                    "buffer", 2 * d.d_k + d.group * d.d_v);
    const size_t need = gdn::mixer_workspace_bytes(d, pj.hidden, batch, batch, false);
    if ((st = check_workspace(workspace, ws_bytes, need)) != GDN_OK) return st;
    const size_t osz = d.out_bf16 ? 2 : 4;
    const Range rx{x, (size_t)batch * pj.hidden * 2}, ry{y, (size_t)batch * pj.hidden * osz};
    const Range rs{state, (size_t)batch * d.h_v * d.d_k * d.d_v * 4};
    const Range rc{conv_state, (size_t)batch * (d.conv_k - 1) * d.conv_dim * 4};
    const Range rws{workspace, need};
    const Range all[] = {rx, ry, rs, rc, rws};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlap(all[i], all[j]))
                return fail(GDN_EINVAL, "x, y, state, conv_state and workspace must not overlap");
    return hip_status(gdn::launch_mixer_decode(d, p, pj, batch, x, conv_state, state, y, workspace,
                                               static_cast<hipStream_t>(stream)),
                      "gdn_mixer_decode launch");
}

const char *gdn_status_string(gdn_status s)
{
    switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_EINVAL: return "GDN_EINVAL";
    case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED";
    case GDN_EWORKSPACE: return "GDN_EWORKSPACE";
    case GDN_EHIP: return "GDN_EHIP";
    }
    return "GDN_UNKNOWN";
}

const char *gdn_last_error(void) { return g_err; }

} // extern "C"
