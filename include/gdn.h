/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet mixer-core library.
 *
 * The operation is the mixer core of Gated DeltaNet hybrid language models
 * ("cherenkov qwen4_exp/cpu.rs", fn deltanet and fn causal_conv; "oxinfer
 * 0.0.5 src/qwen.rs", DeltaRule::run and gdn_forward):
 *
 *   c_t   = silu(causal depthwise conv_K(qkv)_t)       history: last K-1 raw
 *                                                       inputs, oldest first
 *   q^,k^ = per key head L2 norm x (sum x^2 + l2_eps)^-1/2, q^ also * d_k^-1/2
 *   beta  = sigmoid(b),  g = -exp(A_log) softplus(a + dt_bias),  alpha = e^g
 *   S     <- alpha S;  delta = beta (v - S^T k^);  S <- S + k^ delta^T
 *   o     = S^T q^                                      (updated state)
 *   y     = o (mean_{d_v} o^2 + norm_eps)^-1/2 * norm_w * gate(z)
 *
 * with value head hv reading key head hv / (H_v / H_k) (or hv mod H_k, see
 * gdn_head_map), S a per-(sequence, value head) fp32 matrix [d_k][d_v], and
 * gate = SiLU or sigmoid.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is device memory owned by the caller.  The core
 *     entry points (all but gdn_mixer_*) allocate and free nothing; their
 *     only process-wide state is set once and never changes afterwards: a
 *     per-device cache of the compute-unit count (atomic), the kernels'
 *     LDS-size attributes (set on a kernel's first use, in a thread-safe
 *     static initialiser) and the per-device address of the static scratch
 *     array that gdn_prefill_chunked_noalloc uses as its workspace.
 *   - The mixer entry points (gdn_mixer_prefill, gdn_mixer_decode) also keep,
 *     per device, one hipBLASLt handle and one GEMM plan per problem shape.
 *     Both are made on first use, under a lock, and kept until the process
 *     ends; making them allocates host memory and, inside hipBLASLt, device
 *     memory.  Every plan a call needs is resolved before its first launch,
 *     so a failure there still leaves the caller's buffers untouched.
 *   - Layouts are dense row-major with the innermost index last:
 *       qkv   [T][conv_dim], conv_dim = 2*H_k*d_k + H_v*d_v, channels
 *             ordered q (H_k heads) | k (H_k heads) | v (H_v heads), each
 *             head's d lanes contiguous;
 *       z, out [T][H_v*d_v];  a, b [T][H_v];
 *       state [N][H_v][d_k][d_v] fp32 (key lane major, as on the pages);
 *       conv state [N][K-1][conv_dim] fp32, slot 0 the oldest raw input;
 *       params: conv_w [conv_dim][K], a_log or decay_coef [H_v],
 *               dt_bias [H_v], norm_w [d_v], all fp32.
 *   - act_dtype selects bf16 or fp32 for qkv, z, a, b; out_dtype selects
 *     bf16 (round to nearest even) or fp32 for out.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously; no call synchronises the device.
 *   - Arguments are validated on the host before anything is enqueued: a
 *     call that returns an error has written nothing.  gdn_last_error()
 *     then returns a message for the calling thread.
 *   - Supported: H_v % H_k == 0, d_k and d_v in {32, 64, 128},
 *     1 <= K <= 4, chunk == 64.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_EINVAL = 1,        /* bad pointer, shape, alias or cu_seqlens */
    GDN_EUNSUPPORTED = 2,  /* valid but not instantiated (dims, chunk) */
    GDN_EWORKSPACE = 3,    /* workspace missing or too small */
    GDN_EHIP = 4           /* the HIP runtime rejected a launch */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;
typedef enum { GDN_GATE_SILU = 0, GDN_GATE_SIGMOID = 1 } gdn_gate;

/* Which key head value head hv reads ("oxinfer 0.0.5 src/qwen.rs",
 * DeltaRule::run): GROUPED is the contiguous grouping hv / (H_v / H_k) of
 * the original checkpoints, TILED the order hv mod H_k that GGUF
 * conversions use.  The two agree when H_v == H_k. */
typedef enum { GDN_HEADS_GROUPED = 0, GDN_HEADS_TILED = 1 } gdn_head_map;

/* One decay per value head (Gated DeltaNet), or one per key channel of the
 * value head (Kimi Delta Attention: "cortiq-engine 0.8.76 pipeline.rs",
 * AttnKind::Kda, a per-channel decayed delta rule).  With
 * GDN_DECAY_CHANNEL the gate input a is [T][H_v*d_k] and dt_bias
 * [H_v*d_k]; g[i] = coef * softplus(a[i] + dt_bias[i]) and the state update
 * starts with S <- diag(e^g) S.  Every entry point supports it (the
 * chunked prefill then carries the decay inside its q/k operands). */
typedef enum { GDN_DECAY_HEAD = 0, GDN_DECAY_CHANNEL = 1 } gdn_decay_mode;

/* Where the decode entry points (gdn_decode_step, gdn_decode_multi,
 * gdn_rewind, gdn_mixer_decode) expect the fp32 state to be found at the
 * next call: CACHED when the same layer's state is reread soon (it then
 * stays in the last-level cache, 256 MB on MI355X), STREAMED when other work
 * evicts it in between, as in a model with many GDN layers, whose states
 * together exceed the cache.  STREAMED loads and stores the state
 * non-temporally.  Only the speed differs (the results are bit-identical);
 * the persistent kernel for very wide head groups and the prefill ignore it.
 * Measured at B=64, H_k=16, H_v=32, d=128: CACHED 45.2 us per step with the
 * state cached, 60.8 us without; STREAMED 50.7 us and 52.0 us. */
typedef enum { GDN_STATE_CACHED = 0, GDN_STATE_STREAMED = 1 } gdn_state_cache;

typedef struct {
    int32_t h_k, h_v;       /* key heads, value heads */
    int32_t d_k, d_v;       /* lanes per key / value head */
    int32_t conv_k;         /* conv kernel width K */
    int32_t act_dtype;      /* gdn_dtype of qkv, z, a, b */
    int32_t out_dtype;      /* gdn_dtype of out */
    int32_t gate;           /* gdn_gate applied to z */
    float norm_eps;         /* gated RMSNorm epsilon (1e-6 on the pages) */
    float l2_eps;           /* q/k L2-norm epsilon (1e-6 on the pages) */
    int32_t head_map;       /* gdn_head_map */
    int32_t decay_mode;     /* gdn_decay_mode */
    int32_t state_cache;    /* gdn_state_cache (0, CACHED, when zero-initialised) */
} gdn_config;

/* Exactly one of a_log and decay_coef is given, the other is NULL: the
 * log-decay is g = -exp(a_log[hv]) * softplus(a + dt_bias[hv]), or
 * g = decay_coef[hv] * softplus(a + dt_bias[hv]) for layers that store the
 * coefficient -exp(A_log) itself (GGUF ssm_a; "oxinfer 0.0.5 src/qwen.rs",
 * weight loading).
 * conv_w and norm_w must be 16-byte aligned (the kernels read them in
 * 16-byte rows; every torch allocation is); a misaligned one is GDN_EINVAL. */
typedef struct {
    const float *conv_w;    /* [conv_dim][K] depthwise conv taps, no bias */
    const float *a_log;     /* [H_v]  decay magnitude, g = -exp(a_log)... */
    const float *dt_bias;   /* [H_v]  added to a before softplus */
    const float *norm_w;    /* [d_v]  gated-norm weight (plain multiplier) */
    const float *decay_coef;/* [H_v]  or the coefficient itself, g = decay_coef... */
} gdn_params;

/*
 * Causal depthwise conv + SiLU over packed sequences, with history carry
 * ("cherenkov qwen4_exp/cpu.rs" fn causal_conv; "oxinfer 0.0.5
 * src/qwen.rs" gdn_forward, conv-state update).
 *   cu_seqlens_host, cu_seqlens_dev: the same [n_seq+1] offsets (host copy
 *     for validation and grid sizing, device copy for the kernel);
 *     cu[0] = 0, non-decreasing, cu[n_seq] = t_total.
 *   x [t_total][conv_dim] raw inputs (act_dtype);
 *   conv_state [n_seq][K-1][conv_dim] fp32, read then overwritten in place
 *     with each sequence's last K-1 raw inputs (a sequence shorter than K-1
 *     keeps the tail of its old history ahead of its new inputs);
 *   y [t_total][conv_dim] fp32 receives silu(conv).  y must not overlap x
 *     or conv_state.
 */
gdn_status gdn_conv_update(const gdn_config *cfg, const gdn_params *params,
                           int32_t n_seq, int32_t t_total,
                           const int32_t *cu_seqlens_host,
                           const int32_t *cu_seqlens_dev, const void *x,
                           float *conv_state, float *y, void *stream);

/*
 * One decode step: one new token for each of `batch` sequences, one fused
 * kernel for conv, norms, gates, the delta-rule update and the gated norm
 * ("cherenkov qwen4_exp/cpu.rs" fn deltanet).
 *   qkv [batch][conv_dim], z [batch][H_v*d_v], a, b [batch][H_v]
 *     (act_dtype);
 *   conv_state [batch][K-1][conv_dim] and state [batch][H_v][d_k][d_v],
 *     fp32, updated in place;
 *   out [batch][H_v*d_v] (out_dtype); must not overlap any other argument.
 *   batch == 0 is a no-op.
 */
gdn_status gdn_decode_step(const gdn_config *cfg, const gdn_params *params,
                           int32_t batch, const void *qkv, const void *z,
                           const void *a, const void *b, float *conv_state,
                           float *state, void *out, void *stream);

/*
 * Several new tokens per sequence in one call (speculative verification of
 * drafted tokens): the single-token step above applied t_new times in
 * order, with the state read from and written to HBM once per call
 * ("oxinfer 0.0.5 src/qwen.rs", DeltaRule::run over t tokens and the
 * recording forward used for speculative verification).
 *   t_new: tokens per sequence, 1 <= t_new <= 8 (GDN_EUNSUPPORTED beyond,
 *     or when t_new tokens of one key head's conv channels do not fit the
 *     on-chip buffer: t_new * (2*d_k + (H_v/H_k)*d_v) * 4 bytes plus
 *     reduction space must stay within 64 KiB).
 *   n_tok_dev: NULL (every sequence runs t_new tokens) or a device
 *     [batch] int32 array: sequence i runs its first n_tok_dev[i] tokens
 *     (values are clamped to [0, t_new]); later tokens are not read and
 *     their rows of out and state_ckpt are not written.
 *   qkv [batch][t_new][conv_dim], z [batch][t_new][H_v*d_v],
 *     a, b [batch][t_new][H_v] (act_dtype).  z may be NULL when out is.
 *   conv_in / conv_out [batch][K-1][conv_dim] fp32: history before and
 *     after the tokens; may be the same buffer (in place).
 *   state_in / state_out [batch][H_v][d_k][d_v] fp32: may be the same
 *     buffer (in place) but must not partially overlap.
 *   state_ckpt: NULL or [batch][t_new][H_v][d_k][d_v] fp32, the state after
 *     each token (for callers that keep per-token states instead of
 *     replaying; 2 MiB per token and sequence at H_v = 32, d = 128).  With
 *     state_ckpt NULL and t_new = 8 (scalar decay) the call's tokens are
 *     combined in the in-chunk (UT) form, split-bf16 products on the matrix
 *     cores, instead of being stepped one at a time.
 *   out: NULL (no outputs) or [batch][t_new][H_v*d_v] (out_dtype).
 *   batch == 0 is a no-op.
 */
gdn_status gdn_decode_multi(const gdn_config *cfg, const gdn_params *params,
                            int32_t batch, int32_t t_new,
                            const int32_t *n_tok_dev, const void *qkv,
                            const void *z, const void *a, const void *b,
                            const float *conv_in, float *conv_out,
                            const float *state_in, float *state_out,
                            float *state_ckpt, void *out, void *stream);

/*
 * Rewind after speculative verification: a recurrent state cannot be
 * truncated, so the state of each sequence is rebuilt from the state saved
 * before the verified span by replaying the delta rule over the first
 * keep_dev[i] recorded tokens ("oxinfer 0.0.5 src/qwen.rs",
 * QwenSession::rewind and GdnRecord).  The replay is gdn_decode_multi with
 * no outputs, so keeping every recorded token reproduces bit for bit the
 * state that a verification without per-token states (state_ckpt NULL)
 * reached.  (With 8 tokens per call and no per-token states the tokens are
 * combined in the in-chunk form on the matrix cores; a verification that
 * asks for per-token states steps token by token, which agrees with it to
 * rounding, not to the bit.)
 *   t_rec: recorded tokens per sequence (1 <= t_rec <= 8, as t_new above).
 *   keep_dev: NULL (keep all t_rec) or device [batch] int32, clamped to
 *     [0, t_rec].
 *   qkv_rec [batch][t_rec][conv_dim], a_rec, b_rec [batch][t_rec][H_v]: the
 *     recorded raw inputs (act_dtype).
 *   state0 [batch][H_v][d_k][d_v], conv0 [batch][K-1][conv_dim] fp32: the
 *     saved state and history before the span (read only).
 *   state, conv_state: receive the rewound state and history (the last K-1
 *     raw inputs up to the last kept token, reaching into conv0 when fewer
 *     than K-1 tokens are kept).  May equal state0 / conv0.
 */
gdn_status gdn_rewind(const gdn_config *cfg, const gdn_params *params,
                      int32_t batch, int32_t t_rec, const int32_t *keep_dev,
                      const void *qkv_rec, const void *a_rec,
                      const void *b_rec, const float *state0,
                      const float *conv0, float *state, float *conv_state,
                      void *stream);

/*
 * Bytes of device workspace gdn_prefill_chunked needs for these sizes
 * (0 if the configuration is invalid or unsupported).
 */
size_t gdn_prefill_workspace_bytes(const gdn_config *cfg, int32_t n_seq,
                                   int32_t t_total, int32_t chunk);

/*
 * Chunked prefill over packed variable-length sequences.  Exactly the
 * token recurrence above, evaluated chunk by chunk in the UT-transform
 * form (intra-chunk products on matrix cores, the chain of chunk states
 * sequential per sequence and head).  Chunks restart at every sequence
 * start; the last chunk of a sequence may be partial.
 *   chunk: tokens per chunk (64).
 *   cu_seqlens_host / _dev: as in gdn_conv_update.
 *   qkv [t_total][conv_dim], z [t_total][H_v*d_v], a, b [t_total][H_v];
 *     qkv, z and out are read and written in 16-byte pieces and must be
 *     16-byte aligned (GDN_EINVAL otherwise); with GDN_DECAY_CHANNEL so
 *     must a ([t_total][H_v*d_k], read in 16-byte rows too).
 *   state_in [n_seq][H_v][d_k][d_v] fp32, or NULL for zeros;
 *   state_out, same shape: each sequence's final state.  May equal
 *     state_in (in place) but must not partially overlap it.
 *   conv_in [n_seq][K-1][conv_dim] fp32, or NULL for zeros; conv_out, same
 *     shape, the final history.  May equal conv_in.
 *   out [t_total][H_v*d_v] (out_dtype); must not overlap any other buffer.
 *   workspace: device memory of at least
 *     gdn_prefill_workspace_bytes(cfg, n_seq, t_total, chunk) bytes,
 *     256-byte aligned, owned by the caller, contents undefined on return.
 *   A sequence of length 0 copies its state and history through.
 */
gdn_status gdn_prefill_chunked(const gdn_config *cfg, const gdn_params *params,
                               int32_t chunk, int32_t n_seq, int32_t t_total,
                               const int32_t *cu_seqlens_host,
                               const int32_t *cu_seqlens_dev, const void *qkv,
                               const void *z, const void *a, const void *b,
                               const float *state_in, float *state_out,
                               const float *conv_in, float *conv_out,
                               void *out, void *workspace, size_t ws_bytes,
                               void *stream);

/*
 * gdn_prefill_chunked for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, layouts and results as gdn_prefill_chunked
 * (it runs the same kernels), without the workspace: the library takes it
 * from a static device array of GDN_PREFILL_NOALLOC_MAX_BYTES bytes that
 * each device holds from the library's first use until the process ends.
 * The call allocates and frees nothing (the array's address is looked up
 * once per device, on the first call there).
 *   A call whose gdn_prefill_workspace_bytes(cfg, n_seq, t_total, chunk)
 *   exceeds GDN_PREFILL_NOALLOC_MAX_BYTES returns GDN_EUNSUPPORTED and
 *   enqueues nothing (at H_k=16, H_v=32, d=128 the limit is reached near
 *   700 tokens per call).
 *   Every call on one device shares that device's array: calls that
 *   overlap in time on one device (other streams, other threads) race and
 *   must be serialised by the caller.  Nothing in the array needs clearing
 *   between calls.
 */
#define GDN_PREFILL_NOALLOC_MAX_BYTES ((size_t)64 << 20)
gdn_status gdn_prefill_chunked_noalloc(const gdn_config *cfg, const gdn_params *params,
                                       int32_t chunk, int32_t n_seq, int32_t t_total,
                                       const int32_t *cu_seqlens_host,
                                       const int32_t *cu_seqlens_dev, const void *qkv,
                                       const void *z, const void *a, const void *b,
                                       const float *state_in, float *state_out,
                                       const float *conv_in, float *conv_out, void *out,
                                       void *stream);

/*
 * The mixer with its projections ("oxinfer 0.0.5 src/qwen.rs", Gdn struct
 * and gdn_forward): in_proj of the model's hidden states x into qkv, z, b
 * and a, the mixer core above, and out_proj of its output back to the
 * hidden size.  Weights are bf16, row-major [out features][in features],
 * owned by the caller:
 */
typedef struct {
    int32_t hidden;          /* model width H, a positive multiple of 8 */
    const void *w_qkv;       /* [conv_dim][H] */
    const void *w_z;         /* [H_v*d_v][H] */
    const void *w_b;         /* [H_v][H] */
    const void *w_a;         /* [H_v*gate_width][H], gate_width = d_k with
                                GDN_DECAY_CHANNEL, else 1 */
    const void *w_out;       /* [H][H_v*d_v] */
} gdn_proj;

/*
 * Bytes of device workspace gdn_mixer_prefill needs for these sizes (also
 * enough for gdn_mixer_decode with batch <= t_total), 0 if invalid.
 */
size_t gdn_mixer_workspace_bytes(const gdn_config *cfg, int32_t hidden, int32_t n_seq,
                                 int32_t t_total);

/*
 * Mixer over packed sequences (prefill).  The projections are dense GEMMs
 * (bf16 operands, fp32 accumulation); the projected activations stay fp32
 * and the core runs on them; out_proj multiplies the core's fp32 output
 * split into two bf16 parts, so the layer keeps fp32-level accuracy.
 *   cfg->act_dtype must be GDN_BF16: x [t_total][H] bf16.
 *   cfg->out_dtype selects y [t_total][H] bf16 or fp32.
 *   cu_seqlens, state_in/out, conv_in/out: as in gdn_prefill_chunked.
 *   workspace: gdn_mixer_workspace_bytes(cfg, H, n_seq, t_total) bytes,
 *     256-byte aligned.  y must not overlap any other buffer.
 */
gdn_status gdn_mixer_prefill(const gdn_config *cfg, const gdn_params *params,
                             const gdn_proj *proj, int32_t n_seq, int32_t t_total,
                             const int32_t *cu_seqlens_host,
                             const int32_t *cu_seqlens_dev, const void *x,
                             const float *state_in, float *state_out,
                             const float *conv_in, float *conv_out, void *y,
                             void *workspace, size_t ws_bytes, void *stream);

/*
 * Mixer decode step: one token for each of `batch` sequences, x [batch][H]
 * bf16 -> y [batch][H]; conv_state and state updated in place as in
 * gdn_decode_step.  workspace: gdn_mixer_workspace_bytes(cfg, H, batch,
 * batch) bytes.
 */
gdn_status gdn_mixer_decode(const gdn_config *cfg, const gdn_params *params,
                            const gdn_proj *proj, int32_t batch, const void *x,
                            float *conv_state, float *state, void *y,
                            void *workspace, size_t ws_bytes, void *stream);

/* Static name of a status code. */
const char *gdn_status_string(gdn_status status);

/* Message describing the last error returned on the calling thread ("" if
 * none).  The string stays valid until the next call on that thread. */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
