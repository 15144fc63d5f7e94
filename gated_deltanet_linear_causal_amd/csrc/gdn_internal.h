// Host-side launch interface between the C ABI (gdn_api.cpp) and the
// kernels.  Arguments reaching these launchers are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct Dims {
    int h_k, h_v, d_k, d_v, conv_k;
    int group;      // h_v / h_k
    int conv_dim;   // 2*h_k*d_k + h_v*d_v
    int value_dim;  // h_v*d_v
    int act_bf16;   // 1: activations are bf16, 0: fp32
    int out_bf16;   // 1: output is bf16, 0: fp32
    int gate;       // 0: SiLU, 1: sigmoid
    int tiled;      // 0: key head hv / group, 1: key head hv % h_k
    int chan_decay; // 0: one decay per value head, 1: one per key channel
    int out_split;  // 1: out receives bf16 hi parts, then (after all of them) bf16 lo parts
    float norm_eps, l2_eps;
};

struct Params {
    const float *conv_w, *a_log, *dt_bias, *norm_w;
    const float *decay_coef; // replaces -exp(a_log) when not NULL (a_log is then NULL)
};

// Compute units of the current device (queried once per device and kept).
hipError_t device_cu_count(int *n);

hipError_t launch_conv_update(const Dims &d, const Params &p, int n_seq, int max_len,
                              const int32_t *cu_dev, const void *x, float *conv_state,
                              float *y, hipStream_t s);

hipError_t launch_decode(const Dims &d, const Params &p, int batch, const void *qkv,
                         const void *z, const void *a, const void *b, float *conv_state,
                         float *state, void *out, hipStream_t s);

// Several new tokens per sequence (at most kDecodeMultiMaxTokens), and the
// replay of recorded tokens from a saved state (out == NULL).
constexpr int kDecodeMultiMaxTokens = 8;
constexpr size_t kDecodeMultiMaxLds = 65536;
size_t decode_multi_lds_bytes(const Dims &d, int t_new);
hipError_t launch_decode_multi(const Dims &d, const Params &p, int batch, int t_new,
                               const int32_t *n_tok, const void *qkv, const void *z,
                               const void *a, const void *b, const float *conv_in,
                               float *conv_out, const float *state_in, float *state_out,
                               float *ckpt, void *out, hipStream_t s);

// The mixer with its projections (hipBLASLt GEMMs around the core).
struct Proj {
    int hidden;
    const void *w_qkv, *w_z, *w_b, *w_a, *w_out;
};
size_t mixer_workspace_bytes(const Dims &d, int hidden, int n_seq, int t_total, bool prefill);
hipError_t launch_mixer_prefill(const Dims &d, const Params &p, const Proj &pj, int n_seq,
                                int t_total, int max_len, const int32_t *cu_dev, const void *x,
                                const float *state_in, float *state_out, const float *conv_in,
                                float *conv_out, void *y, void *ws, hipStream_t s);
hipError_t launch_mixer_decode(const Dims &d, const Params &p, const Proj &pj, int batch,
                               const void *x, float *conv_state, float *state, void *y, void *ws,
                               hipStream_t s);

// Chunked prefill.  Workspace layout and size are owned by prefill.hip.
size_t prefill_workspace_bytes(const Dims &d, int n_seq, int t_total);
hipError_t launch_prefill(const Dims &d, const Params &p, int n_seq, int t_total,
                          int max_len, const int32_t *cu_dev, const void *qkv,
                          const void *z, const void *a, const void *b,
                          const float *state_in, float *state_out, const float *conv_in,
                          float *conv_out, void *out, void *ws, hipStream_t s);

// Workspace of the allocation-free prefill: a static device array of this
// many bytes per device, its address resolved once per device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void **ptr);

} // namespace gdn
