// Host-side launch interface between the C ABI (gdn_api.cpp) and the
// kernels.  Arguments reaching these launchers are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

typedef uint16_t bf16_t; // (also in gdn_device.h) bf16 as its raw bits

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
    int preconv;    // 1 (decode only): qkv holds silu(conv) already and the history is current
    // Decode inputs as the mixer's split in_proj products (decode_multi only):
    // in_split 2 = every input is the sum of two fp32 partial products
    // in_split_stride elements apart, all four with row stride in_ld; else 1.
    int in_split, in_ld;
    size_t in_split_stride;
    int nt_state;   // 1: decode loads and stores the state non-temporally
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
// From this many tokens per sequence (and without per-token states) a
// multi-token call runs in the in-call UT form (B=64, d = 128, with the
// bench's inputs: t = 8 66.4-67.2 against 68.7-71.0 us stepped; at t = 7
// stepping measured faster).
constexpr int kUtMinTokens = 8;
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
                                int t_total, int max_len, const int32_t *cu_host,
                                const int32_t *cu_dev, const void *x,
                                const float *state_in, float *state_out, const float *conv_in,
                                float *conv_out, void *y, void *ws, hipStream_t s);
hipError_t launch_mixer_decode(const Dims &d, const Params &p, const Proj &pj, int batch,
                               const void *x, float *conv_state, float *state, void *y, void *ws,
                               hipStream_t s);

// Chunked prefill.  Workspace layout and size are owned by prefill.hip.
size_t prefill_workspace_bytes(const Dims &d, int n_seq, int t_total);
// cu_host (host copy of cu_dev, may be NULL) orders the scan's work longest
// sequence first.
hipError_t launch_prefill(const Dims &d, const Params &p, int n_seq, int t_total,
                          int max_len, const int32_t *cu_host, const int32_t *cu_dev, const void *qkv,
                          const void *z, const void *a, const void *b,
                          const float *state_in, float *state_out, const float *conv_in,
                          float *conv_out, void *out, void *ws, hipStream_t s);

// Skinny matrix products of a mixer decode step (skinny.hip): D[M][N] =
// sum over parts of A_part[M][K] . W[N][K]^T, bf16 operands, fp32 partial
// products per contraction slice.  W is the concatenation of up to four
// row blocks: output column n < N lives in w[b] at row n - wstart[b] for the
// last b with wstart[b] <= n.
constexpr int kSkinnyRows = 64;     // rows of A per call, at most
constexpr int kSkinnyCols = 64;     // output columns per workgroup
constexpr int kSkinnyMaxSplit = 16; // contraction slices, at most (K <= 16 slices)
constexpr int kSkinnyDirectRows = 8; // up to this many rows in_proj runs as one slice
struct SkinnyGemm {
    const bf16_t *a[2];
    int M, K, N;
    const bf16_t *w[4];
    int wstart[4];
    float *part; // [skinny_ksplit(K, parts)][M][N]
    int kslice;  // (set by launch_skinny_gemm)
};
// Adds the slices' partials of in_proj and stores them per block (qkv, z,
// b, a), the qkv block through the causal conv + SiLU with its history
// conv_state [M][conv_k-1][qkv columns] moved on in place.
struct ProjEpilogue {
    const float *part;
    int ksplit, M, N;
    int start[5]; // block column starts, start[4] = N
    float *dst[4];
    const float *conv_w;
    float *conv_state;
    int conv_k;
};
// Contraction slices of a skinny product, 0 if K cannot be split for it.
int skinny_ksplit(int K, int nparts);
// With epi (one A part, the whole contraction in one slice: K of 256, 512,
// 1024 or 2048, skinny_direct_ok) the product kernel applies the in_proj
// epilogue itself instead of storing partial products.
bool skinny_direct_ok(int K);
hipError_t launch_skinny_gemm(SkinnyGemm g, int nparts, const ProjEpilogue *epi, hipStream_t s);
hipError_t launch_proj_epilogue(const ProjEpilogue &e, hipStream_t s);
hipError_t launch_out_epilogue(const float *part, int ksplit, size_t n, void *out, int out_bf16,
                               hipStream_t s);

// Workspace of the allocation-free prefill: a static device array of this
// many bytes per device, its address resolved once per device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void **ptr);

} // namespace gdn
