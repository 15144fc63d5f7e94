// Standalone causal depthwise conv + SiLU with history carry over packed
// variable-length sequences ("cherenkov qwen4_exp/cpu.rs" fn causal_conv;
// "oxinfer 0.0.5 src/qwen.rs" gdn_forward and its conv-state update).
//
// Grid: (channel blocks of 256, sequence, 64-token tile).  A thread walks
// its tile of one channel with the K-1 previous raw inputs in registers;
// reads of consecutive channels coalesce.  Only tile 0 of a sequence can
// reach back into the old history (K-1 <= 3 < 64), so the thread of tile 0
// is the one reader and the one writer of that channel's history: the
// in-place update needs no synchronisation.

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kConvTile = 64;

template <typename TIn>
__global__ void __launch_bounds__(256)
conv_update_kernel(const TIn *__restrict__ x, const float *__restrict__ conv_w,
                   const int32_t *__restrict__ cu, float *conv_state, float *__restrict__ y,
                   int conv_dim, int K)
{
    const int ch = blockIdx.x * 256 + threadIdx.x;
    const int n = blockIdx.y;
    const int tile = blockIdx.z;
    if (ch >= conv_dim) return;
    const int s0 = cu[n], e0 = cu[n + 1];
    const int t0 = s0 + tile * kConvTile;
    if (t0 >= e0) return; // also covers L == 0: the history stays as it is

    float w[4];
    for (int j = 0; j < K; ++j) w[j] = conv_w[(size_t)ch * K + j];
    float *hist = conv_state + (size_t)n * (K - 1) * conv_dim + ch;

    // Window of the K-1 raw inputs before t0, oldest first.
    float win[3], old[3];
    for (int j = 0; j < K - 1; ++j) {
        const int tau = t0 - (K - 1) + j;
        if (tau >= s0) {
            win[j] = load_act(x, (size_t)tau * conv_dim + ch);
        } else {
            old[j] = hist[(size_t)(K - 1 + tau - s0) * conv_dim];
            win[j] = old[j];
        }
    }
    const int t1 = min(t0 + kConvTile, e0);
    for (int t = t0; t < t1; ++t) {
        const float cur = load_act(x, (size_t)t * conv_dim + ch);
        float acc = 0.0f;
        for (int j = 0; j < K - 1; ++j) acc = fmaf(w[j], win[j], acc);
        acc = fmaf(w[K - 1], cur, acc);
        y[(size_t)t * conv_dim + ch] = siluf_(acc);
        for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
        if (K > 1) win[K - 2] = cur;
    }
    if (tile == 0) {
        // New history: the last K-1 raw inputs of the sequence, oldest
        // first, reaching into the old history when L < K-1.  For tile 0
        // every old slot was read above (tau = s0-(K-1)+j < s0).
        const int L = e0 - s0;
        for (int sl = 0; sl < K - 1; ++sl) {
            const int tau = L - (K - 1) + sl;
            const float v = tau >= 0 ? load_act(x, (size_t)(s0 + tau) * conv_dim + ch)
                                     : old[K - 1 + tau];
            hist[(size_t)sl * conv_dim] = v;
        }
    }
}

hipError_t launch_conv_update(const Dims &d, const Params &p, int n_seq, int max_len,
                              const int32_t *cu_dev, const void *x, float *conv_state,
                              float *y, hipStream_t s)
{
    const int tiles = (max_len + kConvTile - 1) / kConvTile;
    if (n_seq == 0 || tiles == 0) return hipSuccess;
    const dim3 grid((d.conv_dim + 255) / 256, n_seq, tiles);
    if (d.act_bf16)
        hipLaunchKernelGGL(conv_update_kernel<bf16_t>, grid, dim3(256), 0, s,
                           static_cast<const bf16_t *>(x), p.conv_w, cu_dev, conv_state, y,
                           d.conv_dim, d.conv_k);
    else
        hipLaunchKernelGGL(conv_update_kernel<float>, grid, dim3(256), 0, s,
                           static_cast<const float *>(x), p.conv_w, cu_dev, conv_state, y,
                           d.conv_dim, d.conv_k);
    return hipGetLastError();
}

} // namespace gdn
