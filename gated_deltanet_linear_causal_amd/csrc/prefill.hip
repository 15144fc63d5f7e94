// Chunked prefill of the Gated DeltaNet mixer core on gfx950.
//
// The token recurrence of "cherenkov qwen4_exp/cpu.rs" fn deltanet /
// "oxinfer 0.0.5 src/qwen.rs" DeltaRule::run,
//     S_t = a_t S_{t-1} + k_t d_t^T,  d_t = b_t (v_t - a_t S_{t-1}^T k_t),
//     o_t = S_t^T q_t,
// is evaluated chunk by chunk (C = 64 tokens).  With G_i the in-chunk
// cumulative log-decay and S the state entering the chunk:
//     A    = strict_lower(diag(b) (e^{G_i-G_j}) o K K^T),  T = (I + A)^-1
//     P    = lower(e^{G_i-G_j}) o Q K^T
//     X    = K S,  Y = Q S
//     R    = diag(b) (V - diag(e^G) X)
//     D    = T R
//     O    = diag(e^G) Y + P D
//     S'   = e^{G_C} S + K^T (diag(e^{G_C-G}) D)
// Only differences G_i - G_j with j <= i are exponentiated, so strong
// decay underflows to zero instead of overflowing.
//
// Kernels (one stream, in order):
//   qknorm  grid (16-token tile, key head, seq): causal conv + SiLU and L2
//           norm of q and k, a group of lanes per token row; writes q^, k^
//           split into bf16 hi + lo (ready-made matrix-core operands).
//   tri     grid (chunk, value head, seq): gates and their in-chunk prefix
//           sum, K K^T and Q K^T on MFMA, A, the blocked fp32 triangular
//           inverse T, P; writes T and P rows split into bf16 hi + lo.
//   scan    grid (seq, value head, 16-column slice of d_v): the chain of
//           chunk states, sequential over the chunks of one sequence.  The
//           state slice lives in registers, every matrix operand arrives
//           pre-split, and the next chunk's inputs are in flight while the
//           current one is computed.  conv + SiLU of the slice's v channels
//           happens here.  Writes the pre-norm readout O.
//   norm    grid (rows of (token, value head)): gated RMSNorm + output gate.
//   conv_final: each sequence's last K-1 raw inputs become its history.
//
// Contractions run on v_mfma_f32_16x16x32_bf16 with every fp32 operand
// split into bf16 hi + lo and three products (hi.hi + hi.lo + lo.hi, fp32
// accumulate): plain bf16 operands are far outside the parity tolerance,
// the split form is within it.

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kC = 64;       // tokens per chunk
constexpr int kBV = 16;      // d_v columns per scan workgroup
constexpr int kTileTok = 16; // tokens per qknorm workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Frag {
    bf16x8 hi, lo;
};

__device__ __forceinline__ void split1(float v, __bf16 &h, __bf16 &l)
{
    h = static_cast<__bf16>(v);
    l = static_cast<__bf16>(v - static_cast<float>(h));
}

// fp32 -> (hi, lo) bf16 pair with hi + lo = v to ~16 significant bits.
__device__ __forceinline__ Frag split8(const float (&v)[8])
{
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        __bf16 h, l;
        split1(v[e], h, l);
        f.hi[e] = h;
        f.lo[e] = l;
    }
    return f;
}

// D += A B on one 16x16x32 tile, split-bf16 with three MFMAs.
// Lane l holds A[l%16][8*(l/16) + e], B[8*(l/16) + e][l%16] (e < 8) and
// D[4*(l/16) + e][l%16] (e < 4).
__device__ __forceinline__ f32x4 mma3(const Frag &A, const Frag &B, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.lo, B.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.hi, B.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.hi, B.hi, c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ Frag frag_at(const __bf16 *hi, const __bf16 *lo)
{
    Frag f;
    f.hi = *reinterpret_cast<const bf16x8 *>(hi);
    f.lo = *reinterpret_cast<const bf16x8 *>(lo);
    return f;
}

__device__ __forceinline__ Frag frag_select(bool keep, const Frag &f)
{
    Frag z;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        z.hi[e] = keep ? f.hi[e] : static_cast<__bf16>(0.0f);
        z.lo[e] = keep ? f.lo[e] : static_cast<__bf16>(0.0f);
    }
    return z;
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

template <typename T> __device__ __forceinline__ f32x4 load_act4v(const T *p, size_t i)
{
    const float4 v = load_act4(p, i);
    return f32x4{v.x, v.y, v.z, v.w};
}

// Raw activation bits of 4 channels (loaded now, converted when used).
template <typename T> struct RawAct;
template <> struct RawAct<bf16_t> {
    typedef uint2 type;
    __device__ __forceinline__ static type load(const bf16_t *p, size_t i)
    {
        return *reinterpret_cast<const uint2 *>(p + i);
    }
    __device__ __forceinline__ static f32x4 to_f32(type u)
    {
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
    }
};
template <> struct RawAct<float> {
    typedef f32x4 type;
    __device__ __forceinline__ static type load(const float *p, size_t i)
    {
        return *reinterpret_cast<const f32x4 *>(p + i);
    }
    __device__ __forceinline__ static f32x4 to_f32(type u) { return u; }
};

__device__ __forceinline__ uint32_t pack2(__bf16 a, __bf16 b)
{
    return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// ---------------------------------------------------------------------------
// Workspace layout (sections 256-byte aligned):
//   qk [T][H_k][2: q^,k^][2: hi,lo][d_k] bf16
//   tp [T][H_v][2: T,P][2: hi,lo][C]    bf16 (row of the token's chunk)
//   gb [T][H_v][2]                      fp32 (G in-chunk cumulative, beta)
//   o  [T][H_v*d_v]                     fp32 pre-norm readout
// ---------------------------------------------------------------------------
struct WsLayout {
    size_t qk, tp, gb, o, total;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static WsLayout ws_layout(const Dims &d, int t_total)
{
    WsLayout w;
    const size_t T = (size_t)t_total;
    size_t off = 0;
    w.qk = off;
    off = align256(off + T * d.h_k * 4 * d.d_k * 2);
    w.tp = off;
    off = align256(off + T * d.h_v * 4 * kC * 2);
    w.gb = off;
    off = align256(off + T * d.h_v * 2 * sizeof(float));
    w.o = off;
    off = align256(off + T * d.value_dim * sizeof(float));
    w.total = off;
    return w;
}

size_t prefill_workspace_bytes(const Dims &d, int n_seq, int t_total)
{
    (void)n_seq;
    return ws_layout(d, t_total).total;
}

struct PrefillArgs {
    const void *qkv, *z, *a, *b;
    const float *conv_w, *a_log, *dt_bias, *norm_w;
    const int32_t *cu;
    const float *state_in;
    float *state_out;
    const float *conv_in;
    float *conv_out;
    void *out;
    __bf16 *ws_qk, *ws_tp;
    float *ws_gb, *ws_o;
    int h_k, h_v, d_v, group, conv_k, conv_dim, value_dim;
    int gate, out_bf16;
    float norm_eps, l2_eps;
};

// Conv taps of 4 channels starting at ch, right-aligned to 4 taps (zero
// taps in front when K < 4): w[e][j] multiplies the input 3-j tokens back.
__device__ __forceinline__ void load_taps4(const PrefillArgs &p, int ch, float (&w)[4][4])
{
    const int K = p.conv_k;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int jj = j - (4 - K);
            w[e][j] = jj >= 0 ? p.conv_w[(size_t)(ch + e) * K + jj] : 0.0f;
        }
}

// Raw inputs of 4 channels at sequence position tau (< 0 reaches into the
// incoming history; zero when there is none).
template <typename TIn>
__device__ __forceinline__ f32x4 raw4(const PrefillArgs &p, const TIn *x, int n, int s0, int tau,
                                      int ch)
{
    if (tau >= 0) return load_act4v(x, (size_t)(s0 + tau) * p.conv_dim + ch);
    const int slot = p.conv_k - 1 + tau;
    if (p.conv_in && slot >= 0)
        return ld4(p.conv_in + ((size_t)n * (p.conv_k - 1) + slot) * p.conv_dim + ch);
    return f32x4{0.f, 0.f, 0.f, 0.f};
}

// silu(causal conv) of 4 channels from the 4 taps' raw inputs.
__device__ __forceinline__ f32x4 conv4(const float (&w)[4][4], const f32x4 (&xr)[4])
{
    f32x4 c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = fmaf(w[e][j], xr[j][e], acc);
        c[e] = siluf_(acc);
    }
    return c;
}

// ---------------------------------------------------------------------------
// qknorm: one workgroup per (16-token tile, key head, sequence).  Each token
// row of the key head (q then k, 2*d_k channels) is handled by d_k/2 lanes
// of 4 channels; each L2 norm is a reduction over d_k/4 lanes.
// ---------------------------------------------------------------------------
template <typename TIn, int DK>
__global__ void __launch_bounds__(256)
qknorm_kernel(const PrefillArgs p)
{
    constexpr int LPT = DK / 2;                 // lanes per token row
    constexpr int TPI = 64 / LPT;               // token rows per wave pass
    constexpr int ITERS = kTileTok / (4 * TPI); // passes per wave
    const int tile = blockIdx.x, hk = blockIdx.y, n = blockIdx.z;
    const int s0 = p.cu[n], L = p.cu[n + 1] - s0;
    if (tile * kTileTok >= L) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane / LPT, ll = lane % LPT;
    const bool isk = ll >= DK / 4;
    const int c4 = (isk ? ll - DK / 4 : ll) * 4;
    const int ch = (isk ? p.h_k * DK : 0) + hk * DK + c4;
    const TIn *x = static_cast<const TIn *>(p.qkv);
    float w[4][4];
    load_taps4(p, ch, w);
    const float extra = isk ? 1.0f : rsqrtf((float)DK);

#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int tl = tile * kTileTok + (it * 4 + wave) * TPI + sub;
        const bool valid = tl < L;
        const int tc = valid ? tl : L - 1;
        f32x4 xr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[j] = raw4(p, x, n, s0, tc - 3 + j, ch);
        const f32x4 c = conv4(w, xr);
        float ss = c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3];
        ss = group_sum<DK / 4>(ss);
        const float sc = rsqrtf(ss + p.l2_eps) * extra;
        if (valid) {
            __bf16 h[4], l[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split1(c[e] * sc, h[e], l[e]);
            __bf16 *dst = p.ws_qk + ((size_t)(s0 + tl) * p.h_k + hk) * 4 * DK + (isk ? 2 * DK : 0) + c4;
            *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
            *reinterpret_cast<uint2 *>(dst + DK) = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
        }
    }
}

// ---------------------------------------------------------------------------
// tri: one workgroup per (chunk, value head, sequence), 256 threads.
// ---------------------------------------------------------------------------
template <typename TIn, int DK>
__global__ void __launch_bounds__(256)
tri_kernel(const PrefillArgs p)
{
    constexpr int LC = kC + 4;
    const int c = blockIdx.x, hv = blockIdx.y, n = blockIdx.z;
    const int s0 = p.cu[n];
    const int L = p.cu[n + 1] - s0;
    if (c * kC >= L) return;
    const int t0 = s0 + c * kC;
    const int Lc = min(kC, L - c * kC);
    const int hk = hv / p.group;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;

    __shared__ __attribute__((aligned(16))) float sA[kC * LC];
    __shared__ __attribute__((aligned(16))) float sP[kC * LC];
    __shared__ __attribute__((aligned(16))) float sT[kC * LC];
    __shared__ __attribute__((aligned(16))) float sW[4][16 * 17];
    __shared__ float sG[kC], sB[kC];

    for (int i = tid; i < kC * LC / 4; i += 256) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        reinterpret_cast<f32x4 *>(sA)[i] = z;
        reinterpret_cast<f32x4 *>(sP)[i] = z;
        reinterpret_cast<f32x4 *>(sT)[i] = z;
    }
    // Gates ("cherenkov qwen4_exp/cpu.rs" fn deltanet) and their inclusive
    // prefix sum over the chunk (wave 0).  Past the chunk end: g = 0, b = 0.
    if (wave == 0) {
        float beta = 0.0f, g = 0.0f;
        if (lane < Lc) {
            const size_t gi = (size_t)(t0 + lane) * p.h_v + hv;
            beta = sigmoidf_(load_act(static_cast<const TIn *>(p.b), gi));
            g = -expf(p.a_log[hv]) *
                softplusf_(load_act(static_cast<const TIn *>(p.a), gi) + p.dt_bias[hv]);
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float u = __shfl_up(g, off, 64);
            if (lane >= off) g += u;
        }
        sG[lane] = g;
        sB[lane] = beta;
        if (lane < Lc)
            *reinterpret_cast<float2 *>(p.ws_gb + ((size_t)(t0 + lane) * p.h_v + hv) * 2) =
                make_float2(g, beta);
    }
    __syncthreads();

    // K K^T -> A and Q K^T -> P, lower-triangular 16x16 tiles:
    // 20 tiles (which, mt, nt >= ... nt <= mt); wave w takes every 4th.
    const __bf16 *qk0 = p.ws_qk + ((size_t)t0 * p.h_k + hk) * 4 * DK;
    const size_t rs = (size_t)p.h_k * 4 * DK; // bf16 per token row
    for (int tile = wave; tile < 20; tile += 4) {
        const int which = tile / 10; // 0: K K^T, 1: Q K^T
        int r = tile % 10, mt = 0;
        while (r > mt) {
            r -= mt + 1;
            ++mt;
        }
        const int nt = r;
        const int ra = 16 * mt + col, rb = 16 * nt + col;
        const __bf16 *pA = qk0 + (size_t)(ra < Lc ? ra : 0) * rs + (which == 0 ? 2 * DK : 0) + 8 * kq;
        const __bf16 *pB = qk0 + (size_t)(rb < Lc ? rb : 0) * rs + 2 * DK + 8 * kq;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const Frag A = frag_select(ra < Lc, frag_at(pA + 32 * s, pA + DK + 32 * s));
            const Frag B = frag_select(rb < Lc, frag_at(pB + 32 * s, pB + DK + 32 * s));
            acc = mma3(A, B, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * mt + 4 * kq + e, j = 16 * nt + col;
            const float m = j <= i ? expf(sG[i] - sG[j]) : 0.0f;
            if (which == 0)
                sA[i * LC + j] = j < i ? sB[i] * m * acc[e] : 0.0f;
            else
                sP[i * LC + j] = m * acc[e];
        }
    }
    __syncthreads();

    // T = (I + A)^-1, blocked over 16x16 blocks, fp32.
    // Diagonal blocks by forward substitution: wave b owns block b; lane
    // (col j, quarter q) keeps rows 4q..4q+3 of column j.
    {
        const int b = wave;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (4 * kq + e == col) ? 1.0f : 0.0f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            const f32x4 a4 = ld4(sA + (16 * b + r) * LC + 16 * b + 4 * kq);
            float part = a4[0] * x[0] + a4[1] * x[1] + a4[2] * x[2] + a4[3] * x[3];
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            if (r > col && kq == r / 4) x[r % 4] = -part;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(16 * b + 4 * kq + e) * LC + 16 * b + col] = x[e];
    }
    __syncthreads();
    // Off-diagonal blocks, by distance d from the diagonal:
    //   T_ij = -T_ii (sum_{m=j}^{i-1} A_im T_mj).
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        const bool act = wave < 4 - d;
        const int bi = wave + d, bj = wave;
        if (act) {
            float wv[4] = {0.f, 0.f, 0.f, 0.f};
            for (int m = bj; m < bi; ++m) {
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    float tc[4];
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) tc[kk] = sT[(16 * m + 4 * k4 + kk) * LC + 16 * bj + col];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const f32x4 a4 = ld4(sA + (16 * bi + 4 * kq + e) * LC + 16 * m + 4 * k4);
                        wv[e] = fmaf(a4[0], tc[0], fmaf(a4[1], tc[1], fmaf(a4[2], tc[2], fmaf(a4[3], tc[3], wv[e]))));
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sW[wave][(4 * kq + e) * 17 + col] = wv[e];
        }
        __syncthreads();
        if (act) {
            float tv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                float wk[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) wk[kk] = sW[wave][(4 * k4 + kk) * 17 + col];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x4 t4 = ld4(sT + (16 * bi + 4 * kq + e) * LC + 16 * bi + 4 * k4);
                    tv[e] = fmaf(t4[0], wk[0], fmaf(t4[1], wk[1], fmaf(t4[2], wk[2], fmaf(t4[3], wk[3], tv[e]))));
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * bi + 4 * kq + e) * LC + 16 * bj + col] = -tv[e];
        }
        __syncthreads();
    }

    // T and P rows of the chunk's tokens, split into bf16 hi + lo.
    for (int idx = tid; idx < Lc * 16; idx += 256) {
        const int i = idx >> 4, which = (idx >> 3) & 1, g = idx & 7;
        const float *src = (which ? sP : sT) + i * LC + 8 * g;
        const f32x4 u = ld4(src), v = ld4(src + 4);
        const float vals[8] = {u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
        const Frag f = split8(vals);
        __bf16 *dst = p.ws_tp + ((size_t)(t0 + i) * p.h_v + hv) * 4 * kC + which * 2 * kC + 8 * g;
        *reinterpret_cast<bf16x8 *>(dst) = f.hi;
        *reinterpret_cast<bf16x8 *>(dst + kC) = f.lo;
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, value head, 16-column slice), 256
// threads = 4 waves.  Wave w owns output rows 16w..16w+15 of each chunk and
// the state rows of M-tiles w, w+4, ... (16 rows each).
// ---------------------------------------------------------------------------
template <int DK> constexpr size_t scan_smem_bytes()
{
    constexpr size_t RK = DK + 8, RT = kC + 8;
    return 2 * (4 * kC * RK + 2 * DK * RT + 2 * kBV * RK + 6 * kBV * RT) +
           4 * (kC * kBV + 3 * kC);
}

template <typename TIn, int DK>
__global__ void __launch_bounds__(256)
scan_kernel(const PrefillArgs p, int slices)
{
    constexpr int RK = DK + 8;    // bf16 row stride: q^/k^ rows, S^T rows
    constexpr int RT = kC + 8;    // bf16 row stride: transposed chunk vectors
    constexpr int MTS = DK / 16;  // state M-tiles
    constexpr int MTW = (MTS + 3) / 4;
    constexpr int GPR = DK / 2;   // 16-byte groups per token row (4*DK bf16)
    constexpr int PF = kC * GPR / 256;

    // Map the block index so the slices of one head share an XCD (blocks
    // are dealt round-robin over 8 XCDs): they read the same chunk data.
    const int nheads = gridDim.x / slices;
    int hidx, slice;
    {
        const int b = blockIdx.x;
        if (slices == 8 && nheads % 8 == 0) {
            const int x8 = b % 8, rest = b / 8;
            slice = rest % 8;
            hidx = (rest / 8) * 8 + x8;
        } else {
            slice = b % slices;
            hidx = b / slices;
        }
    }
    const int n = hidx / p.h_v, hv = hidx % p.h_v;
    const int hk = hv / p.group;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const int s0 = p.cu[n];
    const int L = p.cu[n + 1] - s0;
    const int nchunks = (L + kC - 1) / kC;
    const int c0 = hv * p.d_v + slice * kBV; // first value column
    const TIn *x = static_cast<const TIn *>(p.qkv);

    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    __bf16 *sQh = reinterpret_cast<__bf16 *>(smem_raw); // [C][RK]
    __bf16 *sQl = sQh + kC * RK;
    __bf16 *sKh = sQl + kC * RK;
    __bf16 *sKl = sKh + kC * RK;
    __bf16 *sKTh = sKl + kC * RK;  // [DK][RT]  k^ transposed
    __bf16 *sKTl = sKTh + DK * RT;
    __bf16 *sSh = sKTl + DK * RT;  // [16][RK]  state slice transposed
    __bf16 *sSl = sSh + kBV * RK;
    __bf16 *sRh = sSl + kBV * RK;  // [16][RT]  R transposed
    __bf16 *sRl = sRh + kBV * RT;
    __bf16 *sDh = sRl + kBV * RT;  // [16][RT]  D transposed
    __bf16 *sDl = sDh + kBV * RT;
    __bf16 *sEh = sDl + kBV * RT;  // [16][RT]  diag(e^{G_C-G}) D transposed
    __bf16 *sEl = sEh + kBV * RT;
    float *sV = reinterpret_cast<float *>(sEl + kBV * RT); // [C][16] conv(v)
    float *sEG = sV + kC * kBV;    // e^{G_t}
    float *sEGC = sEG + kC;        // e^{G_C - G_t}
    float *sB = sEGC + kC;         // beta_t

    // State slice in registers (D layout): tile mt = wave + 4*u.
    f32x4 S[MTW];
    {
        const float *Sin = p.state_in ? p.state_in + ((size_t)n * p.h_v + hv) * DK * p.d_v : nullptr;
#pragma unroll
        for (int u = 0; u < MTW; ++u) {
            const int mt = wave + 4 * u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * mt + 4 * kq + e;
                S[u][e] = (mt < MTS && Sin) ? Sin[(size_t)i * p.d_v + slice * kBV + col] : 0.0f;
            }
            if (mt < MTS)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    __bf16 h, l;
                    split1(S[u][e], h, l);
                    sSh[col * RK + 16 * mt + 4 * kq + e] = h;
                    sSl[col * RK + 16 * mt + 4 * kq + e] = l;
                }
        }
    }

    // v channels of this thread at staging time: token vt, channels 4*vg..
    const int vt = tid >> 2, vg = tid & 3;
    const int vch = 2 * p.h_k * DK + c0 + 4 * vg;
    float wv[4][4];
    load_taps4(p, vch, wv);

    // Inputs of the next chunk, in flight in registers while the current
    // chunk is computed.  The fetch only issues loads (rows past the chunk
    // end re-read a valid row); every select or conversion that needs the
    // loaded values happens at staging time, after the compute.
    typedef typename RawAct<TIn>::type RawT;
    u32x4 pqk[PF];
    Frag nT[2], nP[2], cT[2], cP[2];
    RawT nxr[4];
    float2 ngb = make_float2(0.f, 0.f);
    float ngc = 0.0f;

#define GDN_SCAN_FETCH(CH)                                                                     \
    {                                                                                          \
        const int ft0 = s0 + (CH) * kC;                                                        \
        const int fLc = min(kC, L - (CH) * kC);                                                \
        _Pragma("unroll") for (int f = 0; f < PF; ++f) {                                       \
            const int idx = tid + 256 * f;                                                     \
            const int t = idx / GPR, g = idx % GPR;                                            \
            const int tr = t < fLc ? t : 0;                                                    \
            pqk[f] = *reinterpret_cast<const u32x4 *>(                                         \
                p.ws_qk + ((size_t)(ft0 + tr) * p.h_k + hk) * 4 * DK + 8 * g);                 \
        }                                                                                      \
        {                                                                                      \
            const int row = 16 * wave + col;                                                   \
            const int rr = row < fLc ? row : 0;                                                \
            const __bf16 *tp = p.ws_tp + ((size_t)(ft0 + rr) * p.h_v + hv) * 4 * kC + 8 * kq;  \
            _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                    \
                nT[s] = frag_at(tp + 32 * s, tp + kC + 32 * s);                                \
                nP[s] = frag_at(tp + 2 * kC + 32 * s, tp + 3 * kC + 32 * s);                   \
            }                                                                                  \
        }                                                                                      \
        {                                                                                      \
            const int tl = (CH) * kC + vt;                                                     \
            const int tc = tl < L ? tl : L - 1;                                                \
            /* positions before the sequence start only occur in chunk 0, whose  */            \
            /* v inputs are read through the history path instead: clamp to 0    */            \
            _Pragma("unroll") for (int j = 0; j < 4; ++j)                                      \
                nxr[j] = RawAct<TIn>::load(                                                    \
                    x, (size_t)(s0 + max(tc - 3 + j, 0)) * p.conv_dim + vch);                  \
        }                                                                                      \
        if (tid < kC) {                                                                        \
            const int tr = tid < fLc ? tid : fLc - 1;                                          \
            ngb = *reinterpret_cast<const float2 *>(p.ws_gb + ((size_t)(ft0 + tr) * p.h_v + hv) * 2); \
            ngc = p.ws_gb[((size_t)(ft0 + fLc - 1) * p.h_v + hv) * 2];                         \
        }                                                                                      \
    }
    // Stage chunk CH (its fetch has landed) into LDS.  XR holds the 4 taps'
    // raw inputs of this thread's v channels.
#define GDN_SCAN_STAGE(CH, XR)                                                                 \
    {                                                                                          \
        const int fLc = min(kC, L - (CH) * kC);                                                \
        _Pragma("unroll") for (int f = 0; f < PF; ++f) {                                       \
            const int idx = tid + 256 * f;                                                     \
            const int t = idx / GPR, g = idx % GPR;                                            \
            const int which = g / (DK / 4), part = (g / (DK / 8)) & 1, cg = g % (DK / 8);     \
            const u32x4 zz = {0u, 0u, 0u, 0u};                                                 \
            const u32x4 v = t < fLc ? pqk[f] : zz;                                             \
            __bf16 *rowdst = (which ? (part ? sKl : sKh) : (part ? sQl : sQh)) + t * RK + 8 * cg; \
            *reinterpret_cast<u32x4 *>(rowdst) = v;                                            \
            if (which) {                                                                       \
                const bf16x8 v8 = __builtin_bit_cast(bf16x8, v);                               \
                __bf16 *tdst = (part ? sKTl : sKTh) + (8 * cg) * RT + t;                       \
                _Pragma("unroll") for (int e = 0; e < 8; ++e) tdst[e * RT] = v8[e];            \
            }                                                                                  \
        }                                                                                      \
        *reinterpret_cast<f32x4 *>(sV + vt * kBV + 4 * vg) = conv4(wv, XR);                    \
        if (tid < kC) {                                                                        \
            const float ng = ngb.x; /* g = 0 past the end: G stays at G_{Lc-1} */              \
            sEG[tid] = expf(ng);                                                               \
            sEGC[tid] = expf(ngc - ng);                                                        \
            sB[tid] = tid < fLc ? ngb.y : 0.0f;                                                \
        }                                                                                      \
        {                                                                                      \
            const bool live = 16 * wave + col < fLc;                                           \
            _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                    \
                cT[s] = frag_select(live, nT[s]);                                              \
                cP[s] = frag_select(live, nP[s]);                                              \
            }                                                                                  \
        }                                                                                      \
    }

    if (nchunks > 0) {
        GDN_SCAN_FETCH(0)
        // chunk 0 may reach into the incoming conv history
        f32x4 x0[4];
        {
            const int tc = vt < L ? vt : L - 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) x0[j] = raw4(p, x, n, s0, tc - 3 + j, vch);
        }
        GDN_SCAN_STAGE(0, x0)
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = s0 + c * kC;
        const int Lc = min(kC, L - c * kC);
        if (c + 1 < nchunks) GDN_SCAN_FETCH(c + 1)

        // X = K S and Y = Q S for rows 16w..16w+15.
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = X;
        {
            const int ro = (16 * wave + col) * RK + 8 * kq;
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const Frag B = frag_at(sSh + col * RK + 32 * s + 8 * kq, sSl + col * RK + 32 * s + 8 * kq);
                X = mma3(frag_at(sKh + ro + 32 * s, sKl + ro + 32 * s), B, X);
                Y = mma3(frag_at(sQh + ro + 32 * s, sQl + ro + 32 * s), B, Y);
            }
        }
        // R = beta (V - e^G X) -> sR (split, transposed);  Y' = e^G Y.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * wave + 4 * kq + e;
            const float eg = sEG[t];
            __bf16 h, l;
            split1(sB[t] * (sV[t * kBV + col] - eg * X[e]), h, l);
            sRh[col * RT + t] = h;
            sRl[col * RT + t] = l;
            Y[e] *= eg;
        }
        __syncthreads();

        // D = T R for rows 16w..16w+15; also diag(e^{G_C-G}) D.
        f32x4 Dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s)
            Dv = mma3(cT[s], frag_at(sRh + col * RT + 32 * s + 8 * kq, sRl + col * RT + 32 * s + 8 * kq), Dv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * wave + 4 * kq + e;
            __bf16 h, l;
            split1(Dv[e], h, l);
            sDh[col * RT + t] = h;
            sDl[col * RT + t] = l;
            split1(Dv[e] * sEGC[t], h, l);
            sEh[col * RT + t] = h;
            sEl[col * RT + t] = l;
        }
        __syncthreads();

        // O = Y' + P D
#pragma unroll
        for (int s = 0; s < 2; ++s)
            Y = mma3(cP[s], frag_at(sDh + col * RT + 32 * s + 8 * kq, sDl + col * RT + 32 * s + 8 * kq), Y);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * wave + 4 * kq + e;
            if (t < Lc) p.ws_o[(size_t)(t0 + t) * p.value_dim + c0 + col] = Y[e];
        }

        // S' = e^{G_C} S + K^T diag(e^{G_C-G}) D
        {
            const float gam = sEG[kC - 1];
            Frag Bs[2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
                Bs[s] = frag_at(sEh + col * RT + 32 * s + 8 * kq, sEl + col * RT + 32 * s + 8 * kq);
#pragma unroll
            for (int u = 0; u < MTW; ++u) {
                const int mt = wave + 4 * u;
                if (mt < MTS) {
                    f32x4 acc = gam * S[u];
                    const int ro = (16 * mt + col) * RT + 8 * kq;
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        acc = mma3(frag_at(sKTh + ro + 32 * s, sKTl + ro + 32 * s), Bs[s], acc);
                    S[u] = acc;
                }
            }
        }
        __syncthreads(); // every read of this chunk's LDS data is done

        // State slice for the next chunk's products, split and transposed.
#pragma unroll
        for (int u = 0; u < MTW; ++u) {
            const int mt = wave + 4 * u;
            if (mt < MTS)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    __bf16 h, l;
                    split1(S[u][e], h, l);
                    sSh[col * RK + 16 * mt + 4 * kq + e] = h;
                    sSl[col * RK + 16 * mt + 4 * kq + e] = l;
                }
        }
        if (c + 1 < nchunks) {
            f32x4 xr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[j] = RawAct<TIn>::to_f32(nxr[j]);
            GDN_SCAN_STAGE(c + 1, xr)
        }
        __syncthreads();
    }
#undef GDN_SCAN_FETCH
#undef GDN_SCAN_STAGE

    // Final state slice.
    float *Sout = p.state_out + ((size_t)n * p.h_v + hv) * DK * p.d_v;
#pragma unroll
    for (int u = 0; u < MTW; ++u) {
        const int mt = wave + 4 * u;
        if (mt < MTS)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Sout[(size_t)(16 * mt + 4 * kq + e) * p.d_v + slice * kBV + col] = S[u][e];
    }
}

// ---------------------------------------------------------------------------
// norm: gated RMSNorm of each (token, value head) row: d_v/4 lanes per row,
// float4 per lane ("oxinfer 0.0.5 src/qwen.rs" gdn_forward, gated norm).
// ---------------------------------------------------------------------------
template <typename TIn, int DV>
__global__ void __launch_bounds__(256)
norm_kernel(const PrefillArgs p, int rows)
{
    constexpr int LPR = DV / 4;   // lanes per row
    constexpr int RPW = 64 / LPR; // rows per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = (blockIdx.x * 4 + wave) * RPW + lane / LPR;
    const int c4 = (lane % LPR) * 4;
    const bool valid = row < rows;
    const int rr = valid ? row : rows - 1;
    const int t = rr / p.h_v, hv = rr % p.h_v;
    const size_t base = (size_t)t * p.value_dim + (size_t)hv * DV + c4;
    const f32x4 o = ld4(p.ws_o + base);
    float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
    ss = group_sum<LPR>(ss);
    const float rn = rsqrtf(ss / DV + p.norm_eps);
    const f32x4 z = load_act4v(static_cast<const TIn *>(p.z), base);
    const f32x4 w = ld4(p.norm_w + c4);
    float4 y;
    y.x = o[0] * rn * w[0] * gatef_(z[0], p.gate);
    y.y = o[1] * rn * w[1] * gatef_(z[1], p.gate);
    y.z = o[2] * rn * w[2] * gatef_(z[2], p.gate);
    y.w = o[3] * rn * w[3] * gatef_(z[3], p.gate);
    if (valid) store_out4(p.out, base, y, p.out_bf16);
}

template <typename TIn>
__global__ void __launch_bounds__(256)
conv_final_kernel(const PrefillArgs p)
{
    const int ch = blockIdx.x * 256 + threadIdx.x;
    const int n = blockIdx.y;
    if (ch >= p.conv_dim) return;
    const int K = p.conv_k, CD = p.conv_dim;
    const int s0 = p.cu[n], L = p.cu[n + 1] - s0;
    const TIn *x = static_cast<const TIn *>(p.qkv);
    float old[3];
    for (int j = 0; j < K - 1; ++j)
        old[j] = p.conv_in ? p.conv_in[((size_t)n * (K - 1) + j) * CD + ch] : 0.0f;
    for (int sl = 0; sl < K - 1; ++sl) {
        const int tau = L - (K - 1) + sl;
        const float v = tau >= 0 ? load_act(x, (size_t)(s0 + tau) * CD + ch) : old[K - 1 + tau];
        p.conv_out[((size_t)n * (K - 1) + sl) * CD + ch] = v;
    }
}

template <typename TIn, int DV>
static hipError_t launch_norm(const PrefillArgs &a, int rows, hipStream_t s)
{
    constexpr int RPB = 4 * (64 / (DV / 4)); // rows per block
    hipLaunchKernelGGL((norm_kernel<TIn, DV>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, s, a,
                       rows);
    return hipGetLastError();
}

template <typename TIn, int DK>
static hipError_t launch_prefill_t(const PrefillArgs &a, int n_seq, int t_total, int max_len,
                                   hipStream_t s)
{
    hipError_t e;
    if (max_len > 0) {
        hipLaunchKernelGGL((qknorm_kernel<TIn, DK>),
                           dim3((max_len + kTileTok - 1) / kTileTok, a.h_k, n_seq), dim3(256), 0,
                           s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((tri_kernel<TIn, DK>), dim3((max_len + kC - 1) / kC, a.h_v, n_seq),
                           dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (n_seq > 0) {
        const int slices = a.d_v / kBV;
        hipLaunchKernelGGL((scan_kernel<TIn, DK>), dim3(n_seq * a.h_v * slices), dim3(256),
                           scan_smem_bytes<DK>(), s, a, slices);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int rows = t_total * a.h_v;
    if (rows > 0) {
        if (a.d_v == 32) e = launch_norm<TIn, 32>(a, rows, s);
        else if (a.d_v == 64) e = launch_norm<TIn, 64>(a, rows, s);
        else e = launch_norm<TIn, 128>(a, rows, s);
        if (e != hipSuccess) return e;
    }
    if (n_seq > 0 && a.conv_k > 1) {
        hipLaunchKernelGGL((conv_final_kernel<TIn>), dim3((a.conv_dim + 255) / 256, n_seq),
                           dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK>
static void set_smem_limits()
{
    hipFuncSetAttribute(reinterpret_cast<const void *>(scan_kernel<bf16_t, DK>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)scan_smem_bytes<DK>());
    hipFuncSetAttribute(reinterpret_cast<const void *>(scan_kernel<float, DK>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)scan_smem_bytes<DK>());
}

hipError_t launch_prefill(const Dims &d, const Params &pr, int n_seq, int t_total, int max_len,
                          const int32_t *cu_dev, const void *qkv, const void *z, const void *a,
                          const void *b, const float *state_in, float *state_out,
                          const float *conv_in, float *conv_out, void *out, void *ws,
                          hipStream_t s)
{
    const WsLayout w = ws_layout(d, t_total);
    char *base = static_cast<char *>(ws);
    PrefillArgs A;
    A.qkv = qkv;
    A.z = z;
    A.a = a;
    A.b = b;
    A.conv_w = pr.conv_w;
    A.a_log = pr.a_log;
    A.dt_bias = pr.dt_bias;
    A.norm_w = pr.norm_w;
    A.cu = cu_dev;
    A.state_in = state_in;
    A.state_out = state_out;
    A.conv_in = conv_in;
    A.conv_out = conv_out;
    A.out = out;
    A.ws_qk = reinterpret_cast<__bf16 *>(base + w.qk);
    A.ws_tp = reinterpret_cast<__bf16 *>(base + w.tp);
    A.ws_gb = reinterpret_cast<float *>(base + w.gb);
    A.ws_o = reinterpret_cast<float *>(base + w.o);
    A.h_k = d.h_k;
    A.h_v = d.h_v;
    A.d_v = d.d_v;
    A.group = d.group;
    A.conv_k = d.conv_k;
    A.conv_dim = d.conv_dim;
    A.value_dim = d.value_dim;
    A.gate = d.gate;
    A.out_bf16 = d.out_bf16;
    A.norm_eps = d.norm_eps;
    A.l2_eps = d.l2_eps;

    static bool limits_set = false;
    if (!limits_set) {
        set_smem_limits<32>();
        set_smem_limits<64>();
        set_smem_limits<128>();
        limits_set = true;
    }
#define GDN_PF_CASE(DK_)                                                                      \
    if (d.d_k == DK_)                                                                         \
        return d.act_bf16 ? launch_prefill_t<bf16_t, DK_>(A, n_seq, t_total, max_len, s)      \
                          : launch_prefill_t<float, DK_>(A, n_seq, t_total, max_len, s);
    GDN_PF_CASE(32)
    GDN_PF_CASE(64)
    GDN_PF_CASE(128)
#undef GDN_PF_CASE
    return hipErrorInvalidValue;
}

} // namespace gdn
