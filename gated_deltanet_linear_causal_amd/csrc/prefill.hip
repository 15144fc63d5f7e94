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
//     S'   = e^{G_C} S + (diag(e^{G_C-G}) K)^T D
// Only differences G_i - G_j with j <= i are exponentiated, so strong
// decay underflows to zero instead of overflowing.
//
// Kernels (one stream, in order):
//   prep  grid (chunk, key head, seq): conv + SiLU, L2 norms, gates and
//         their in-chunk prefix sum, K K^T and Q K^T on MFMA, A, the
//         triangular inverse T in fp32, P.  Writes q^, k^, conv(v), T, P,
//         G, b to the workspace.  Fully parallel.
//   scan  grid (seq, value head, 16-column slice of d_v): the chain of
//         chunk states, sequential over the chunks of one sequence; the
//         state slice lives in registers.  Writes the pre-norm readout O.
//   norm  grid (token, value head): gated RMSNorm + output gate -> out;
//         plus the final conv history.
//
// Contractions run on v_mfma_f32_16x16x32_bf16 with each fp32 operand split
// into bf16 hi + lo and three products (hi.hi + hi.lo + lo.hi, fp32
// accumulate): plain bf16 operands are far outside the parity tolerance,
// the split form is within it.

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kC = 64;      // tokens per chunk
constexpr int kBV = 16;     // d_v columns per scan workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Frag {
    bf16x8 hi, lo;
};

// fp32 -> (hi, lo) bf16 pair with hi + lo = v to ~16 significant bits.
__device__ __forceinline__ Frag split8(const float (&v)[8])
{
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(v[e]);
        f.hi[e] = h;
        f.lo[e] = static_cast<__bf16>(v[e] - static_cast<float>(h));
    }
    return f;
}

__device__ __forceinline__ Frag split8(float4 a, float4 b)
{
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return split8(v);
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

__device__ __forceinline__ Frag lds_frag(const float *row8)
{
    const float4 a = *reinterpret_cast<const float4 *>(row8);
    const float4 b = *reinterpret_cast<const float4 *>(row8 + 4);
    return split8(a, b);
}

// ---------------------------------------------------------------------------
// Workspace layout (all fp32, each section 256-byte aligned):
//   qk [T][H_k][2][d_k]   q^ then k^ of each key head
//   v  [T][H_v*d_v]       conv(v)
//   tp [T][H_v][2][C]     row of T, then row of P, for the token's chunk
//   gb [T][H_v][2]        G (in-chunk cumulative log decay), beta
//   o  [T][H_v*d_v]       pre-norm readout
// ---------------------------------------------------------------------------
struct WsLayout {
    size_t qk, v, tp, gb, o, total;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static WsLayout ws_layout(const Dims &d, int t_total)
{
    WsLayout w;
    const size_t T = (size_t)t_total;
    size_t off = 0;
    w.qk = off;
    off = align256(off + T * d.h_k * 2 * d.d_k * sizeof(float));
    w.v = off;
    off = align256(off + T * d.value_dim * sizeof(float));
    w.tp = off;
    off = align256(off + T * d.h_v * 2 * kC * sizeof(float));
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
    float *ws_qk, *ws_v, *ws_tp, *ws_gb, *ws_o;
    int h_k, h_v, d_v, group, conv_k, conv_dim, value_dim;
    int gate, out_bf16;
    float norm_eps, l2_eps;
};

// ---------------------------------------------------------------------------
// prep: one workgroup per (chunk, key head, sequence), 256 threads.
// ---------------------------------------------------------------------------
template <typename TIn, int DK>
__global__ void __launch_bounds__(256)
prep_kernel(const PrefillArgs p)
{
    constexpr int LDK = DK + 4;   // padded row of q^/k^ in LDS
    constexpr int LC = kC + 4;    // padded row of the C x C matrices
    const int c = blockIdx.x, hk = blockIdx.y, n = blockIdx.z;
    const int s0 = p.cu[n];
    const int L = p.cu[n + 1] - s0;
    if (c * kC >= L) return;
    const int t0 = s0 + c * kC;
    const int Lc = min(kC, L - c * kC);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = p.conv_k, CD = p.conv_dim;
    const TIn *x = static_cast<const TIn *>(p.qkv);

    extern __shared__ float smem[];
    float *sQ = smem;                 // [C][LDK]   later reused as sA / sT
    float *sK = sQ + kC * LDK;        // [C][LDK]
    float *sKK = sK + kC * LDK;       // [C][LC]
    float *sQKm = sKK + kC * LC;      // [C][LC]
    float *sG = sQKm + kC * LC;       // [C]
    float *sB = sG + kC;              // [C]
    float *sA = sQ;                   // [C][LC], valid once q^/k^ are consumed

    // --- conv + SiLU of the chunk, history from the previous chunk's raw
    //     inputs or from conv_in ---------------------------------------
    auto conv_channel = [&](int ch, auto &&emit) {
        float w[4];
        for (int j = 0; j < K; ++j) w[j] = p.conv_w[(size_t)ch * K + j];
        float win[3];
        for (int j = 0; j < K - 1; ++j) {
            const int tau = t0 - (K - 1) + j;
            if (tau >= s0)
                win[j] = load_act(x, (size_t)tau * CD + ch);
            else
                win[j] = p.conv_in ? p.conv_in[((size_t)n * (K - 1) + (K - 1 + tau - s0)) * CD + ch]
                                   : 0.0f;
        }
        for (int t = 0; t < Lc; ++t) {
            const float cur = load_act(x, (size_t)(t0 + t) * CD + ch);
            float acc = 0.0f;
            for (int j = 0; j < K - 1; ++j) acc = fmaf(w[j], win[j], acc);
            acc = fmaf(w[K - 1], cur, acc);
            emit(t, siluf_(acc));
            for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
            if (K > 1) win[K - 2] = cur;
        }
    };
    for (int l = tid; l < 2 * DK; l += 256) {
        const bool isq = l < DK;
        const int ch = isq ? hk * DK + l : p.h_k * DK + hk * DK + (l - DK);
        float *dst = (isq ? sQ : sK) + (isq ? l : l - DK);
        conv_channel(ch, [&](int t, float v) { dst[t * LDK] = v; });
        for (int t = Lc; t < kC; ++t) dst[t * LDK] = 0.0f;
    }
    {
        const int vbase = 2 * p.h_k * DK + hk * p.group * p.d_v;
        const int nv = p.group * p.d_v;
        for (int l = tid; l < nv; l += 256) {
            float *dst = p.ws_v + (size_t)t0 * p.value_dim + (size_t)hk * nv + l;
            conv_channel(vbase + l, [&](int t, float v) { dst[(size_t)t * p.value_dim] = v; });
        }
    }
    __syncthreads();

    // --- L2 norms (rows past Lc are zero and stay zero) -----------------
    for (int r = wave; r < 2 * kC; r += 4) {
        float *row = (r < kC ? sQ : sK) + (r % kC) * LDK;
        float ss = 0.0f;
        for (int i = lane; i < DK; i += 64) ss = fmaf(row[i], row[i], ss);
        ss = group_sum<64>(ss);
        const float sc = rsqrtf(ss + p.l2_eps) * (r < kC ? rsqrtf((float)DK) : 1.0f);
        for (int i = lane; i < DK; i += 64) row[i] *= sc;
    }
    __syncthreads();

    // q^, k^ to the workspace for the scan.
    for (int idx = tid; idx < Lc * 2 * (DK / 4); idx += 256) {
        const int t = idx / (2 * (DK / 4));
        const int rem = idx % (2 * (DK / 4));
        const int which = rem / (DK / 4), q4 = rem % (DK / 4);
        const float4 v = *reinterpret_cast<const float4 *>((which ? sK : sQ) + t * LDK + 4 * q4);
        *reinterpret_cast<float4 *>(p.ws_qk + (((size_t)(t0 + t) * p.h_k + hk) * 2 + which) * DK +
                                    4 * q4) = v;
    }

    // --- K K^T and Q K^T, lower-triangular 16x16 tiles -------------------
    // 20 tiles: (which, mt, nt) with nt <= mt; wave w takes every 4th.
    for (int tile = wave; tile < 20; tile += 4) {
        const int which = tile / 10;  // 0: K K^T, 1: Q K^T
        int r = tile % 10, mt = 0;
        while (r > mt) { r -= mt + 1; ++mt; }
        const int nt = r;
        const float *Arow = (which ? sQ : sK) + (16 * mt + (lane & 15)) * LDK + 8 * (lane >> 4);
        const float *Brow = sK + (16 * nt + (lane & 15)) * LDK + 8 * (lane >> 4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) acc = mma3(lds_frag(Arow + 32 * s), lds_frag(Brow + 32 * s), acc);
        float *D = (which ? sQKm : sKK) + (16 * mt + 4 * (lane >> 4)) * LC + 16 * nt + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) D[e * LC] = acc[e];
    }
    __syncthreads();

    // --- per value head of the group: gates, A, T = (I+A)^-1, P ----------
    const TIn *pa = static_cast<const TIn *>(p.a);
    const TIn *pb = static_cast<const TIn *>(p.b);
    for (int hl = 0; hl < p.group; ++hl) {
        const int hv = hk * p.group + hl;
        if (wave == 0) {
            float beta = 0.0f, g = 0.0f;
            if (lane < Lc) {
                const size_t gi = (size_t)(t0 + lane) * p.h_v + hv;
                beta = sigmoidf_(load_act(pb, gi));
                g = -expf(p.a_log[hv]) * softplusf_(load_act(pa, gi) + p.dt_bias[hv]);
            }
            // inclusive prefix sum over the chunk
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float u = __shfl_up(g, off, 64);
                if (lane >= off) g += u;
            }
            sG[lane] = g;
            sB[lane] = beta;
            if (lane < Lc) {
                float *gb = p.ws_gb + ((size_t)(t0 + lane) * p.h_v + hv) * 2;
                gb[0] = g;
                gb[1] = beta;
            }
        }
        __syncthreads();
        // A (strict lower) into sA; P (lower incl. diagonal) to the workspace.
        for (int idx = tid; idx < kC * (kC / 4); idx += 256) {
            const int i = idx / (kC / 4), j0 = 4 * (idx % (kC / 4));
            const float Gi = sG[i], bi = sB[i];
            float av[4], pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + e;
                const float m = j <= i ? expf(Gi - sG[j]) : 0.0f;
                av[e] = j < i ? bi * m * sKK[i * LC + j] : 0.0f;
                pv[e] = j <= i ? m * sQKm[i * LC + j] : 0.0f;
            }
            *reinterpret_cast<float4 *>(sA + i * LC + j0) = make_float4(av[0], av[1], av[2], av[3]);
            if (i < Lc)
                *reinterpret_cast<float4 *>(p.ws_tp + (((size_t)(t0 + i) * p.h_v + hv) * 2 + 1) * kC + j0) =
                    make_float4(pv[0], pv[1], pv[2], pv[3]);
        }
        __syncthreads();
        // Forward substitution, fp32: thread (column j, quarter q) keeps rows
        // 16q .. 16q+15 of column j of T in registers.
        {
            const int j = tid >> 2, q = tid & 3;
            float r[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) r[s] = (16 * q + s == j) ? 1.0f : 0.0f;
#pragma unroll
            for (int i = 1; i < kC; ++i) {
                const float *Ai = sA + i * LC + 16 * q;
                float part = 0.0f;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const float4 av = *reinterpret_cast<const float4 *>(Ai + 4 * s4);
                    part = fmaf(av.x, r[4 * s4 + 0], part);
                    part = fmaf(av.y, r[4 * s4 + 1], part);
                    part = fmaf(av.z, r[4 * s4 + 2], part);
                    part = fmaf(av.w, r[4 * s4 + 3], part);
                }
                part += __shfl_xor(part, 1, 64);
                part += __shfl_xor(part, 2, 64);
                if (q == i / 16 && i > j) r[i % 16] = -part;
            }
            __syncthreads(); // every thread is done reading A
#pragma unroll
            for (int s = 0; s < 16; ++s) sA[(16 * q + s) * LC + j] = r[s];
        }
        __syncthreads();
        for (int idx = tid; idx < Lc * (kC / 4); idx += 256) {
            const int i = idx / (kC / 4), j0 = 4 * (idx % (kC / 4));
            *reinterpret_cast<float4 *>(p.ws_tp + (((size_t)(t0 + i) * p.h_v + hv) * 2 + 0) * kC + j0) =
                *reinterpret_cast<const float4 *>(sA + i * LC + j0);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, value head, 16-column slice), 256
// threads = 4 waves.  Wave w owns output rows 16w..16w+15 of each chunk and
// the state rows of M-tiles w, w+4, ... (16 rows each).
// ---------------------------------------------------------------------------
template <int DK>
__global__ void __launch_bounds__(256)
scan_kernel(const PrefillArgs p, int slices)
{
    constexpr int LDK = DK + 4;
    constexpr int LT = kC + 4;    // padded row of the transposed C-vectors
    constexpr int MTS = DK / 16;  // state M-tiles
    constexpr int MTW = (MTS + 3) / 4; // state M-tiles per wave (max)
    constexpr int PF = (kC * DK / 4) / 256; // float4 prefetch per thread per matrix

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

    extern __shared__ float smem[];
    float *sK = smem;              // [C][LDK]
    float *sQ = sK + kC * LDK;     // [C][LDK]
    float *sST = sQ + kC * LDK;    // [16][LDK]  state slice, transposed
    float *sRT = sST + kBV * LDK;  // [16][LT]   R, transposed
    float *sDT = sRT + kBV * LT;   // [16][LT]   D, transposed
    float *sV = sDT + kBV * LT;    // [C][16]
    float *sG = sV + kC * kBV;     // [C]
    float *sB = sG + kC;           // [C]

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
                for (int e = 0; e < 4; ++e) sST[col * LDK + 16 * mt + 4 * kq + e] = S[u][e];
        }
    }

    // Chunk inputs staged through registers one chunk ahead.
    constexpr int PV = kC * kBV / 256;  // v values per thread per chunk
    float4 pk[PF], pq[PF];
    float pv_[PV], pg_ = 0.0f, pb_ = 0.0f;
    auto fetch = [&](int c) {
        const int t0 = s0 + c * kC;
        const int Lc = min(kC, L - c * kC);
#pragma unroll
        for (int f = 0; f < PF; ++f) {
            const int idx = tid + 256 * f;
            const int t = idx / (DK / 4), i4 = idx % (DK / 4);
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            const float *base = p.ws_qk + (((size_t)(t0 + t) * p.h_k + hk) * 2) * DK + 4 * i4;
            pq[f] = t < Lc ? *reinterpret_cast<const float4 *>(base) : z;
            pk[f] = t < Lc ? *reinterpret_cast<const float4 *>(base + DK) : z;
        }
#pragma unroll
        for (int f = 0; f < PV; ++f) {
            const int idx = tid + 256 * f;
            const int t = idx / kBV, cc = idx % kBV;
            pv_[f] = t < Lc ? p.ws_v[(size_t)(t0 + t) * p.value_dim + c0 + cc] : 0.0f;
        }
        if (tid < kC) {
            if (tid < Lc) {
                const float *gb = p.ws_gb + ((size_t)(t0 + tid) * p.h_v + hv) * 2;
                pg_ = gb[0];
                pb_ = gb[1];
            } else {
                pg_ = p.ws_gb[((size_t)(t0 + Lc - 1) * p.h_v + hv) * 2]; // g = 0 past the end
                pb_ = 0.0f;
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int f = 0; f < PF; ++f) {
            const int idx = tid + 256 * f;
            const int t = idx / (DK / 4), i4 = idx % (DK / 4);
            *reinterpret_cast<float4 *>(sQ + t * LDK + 4 * i4) = pq[f];
            *reinterpret_cast<float4 *>(sK + t * LDK + 4 * i4) = pk[f];
        }
#pragma unroll
        for (int f = 0; f < PV; ++f) sV[tid + 256 * f] = pv_[f];
        if (tid < kC) {
            sG[tid] = pg_;
            sB[tid] = pb_;
        }
    };

    if (nchunks > 0) {
        fetch(0);
        stage();
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = s0 + c * kC;
        const int Lc = min(kC, L - c * kC);
        // T and P rows of this wave's output tile (A operands), issued early.
        const int row = 16 * wave + col;
        float Tf[2][8], Pf[2][8];
        {
            const float *tp = p.ws_tp + (((size_t)(t0 + row) * p.h_v + hv) * 2) * kC;
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int e4 = 0; e4 < 2; ++e4) {
                    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                    const float4 tv = row < Lc ? *reinterpret_cast<const float4 *>(tp + 32 * s + 8 * kq + 4 * e4) : z;
                    const float4 pv = row < Lc ? *reinterpret_cast<const float4 *>(tp + kC + 32 * s + 8 * kq + 4 * e4) : z;
                    Tf[s][4 * e4 + 0] = tv.x; Tf[s][4 * e4 + 1] = tv.y;
                    Tf[s][4 * e4 + 2] = tv.z; Tf[s][4 * e4 + 3] = tv.w;
                    Pf[s][4 * e4 + 0] = pv.x; Pf[s][4 * e4 + 1] = pv.y;
                    Pf[s][4 * e4 + 2] = pv.z; Pf[s][4 * e4 + 3] = pv.w;
                }
        }
        if (c + 1 < nchunks) fetch(c + 1);

        // X = K S and Y = Q S for rows 16w..16w+15.
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = X;
        {
            const float *Ka = sK + (16 * wave + col) * LDK + 8 * kq;
            const float *Qa = sQ + (16 * wave + col) * LDK + 8 * kq;
            const float *Bs = sST + col * LDK + 8 * kq;
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const Frag B = lds_frag(Bs + 32 * s);
                X = mma3(lds_frag(Ka + 32 * s), B, X);
                Y = mma3(lds_frag(Qa + 32 * s), B, Y);
            }
        }
        const float GC = sG[kC - 1];
        // R = beta (V - e^G X) -> sRT;  Y' = e^G Y stays in registers.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * wave + 4 * kq + e;
            const float eg = expf(sG[t]);
            sRT[col * LT + t] = sB[t] * (sV[t * kBV + col] - eg * X[e]);
            Y[e] *= eg;
        }
        __syncthreads();

        // D = T R for rows 16w..16w+15.
        f32x4 Dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s)
            Dv = mma3(split8(Tf[s]), lds_frag(sRT + col * LT + 32 * s + 8 * kq), Dv);
#pragma unroll
        for (int e = 0; e < 4; ++e) sDT[col * LT + 16 * wave + 4 * kq + e] = Dv[e];
        __syncthreads();

        // O = Y' + P D
#pragma unroll
        for (int s = 0; s < 2; ++s)
            Y = mma3(split8(Pf[s]), lds_frag(sDT + col * LT + 32 * s + 8 * kq), Y);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * wave + 4 * kq + e;
            if (t < Lc) p.ws_o[(size_t)(t0 + t) * p.value_dim + c0 + col] = Y[e];
        }

        // S' = e^{G_C} S + (diag(e^{G_C - G}) K)^T D
        const float gam = expf(GC);
#pragma unroll
        for (int u = 0; u < MTW; ++u) {
            const int mt = wave + 4 * u;
            if (mt >= MTS) break;
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = gam * S[u][e];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                float av[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = 32 * s + 8 * kq + e;
                    av[e] = expf(GC - sG[t]) * sK[t * LDK + 16 * mt + col];
                }
                acc = mma3(split8(av), lds_frag(sDT + col * LT + 32 * s + 8 * kq), acc);
            }
            S[u] = acc;
        }
        __syncthreads(); // all reads of sK, sQ, sST, sDT for this chunk done
#pragma unroll
        for (int u = 0; u < MTW; ++u) {
            const int mt = wave + 4 * u;
            if (mt >= MTS) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) sST[col * LDK + 16 * mt + 4 * kq + e] = S[u][e];
        }
        if (c + 1 < nchunks) stage();
        __syncthreads();
    }

    // Final state slice.
    float *Sout = p.state_out + ((size_t)n * p.h_v + hv) * DK * p.d_v;
#pragma unroll
    for (int u = 0; u < MTW; ++u) {
        const int mt = wave + 4 * u;
        if (mt >= MTS) break;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Sout[(size_t)(16 * mt + 4 * kq + e) * p.d_v + slice * kBV + col] = S[u][e];
    }
}

// ---------------------------------------------------------------------------
// norm: gated RMSNorm of each (token, value head) row; one wave per row.
// conv_final: each sequence's last K-1 raw inputs become its new history.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ void __launch_bounds__(256)
norm_kernel(const PrefillArgs p, int rows)
{
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const int t = r / p.h_v, hv = r % p.h_v;
    const int DV = p.d_v;
    const size_t base = (size_t)t * p.value_dim + (size_t)hv * DV;
    float o[2], ss = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = lane + 64 * u;
        o[u] = j < DV ? p.ws_o[base + j] : 0.0f;
        ss = fmaf(o[u], o[u], ss);
    }
    ss = group_sum<64>(ss);
    const float rn = rsqrtf(ss / DV + p.norm_eps);
    const TIn *z = static_cast<const TIn *>(p.z);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = lane + 64 * u;
        if (j < DV) {
            const float y = o[u] * rn * p.norm_w[j] * gatef_(load_act(z, base + j), p.gate);
            store_out1(p.out, base + j, y, p.out_bf16);
        }
    }
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

template <typename TIn, int DK>
static hipError_t launch_prefill_t(const PrefillArgs &a, int n_seq, int t_total, int max_len,
                                   hipStream_t s)
{
    const int max_chunks = (max_len + kC - 1) / kC;
    if (max_chunks > 0) {
        const size_t sh = sizeof(float) * (2 * kC * (DK + 4) + 2 * kC * (kC + 4) + 2 * kC);
        hipLaunchKernelGGL((prep_kernel<TIn, DK>), dim3(max_chunks, a.h_k, n_seq), dim3(256), sh,
                           s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (n_seq > 0) {
        const int slices = a.d_v / kBV;
        const size_t sh = sizeof(float) * (2 * kC * (DK + 4) + kBV * (DK + 4) +
                                           2 * kBV * (kC + 4) + kC * kBV + 2 * kC);
        hipLaunchKernelGGL((scan_kernel<DK>), dim3(n_seq * a.h_v * slices), dim3(256), sh, s, a,
                           slices);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int rows = t_total * a.h_v;
    if (rows > 0) {
        hipLaunchKernelGGL((norm_kernel<TIn>), dim3((rows + 3) / 4), dim3(256), 0, s, a, rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (n_seq > 0 && a.conv_k > 1) {
        hipLaunchKernelGGL((conv_final_kernel<TIn>), dim3((a.conv_dim + 255) / 256, n_seq),
                           dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK>
static void set_smem_limits()
{
    const int big = (int)sizeof(float) * (2 * kC * (DK + 4) + 2 * kC * (kC + 4) + 2 * kC);
    hipFuncSetAttribute(reinterpret_cast<const void *>(prep_kernel<bf16_t, DK>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, big);
    hipFuncSetAttribute(reinterpret_cast<const void *>(prep_kernel<float, DK>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, big);
    const int sc = (int)sizeof(float) * (2 * kC * (DK + 4) + kBV * (DK + 4) + 2 * kBV * (kC + 4) +
                                         kC * kBV + 2 * kC);
    hipFuncSetAttribute(reinterpret_cast<const void *>(scan_kernel<DK>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, sc);
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
    A.ws_qk = reinterpret_cast<float *>(base + w.qk);
    A.ws_v = reinterpret_cast<float *>(base + w.v);
    A.ws_tp = reinterpret_cast<float *>(base + w.tp);
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
