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
//   qknorm  grid (chunk, key head, seq): causal conv + SiLU and L2 norm of
//           q and k, a group of lanes per token row; writes q^, k^ rows split
//           into bf16 hi + lo (ready-made matrix-core operands) and a
//           transposed, bank-swizzled copy of the chunk's k^.
//   tri     grid (chunk, value head, seq): gates and their in-chunk prefix
//           sum, K K^T and Q K^T on MFMA, A, the blocked fp32 triangular
//           inverse T, P; writes T and P rows split into bf16 hi + lo.
//   scan    grid (seq, value head, 16-column slice of d_v), 8 waves: four
//           consumer waves run the chain of chunk states (state slice in
//           registers, every matrix operand pre-split); four producer waves
//           stream the next chunk's operands straight into LDS
//           (global_load_lds, no register staging), convolve the slice's v
//           channels and stage the gates.  Writes the pre-norm readout O.
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
// Workspace layout (sections 256-byte aligned; head-major so that a chunk's
// data of one head is contiguous):
//   qk [H_k][T][2: q^,k^][2: hi,lo][d_k] bf16
//   kT [T + C*N slots][H_k*2*d_k] bf16: chunk (n, c) owns the 64 slot rows
//       from s0 + C*n + C*c, holding per key head [hi,lo][d_k][C] (k^
//       transposed); the 16-byte groups of a row are permuted by
//       (group ^ (row & 7)) so that matrix-operand reads spread over banks
//   tp [H_v][T][2: T,P][2: hi,lo][C]    bf16 (row of the token's chunk)
//   gb [H_v][T][2]                      fp32 (G in-chunk cumulative, beta)
//   o  [H_v][T][d_v]                    fp32 pre-norm readout
// ---------------------------------------------------------------------------
struct WsLayout {
    size_t qk, kt, tp, gb, o, total;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static WsLayout ws_layout(const Dims &d, int n_seq, int t_total)
{
    WsLayout w;
    const size_t T = (size_t)t_total;
    size_t off = 0;
    w.qk = off;
    off = align256(off + T * d.h_k * 4 * d.d_k * 2);
    w.kt = off;
    off = align256(off + (T + (size_t)kC * n_seq) * d.h_k * 2 * d.d_k * 2);
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
    return t_total > 0 ? ws_layout(d, n_seq, t_total).total : 0;
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
    __bf16 *ws_qk, *ws_kt, *ws_tp;
    float *ws_gb, *ws_o;
    int t_total;
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
// qknorm: one workgroup per (chunk, key head, sequence).  Each token row of
// the key head (q then k, 2*d_k channels) is handled by d_k/2 lanes of 4
// channels; each L2 norm is a reduction over d_k/4 lanes.  The k^ rows are
// also gathered in LDS and written out transposed for the scan.
// ---------------------------------------------------------------------------
template <typename TIn, int DK>
__global__ void __launch_bounds__(256)
qknorm_kernel(const PrefillArgs p)
{
    constexpr int LPT = DK / 2;              // lanes per token row
    constexpr int TPI = 64 / LPT;            // token rows per wave pass
    constexpr int TPL = kC / (4 * TPI);      // consecutive tokens per lane
    constexpr int WIN = TPL + 3;             // raw rows a lane reads
    constexpr int RT = kC + 8;               // LDS row stride of the transpose
    const int c = blockIdx.x, hk = blockIdx.y, n = blockIdx.z;
    const int s0 = p.cu[n], L = p.cu[n + 1] - s0;
    if (c * kC >= L) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane / LPT, ll = lane % LPT;
    const bool isk = ll >= DK / 4;
    const int c4 = (isk ? ll - DK / 4 : ll) * 4;
    const int ch = (isk ? p.h_k * DK : 0) + hk * DK + c4;
    const TIn *x = static_cast<const TIn *>(p.qkv);
    __shared__ __attribute__((aligned(16))) __bf16 sKt[2][DK][RT];
    __bf16 *qkrow0 = p.ws_qk + ((size_t)hk * p.t_total + s0) * 4 * DK;
    const int r0 = kC / 4 * wave + TPL * sub; // first chunk row of this lane
    const int tl0 = c * kC + r0;              // its position in the sequence

    // Every raw input the lane needs, loaded at once (positions clamped into
    // the sequence; positions before its start are replaced below).
    typedef typename RawAct<TIn>::type RawT;
    RawT raw[WIN];
#pragma unroll
    for (int j = 0; j < WIN; ++j) {
        const int tau = min(max(tl0 - 3 + j, 0), L - 1);
        raw[j] = RawAct<TIn>::load(x, (size_t)(s0 + tau) * p.conv_dim + ch);
    }
    float w[4][4];
    load_taps4(p, ch, w);
    const float extra = isk ? 1.0f : rsqrtf((float)DK);
    f32x4 xv[WIN];
#pragma unroll
    for (int j = 0; j < WIN; ++j) xv[j] = RawAct<TIn>::to_f32(raw[j]);
    if (tl0 < 3) { // the first rows of a sequence reach into its history
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (tl0 - 3 + j < 0) xv[j] = raw4(p, x, n, s0, tl0 - 3 + j, ch);
    }

#pragma unroll
    for (int k = 0; k < TPL; ++k) {
        const int r = r0 + k, tl = tl0 + k;
        const bool valid = tl < L;
        const f32x4 xr[4] = {xv[k], xv[k + 1], xv[k + 2], xv[k + 3]};
        const f32x4 cv = conv4(w, xr);
        float ss = cv[0] * cv[0] + cv[1] * cv[1] + cv[2] * cv[2] + cv[3] * cv[3];
        ss = group_sum<DK / 4>(ss);
        const float sc = valid ? rsqrtf(ss + p.l2_eps) * extra : 0.0f;
        __bf16 h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split1(cv[e] * sc, h[e], l[e]);
        if (valid) {
            __bf16 *dst = qkrow0 + (size_t)tl * 4 * DK + (isk ? 2 * DK : 0) + c4;
            *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
            *reinterpret_cast<uint2 *>(dst + DK) = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
        }
        if (isk) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sKt[0][c4 + e][r] = h[e];
                sKt[1][c4 + e][r] = l[e];
            }
        }
    }
    __syncthreads();
    // chunk block of k^ transposed: [hi,lo][d_k][C], 16-byte groups of row i
    // stored at group (g ^ (i & 7)).
    __bf16 *kt = p.ws_kt + (size_t)(s0 + kC * n + kC * c) * p.h_k * 2 * DK + (size_t)hk * 2 * DK * kC;
    for (int idx = tid; idx < 2 * DK * 8; idx += 256) {
        const int part = idx / (DK * 8), rem = idx % (DK * 8);
        const int i = rem >> 3, g = rem & 7;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(&sKt[part][i][8 * g]);
        *reinterpret_cast<u32x4 *>(kt + (size_t)part * DK * kC + (size_t)i * kC + 8 * (g ^ (i & 7))) = v;
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

    // Issue every global load first: the gate inputs (wave 0) and, per
    // wave w (row block w), the pre-split fragments of Q^ and K^ rows
    // 16w.. and of K^ rows 16nt.. for the column blocks nt <= w.
    const TIn *pa = static_cast<const TIn *>(p.a);
    const TIn *pb = static_cast<const TIn *>(p.b);
    float a_raw = 0.0f, b_raw = 0.0f;
    if (wave == 0 && lane < Lc) {
        const size_t gi = (size_t)(t0 + lane) * p.h_v + hv;
        a_raw = load_act(pa, gi);
        b_raw = load_act(pb, gi);
    }
    const __bf16 *qk0 = p.ws_qk + ((size_t)hk * p.t_total + t0) * 4 * DK;
    constexpr int KS = DK / 32;
    Frag fq[KS], fk[4][KS];
    {
        const int ra = 16 * wave + col;
        const __bf16 *pr = qk0 + (size_t)(ra < Lc ? ra : 0) * 4 * DK + 8 * kq;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            fq[s] = frag_at(pr + 32 * s, pr + DK + 32 * s);
            fk[3][s] = frag_at(pr + 2 * DK + 32 * s, pr + 3 * DK + 32 * s);
        }
#pragma unroll
        for (int nt = 0; nt < 3; ++nt) {
            if (nt < wave) {
                const int rb = 16 * nt + col;
                const __bf16 *pk = qk0 + (size_t)(rb < Lc ? rb : 0) * 4 * DK + 2 * DK + 8 * kq;
#pragma unroll
                for (int s = 0; s < KS; ++s) fk[nt][s] = frag_at(pk + 32 * s, pk + DK + 32 * s);
            }
        }
    }
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
            beta = sigmoidf_(b_raw);
            g = -expf(p.a_log[hv]) * softplusf_(a_raw + p.dt_bias[hv]);
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float u = __shfl_up(g, off, 64);
            if (lane >= off) g += u;
        }
        sG[lane] = g;
        sB[lane] = beta;
        if (lane < Lc)
            *reinterpret_cast<float2 *>(p.ws_gb + ((size_t)hv * p.t_total + t0 + lane) * 2) =
                make_float2(g, beta);
    }
    __syncthreads();

    // K K^T -> A and Q K^T -> P for row block mt = w, column blocks nt <= w.
    {
        const int mt = wave;
        const bool arow = 16 * mt + col < Lc;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            if (nt <= mt) {
                const bool brow = 16 * nt + col < Lc;
                f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = akk;
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const Frag B = frag_select(brow, nt == mt ? fk[3][s] : fk[nt < 3 ? nt : 0][s]);
                    akk = mma3(frag_select(arow, fk[3][s]), B, akk);
                    aqk = mma3(frag_select(arow, fq[s]), B, aqk);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * mt + 4 * kq + e, j = 16 * nt + col;
                    const float m = j <= i ? expf(sG[i] - sG[j]) : 0.0f;
                    sA[i * LC + j] = j < i ? sB[i] * m * akk[e] : 0.0f;
                    sP[i * LC + j] = m * aqk[e];
                }
            }
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
        __bf16 *dst = p.ws_tp + ((size_t)hv * p.t_total + t0 + i) * 4 * kC + which * 2 * kC + 8 * g;
        *reinterpret_cast<bf16x8 *>(dst) = f.hi;
        *reinterpret_cast<bf16x8 *>(dst + kC) = f.lo;
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, value head, 16-column slice), 512
// threads.  Waves 0-3 (consumers): wave w owns output rows 16w..16w+15 of
// each chunk and the state rows of M-tiles w, w+4, ...; it loads the matrix
// operands that only it uses (its q^/k^ rows, its T and P rows) straight
// into registers one chunk ahead.  Waves 4-7 (producers): while the
// consumers compute chunk c they stream chunk c+1's transposed k^ block
// into LDS (global_load_lds, double buffered), convolve the slice's v
// channels and stage the gates.  Per chunk:
//   consumers  operand loads(c+1); X, Y, R | D | O, S update, S^T split
//   producers  k^T(c+1), v/gates loads(c+1) | sV, b, e^G (c+1)
//              | e^{G_C-G}(c+1), wait
// with a workgroup barrier at each '|' and one at the end.
// ---------------------------------------------------------------------------
template <int DK> struct ScanLds {
    static constexpr int KT_BYTES = 2 * DK * kC * 2; // one transposed k^ block
    static constexpr int RK = DK + 8;        // bf16 stride of S^T rows
    static constexpr int RT = kC + 8;        // bf16 stride of R, D, E rows
    static constexpr int o_kt = 0;           // two buffers
    static constexpr int o_s = o_kt + 2 * KT_BYTES;    // [hi,lo][16][RK]
    static constexpr int o_r = o_s + 2 * kBV * RK * 2; // [hi,lo][16][RT]
    static constexpr int o_d = o_r + 2 * kBV * RT * 2;
    static constexpr int o_e = o_d + 2 * kBV * RT * 2;
    static constexpr int o_v = o_e + 2 * kBV * RT * 2; // fp32 [C][16]
    static constexpr int o_g = o_v + kC * kBV * 4;     // fp32 e^G, e^{G_C-G}, beta
    static constexpr int total = o_g + 3 * kC * 4;
};
template <int DK> constexpr size_t scan_smem_bytes() { return ScanLds<DK>::total; }

// 16 bytes per lane, global -> LDS without register staging: lane l's
// bytes land at lds_base + 16 l.
__device__ __forceinline__ void lds_load16(const void *g, void *lds_base)
{
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void *)g,
        (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also
// waits for every outstanding global-to-LDS load of the calling wave (they
// write LDS), which would stall the producers' prefetch at every barrier;
// here each wave only drains its own LDS reads/writes, and the producers
// drain their global-to-LDS loads explicitly before the barrier that
// publishes them.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename TIn, int DK>
__global__ void __launch_bounds__(512)
scan_kernel(const PrefillArgs p, int slices)
{
    using LY = ScanLds<DK>;
    constexpr int RK = LY::RK, RT = LY::RT;
    constexpr int KS = DK / 32;        // k-steps over d_k
    constexpr int MTS = DK / 16;       // state M-tiles
    constexpr int MTW = (MTS + 3) / 4; // per consumer wave

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
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: role branches stay wave-uniform, so each
    // role's waits (e.g. the producers' drain of LDS-direct loads) stay on
    // that role's path
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave >= 4;
    const int cw = wave & 3; // consumer or producer wave index
    const int col = lane & 15, kq = lane >> 4;
    const int s0 = p.cu[n];
    const int L = p.cu[n + 1] - s0;
    const int nchunks = (L + kC - 1) / kC;
    const int c0 = hv * p.d_v + slice * kBV; // first value column
    const TIn *x = static_cast<const TIn *>(p.qkv);

    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *sKT = smem + LY::o_kt;
    __bf16 *sSh = reinterpret_cast<__bf16 *>(smem + LY::o_s), *sSl = sSh + kBV * RK;
    __bf16 *sRh = reinterpret_cast<__bf16 *>(smem + LY::o_r), *sRl = sRh + kBV * RT;
    __bf16 *sDh = reinterpret_cast<__bf16 *>(smem + LY::o_d), *sDl = sDh + kBV * RT;
    __bf16 *sEh = reinterpret_cast<__bf16 *>(smem + LY::o_e), *sEl = sEh + kBV * RT;
    float *sV = reinterpret_cast<float *>(smem + LY::o_v);
    float *sEG = reinterpret_cast<float *>(smem + LY::o_g), *sEGC = sEG + kC, *sB = sEGC + kC;

    const __bf16 *qk_head = p.ws_qk + (size_t)hk * p.t_total * 4 * DK;
    const __bf16 *kt_seq = p.ws_kt + (size_t)(s0 + kC * n) * p.h_k * 2 * DK + (size_t)hk * 2 * DK * kC;
    const __bf16 *tp_head = p.ws_tp + (size_t)hv * p.t_total * 4 * kC;
    const float *gb_head = p.ws_gb + (size_t)hv * p.t_total * 2;
    float *o_head = p.ws_o + (size_t)hv * p.t_total * p.d_v;

    // ---- producer state: thread (token vt, channels 4 vg) of the v slice
    typedef typename RawAct<TIn>::type RawT;
    const int pt = tid - 256;
    const int vt = (pt & 255) >> 2, vg = pt & 3;
    const int vch = 2 * p.h_k * DK + c0 + 4 * vg;
    float wv[4][4];
    RawT nxr[4];
    float2 ngb = make_float2(0.f, 0.f);
    float ngc = 0.0f;
    if (producer) load_taps4(p, vch, wv);

    // ---- consumer state: state slice and this wave's operand fragments;
    // each fragment is reloaded with the next chunk's data right after its
    // last use in the current chunk.
    f32x4 S[MTW];
    Frag cK[KS], cQ[KS], cT[2], cP[2];

#define GDN_PROD_KT(CH, BUF)                                                                   \
    {                                                                                          \
        const char *src = reinterpret_cast<const char *>(kt_seq + (size_t)(CH) * kC * p.h_k * 2 * DK); \
        for (int k = cw; k < LY::KT_BYTES / 1024; k += 4)                                      \
            lds_load16(src + k * 1024 + lane * 16, sKT + (BUF) * LY::KT_BYTES + k * 1024);     \
    }
#define GDN_PROD_REGS(CH)                                                                      \
    {                                                                                          \
        const int fLc = min(kC, L - (CH) * kC);                                                \
        const int tl = (CH) * kC + vt;                                                         \
        const int tc = tl < L ? tl : L - 1;                                                    \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                          \
            nxr[j] = RawAct<TIn>::load(x, (size_t)(s0 + max(tc - 3 + j, 0)) * p.conv_dim + vch); \
        if (pt < kC) {                                                                         \
            const int tr = pt < fLc ? pt : fLc - 1;                                            \
            ngb = *reinterpret_cast<const float2 *>(gb_head + (size_t)(s0 + (CH) * kC + tr) * 2); \
            ngc = gb_head[(size_t)(s0 + (CH) * kC + fLc - 1) * 2];                             \
        }                                                                                      \
    }
#define GDN_PROD_STAGE_V(CH, XR)                                                               \
    {                                                                                          \
        const int fLc = min(kC, L - (CH) * kC);                                                \
        *reinterpret_cast<f32x4 *>(sV + vt * kBV + 4 * vg) = conv4(wv, XR);                    \
        if (pt < kC) {                                                                         \
            sEG[pt] = expf(ngb.x); /* g = 0 past the end: G stays at G_{Lc-1} */               \
            sB[pt] = pt < fLc ? ngb.y : 0.0f;                                                  \
        }                                                                                      \
    }
#define GDN_PROD_STAGE_EGC()                                                                   \
    {                                                                                          \
        if (pt < kC) sEGC[pt] = expf(ngc - ngb.x);                                             \
    }
    // Consumer operand loads of chunk CH: row 16w+col of q^, k^ (A of X, Y)
    // and of T, P (A of D and of O).  Rows past the end read a valid row;
    // their X, Y rows are never used, and T, P are zeroed at use.
#define GDN_CONS_ROWOFF(CH) ((size_t)(s0 + (CH) * kC + (16 * cw + col < min(kC, L - (CH) * kC) ? 16 * cw + col : 0)))
#define GDN_CONS_LOAD_QK(CH)                                                                   \
    {                                                                                          \
        const __bf16 *qr = qk_head + GDN_CONS_ROWOFF(CH) * 4 * DK + 8 * kq;                    \
        _Pragma("unroll") for (int s = 0; s < KS; ++s) {                                       \
            cQ[s] = frag_at(qr + 32 * s, qr + DK + 32 * s);                                    \
            cK[s] = frag_at(qr + 2 * DK + 32 * s, qr + 3 * DK + 32 * s);                       \
        }                                                                                      \
    }
#define GDN_CONS_LOAD_T(CH)                                                                    \
    {                                                                                          \
        const __bf16 *tp = tp_head + GDN_CONS_ROWOFF(CH) * 4 * kC + 8 * kq;                    \
        _Pragma("unroll") for (int s = 0; s < 2; ++s) cT[s] = frag_at(tp + 32 * s, tp + kC + 32 * s); \
    }
#define GDN_CONS_LOAD_P(CH)                                                                    \
    {                                                                                          \
        const __bf16 *tp = tp_head + GDN_CONS_ROWOFF(CH) * 4 * kC + 2 * kC + 8 * kq;           \
        _Pragma("unroll") for (int s = 0; s < 2; ++s) cP[s] = frag_at(tp + 32 * s, tp + kC + 32 * s); \
    }

    // ---- prologue: chunk 0 ----------------------------------------------
    if (producer) {
        if (nchunks > 0) {
            GDN_PROD_KT(0, 0)
            GDN_PROD_REGS(0)
            // chunk 0 may reach into the incoming conv history
            f32x4 x0[4];
            {
                const int tc = vt < L ? vt : L - 1;
#pragma unroll
                for (int j = 0; j < 4; ++j) x0[j] = raw4(p, x, n, s0, tc - 3 + j, vch);
            }
            GDN_PROD_STAGE_V(0, x0)
            GDN_PROD_STAGE_EGC()
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); // LDS-direct loads have landed
    } else {
        const float *Sin = p.state_in ? p.state_in + ((size_t)n * p.h_v + hv) * DK * p.d_v : nullptr;
#pragma unroll
        for (int u = 0; u < MTW; ++u) {
            const int mt = cw + 4 * u;
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
        if (nchunks > 0) {
            GDN_CONS_LOAD_QK(0)
            GDN_CONS_LOAD_T(0)
            GDN_CONS_LOAD_P(0)
        }
    }
    lds_barrier();

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = s0 + c * kC;
        const int Lc = min(kC, L - c * kC);
        const bool more = c + 1 < nchunks;
        f32x4 Y = {0.f, 0.f, 0.f, 0.f};
        float gam = 0.0f;

        // ---- phase 1: X, Y, R = beta (V - e^G X) -> sR | k^T, v/gates (c+1)
        const bool live = 16 * cw + col < Lc; // this lane's T / P row exists
        if (!producer) {
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const Frag B = frag_at(sSh + col * RK + 32 * s + 8 * kq, sSl + col * RK + 32 * s + 8 * kq);
                X = mma3(cK[s], B, X);
                Y = mma3(cQ[s], B, Y);
            }
            if (more) GDN_CONS_LOAD_QK(c + 1)
            gam = sEG[kC - 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * cw + 4 * kq + e;
                const float eg = sEG[t];
                __bf16 h, l;
                split1(sB[t] * (sV[t * kBV + col] - eg * X[e]), h, l);
                sRh[col * RT + t] = h;
                sRl[col * RT + t] = l;
                Y[e] *= eg;
            }
        } else if (more) {
            GDN_PROD_KT(c + 1, (c + 1) & 1)
            GDN_PROD_REGS(c + 1)
        }
        lds_barrier();

        // ---- phase 2: D = T R -> sD, sE | sV, beta, e^G (c+1) -------------
        if (!producer) {
            f32x4 Dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s)
                Dv = mma3(frag_select(live, cT[s]),
                          frag_at(sRh + col * RT + 32 * s + 8 * kq, sRl + col * RT + 32 * s + 8 * kq), Dv);
            if (more) GDN_CONS_LOAD_T(c + 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * cw + 4 * kq + e;
                __bf16 h, l;
                split1(Dv[e], h, l);
                sDh[col * RT + t] = h;
                sDl[col * RT + t] = l;
                split1(Dv[e] * sEGC[t], h, l);
                sEh[col * RT + t] = h;
                sEl[col * RT + t] = l;
            }
        } else if (more) {
            f32x4 xr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xr[j] = RawAct<TIn>::to_f32(nxr[j]);
            GDN_PROD_STAGE_V(c + 1, xr)
        }
        lds_barrier();

        // ---- phase 3: O = Y' + P D; S' = gam S + K^T E | e^{G_C-G} (c+1) --
        if (!producer) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
                Y = mma3(frag_select(live, cP[s]),
                         frag_at(sDh + col * RT + 32 * s + 8 * kq, sDl + col * RT + 32 * s + 8 * kq), Y);
            if (more) GDN_CONS_LOAD_P(c + 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * cw + 4 * kq + e;
                if (t < Lc) o_head[(size_t)(t0 + t) * p.d_v + slice * kBV + col] = Y[e];
            }
            Frag Bs[2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
                Bs[s] = frag_at(sEh + col * RT + 32 * s + 8 * kq, sEl + col * RT + 32 * s + 8 * kq);
            const char *kt = sKT + (c & 1) * LY::KT_BYTES;
#pragma unroll
            for (int u = 0; u < MTW; ++u) {
                const int mt = cw + 4 * u;
                if (mt < MTS) {
                    const int i = 16 * mt + col;
                    f32x4 acc = gam * S[u];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int g = (4 * s + kq) ^ (i & 7);
                        const __bf16 *ah = reinterpret_cast<const __bf16 *>(kt + (size_t)i * kC * 2 + g * 16);
                        acc = mma3(frag_at(ah, ah + DK * kC), Bs[s], acc);
                    }
                    S[u] = acc;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        __bf16 h, l;
                        split1(acc[e], h, l);
                        sSh[col * RK + 16 * mt + 4 * kq + e] = h;
                        sSl[col * RK + 16 * mt + 4 * kq + e] = l;
                    }
                }
            }
        } else {
            if (more) GDN_PROD_STAGE_EGC()
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); // chunk c+1's LDS-direct loads landed
        }
        lds_barrier();
    }
#undef GDN_PROD_KT
#undef GDN_PROD_REGS
#undef GDN_PROD_STAGE_V
#undef GDN_PROD_STAGE_EGC
#undef GDN_CONS_ROWOFF
#undef GDN_CONS_LOAD_QK
#undef GDN_CONS_LOAD_T
#undef GDN_CONS_LOAD_P

    // Final state slice.
    if (!producer) {
        float *Sout = p.state_out + ((size_t)n * p.h_v + hv) * DK * p.d_v;
#pragma unroll
        for (int u = 0; u < MTW; ++u) {
            const int mt = cw + 4 * u;
            if (mt < MTS)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Sout[(size_t)(16 * mt + 4 * kq + e) * p.d_v + slice * kBV + col] = S[u][e];
        }
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
    constexpr int RPW = 64 / LPR; // rows per wave and slot
    constexpr int RPT = 4;        // rows per lane (independent loads in flight)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rbase = (blockIdx.x * 4 + wave) * RPT * RPW + lane / LPR;
    const int c4 = (lane % LPR) * 4;
    const TIn *zp = static_cast<const TIn *>(p.z);
    f32x4 o[RPT], z[RPT];
    size_t base[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int row = rbase + k * RPW;
        const int rr = row < rows ? row : rows - 1;
        const int t = rr / p.h_v, hv = rr % p.h_v;
        base[k] = (size_t)t * p.value_dim + (size_t)hv * DV + c4;
        o[k] = ld4(p.ws_o + ((size_t)hv * p.t_total + t) * DV + c4);
        z[k] = load_act4v(zp, base[k]);
    }
    const f32x4 w = ld4(p.norm_w + c4);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        float ss = o[k][0] * o[k][0] + o[k][1] * o[k][1] + o[k][2] * o[k][2] + o[k][3] * o[k][3];
        ss = group_sum<LPR>(ss);
        const float rn = rsqrtf(ss / DV + p.norm_eps);
        float4 y;
        y.x = o[k][0] * rn * w[0] * gatef_(z[k][0], p.gate);
        y.y = o[k][1] * rn * w[1] * gatef_(z[k][1], p.gate);
        y.z = o[k][2] * rn * w[2] * gatef_(z[k][2], p.gate);
        y.w = o[k][3] * rn * w[3] * gatef_(z[k][3], p.gate);
        if (rbase + k * RPW < rows) store_out4(p.out, base[k], y, p.out_bf16);
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

template <typename TIn, int DV>
static hipError_t launch_norm(const PrefillArgs &a, int rows, hipStream_t s)
{
    constexpr int RPB = 4 * 4 * (64 / (DV / 4)); // rows per block
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
        hipLaunchKernelGGL((qknorm_kernel<TIn, DK>), dim3((max_len + kC - 1) / kC, a.h_k, n_seq),
                           dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((tri_kernel<TIn, DK>), dim3((max_len + kC - 1) / kC, a.h_v, n_seq),
                           dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (n_seq > 0) {
        const int slices = a.d_v / kBV;
        hipLaunchKernelGGL((scan_kernel<TIn, DK>), dim3(n_seq * a.h_v * slices), dim3(512),
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
    const WsLayout w = ws_layout(d, n_seq, t_total);
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
    A.ws_kt = reinterpret_cast<__bf16 *>(base + w.kt);
    A.t_total = t_total;
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
