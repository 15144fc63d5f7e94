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
//     W    = T diag(b e^G) K,      U = T diag(b) V      (no dependence on S)
//     D    = U - W S               (= T diag(b) (V - diag(e^G) K S))
//     O    = diag(e^G) Q S + P D
//     S'   = e^{G_C} S + K^T (diag(e^{G_C-G}) D)
// Only differences G_i - G_j with j <= i are exponentiated, so strong
// decay underflows to zero instead of overflowing.
//
// Kernels (one stream, in order):
//   qknorm  grid (chunk, key head, seq): causal conv + SiLU and L2 norm of
//           q and k; writes q^ and k^T as ready-made matrix-core operands
//           (split into bf16 hi + lo, one 1 KB fragment per 16x32 tile) and
//           the chunk's Gram matrices K K^T and Q K^T (fp32, MFMA).
//   tri     grid (chunk, value head, seq): gates and their in-chunk prefix
//           sum, A and P from the Gram matrices, the blocked fp32
//           triangular inverse T, the v conv, and W, U on MFMA; writes W
//           (negated), P as fragments, U in the accumulator layout of the
//           scan, and the decay factors e^G, e^{G_C-G}.
//   scan    grid (seq, value head, 16-column slice of d_v), 8 waves: four
//           carry the chain of chunk states (D = U - W S | S'), four trail
//           them by a chunk and form O = e^G Q S + P D; every operand of the
//           next chunk is loaded into registers right after its last use.
//   norm    grid (rows of (token, value head)): gated RMSNorm + output gate;
//           its first workgroups write each sequence's last K-1 raw inputs
//           as its conv history.
//
// Contractions run on v_mfma_f32_16x16x32_bf16 with every fp32 operand
// split into bf16 hi + lo and three products (hi.hi + hi.lo + lo.hi, fp32
// accumulate): plain bf16 operands are far outside the parity tolerance,
// the split form is within it.

#include "gdn_device.h"
#include "gdn_internal.h"

#include <algorithm>
#include <mutex>

namespace gdn {

constexpr int kC = 64;       // tokens per chunk
constexpr int kBV = 16;      // d_v columns per scan tile
constexpr int kSeqOrder = 64; // sequences the scan orders by length
constexpr int kQkChunks = 2; // chunks per qknorm workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Frag {
    bf16x8 hi, lo;
};

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
    // channels i..i+7 (16 bytes) as two quads
    __device__ __forceinline__ static void load8(const bf16_t *p, size_t i, type &a, type &b)
    {
        const uint4 v = *reinterpret_cast<const uint4 *>(p + i);
        a = make_uint2(v.x, v.y);
        b = make_uint2(v.z, v.w);
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
    __device__ __forceinline__ static void load8(const float *p, size_t i, type &a, type &b)
    {
        a = load(p, i);
        b = load(p, i + 4);
    }
    __device__ __forceinline__ static f32x4 to_f32(type u) { return u; }
};

__device__ __forceinline__ uint32_t pack2(__bf16 a, __bf16 b)
{
    return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Workgroup barrier that orders LDS traffic only: each wave drains its own
// LDS reads/writes, then all waves meet.  (No global memory is exchanged
// between the waves of a workgroup here, so no global fence is needed; the
// empty asm statements keep the compiler from moving memory accesses
// across the barrier.)
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xf << 8);

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Workspace (sections 256-byte aligned).  Chunk c of sequence n lives in
// chunk slot  cu[n]/C + n + c  (slots never overlap: a sequence of length L
// starting at s0 spans at most floor((s0+L)/C) - floor(s0/C) + 1 slots), so
// every chunk owns 64 whole rows, the rows past a sequence's end included.
//
// A "fragment" is one 16x32 bf16 operand tile of v_mfma_f32_16x16x32_bf16
// as the 64 lanes hold it: 1 KB, lane l's 8 values at byte 16 l.  For a
// matrix M (rows r, contraction index k), fragment (rb, s) holds
// M[16 rb + l%16][k(s, l/16, e)], stored hi part then lo part.
//   natural k order:   k = 32 s + 8 q + e
//   d_k-permuted order: k = 32 s + 4 q + e (e < 4), 32 s + 16 + 4 q + (e-4)
// The permuted order is the one the scan keeps its state operand in (the
// state tile of the accumulator layout lands in it with 8-byte writes).
//
//   qf   [H_k][slot][rb 4][s d_k/32][hi,lo] fragments of q^ (permuted)
//   ktf  [H_k][slot][rb d_k/16][s 2][hi,lo] fragments of k^T (natural,
//        k = token)
//   gram [H_k][slot][K K^T, Q K^T][64][64] fp32 (tiles on/below the
//        diagonal written)
//   wf   [H_v][slot][rb 4][s d_k/32][hi,lo] fragments of -W (permuted)
//   pf   [H_v][slot][rb 4][s 2][hi,lo] fragments of P (natural)
//   uf   [H_v][slot][slice d_v/16][rb 4][64 lanes][4] fp32: U in the
//        accumulator layout (lane l: rows 16 rb + 4 (l/16) + e, column
//        16 slice + l%16)
//   gf   [H_v][slot][e^G, e^{G_C-G}][64] fp32
//   o    [H_v][T][d_v] fp32 pre-norm readout
//
// With one decay per key channel (Kimi Delta Attention) the decay sits
// inside the q/k operands, so qf, ktf and gram are per value head and hold
// q^ (.) e^G, (k^ (.) e^{G_C-G})^T and the decayed Gram tiles; kw
// [H_v][slot] (ktf layout) holds (k^ (.) e^G)^T for W, and gf the chunk
// decay e^{G_C} of each key channel ([d_k] of the 128 floats).
// ---------------------------------------------------------------------------
struct WsLayout {
    size_t qf, ktf, gram, wf, pf, uf, gf, o, kw, total;
    int ns;
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int chunk_slots(int n_seq, int t_total) { return t_total / kC + n_seq + 1; }

static WsLayout ws_layout(const Dims &d, int n_seq, int t_total)
{
    WsLayout w;
    w.ns = chunk_slots(n_seq, t_total);
    const size_t NS = (size_t)w.ns;
    const size_t frag_dk = (size_t)kC * d.d_k * 2 * 2; // bytes of a 64 x d_k hi/lo block
    // With one decay per key channel the q/k operands and the Gram tiles
    // carry that decay, so they exist per value head.
    const size_t hq = d.chan_decay ? d.h_v : d.h_k;
    size_t off = 0;
    w.qf = off;
    off = align256(off + hq * NS * frag_dk);
    w.ktf = off;
    off = align256(off + hq * NS * frag_dk);
    w.gram = off;
    off = align256(off + hq * NS * 2 * kC * kC * sizeof(float));
    w.wf = off;
    off = align256(off + d.h_v * NS * frag_dk);
    w.pf = off;
    off = align256(off + d.h_v * NS * (size_t)kC * kC * 2 * 2);
    w.uf = off;
    off = align256(off + d.h_v * NS * (size_t)kC * d.d_v * sizeof(float));
    w.gf = off;
    off = align256(off + d.h_v * NS * 2 * kC * sizeof(float));
    w.o = off;
    off = align256(off + (size_t)t_total * d.value_dim * sizeof(float));
    w.kw = off; // per-channel decay only: k^ (.) e^G fragments for W
    off = align256(off + (d.chan_decay ? d.h_v * NS * frag_dk : 0));
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
    const float *decay_coef; // when not NULL, the log-decay coefficient itself (a_log NULL)
    const int32_t *cu;
    const float *state_in;
    float *state_out;
    const float *conv_in;
    float *conv_out;
    void *out;
    __bf16 *ws_qf, *ws_ktf, *ws_wf, *ws_pf, *ws_kw;
    float *ws_gram, *ws_uf, *ws_gf, *ws_o;
    int ns, t_total;
    int h_k, h_v, d_v, group, conv_k, conv_dim, value_dim;
    int gate, out_bf16, tiled, kda;
    int out_split;   // out: bf16 hi parts, then the lo parts at out + t_total * value_dim
    float norm_eps, l2_eps;
    // The scan's sequences in the order its workgroups take them: longest
    // first (the first kSeqOrder sequences of the call; later ones keep
    // their own index).
    uint8_t seq_order[kSeqOrder];
};

// Conv taps of 4 channels starting at ch, right-aligned to 4 taps (zero
// taps in front when K < 4): w[e][j] multiplies the input 3-j tokens back.
// Every tap is loaded unconditionally (K = 4: one 16-byte row per channel;
// K < 4: clamped single loads, the missing front taps selected to zero), so
// the loads stay in flight until the conv uses them.
__device__ __forceinline__ void load_taps4(const PrefillArgs &p, int ch, float (&w)[4][4])
{
    const int K = p.conv_k;
    f32x4 t[4];
    if (K == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = ld4(p.conv_w + (size_t)(ch + e) * 4);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < 4; ++j) t[e][j] = p.conv_w[(size_t)(ch + e) * K + max(j - (4 - K), 0)];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[e][j] = j >= 4 - K ? t[e][j] : 0.0f;
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

// Sum over aligned groups of W lanes (W = 4, 8 or 16, inside one row of 16
// lanes), every lane of a group ending with the group's sum: DPP moves only
// (quad permutations, half-row and row mirrors), no LDS traffic.
template <int CTRL> __device__ __forceinline__ float dppf(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xf, 0xf, false));
}
template <int W> __device__ __forceinline__ float row_sum(float v)
{
    static_assert(W == 4 || W == 8 || W == 16, "group size");
    v += dppf<0xb1>(v);                  // quad_perm [1,0,3,2]
    v += dppf<0x4e>(v);                  // quad_perm [2,3,0,1]
    if (W >= 8) v += dppf<0x141>(v);     // row_half_mirror
    if (W >= 16) v += dppf<0x140>(v);    // row_mirror
    return v;
}

// silu with the hardware exponential and reciprocal (a few ulp; the
// parity tolerance is orders of magnitude wider).
__device__ __forceinline__ float silu_fast(float x)
{
    return x * sigmoid_hw(x);
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
        c[e] = silu_fast(acc);
    }
    return c;
}

// ---------------------------------------------------------------------------
// qknorm: one workgroup per (two consecutive chunks, key head, sequence).  Each token row of
// the key head (q then k, 2*d_k channels) is handled by d_k/4 lanes of 8
// channels; each L2 norm is a DPP reduction over d_k/8 lanes.  The normalised
// rows (split hi/lo, zero past the sequence end) are gathered in LDS, then
// written out as q^ and k^T fragments, and the Gram tiles on and below the
// diagonal are formed on MFMA.
// ---------------------------------------------------------------------------
template <int DK> constexpr size_t qknorm_smem_bytes() { return 2 * 2 * kC * (DK + 8) * 2; }

template <typename TIn, int DK>
__global__ void __launch_bounds__(256)
qknorm_kernel(const PrefillArgs p)
{
    constexpr int LPT = DK / 4;              // lanes per token row (8 channels each)
    constexpr int TPI = 64 / LPT;            // token rows per wave pass
    constexpr int TPL = kC / (4 * TPI);      // consecutive tokens per lane
    constexpr int WIN = TPL + 3;             // raw rows a lane reads
    constexpr int KS = DK / 32, MTS = DK / 16;
    constexpr int RS = DK + 8;               // LDS row stride (bf16)
    const int hk = blockIdx.y, n = blockIdx.z;
    const int s0 = p.cu[n], L = p.cu[n + 1] - s0;
    const int cfirst = blockIdx.x * kQkChunks;
    if (cfirst * kC >= L) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane / LPT, ll = lane % LPT;
    const bool isk = ll >= DK / 8;           // q lanes, then k lanes (DK/8 each)
    const int c8 = (isk ? ll - DK / 8 : ll) * 8;
    const int ch = (isk ? p.h_k * DK : 0) + hk * DK + c8;
    const TIn *x = static_cast<const TIn *>(p.qkv);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // [q,k][hi,lo][row][RS]
    __bf16 *sQK = reinterpret_cast<__bf16 *>(smem);
    const int r0 = kC / 4 * wave + TPL * sub; // first chunk row of this lane
    const int col = lane & 15, kq = lane >> 4;
    auto row = [&](int m, int hl, int r) { return sQK + ((2 * m + hl) * kC + r) * RS; };

    // Every raw input the lane needs for a chunk (8 channels per row),
    // loaded at once (positions clamped into the sequence; positions before
    // its start are replaced when used).  The raw inputs of all the
    // workgroup's chunks are put in flight first, so the later chunks' loads
    // overlap the earlier chunks' work and stores.
    typedef typename RawAct<TIn>::type RawT;
    auto load_raw = [&](int c, RawT (&raw)[WIN][2]) {
        const int tl0 = c * kC + r0;
#pragma unroll
        for (int j = 0; j < WIN; ++j) {
            const int tau = min(max(tl0 - 3 + j, 0), L - 1);
            const size_t base = (size_t)(s0 + tau) * p.conv_dim + ch;
            RawAct<TIn>::load8(x, base, raw[j][0], raw[j][1]);
        }
    };
    RawT rawA[WIN][2], rawB[WIN][2];
    const bool second = (cfirst + 1) * kC < L;
    // (the taps, which the first chunk's conv needs, go ahead of the second
    // chunk's rows: loads complete in issue order)
    load_raw(cfirst, rawA);
    float w0[4][4], w1[4][4];
    load_taps4(p, ch, w0);
    load_taps4(p, ch + 4, w1);
    if (second) load_raw(cfirst + 1, rawB);
    const float extra = isk ? 1.0f : rsqrtf((float)DK);

    auto process = [&](int c, const RawT (&raw)[WIN][2]) {
        const int slot = s0 / kC + n + c;
        const int tl0 = c * kC + r0; // position in the sequence of row r0
        f32x4 xv[WIN][2];
#pragma unroll
        for (int j = 0; j < WIN; ++j) {
            xv[j][0] = RawAct<TIn>::to_f32(raw[j][0]);
            xv[j][1] = RawAct<TIn>::to_f32(raw[j][1]);
        }
        if (tl0 < 3) { // the first rows of a sequence reach into its history
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (tl0 - 3 + j < 0) {
                    xv[j][0] = raw4(p, x, n, s0, tl0 - 3 + j, ch);
                    xv[j][1] = raw4(p, x, n, s0, tl0 - 3 + j, ch + 4);
                }
        }

#pragma unroll
        for (int k = 0; k < TPL; ++k) {
            const int r = r0 + k, tl = tl0 + k;
            const f32x4 xa[4] = {xv[k][0], xv[k + 1][0], xv[k + 2][0], xv[k + 3][0]};
            const f32x4 xb[4] = {xv[k][1], xv[k + 1][1], xv[k + 2][1], xv[k + 3][1]};
            const f32x4 ca = conv4(w0, xa), cb = conv4(w1, xb);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += ca[e] * ca[e] + cb[e] * cb[e];
            ss = row_sum<DK / 8>(ss);
            const float sc = tl < L ? rsqrtf(ss + p.l2_eps) * extra : 0.0f;
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = ca[e] * sc;
                v[4 + e] = cb[e] * sc;
            }
            const Frag f = split8(v);
            __bf16 *dst = sQK + ((isk ? 2 : 0) * kC + r) * RS + c8;
            *reinterpret_cast<bf16x8 *>(dst) = f.hi;
            *reinterpret_cast<bf16x8 *>(dst + kC * RS) = f.lo;
        }
        lds_barrier();

        // q^ fragments, d_k-permuted order.
        __bf16 *qf = p.ws_qf + ((size_t)hk * p.ns + slot) * (2 * kC * DK);
        for (int f = wave; f < 4 * KS * 2; f += 4) {
            const int hl = f & 1, s = (f >> 1) % KS, rb = (f >> 1) / KS;
            const __bf16 *src = row(0, hl, 16 * rb + col) + 32 * s + 4 * kq;
            const uint2 x0 = *reinterpret_cast<const uint2 *>(src);
            const uint2 x1 = *reinterpret_cast<const uint2 *>(src + 16);
            *reinterpret_cast<u32x4 *>(qf + (size_t)f * 512 + lane * 8) = u32x4{x0.x, x0.y, x1.x, x1.y};
        }
        // k^T fragments, natural (token) order: lane (i, q) of fragment
        // (rb, s) gathers k^[32 s + 8 q + e][16 rb + i].
        __bf16 *ktf = p.ws_ktf + ((size_t)hk * p.ns + slot) * (2 * kC * DK);
        for (int f = wave; f < MTS * 4; f += 4) {
            const int hl = f & 1, s = (f >> 1) & 1, rb = f >> 2;
            const int i = 16 * rb + col, t = 32 * s + 8 * kq;
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = pack2(row(1, hl, t + 2 * e)[i], row(1, hl, t + 2 * e + 1)[i]);
            *reinterpret_cast<u32x4 *>(ktf + (size_t)f * 512 + lane * 8) = v;
        }
        // Gram tiles (mt, nt), nt <= mt, listed row by row; wave w takes
        // tiles w, w+4, w+8.
        float *gram = p.ws_gram + ((size_t)hk * p.ns + slot) * (2 * kC * kC);
        for (int tile = wave; tile < 10; tile += 4) {
            const int mt = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int nt = tile - mt * (mt + 1) / 2;
            f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = akk;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int o = 32 * s + 8 * kq;
                const Frag bk = frag_at(row(1, 0, 16 * nt + col) + o, row(1, 1, 16 * nt + col) + o);
                const Frag ak = frag_at(row(1, 0, 16 * mt + col) + o, row(1, 1, 16 * mt + col) + o);
                const Frag aq = frag_at(row(0, 0, 16 * mt + col) + o, row(0, 1, 16 * mt + col) + o);
                akk = mma3(ak, bk, akk);
                aqk = mma3(aq, bk, aqk);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * mt + 4 * kq + e, j = 16 * nt + col;
                // (non-temporal: only tri reads the Gram tiles; cached, they
                // crowd the scan's operands out later; scan 1.5 and tri 1.1 us
                // faster at T=4096)
                __builtin_nontemporal_store(akk[e], gram + i * kC + j);
                __builtin_nontemporal_store(aqk[e], gram + kC * kC + i * kC + j);
            }
        }
    };

    process(cfirst, rawA);
    if (second) {
        lds_barrier(); // the first chunk's LDS reads are done
        process(cfirst + 1, rawB);
    }
}

// ---------------------------------------------------------------------------
// kda_intra: the intra-chunk operands when each key channel has its own
// decay (Kimi Delta Attention, "cortiq-engine 0.8.76 pipeline.rs",
// AttnKind::Kda).  The decay then sits inside the key/query dot products,
//   A'[i][j] = sum_d k[i][d] k[j][d] e^{G[i][d] - G[j][d]},
//   P'[i][j] = sum_d q[i][d] k[j][d] e^{G[i][d] - G[j][d]}     (j <= i),
// with G[t][d] the prefix over the chunk of g[t][d] = c softplus(a + dt_bias)
// (G <= 0, non-increasing in t), so no Gram matrix can be shared by the
// value heads of a group.  A workgroup (16 waves at d_k = 128, 8 below; its
// fp32 rows fill ~110 KB of LDS, so one per CU) walks up to 8 consecutive
// chunks of one (value head, sequence), issuing each chunk's input loads
// while the previous chunk is processed.  Per chunk:
//   1. conv + SiLU + L2 norm of the chunk's q and k rows (fp32 in LDS) and
//      the per-channel prefix G;
//   2. A' and P': 16x16 blocks below the diagonal on the matrix cores with
//      both factors taken relative to the last row r of the column block
//      (e^{G[i]-G[r]} <= 1 for i > r, e^{G[r]-G[j]} <= 1 for j <= r, so
//      nothing overflows); the diagonal blocks the same way at the level of
//      4-row sub-blocks, and inside the sub-blocks one exponential per
//      (i, j, d);
//   3. the fragments the later kernels read: (k^ (.) e^G)^T for W, q^ (.) e^G
//      for the read-out, (k^ (.) e^{G_C-G})^T for the state update, and the
//      chunk decay e^{G_C} of each channel.
// ---------------------------------------------------------------------------
// LDS: the q, k and G rows (fp32, stride d_k + 4), the head's conv taps
// (q then k channels, four taps each), its dt_bias row and the three
// incoming history rows of its q and k channels (first chunk only)
template <int DK> constexpr size_t kda_smem_bytes()
{
    return 3 * (size_t)kC * (DK + 4) * 4 + 2 * DK * 16 + DK * 4 + 3 * 2 * DK * 4;
}
// Waves of kda_intra: its LDS rows allow one workgroup per CU, so at d_k = 128
// it runs 16 waves (twice the latency hiding of 8 for the same LDS).
template <int DK> constexpr int kda_waves() { return DK == 128 ? 16 : 8; }

// Lane roles of kda_intra (from the thread index): the conv rows and
// channels it loads, its gate channel and part, its fragment row and quad.
template <int DK> struct KdaLane {
    static constexpr int NW = kda_waves<DK>(), LPT = DK / 4, TPI = 64 / LPT;
    static constexpr int TPL = kC / (NW * TPI), NPART = 64 * NW / DK, TPP = kC / NPART;
    static constexpr int GL = DK / 8;            // lanes per gate row (8 channels each)
    int tid, lane, col, kq, c8, ch, r0, gd, gpart, gt, g8;
    bool isk;
    __device__ __forceinline__ KdaLane(int t, int wave, int hk, int h_k)
    {
        tid = t;
        lane = t & 63;
        col = lane & 15;
        kq = lane >> 4;
        const int sub = lane / LPT, ll = lane % LPT;
        isk = ll >= DK / 8;
        c8 = (isk ? ll - DK / 8 : ll) * 8;
        ch = (isk ? h_k * DK : 0) + hk * DK + c8;
        r0 = kC / NW * wave + TPL * sub;
        gd = t % DK;
        gpart = t / DK;
        gt = t / GL;
        g8 = 8 * (t % GL);
    }
};

template <typename TIn, int DK>
__global__ void __launch_bounds__(64 * kda_waves<DK>())
kda_intra_kernel(const PrefillArgs p, int per)
{
    typedef KdaLane<DK> Lane;
    constexpr int NW = Lane::NW;             // waves
    constexpr int RQ = DK + 4;               // fp32 LDS row stride
    constexpr int TPL = Lane::TPL;           // consecutive tokens per lane
    constexpr int WIN = TPL + 3;             // raw rows a lane reads
    constexpr int KS = DK / 32, MTS = DK / 16;
    constexpr int TPP = Lane::TPP;           // gate prefix: tokens per part of the chunk
    const int hv = blockIdx.y, n = blockIdx.z;
    const int s0 = p.cu[n], L = p.cu[n + 1] - s0;
    const int cbeg = blockIdx.x * per, cend = min(cbeg + per, (L + kC - 1) / kC);
    if (cbeg >= cend) return;
    const int hk = key_head_of(hv, p.h_k, p.group, p.tiled);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float *sQ = reinterpret_cast<float *>(smem);
    float *sK = sQ + kC * RQ;
    float *sG = sK + kC * RQ;
    float *sW = sG + kC * RQ;
    float *sDt = sW + 8 * DK;
    float *sH = sDt + DK;
    const TIn *x = static_cast<const TIn *>(p.qkv);
    const TIn *pa = static_cast<const TIn *>(p.a);

    // ---- per-head constants: conv taps (in LDS), gate parameters
    const int tid = threadIdx.x;
    if (tid < 2 * DK) {
        const int ct = (tid >= DK ? p.h_k * DK : 0) + hk * DK + (tid % DK);
        f32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int jj = j - (4 - p.conv_k);
            t[j] = jj >= 0 ? p.conv_w[(size_t)ct * p.conv_k + jj] : 0.0f;
        }
        *reinterpret_cast<f32x4 *>(sW + 4 * tid) = t;
    }
    if (tid < DK) sDt[tid] = p.dt_bias[(size_t)hv * DK + tid];
    if (cbeg == 0) // the raw inputs 3, 2, 1 tokens before the sequence
        for (int i = tid; i < 3 * 2 * DK / 4; i += 64 * NW) {
            const int j = i / (2 * DK / 4), c4 = 4 * (i % (2 * DK / 4));
            const int chh = (c4 >= DK ? p.h_k * DK : 0) + hk * DK + c4 % DK;
            *reinterpret_cast<f32x4 *>(sH + j * 2 * DK + c4) = raw4(p, x, n, s0, j - 3, chh);
        }
    const float coef = decay_coef_of(p.a_log, p.decay_coef, hv);

    // Raw q/k rows (as the scalar-decay path) and gate inputs of chunk cc.
    // A workgroup walks the chunks [cbeg, cend) of its head; each chunk's
    // loads are issued while the previous chunk is still being processed,
    // so their latency and the previous chunk's stores overlap its work.
    // (fp32 inputs take twice the registers: in flight across the Gram phase
    // they would spill, so they are loaded when the chunk starts)
    constexpr bool kPrefetch = sizeof(TIn) == 2;
    typedef typename RawAct<TIn>::type RawT;
    RawT raw[WIN][2], araw[2];
    auto load_chunk = [&](int cc, const Lane &q) {
        const int tl = cc * kC + q.r0, lc = min(kC, L - cc * kC);
#pragma unroll
        for (int j = 0; j < WIN; ++j) {
            const int tau = min(max(tl - 3 + j, 0), L - 1);
            const size_t base = (size_t)(s0 + tau) * p.conv_dim + q.ch;
            RawAct<TIn>::load8(x, base, raw[j][0], raw[j][1]);
        }
        // gate inputs: 8 channels of token gt (rows past the end, and the
        // spare threads when d_k < 64, re-read the last row: unused)
        const int t = min(q.gt, lc - 1);
        RawAct<TIn>::load8(pa, (size_t)(s0 + cc * kC + t) * p.h_v * DK + (size_t)hv * DK + q.g8, araw[0],
                           araw[1]);
    };
    if (kPrefetch) load_chunk(cbeg, Lane(tid, wave, hk, p.h_k));
    lds_barrier(); // taps, dt_bias and history stored

    for (int c = cbeg;;) {
        // The lane roles are recomputed per chunk from an opaque zero, which
        // keeps the compiler from hoisting their address arithmetic out of
        // the chunk loop (held there, it spills, and every spill reload
        // waits for the loads in flight).
        int lz;
        asm volatile("s_mov_b32 %0, 0" : "=s"(lz));
        const Lane q(tid + lz, wave, hk, p.h_k);
        const int lane = q.lane, col = q.col, kq = q.kq, c8 = q.c8, ch = q.ch, r0 = q.r0;
        const int gd = q.gd, gpart = q.gpart;
        const bool isk = q.isk;
        const float extra = isk ? 1.0f : rsqrtf((float)DK);
        const int Lc = min(kC, L - c * kC);
        const int slot = s0 / kC + n + c;
        const int tl0 = c * kC + r0;
        if (!kPrefetch) load_chunk(c, q);

        // ---- 1. conv + SiLU + L2 norm, fp32 rows (zero past the sequence end)
        {
            f32x4 xv[WIN][2];
#pragma unroll
            for (int j = 0; j < WIN; ++j) {
                xv[j][0] = RawAct<TIn>::to_f32(raw[j][0]);
                xv[j][1] = RawAct<TIn>::to_f32(raw[j][1]);
            }
            if (tl0 < 3) { // (from LDS: a global load here would wait for every store in flight)
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    if (tl0 - 3 + j < 0) {
                        const float *h = sH + (tl0 + j) * 2 * DK + (isk ? DK : 0) + c8;
                        xv[j][0] = ld4(h);
                        xv[j][1] = ld4(h + 4);
                    }
            }
            float w0[4][4], w1[4][4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x4 ta = ld4(sW + 4 * ((isk ? DK : 0) + c8 + e));
                const f32x4 tb = ld4(sW + 4 * ((isk ? DK : 0) + c8 + 4 + e));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    w0[e][j] = ta[j];
                    w1[e][j] = tb[j];
                }
            }
#pragma unroll
            for (int k = 0; k < TPL; ++k) {
                const int r = r0 + k, tl = tl0 + k;
                const f32x4 xa[4] = {xv[k][0], xv[k + 1][0], xv[k + 2][0], xv[k + 3][0]};
                const f32x4 xb[4] = {xv[k][1], xv[k + 1][1], xv[k + 2][1], xv[k + 3][1]};
                const f32x4 ca = conv4(w0, xa), cb = conv4(w1, xb);
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) ss += ca[e] * ca[e] + cb[e] * cb[e];
                ss = row_sum<DK / 8>(ss);
                const float sc = tl < L ? rsqrtf(ss + p.l2_eps) * extra : 0.0f;
                float *dst = (isk ? sK : sQ) + r * RQ + c8;
                *reinterpret_cast<f32x4 *>(dst) = ca * sc;
                *reinterpret_cast<f32x4 *>(dst + 4) = cb * sc;
            }
        }
        // per-channel log-decays g (zero past the end), then their prefix
        // within each part of the chunk, then the parts' offsets
        if (q.gt < kC) {
            const f32x4 ga = RawAct<TIn>::to_f32(araw[0]), gb = RawAct<TIn>::to_f32(araw[1]);
            const f32x4 da = ld4(sDt + q.g8), db = ld4(sDt + q.g8 + 4);
            f32x4 oa, ob;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // (8192 softplus per chunk: the hardware exp/log form)
                const float xg = (e < 4 ? ga[e] : gb[e - 4]) + (e < 4 ? da[e] : db[e - 4]);
                const float g = q.gt < Lc ? coef * softplus_hw(xg) : 0.0f;
                if (e < 4) oa[e] = g; else ob[e - 4] = g;
            }
            *reinterpret_cast<f32x4 *>(sG + q.gt * RQ + q.g8) = oa;
            *reinterpret_cast<f32x4 *>(sG + q.gt * RQ + q.g8 + 4) = ob;
        }
        // the next chunk's loads go out now (its raw rows and gates are
        // free); no barrier below waits for them
        const bool more = c + 1 < cend;
        if (kPrefetch && more) load_chunk(c + 1, q);
        lds_barrier();
        {
            float G = 0.0f;
#pragma unroll
            for (int tt = 0; tt < TPP; ++tt) {
                const int t = gpart * TPP + tt;
                G += sG[t * RQ + gd];
                sG[t * RQ + gd] = G;
            }
        }
        lds_barrier();
        {
            float off = 0.0f;
            for (int pp = 0; pp < gpart; ++pp) off += sG[((pp + 1) * TPP - 1) * RQ + gd];
            lds_barrier();
            if (gpart > 0)
#pragma unroll
                for (int tt = 0; tt < TPP; ++tt) sG[(gpart * TPP + tt) * RQ + gd] += off;
        }
        lds_barrier();

        // ---- 2. decayed Gram tiles, in 22 jobs of three kinds:
        //  off(pr), pr < 6: the 16x16 blocks (I, J), I > J, pair pr of
        //   (1,0) (2,0) (3,0) (2,1) (3,1) (3,2), on the matrix cores with both
        //   factors relative to the last row r of column block J
        //   (e^{G_i-G_r} <= 1, e^{G_r-G_j} <= 1: nothing overflows however
        //   strong the decay);
        //  diag(m), m < 12: diagonal block b = m / 3 split into 4-row
        //   sub-blocks, the pairs (i, j) with j in sub-block J = m % 3 and i
        //   in a later one, on the matrix cores relative to J's last row r
        //   (rows scaled by e^{G_i-G_r}, the 4 columns by e^{G_r-G_j}; one
        //   exponential per (lane, d), its sign set by the lane's role); the
        //   mirrored entries above the diagonal are written as zeros;
        //  within(b), b < 4: the 10 pairs j <= i inside each sub-block of
        //   diagonal block b, one per lane with one exponential per (i, j, d)
        //   (e^{G_i-G_j} <= 1); lanes 40-63 write the 24 zeros above the
        //   diagonal inside the sub-blocks.
        // An off or within job costs about two diag jobs; with 16 waves:
        // waves 0-5 off, 6-9 within, 10-15 two diag jobs each; with 8: waves
        // 0-5 off + two diag, 6-7 two within.
        float *gram = p.ws_gram + ((size_t)hv * p.ns + slot) * (2 * kC * kC);
        auto job_off = [&](int pr) {
            const int bI = pr < 3 ? pr + 1 : (pr < 5 ? pr - 1 : 3);
            const int bJ = pr < 3 ? 0 : (pr < 5 ? 1 : 2);
            const int r = 16 * bJ + 15, i = 16 * bI + col, j = 16 * bJ + col;
            f32x4 aa = {0.f, 0.f, 0.f, 0.f}, ap = aa;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const int d0 = 32 * st + 8 * kq;
                float va[8], vq[8], vb[8];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4 gr = ld4(sG + r * RQ + d0 + 4 * h);
                    const f32x4 gi = ld4(sG + i * RQ + d0 + 4 * h), gj = ld4(sG + j * RQ + d0 + 4 * h);
                    const f32x4 ki = ld4(sK + i * RQ + d0 + 4 * h), qi = ld4(sQ + i * RQ + d0 + 4 * h);
                    const f32x4 kj = ld4(sK + j * RQ + d0 + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ei = __expf(gi[e] - gr[e]), ej = __expf(gr[e] - gj[e]);
                        va[4 * h + e] = ki[e] * ei;
                        vq[4 * h + e] = qi[e] * ei;
                        vb[4 * h + e] = kj[e] * ej;
                    }
                }
                const Frag fb = split8(vb);
                aa = mma3(split8(va), fb, aa);
                ap = mma3(split8(vq), fb, ap);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ri = 16 * bI + 4 * kq + e, cj = 16 * bJ + col;
                gram[ri * kC + cj] = aa[e];
                gram[kC * kC + ri * kC + cj] = ap[e];
            }
        };
        auto job_diag = [&](int m) {
            const int b = m / 3, J = m % 3;
            const int r = 16 * b + 4 * J + 3, i = 16 * b + col;
            const bool arow = col > 4 * J + 3, bcol = (col >> 2) == J;
            f32x4 aa = {0.f, 0.f, 0.f, 0.f}, ap = aa;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const int d0 = 32 * st + 8 * kq;
                float va[8], vq[8], vb[8];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4 gr = ld4(sG + r * RQ + d0 + 4 * h), gi = ld4(sG + i * RQ + d0 + 4 * h);
                    const f32x4 ki = ld4(sK + i * RQ + d0 + 4 * h), qi = ld4(sQ + i * RQ + d0 + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float ex = __expf(arow ? gi[e] - gr[e] : gr[e] - gi[e]);
                        va[4 * h + e] = arow ? ki[e] * ex : 0.0f;
                        vq[4 * h + e] = arow ? qi[e] * ex : 0.0f;
                        vb[4 * h + e] = bcol ? ki[e] * ex : 0.0f;
                    }
                }
                const Frag fb = split8(vb);
                aa = mma3(split8(va), fb, aa);
                ap = mma3(split8(vq), fb, ap);
            }
            // accumulator lane: rows 4 kq + e, column col of the block
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ri = 4 * kq + e, at = (16 * b + ri) * kC + 16 * b + col;
                if (ri > 4 * J + 3 && (col >> 2) == J) {
                    gram[at] = aa[e];
                    gram[kC * kC + at] = ap[e];
                }
                if ((ri >> 2) == J && col > 4 * J + 3) {
                    gram[at] = 0.0f;
                    gram[kC * kC + at] = 0.0f;
                }
            }
        };
        auto job_within = [&](int b) {
            if (lane < 40) {
                const int sb = lane / 10, pp = lane % 10;
                const int il = pp >= 6 ? 3 : (pp >= 3 ? 2 : (pp >= 1 ? 1 : 0));
                const int jl = pp - il * (il + 1) / 2;
                const int i = 16 * b + 4 * sb + il, j = 16 * b + 4 * sb + jl;
                float acc_a = 0.0f, acc_p = 0.0f;
                for (int d4 = 0; d4 < DK / 4; ++d4) {
                    const f32x4 ki = ld4(sK + i * RQ + 4 * d4), qi = ld4(sQ + i * RQ + 4 * d4);
                    const f32x4 gi = ld4(sG + i * RQ + 4 * d4);
                    const f32x4 kj = ld4(sK + j * RQ + 4 * d4), gj = ld4(sG + j * RQ + 4 * d4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float w = kj[e] * __expf(gi[e] - gj[e]);
                        acc_a = fmaf(ki[e], w, acc_a);
                        acc_p = fmaf(qi[e], w, acc_p);
                    }
                }
                gram[i * kC + j] = acc_a;
                gram[kC * kC + i * kC + j] = acc_p;
            } else {
                const int u = lane - 40, sb = u / 6, pu = u % 6;
                const int il = pu < 3 ? 0 : (pu < 5 ? 1 : 2);
                const int jl = pu < 3 ? pu + 1 : (pu < 5 ? pu - 1 : 3);
                const int i = 16 * b + 4 * sb + il, j = 16 * b + 4 * sb + jl;
                gram[i * kC + j] = 0.0f;
                gram[kC * kC + i * kC + j] = 0.0f;
            }
        };
        if (NW == 16) {
            if (wave < 6) {
                job_off(wave);
            } else if (wave < 10) {
                job_within(wave - 6);
            } else {
                job_diag(2 * (wave - 10));
                job_diag(2 * (wave - 10) + 1);
            }
        } else {
            if (wave < 6) {
                job_off(wave);
                job_diag(2 * wave);
                job_diag(2 * wave + 1);
            } else {
                job_within(2 * (wave - 6));
                job_within(2 * (wave - 6) + 1);
            }
        }
        // ---- 3. decayed operand fragments and the chunk decay
        {
            const size_t fbase = ((size_t)hv * p.ns + slot) * (2 * kC * DK) + lane * 8;
            // (k^ (.) e^G)^T for W, and (k^ (.) e^{G_C - G})^T for the state
            // update: lane (i, q) of fragment (rb, s) holds tokens 32 s + 8 q + e
            // of channel 16 rb + i
            for (int f = wave; f < MTS * 2; f += NW) {
                const int st = f & 1, rb = f >> 1;
                const int d = 16 * rb + col, t = 32 * st + 8 * kq;
                const float gC = sG[(kC - 1) * RQ + d];
                float vw[8], vs[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float kv = sK[(t + e) * RQ + d], g = sG[(t + e) * RQ + d];
                    vw[e] = kv * __expf(g);
                    vs[e] = kv * __expf(gC - g);
                }
                const Frag a = split8(vw), bq = split8(vs);
                const int fi = (rb * 2 + st) * 2;
                *reinterpret_cast<bf16x8 *>(p.ws_kw + fbase + (size_t)fi * 512) = a.hi;
                *reinterpret_cast<bf16x8 *>(p.ws_kw + fbase + (size_t)(fi + 1) * 512) = a.lo;
                *reinterpret_cast<bf16x8 *>(p.ws_ktf + fbase + (size_t)fi * 512) = bq.hi;
                *reinterpret_cast<bf16x8 *>(p.ws_ktf + fbase + (size_t)(fi + 1) * 512) = bq.lo;
            }
            // q^ (.) e^G, d_k-permuted: lane (row col, q) of fragment (rb, s) holds
            // channels 32 s + 4 q + e and 32 s + 16 + 4 q + e of row 16 rb + col
            for (int f = wave; f < 4 * KS; f += NW) {
                const int st = f % KS, rb = f / KS;
                const int t = 16 * rb + col, d0 = 32 * st + 4 * kq;
                const f32x4 q0 = ld4(sQ + t * RQ + d0), q1 = ld4(sQ + t * RQ + d0 + 16);
                const f32x4 g0 = ld4(sG + t * RQ + d0), g1 = ld4(sG + t * RQ + d0 + 16);
                float v[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = q0[e] * __expf(g0[e]);
                    v[4 + e] = q1[e] * __expf(g1[e]);
                }
                const Frag fq = split8(v);
                *reinterpret_cast<bf16x8 *>(p.ws_qf + fbase + (size_t)(2 * f) * 512) = fq.hi;
                *reinterpret_cast<bf16x8 *>(p.ws_qf + fbase + (size_t)(2 * f + 1) * 512) = fq.lo;
            }
            if (q.tid < DK)
                p.ws_gf[((size_t)hv * p.ns + slot) * (2 * kC) + q.tid] = __expf(sG[(kC - 1) * RQ + q.tid]);
        }
        if (!more) break;
        ++c;
        lds_barrier(); // this chunk's LDS reads are done before the next one's writes
    }
}

// ---------------------------------------------------------------------------
// tri: one workgroup per (chunk, value head, sequence), 256 threads.
// ---------------------------------------------------------------------------
template <int DV> struct TriLds {
    static constexpr int LC = kC + 4;    // fp32 stride of A, P, T and V^T rows
    static constexpr int o_t = 0;
    static constexpr int o_g = o_t + kC * LC * 4;     // G, beta, beta e^G
    static constexpr int o_u = o_g + 3 * kC * 4;      // A, P, later V^T
    static constexpr int ap = 2 * kC * LC * 4, vt = DV * LC * 4;
    static constexpr int total = o_u + (ap > vt ? ap : vt);
};

template <typename TIn, int DK, int DV, bool KDA>
__global__ void __launch_bounds__(256)
tri_kernel(const PrefillArgs p)
{
    using LY = TriLds<DV>;
    constexpr int LC = LY::LC;
    constexpr int KS = DK / 32, VS = DV / 16;
    constexpr int CG = DV / 4;            // v channel groups of 4
    constexpr int TPG = kC * CG / 256;    // consecutive tokens per thread in the v conv
    constexpr int VWIN = TPG + 3;
    const int c = blockIdx.x, hv = blockIdx.y, n = blockIdx.z;
    const int s0 = p.cu[n];
    const int L = p.cu[n + 1] - s0;
    if (c * kC >= L) return;
    const int t0 = s0 + c * kC;
    const int Lc = min(kC, L - c * kC);
    const int hk = key_head_of(hv, p.h_k, p.group, p.tiled);
    const int slot = s0 / kC + n + c;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    float *sT = reinterpret_cast<float *>(smem + LY::o_t);
    float *sG = reinterpret_cast<float *>(smem + LY::o_g), *sB = sG + kC, *sBE = sB + kC;
    float *sA = reinterpret_cast<float *>(smem + LY::o_u), *sP = sA + kC * LC;
    float *sV = reinterpret_cast<float *>(smem + LY::o_u); // V^T [DV][LC]

    // ---- loads of the first phases: gates (wave 0) and Gram rows --------
    const TIn *pa = static_cast<const TIn *>(p.a);
    const TIn *pb = static_cast<const TIn *>(p.b);
    // (every wave loads them, rows past the end clamped to the last one and
    // masked where used: a load under a branch would be waited for at once)
    const size_t gi = (size_t)(t0 + min(lane, Lc - 1)) * p.h_v + hv;
    const float a_raw = KDA ? 0.0f : load_act(pa, gi), b_raw = load_act(pb, gi);
    const float dt_b = KDA ? 0.0f : p.dt_bias[hv];
    // Gram rows: thread (i, jq) holds row i, columns 16 jq .. 16 jq + 15 of
    // tiles on or below the diagonal.  A thread whose tile lies above the
    // diagonal reads the diagonal tile of its row instead (finite values,
    // all multiplied by the zero mask below; unconditional loads are not
    // waited for where they are issued).
    const int gi_ = tid >> 2, gq = tid & 3;
    f32x4 gkk[4], gqk[4];
    {
        const float *g = p.ws_gram + ((size_t)(KDA ? hv : hk) * p.ns + slot) * (2 * kC * kC) +
                         gi_ * kC + 16 * min(gq, gi_ >> 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            gkk[m] = ld4(g + 4 * m);
            gqk[m] = ld4(g + kC * kC + 4 * m);
        }
    }
    // ---- loads needed only after the solve, issued right after the Gram
    // rows (loads complete in issue order, so they do not delay the Gram
    // rows) and in flight during the gates, A, P and the solve: raw v
    // inputs, thread (channel group cg, token group tg), and the v taps
    typedef typename RawAct<TIn>::type RawT;
    const TIn *x = static_cast<const TIn *>(p.qkv);
    const int cg = tid % CG, tg = tid / CG;
    const int vch = 2 * p.h_k * DK + hv * DV + 4 * cg;
    const int vt0 = c * kC + tg * TPG; // first token (sequence position)
    RawT vraw[VWIN];
#pragma unroll
    for (int j = 0; j < VWIN; ++j) {
        const int tau = min(max(vt0 - 3 + j, 0), L - 1);
        vraw[j] = RawAct<TIn>::load(x, (size_t)(s0 + tau) * p.conv_dim + vch);
    }
    float wv[4][4];
    load_taps4(p, vch, wv);
    // ---- gates ("cherenkov qwen4_exp/cpu.rs" fn deltanet) and their
    // inclusive prefix sum over the chunk (wave 0); past the chunk end
    // g = 0 and b = 0.
    // (with one decay per key channel the decay is already inside the Gram
    // tiles and the k operand: only beta is needed here)
    if (KDA && wave == 0) {
        const float beta = lane < Lc ? sigmoid_hw(b_raw) : 0.0f;
        sG[lane] = 0.0f;
        sB[lane] = beta;
        sBE[lane] = beta;
    }
    if (!KDA && wave == 0) {
        float beta = 0.0f, g = 0.0f;
        if (lane < Lc) {
            beta = sigmoid_hw(b_raw);
            g = decay_coef_of(p.a_log, p.decay_coef, hv) * softplus_hw(a_raw + dt_b);
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float u = __shfl_up(g, off, 64);
            if (lane >= off) g += u;
        }
        const float gC = __shfl(g, 63, 64);
        const float eg = __expf(g);
        sG[lane] = g;
        sB[lane] = beta;
        sBE[lane] = beta * eg;
        float *gf = p.ws_gf + ((size_t)hv * p.ns + slot) * (2 * kC);
        gf[lane] = eg;
        gf[kC + lane] = __expf(gC - g);
    }
    __syncthreads();

    // ---- A and P rows from the Gram rows.
    {
        const int i = gi_;
        const float Gi = sG[i], bi = sB[i];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 av, pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * gq + 4 * m + e;
                // e^{G_i - G_j} <= 1: the hardware exponential (relative
                // error ~1e-7 where the factor is not negligible)
                const float md = j <= i ? (KDA ? 1.0f : __expf(Gi - sG[j])) : 0.0f;
                av[e] = j < i ? bi * md * gkk[m][e] : 0.0f;
                pv[e] = md * gqk[m][e];
            }
            *reinterpret_cast<f32x4 *>(sA + i * LC + 16 * gq + 4 * m) = av;
            *reinterpret_cast<f32x4 *>(sP + i * LC + 16 * gq + 4 * m) = pv;
        }
    }
    __syncthreads();

    // ---- P fragments (natural order): wave w takes (rb, s) = pairs w, w+4.
    // Rows 0-31 are zero in columns 32-63 (P is lower triangular): those two
    // fragments are never read, so they are not written.
    {
        __bf16 *pf = p.ws_pf + ((size_t)hv * p.ns + slot) * (2 * kC * kC) + lane * 8;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int pr = wave + 4 * k, rb = pr >> 1, s = pr & 1;
            if (rb < 2 && s == 1) continue;
            const float *src = sP + (16 * rb + col) * LC + 32 * s + 8 * kq;
            const f32x4 u = ld4(src), v = ld4(src + 4);
            const float vals[8] = {u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
            const Frag f = split8(vals);
            *reinterpret_cast<bf16x8 *>(pf + (size_t)(2 * pr) * 512) = f.hi;
            *reinterpret_cast<bf16x8 *>(pf + (size_t)(2 * pr + 1) * 512) = f.lo;
        }
    }


    // ---- T = (I + A)^-1, blocked over 16x16 blocks, fp32.
    // Diagonal blocks by forward substitution: wave b owns block b; lane
    // (col j, quarter q) keeps rows 4q..4q+3 of column j.
    {
        const int b = wave;
        float xs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[e] = (4 * kq + e == col) ? 1.0f : 0.0f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            const f32x4 a4 = ld4(sA + (16 * b + r) * LC + 16 * b + 4 * kq);
            float part = a4[0] * xs[0] + a4[1] * xs[1] + a4[2] * xs[2] + a4[3] * xs[3];
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            if (r > col && kq == r / 4) xs[r % 4] = -part;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(16 * b + 4 * kq + e) * LC + 16 * b + col] = xs[e];
        // blocks above the diagonal are zero
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
            if (bj > b)
#pragma unroll
                for (int e = 0; e < 4; ++e) sT[(16 * b + 4 * kq + e) * LC + 16 * bj + col] = 0.0f;
    }
    __syncthreads();
    // k^T fragments for the W^T tiles of this wave: column blocks 2 sp and
    // 2 sp + 1 of d_k (sp = wave), both token steps.  Issued only now, in
    // flight during the off-diagonal blocks and the v conv: issued with the
    // Gram rows, every resident workgroup's 32 KB of them queued ahead of
    // the next workgroups' gates and Gram rows (bench-step prefill 269-272
    // against 274-280 us).
    const int sp = wave;
    const bool wact = sp < KS;
    Frag kA[2][2];
    if (wact) {
        const __bf16 *kt = (KDA ? p.ws_kw + ((size_t)hv * p.ns + slot) * (2 * kC * DK)
                                : p.ws_ktf + ((size_t)hk * p.ns + slot) * (2 * kC * DK)) + lane * 8;
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int f = ((2 * sp + n2) * 2 + s) * 2;
                kA[n2][s] = frag_at(kt + (size_t)f * 512, kt + (size_t)(f + 1) * 512);
            }
    }
    // Off-diagonal blocks, by distance d from the diagonal, on the matrix
    // cores (split products, fp32 accumulate):
    //   T_ij = -T_ii (sum_{m=j}^{i-1} A_im T_mj);
    // the accumulated sum is already the B operand of the product with T_ii.
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int bi = wave + d, bj = wave;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int m = bj; m < bi; ++m) {
                const Frag4 fa = split4(ld4(sA + (16 * bi + col) * LC + 16 * m + 4 * kq));
                f32x4 tb;
#pragma unroll
                for (int e = 0; e < 4; ++e) tb[e] = sT[(16 * m + 4 * kq + e) * LC + 16 * bj + col];
                acc = mma3k16(fa, split4(tb), acc);
            }
            const Frag4 ft = split4(ld4(sT + (16 * bi + col) * LC + 16 * bi + 4 * kq));
            const f32x4 t = mma3k16(ft, split4(acc), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * bi + 4 * kq + e) * LC + 16 * bj + col] = -t[e];
        }
        __syncthreads();
    }

    // ---- v: silu(causal conv), transposed into LDS (A and P are dead).
    {
        f32x4 xv[VWIN];
#pragma unroll
        for (int j = 0; j < VWIN; ++j) xv[j] = RawAct<TIn>::to_f32(vraw[j]);
        if (vt0 < 3) {
#pragma unroll
            for (int j = 0; j < 3; ++j)
                if (vt0 - 3 + j < 0) xv[j] = raw4(p, x, n, s0, vt0 - 3 + j, vch);
        }
        float vt[4][TPG];
#pragma unroll
        for (int k = 0; k < TPG; ++k) {
            const f32x4 xr[4] = {xv[k], xv[k + 1], xv[k + 2], xv[k + 3]};
            const f32x4 cv = conv4(wv, xr);
#pragma unroll
            for (int e = 0; e < 4; ++e) vt[e][k] = cv[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float *dst = sV + (4 * cg + e) * LC + tg * TPG;
#pragma unroll
            for (int k = 0; k < TPG; k += 2)
                *reinterpret_cast<float2 *>(dst + k) = make_float2(vt[e][k], vt[e][k + 1]);
        }
    }
    __syncthreads();

    // ---- W^T = K^T diag(b e^G) T^T (tile (d_k block, row block rb)) and
    // U = T diag(b) V (tile (rb, d_v block)).  T is lower triangular, so row
    // blocks 0 and 1 only have the first token step.
    __bf16 *wf = p.ws_wf + ((size_t)hv * p.ns + slot) * (2 * kC * DK) + lane * 8;
    float *uf = p.ws_uf + ((size_t)hv * p.ns + slot) * ((size_t)kC * DV) + lane * 4;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int steps = rb < 2 ? 1 : 2;
        Frag Tw[2], Tu[2]; // rows 16 rb + col, tokens 32 s + 8 kq + e, scaled
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (s < steps) {
                const int t = 32 * s + 8 * kq;
                const float *src = sT + (16 * rb + col) * LC + t;
                const f32x4 u0 = ld4(src), u1 = ld4(src + 4);
                const f32x4 be0 = ld4(sBE + t), be1 = ld4(sBE + t + 4);
                const f32x4 b0 = ld4(sB + t), b1 = ld4(sB + t + 4);
                const float vw[8] = {u0[0] * be0[0], u0[1] * be0[1], u0[2] * be0[2], u0[3] * be0[3],
                                     u1[0] * be1[0], u1[1] * be1[1], u1[2] * be1[2], u1[3] * be1[3]};
                const float vu[8] = {u0[0] * b0[0], u0[1] * b0[1], u0[2] * b0[2], u0[3] * b0[3],
                                     u1[0] * b1[0], u1[1] * b1[1], u1[2] * b1[2], u1[3] * b1[3]};
                Tw[s] = split8(vw);
                Tu[s] = split8(vu);
            }
        }
        if (wact) {
            f32x4 wt[2];
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s < steps) acc = mma3(kA[n2][s], Tw[s], acc);
                wt[n2] = acc;
            }
            // lane (row 16 rb + col, q) holds W columns 32 sp + 4 q + e and
            // 32 sp + 16 + 4 q + e: fragment (rb, sp) of -W in permuted order
            const float vals[8] = {-wt[0][0], -wt[0][1], -wt[0][2], -wt[0][3],
                                   -wt[1][0], -wt[1][1], -wt[1][2], -wt[1][3]};
            const Frag f = split8(vals);
            const int fi = (rb * KS + sp) * 2;
            *reinterpret_cast<bf16x8 *>(wf + (size_t)fi * 512) = f.hi;
            *reinterpret_cast<bf16x8 *>(wf + (size_t)(fi + 1) * 512) = f.lo;
        }
#pragma unroll
        for (int nb = wave; nb < VS; nb += 4) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s)
                if (s < steps) {
                    const float *src = sV + (16 * nb + col) * LC + 32 * s + 8 * kq;
                    const f32x4 u0 = ld4(src), u1 = ld4(src + 4);
                    const float vals[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                    acc = mma3(Tu[s], split8(vals), acc);
                }
            // (U is read once, by one scan workgroup: stored non-temporally,
            // as the scan loads it, so it does not crowd the shared chunk
            // operands out of the cache; scan 129.4 against 139 us, tri 2 us
            // slower)
            __builtin_nontemporal_store(acc, reinterpret_cast<f32x4 *>(uf + (size_t)(nb * 4 + rb) * 256));
        }
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, value head, slice of NT 16-column tiles
// of d_v), 8 waves in two roles, one wave of each per SIMD:
//   chain waves 0-3: wave w carries rows 16w..16w+15 of D = U - W S and the
//     state rows of M-tiles w, w+4, ... through S' = e^{G_C} S + K^T E, for
//     every column tile of the slice;
//   output waves 4-7: one chunk behind, wave w forms rows 16w.. of
//     O = e^G (Q S) + P D from the state and D the chain left in LDS.
// Each role loads only its own operands, pre-split, into registers, each
// reloaded with the next chunk's data right after its last use; LDS holds
// what the roles exchange: the state slice S^T (d_k-permuted, B operand,
// double-buffered by chunk parity), D (double-buffered) and e^{G_C-G} D.
// Both roles meet at the same two barriers per chunk.  Every operand
// fragment a wave loads serves all NT column tiles, so wider slices cut the
// operand stream per column (the slices of one head all read the same W,
// K^T, Q and P of a chunk).
// ---------------------------------------------------------------------------
template <int DK, bool KDA, int NT>
__global__ void __launch_bounds__(512)
scan_kernel(const PrefillArgs p, int slices)
{
    constexpr int RK = DK + 8;         // bf16 stride of S^T rows
    constexpr int RT = kC + 8;         // bf16 stride of D, E rows
    constexpr int KS = DK / 32;        // k-steps over d_k
    constexpr int MTS = DK / 16;       // state M-tiles
    constexpr int MTW = (MTS + 3) / 4; // per chain wave
    constexpr int NC = kBV * NT;       // columns of the slice

    // Map the block index so the slices of one head share an XCD (blocks
    // are dealt round-robin over 8 XCDs): they read the same chunk data.
    const int nheads = gridDim.x / slices;
    int hidx, slice;
    {
        const int b = blockIdx.x;
        if (slices > 1 && nheads % 8 == 0) {
            const int x8 = b % 8, rest = b / 8;
            slice = rest % slices;
            hidx = (rest / slices) * 8 + x8;
        } else {
            slice = b % slices;
            hidx = b / slices;
        }
    }
    const int nq = hidx / p.h_v, hv = hidx % p.h_v;
    const int n = nq < kSeqOrder ? p.seq_order[nq] : nq;
    const int hk = key_head_of(hv, p.h_k, p.group, p.tiled);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = wave & 3;
    const int col = lane & 15, kq = lane >> 4;
    const int s0 = p.cu[n];
    const int L = p.cu[n + 1] - s0;
    const int nchunks = (L + kC - 1) / kC;
    const int slot0 = s0 / kC + n;
    const int c0 = slice * NC; // first d_v column of the slice

    __shared__ __attribute__((aligned(16))) __bf16 sS[2][2][NC * RK]; // [parity][hi,lo]
    __shared__ __attribute__((aligned(16))) __bf16 sD[2][2][NC * RT]; // [parity][hi,lo]
    __shared__ __attribute__((aligned(16))) __bf16 sE[2][NC * RT];    // [hi,lo]

    if (wave < 4) {
        // ================= chain waves ===================================
        // (per value head when each key channel has its own decay)
        const int hq = KDA ? hv : hk;
        const __bf16 *ktf = p.ws_ktf + ((size_t)hq * p.ns + slot0) * (2 * kC * DK) + lane * 8;
        const __bf16 *wf = p.ws_wf + ((size_t)hv * p.ns + slot0) * (2 * kC * DK) + lane * 8;
        const float *uf = p.ws_uf + ((size_t)hv * p.ns + slot0) * ((size_t)kC * p.d_v) +
                          (size_t)slice * NT * 4 * 256 + w * 256 + lane * 4;
        const float *gf = p.ws_gf + ((size_t)hv * p.ns + slot0) * (2 * kC);
        f32x4 S[MTW][NT];
        Frag cW[KS], cK[MTW][2];
        f32x4 cU[NT], cEGC;
        float gam = 0.0f;
        f32x4 gam4[MTW]; // per-channel chunk decay of this wave's state rows
#pragma unroll
        for (int u = 0; u < MTW; ++u) gam4[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Load groups, each issued right after the last use of what it
        // replaces: W rows and U (phase 1), e^{G_C-G} rows (after E), k^T rows
        // and e^{G_C} (phase 2).  The loads are unconditional (the last chunk
        // reloads itself) so that the compiler's load counters stay exact and
        // each wait covers only its own group, never the prefetch behind it.
        // U is the one operand only this workgroup reads, once: its loads are
        // non-temporal, which leaves the cache to the operands the head's
        // slices share (T=4096: 139.4 against 146.2 us).
#define GDN_CHAIN_LOAD1(CH)                                                                    \
        {                                                                                      \
            const size_t off = (size_t)(CH) * (2 * kC * DK);                                   \
            _Pragma("unroll") for (int s = 0; s < KS; ++s) {                                   \
                const int f = (w * KS + s) * 2;                                                \
                cW[s] = frag_at(wf + off + f * 512, wf + off + (f + 1) * 512);                 \
            }                                                                                  \
            _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                                  \
                cU[nt] = __builtin_nontemporal_load(                                           \
                    reinterpret_cast<const f32x4 *>(uf + (size_t)(CH) * kC * p.d_v + nt * 4 * 256)); \
        }
#define GDN_CHAIN_LOAD1B(CH) cEGC = ld4(gf + (size_t)(CH) * (2 * kC) + kC + 16 * w + 4 * kq);
#define GDN_CHAIN_LOAD2(CH)                                                                    \
        {                                                                                      \
            const size_t off = (size_t)(CH) * (2 * kC * DK);                                   \
            _Pragma("unroll") for (int u = 0; u < MTW; ++u) {                                  \
                const int mt = min(w + 4 * u, MTS - 1);                                        \
                _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                \
                    const int f = (mt * 2 + s) * 2;                                            \
                    cK[u][s] = frag_at(ktf + off + f * 512, ktf + off + (f + 1) * 512);        \
                }                                                                              \
            }                                                                                  \
            if (KDA) {                                                                         \
                _Pragma("unroll") for (int u = 0; u < MTW; ++u) {                              \
                    const int mt = min(w + 4 * u, MTS - 1);                                    \
                    gam4[u] = ld4(gf + (size_t)(CH) * (2 * kC) + 16 * mt + 4 * kq);            \
                }                                                                              \
            } else {                                                                           \
                gam = gf[(size_t)(CH) * (2 * kC) + kC - 1];                                    \
            }                                                                                  \
        }
        // State tile (mt, column tile nt) into S^T (buffer par) at its
        // d_k-permuted position.
        auto put_state = [&](int par, int mt, int nt, const f32x4 &v) {
            __bf16 h[4], l[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split1(v[e], h[e], l[e]);
            const int pos = (16 * nt + col) * RK + 32 * (mt >> 1) + 8 * kq + 4 * (mt & 1);
            *reinterpret_cast<uint2 *>(&sS[par][0][pos]) = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
            *reinterpret_cast<uint2 *>(&sS[par][1][pos]) = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
        };
        {
            const float *Sin = p.state_in ? p.state_in + ((size_t)n * p.h_v + hv) * DK * p.d_v : nullptr;
#pragma unroll
            for (int u = 0; u < MTW; ++u) {
                const int mt = w + 4 * u;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * mt + 4 * kq + e;
                        S[u][nt][e] = (mt < MTS && Sin) ? Sin[(size_t)i * p.d_v + c0 + 16 * nt + col] : 0.0f;
                    }
                    if (mt < MTS) put_state(0, mt, nt, S[u][nt]);
                }
            }
        }
        if (nchunks > 0) {
            GDN_CHAIN_LOAD1(0)
            GDN_CHAIN_LOAD1B(0)
            GDN_CHAIN_LOAD2(0)
        }
        // Drain the prologue's loads (issued in whatever order the compiler
        // chose) so that only the loop's own issue order decides its waits.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            const int par = c & 1;
            const int cn = c + 1 < nchunks ? c + 1 : c; // chunk whose operands are prefetched
            // ---- phase 1: D = U - W S -> sD, e^{G_C-G} D -> sE
            f32x4 Dv[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) Dv[nt] = cU[nt];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int o = (16 * nt + col) * RK + 32 * s + 8 * kq;
                    Dv[nt] = mma3(cW[s], frag_at(&sS[par][0][o], &sS[par][1][o]), Dv[nt]);
                }
            }
            GDN_CHAIN_LOAD1(cn)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                // this lane's 4 consecutive tokens: 8-byte writes
                __bf16 dh[4], dl[4], eh[4], el[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    split1(Dv[nt][e], dh[e], dl[e]);
                    split1(KDA ? Dv[nt][e] : Dv[nt][e] * cEGC[e], eh[e], el[e]);
                }
                const int o = (16 * nt + col) * RT + 16 * w + 4 * kq;
                *reinterpret_cast<uint2 *>(&sD[par][0][o]) = make_uint2(pack2(dh[0], dh[1]), pack2(dh[2], dh[3]));
                *reinterpret_cast<uint2 *>(&sD[par][1][o]) = make_uint2(pack2(dl[0], dl[1]), pack2(dl[2], dl[3]));
                *reinterpret_cast<uint2 *>(&sE[0][o]) = make_uint2(pack2(eh[0], eh[1]), pack2(eh[2], eh[3]));
                *reinterpret_cast<uint2 *>(&sE[1][o]) = make_uint2(pack2(el[0], el[1]), pack2(el[2], el[3]));
            }
            GDN_CHAIN_LOAD1B(cn)
            lds_barrier();
            // ---- phase 2: S' = e^{G_C} S + K^T E -> sS (other parity)
            // (the state is pinned here so that e^{G_C} S, which waits for the
            // phase-2 loads, is not hoisted into phase 1)
#pragma unroll
            for (int u = 0; u < MTW; ++u)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(S[u][nt]));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                Frag Be[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int o = (16 * nt + col) * RT + 32 * s + 8 * kq;
                    Be[s] = frag_at(&sE[0][o], &sE[1][o]);
                }
#pragma unroll
                for (int u = 0; u < MTW; ++u) {
                    const int mt = w + 4 * u;
                    if (mt < MTS) {
                        f32x4 acc = KDA ? gam4[u] * S[u][nt] : gam * S[u][nt];
#pragma unroll
                        for (int s = 0; s < 2; ++s) acc = mma3(cK[u][s], Be[s], acc);
                        S[u][nt] = acc;
                        put_state(par ^ 1, mt, nt, acc);
                    }
                }
            }
            GDN_CHAIN_LOAD2(cn)
            lds_barrier();
        }
#undef GDN_CHAIN_LOAD1B
#undef GDN_CHAIN_LOAD1
#undef GDN_CHAIN_LOAD2
        float *Sout = p.state_out + ((size_t)n * p.h_v + hv) * DK * p.d_v;
#pragma unroll
        for (int u = 0; u < MTW; ++u) {
            const int mt = w + 4 * u;
            if (mt < MTS)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Sout[(size_t)(16 * mt + 4 * kq + e) * p.d_v + c0 + 16 * nt + col] = S[u][nt][e];
        }
    } else {
        // ================= output waves (one chunk behind) ==============
        // Issue priority: the output waves' products gate the barriers both
        // roles meet at, so they run at priority 3 over the chain waves
        // sharing their SIMD, and drop to 0 while issuing their loads so
        // that the chain's loads are not queued behind them.
        const __bf16 *qf = p.ws_qf + ((size_t)(KDA ? hv : hk) * p.ns + slot0) * (2 * kC * DK) + lane * 8;
        const __bf16 *pf = p.ws_pf + ((size_t)hv * p.ns + slot0) * (2 * kC * kC) + lane * 8;
        const float *gf = p.ws_gf + ((size_t)hv * p.ns + slot0) * (2 * kC);
        float *o_head = p.ws_o + (size_t)hv * p.t_total * p.d_v + c0 + col;
        Frag cQ[KS], cP[2];
        f32x4 cEG, Y[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) Y[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#define GDN_OUT_LOAD1(CH)                                                                      \
        {                                                                                      \
            const size_t off = (size_t)(CH) * (2 * kC * DK);                                   \
            _Pragma("unroll") for (int s = 0; s < KS; ++s) {                                   \
                const int f = (w * KS + s) * 2;                                                \
                cQ[s] = frag_at(qf + off + f * 512, qf + off + (f + 1) * 512);                 \
            }                                                                                  \
            cEG = ld4(gf + (size_t)(CH) * (2 * kC) + 16 * w + 4 * kq);                         \
        }
#define GDN_OUT_LOAD2(CH)                                                                      \
        {                                                                                      \
            const size_t off = (size_t)(CH) * (2 * kC * kC);                                   \
            _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                    \
                const int f = (w * 2 + s) * 2;                                                 \
                if (s == 0 || w >= 2) /* rows 0-31 of P are zero in columns 32-63 */           \
                    cP[s] = frag_at(pf + off + f * 512, pf + off + (f + 1) * 512);             \
            }                                                                                  \
        }
        // Y = e^G (Q S) of chunk cc from the state buffer of its parity.
        auto readout = [&](int cc) {
            const int par = cc & 1;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int o = (16 * nt + col) * RK + 32 * s + 8 * kq;
                    acc = mma3(cQ[s], frag_at(&sS[par][0][o], &sS[par][1][o]), acc);
                }
                Y[nt] = KDA ? acc : acc * cEG; // (q already carries e^G per channel)
            }
        };
        // O = Y + P D of chunk cc, stored for its rows inside the sequence.
        auto finish = [&](int cc) {
            const int par = cc & 1;
            const int Lc = min(kC, L - cc * kC);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 y = Y[nt];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if (s == 0 || w >= 2) { // P is lower triangular
                        const int o = (16 * nt + col) * RT + 32 * s + 8 * kq;
                        y = mma3(cP[s], frag_at(&sD[par][0][o], &sD[par][1][o]), y);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * w + 4 * kq + e;
                    if (t < Lc) o_head[(size_t)(s0 + cc * kC + t) * p.d_v + 16 * nt] = y[e];
                }
            }
        };
        if (nchunks > 0) {
            GDN_OUT_LOAD1(0)
            GDN_OUT_LOAD2(0)
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            // phase 1: readout of chunk c-1 (its state is still in LDS)
            __builtin_amdgcn_s_setprio(3);
            if (c > 0) readout(c - 1);
            __builtin_amdgcn_s_setprio(0);
            GDN_OUT_LOAD1(c)
            lds_barrier();
            // phase 2: finish chunk c-1 (its D is still in LDS)
            __builtin_amdgcn_s_setprio(3);
            if (c > 0) finish(c - 1);
            __builtin_amdgcn_s_setprio(0);
            GDN_OUT_LOAD2(c)
            lds_barrier();
        }
#undef GDN_OUT_LOAD1
#undef GDN_OUT_LOAD2
        // the last chunk: the chain has left its state and D in LDS
        if (nchunks > 0) {
            readout(nchunks - 1);
            finish(nchunks - 1);
        }
    }
}

// ---------------------------------------------------------------------------
// conv history: each sequence's last K-1 raw inputs, oldest first, reaching
// into its initial history when it is shorter ("oxinfer 0.0.5 src/qwen.rs"
// gdn_forward, GdnState).  Thread per (channel, sequence).
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ void conv_final_channel(const PrefillArgs &p, int ch, int n)
{
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

// ---------------------------------------------------------------------------
// norm: gated RMSNorm of each (token, value head) row: d_v/4 lanes per row,
// float4 per lane ("oxinfer 0.0.5 src/qwen.rs" gdn_forward, gated norm).
// The first conv_blocks workgroups of the launch write the conv history
// instead (conv_bx blocks of 256 channels per sequence): that work needs
// only the raw inputs and the initial history, which every earlier launch
// of the call has finished reading, and it hides under the norm's stream.
// ---------------------------------------------------------------------------
template <typename TIn, int DV>
__global__ void __launch_bounds__(256)
norm_kernel(const PrefillArgs p, int rows, int conv_blocks, int conv_bx)
{
    if ((int)blockIdx.x < conv_blocks) {
        const int b = blockIdx.x;
        conv_final_channel<TIn>(p, (b % conv_bx) * 256 + threadIdx.x, b / conv_bx);
        return;
    }
    const int blk = blockIdx.x - conv_blocks;
    constexpr int LPR = DV / 4;   // lanes per row
    constexpr int RPW = 64 / LPR; // rows per wave and slot
    constexpr int RPT = 4;        // rows per lane (independent loads in flight)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rbase = (blk * 4 + wave) * RPT * RPW + lane / LPR;
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
        // (the pre-norm output is read exactly once: non-temporal loads, 24.3
        // against 26.5 us at T=4096)
        o[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.ws_o + ((size_t)hv * p.t_total + t) * DV + c4));
        z[k] = load_act4v(zp, base[k]);
    }
    const f32x4 w = ld4(p.norm_w + c4);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        float ss = o[k][0] * o[k][0] + o[k][1] * o[k][1] + o[k][2] * o[k][2] + o[k][3] * o[k][3];
        ss = group_sum<LPR>(ss);
        const float rn = rsqrtf(ss / DV + p.norm_eps);
        float4 y;
        y.x = o[k][0] * rn * w[0] * gate_hw(z[k][0], p.gate);
        y.y = o[k][1] * rn * w[1] * gate_hw(z[k][1], p.gate);
        y.z = o[k][2] * rn * w[2] * gate_hw(z[k][2], p.gate);
        y.w = o[k][3] * rn * w[3] * gate_hw(z[k][3], p.gate);
        if (rbase + k * RPW < rows) {
            if (p.out_split)
                store_split4(p.out, base[k], (size_t)p.t_total * p.value_dim, y);
            else
                store_out4(p.out, base[k], y, p.out_bf16);
        }
    }
}

// The gated norm of `rows` rows, with the conv history of n_seq sequences
// written by extra workgroups of the same launch (none when conv_k == 1).
template <typename TIn, int DV>
static hipError_t launch_norm(const PrefillArgs &a, int rows, int n_seq, hipStream_t s)
{
    constexpr int RPB = 4 * 4 * (64 / (DV / 4)); // rows per block
    const int conv_bx = (a.conv_dim + 255) / 256;
    const int conv_blocks = a.conv_k > 1 ? conv_bx * n_seq : 0;
    const int blocks = conv_blocks + (rows + RPB - 1) / RPB;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((norm_kernel<TIn, DV>), dim3(blocks), dim3(256), 0, s, a, rows,
                       conv_blocks, conv_bx);
    return hipGetLastError();
}

// 16-column tiles of d_v per scan workgroup.  Every slice of a head loads
// the same chunk operands, so wider slices cut the operand stream per
// column, but they lengthen each workgroup's per-chunk critical path.
// Widen (up to 4 tiles, the LDS limit) only while at least one workgroup per
// compute unit remains.  Measured at H_v=32, d=128: one sequence of 4096
// tokens (32 heads) is fastest at one tile (prefill 284 us against 294 at
// two and 362 at four); 8 packed sequences (256 heads) at four (1282 us
// against 1323 at two and 1560 at one).
static int scan_tiles(int heads, int tiles_per_head, int ncu)
{
    int nt = 1;
    while (nt < 4 && nt * 2 <= tiles_per_head && heads * (tiles_per_head / (nt * 2)) >= ncu)
        nt *= 2;
    return nt;
}

// Every sequence of the call is empty: each final state is its initial
// state (zeros when none is given).  One thread per float (the state
// pointers carry no alignment promise beyond 4 bytes); nothing to do when the
// update is in place.
__global__ void __launch_bounds__(256) state_pass_kernel(const float *__restrict__ sin,
                                                         float *__restrict__ sout, size_t n)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    sout[i] = sin ? sin[i] : 0.0f;
}

// Chunks one kda_intra workgroup walks through: as many as keeps about one
// workgroup per CU (its LDS rows allow no second one), at most 8 so that
// the last round of a packed batch stays short.
static int kda_chunks_per_block(int nch_max, int heads, int ncu)
{
    return std::max(1, std::min(8, (int)((long long)nch_max * heads / std::max(ncu, 1))));
}

template <typename TIn, int DK, int DV, bool KDA>
static hipError_t launch_prefill_t(const PrefillArgs &a, int n_seq, int t_total, int max_len,
                                   hipStream_t s)
{
    hipError_t e;
    if (max_len == 0) {
        // No chunk exists, so there is no workspace to read: the scan (whose
        // prologue loads chunk 0's operands) must not run.
        const size_t n = (size_t)n_seq * a.h_v * DK * DV;
        if (n > 0 && a.state_in != a.state_out) {
            hipLaunchKernelGGL(state_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               s, a.state_in, a.state_out, n);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        return launch_norm<TIn, DV>(a, 0, n_seq, s);
    }
    {
        const int nch_max = (max_len + kC - 1) / kC;
        const dim3 grid_v((max_len + kC - 1) / kC, a.h_v, n_seq);
        if (KDA) {
            int ncu = 0;
            if ((e = device_cu_count(&ncu)) != hipSuccess) return e;
            const int per = kda_chunks_per_block(nch_max, a.h_v * n_seq, ncu);
            const dim3 grid_c((nch_max + per - 1) / per, a.h_v, n_seq);
            hipLaunchKernelGGL((kda_intra_kernel<TIn, DK>), grid_c, dim3(64 * kda_waves<DK>()),
                               kda_smem_bytes<DK>(), s, a, per);
        } else {
            const dim3 grid_k((nch_max + kQkChunks - 1) / kQkChunks, a.h_k, n_seq);
            hipLaunchKernelGGL((qknorm_kernel<TIn, DK>), grid_k, dim3(256), qknorm_smem_bytes<DK>(),
                               s, a);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((tri_kernel<TIn, DK, DV, KDA>), grid_v, dim3(256), TriLds<DV>::total, s,
                           a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (n_seq > 0) {
        int ncu = 0;
        if ((e = device_cu_count(&ncu)) != hipSuccess) return e;
        const int nt = scan_tiles(n_seq * a.h_v, DV / kBV, ncu);
        const int slices = DV / kBV / nt;
        const dim3 grid(n_seq * a.h_v * slices);
        if (nt == 4)
            hipLaunchKernelGGL((scan_kernel<DK, KDA, 4>), grid, dim3(512), 0, s, a, slices);
        else if (nt == 2)
            hipLaunchKernelGGL((scan_kernel<DK, KDA, 2>), grid, dim3(512), 0, s, a, slices);
        else
            hipLaunchKernelGGL((scan_kernel<DK, KDA, 1>), grid, dim3(512), 0, s, a, slices);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return launch_norm<TIn, DV>(a, t_total * a.h_v, n_seq, s);
}

// Dynamic LDS above the default 64 KB needs the attribute raised once.
template <typename TIn, int DK, int DV>
static hipError_t set_smem_limits()
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(qknorm_kernel<TIn, DK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)qknorm_smem_bytes<DK>());
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kda_intra_kernel<TIn, DK>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kda_smem_bytes<DK>());
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(tri_kernel<TIn, DK, DV, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)TriLds<DV>::total);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(tri_kernel<TIn, DK, DV, false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)TriLds<DV>::total);
}

template <typename TIn, int DK, int DV>
static hipError_t run_prefill(const PrefillArgs &a, int n_seq, int t_total, int max_len,
                              hipStream_t s)
{
    static const hipError_t limits = set_smem_limits<TIn, DK, DV>();
    if (limits != hipSuccess) return limits;
    if (a.kda) return launch_prefill_t<TIn, DK, DV, true>(a, n_seq, t_total, max_len, s);
    return launch_prefill_t<TIn, DK, DV, false>(a, n_seq, t_total, max_len, s);
}

template <typename TIn, int DK>
static hipError_t dispatch_dv(const PrefillArgs &a, int n_seq, int t_total, int max_len,
                              hipStream_t s)
{
    switch (a.d_v) {
    case 32: return run_prefill<TIn, DK, 32>(a, n_seq, t_total, max_len, s);
    case 64: return run_prefill<TIn, DK, 64>(a, n_seq, t_total, max_len, s);
    case 128: return run_prefill<TIn, DK, 128>(a, n_seq, t_total, max_len, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill(const Dims &d, const Params &pr, int n_seq, int t_total, int max_len,
                          const int32_t *cu_host, const int32_t *cu_dev, const void *qkv,
                          const void *z, const void *a, const void *b,
                          const float *state_in, float *state_out,
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
    A.decay_coef = pr.decay_coef;
    A.dt_bias = pr.dt_bias;
    A.norm_w = pr.norm_w;
    A.cu = cu_dev;
    A.state_in = state_in;
    A.state_out = state_out;
    A.conv_in = conv_in;
    A.conv_out = conv_out;
    A.out = out;
    A.ws_qf = reinterpret_cast<__bf16 *>(base + w.qf);
    A.ws_ktf = reinterpret_cast<__bf16 *>(base + w.ktf);
    A.ws_wf = reinterpret_cast<__bf16 *>(base + w.wf);
    A.ws_pf = reinterpret_cast<__bf16 *>(base + w.pf);
    A.ws_gram = reinterpret_cast<float *>(base + w.gram);
    A.ws_uf = reinterpret_cast<float *>(base + w.uf);
    A.ws_gf = reinterpret_cast<float *>(base + w.gf);
    A.ws_o = reinterpret_cast<float *>(base + w.o);
    A.ws_kw = reinterpret_cast<__bf16 *>(base + w.kw);
    A.ns = w.ns;
    A.t_total = t_total;
    A.h_k = d.h_k;
    A.h_v = d.h_v;
    A.d_v = d.d_v;
    A.group = d.group;
    A.conv_k = d.conv_k;
    A.conv_dim = d.conv_dim;
    A.value_dim = d.value_dim;
    A.gate = d.gate;
    A.tiled = d.tiled;
    A.kda = d.chan_decay;
    A.out_split = d.out_split;
    A.out_bf16 = d.out_bf16;
    A.norm_eps = d.norm_eps;
    A.l2_eps = d.l2_eps;
    // Longest sequence first: a scan workgroup walks its sequence's whole
    // chain, so with more workgroups than CUs (packed sequences) the long
    // chains should start in the first round (8 packed sequences of 709 to
    // 4,688 tokens: prefill 1.25 against 1.28 ms, bit-identical).
    for (int i = 0; i < kSeqOrder; ++i) A.seq_order[i] = (uint8_t)i;
    if (cu_host && n_seq > 1) {
        const int m = std::min(n_seq, kSeqOrder);
        std::stable_sort(A.seq_order, A.seq_order + m, [&](uint8_t x, uint8_t y) {
            return cu_host[x + 1] - cu_host[x] > cu_host[y + 1] - cu_host[y];
        });
    }

#define GDN_PF_CASE(DK_)                                                                      \
    if (d.d_k == DK_)                                                                         \
        return d.act_bf16 ? dispatch_dv<bf16_t, DK_>(A, n_seq, t_total, max_len, s)           \
                          : dispatch_dv<float, DK_>(A, n_seq, t_total, max_len, s);
    GDN_PF_CASE(32)
    GDN_PF_CASE(64)
    GDN_PF_CASE(128)
#undef GDN_PF_CASE
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate: the workspace of the
// allocation-free prefill entry point.  One copy per device, held until the
// process ends; every call on a device shares it, so calls that overlap on
// one device race.  Every workspace value the prefill uses was written
// earlier in the same call (a few loads whose values go unused may read what
// an earlier call left), so nothing needs clearing between calls.  Host code
// never uses the array's name as a device address: the address comes from
// hipGetSymbolAddress, once per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kStaticScratchBytes];

hipError_t static_scratch(void **ptr)
{
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

} // namespace gdn
