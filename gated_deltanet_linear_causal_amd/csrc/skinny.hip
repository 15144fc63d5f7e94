// The projections of a mixer decode step on the matrix cores ("oxinfer 0.0.5
// src/qwen.rs", gdn_forward: in_proj of the hidden states into qkv, z, b
// and a; out_proj of the core's output), for the few rows (one per
// sequence) a decode step carries.
//
// A decode step multiplies at most 64 rows by weight matrices thousands of
// rows long, so its time is the weight stream.  One kernel serves both
// projections: a workgroup takes 64 output columns (16 per wave) and one
// slice of the contraction, and streams the A rows (the hidden states, or
// the core output as bf16 hi and lo parts) and its weight rows through LDS
// in 64-wide chunks of the contraction.  The partial products of the
// slices go to a workspace and a second, element-wise kernel adds them in
// slice order (so the result does not depend on timing) and applies the
// epilogue:
//   in_proj:  the causal conv + SiLU of the qkv columns over the conv
//             history, with the history moved on by one token ("cherenkov
//             qwen4_exp/cpu.rs" fn causal_conv), so the core receives the
//             convolved activations; z, b and a pass through;
//   out_proj: the sum of the hi and lo products (the core output split so
//             that the layer keeps fp32-level accuracy), stored as fp32 or
//             bf16.
// Up to 8 rows the in_proj contraction is one slice and the product kernel
// applies the in_proj epilogue itself (no partial products, no second
// kernel); above 8 rows at d_k = d_v = 128 the core decode kernel adds the
// two in_proj slices as it loads them and runs the conv itself.
// bf16 x bf16 products are exact in fp32 and accumulate in fp32.

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// (native vectors: arrays of HIP's uint4 wrapper are not kept in registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier that orders LDS only: each wave drains its LDS writes,
// then all meet.  The weight and A loads in flight stay in flight (a
// __syncthreads() fence would wait for them).
__device__ __forceinline__ void sk_lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr int kSkKC = 64;        // k per staged chunk
constexpr int kSkRS = kSkKC + 8; // LDS row stride (bf16): fragment reads hit distinct banks
// Chunks in flight per thread (measured: 8 was slower than 4).
template <int KSL> constexpr int sk_depth() { return 4; }

// Both operands stream through LDS chunk by chunk: every thread loads two
// 16-byte pieces of each 64 x 64 tile (a wave covers eight whole 128-byte
// rows, so each load instruction reads whole cache lines), sk_depth() chunks
// ahead in a register ring; the MFMA fragments are then read from LDS.
// The contraction slice KSL is a multiple of kSkKC * sk_depth() and the
// slices tile K exactly, so every staged chunk lies inside the matrices:
// rows past M and columns past N read clamped rows and their results are
// dropped.  No load is conditional and no arithmetic touches the loaded
// pieces before they are stored, so the compiler's count of loads in
// flight stays exact and a wait for one chunk never drains the ones behind.
template <int NPART, int KSL, bool EPI>
__global__ void __launch_bounds__(256, 2) skinny_gemm_kernel(const SkinnyGemm p, const ProjEpilogue e)
{
    __shared__ __attribute__((aligned(16))) __bf16 sa[2][NPART][kSkinnyRows * kSkRS];
    __shared__ __attribute__((aligned(16))) __bf16 sw[2][kSkinnyCols * kSkRS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;
    constexpr int nch = KSL / kSkKC;
    constexpr int D = sk_depth<KSL>();
    static_assert(nch % D == 0, "ring depth");
    // Row tiles of 16 A rows: the direct path (the epilogue in the product)
    // carries at most 8 rows, so it stages and multiplies one tile, a
    // quarter of the A loads and products of the four-tile form.
    constexpr int MT = EPI ? 1 : 4;
    const int k0 = blockIdx.y * KSL;
    const int n0 = blockIdx.x * kSkinnyCols;

    // the two pieces of this thread: tile row tid/8 (+32), 16-byte column
    // tid%8 (one row tile of A: one 8-byte piece, row tid/16, 8-byte column
    // tid%16)
    const int prow = tid >> 3, pc = tid & 7;
    const int arow1 = tid >> 4, ac1 = tid & 15;
    const bf16_t *ap[2][NPART];
    const bf16_t *wp[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = prow + 32 * q;
#pragma unroll
        for (int part = 0; part < NPART; ++part)
            ap[q][part] = MT == 4 ? p.a[part] + (size_t)min(r, p.M - 1) * p.K + k0 + 8 * pc
                                  : p.a[part] + (size_t)min(arow1, p.M - 1) * p.K + k0 + 4 * ac1;
        const int n = min(n0 + r, p.N - 1);
        int blk = 0;
#pragma unroll
        for (int b = 1; b < 4; ++b)
            if (n >= p.wstart[b]) blk = b;
        wp[q] = p.w[blk] + (size_t)(n - p.wstart[blk]) * p.K + k0 + 8 * pc;
    }
    // The ring's slots are separate arrays and every step is written out
    // (macros), so each access has a literal index and the ring stays in
    // registers.  Chunks past the slice, issued by the last steps, reread its
    // last chunk and are never stored.
    u32x4 r0[2][NPART + 1], r1[2][NPART + 1], r2[2][NPART + 1], r3[2][NPART + 1];
    u32x4 r4[2][NPART + 1], r5[2][NPART + 1], r6[2][NPART + 1], r7[2][NPART + 1];
    // Every workgroup of a launch reads the same A rows; each visits the
    // slice's chunks in a rotated order (a fixed rotation per column tile, so
    // every result is the same from run to run) so that they do not all
    // request the same lines at once.
    const int rot = (int)(blockIdx.x % nch);
#define GDN_SK_ISSUE(R, CH)                                                                    \
    {                                                                                          \
        const int off_ = ((min((CH), nch - 1) + rot) % nch) * kSkKC;                           \
        _Pragma("unroll") for (int q = 0; q < 2; ++q) {                                        \
            _Pragma("unroll") for (int part = 0; part < NPART; ++part) {                       \
                if (MT == 4) {                                                                 \
                    R[q][part] = *reinterpret_cast<const u32x4 *>(ap[q][part] + off_);         \
                } else if (q == 0) {                                                           \
                    const uint2 v_ = *reinterpret_cast<const uint2 *>(ap[0][part] + off_);     \
                    R[0][part] = u32x4{v_.x, v_.y, 0u, 0u};                                    \
                }                                                                              \
            }                                                                                  \
            R[q][NPART] = *reinterpret_cast<const u32x4 *>(wp[q] + off_);                      \
        }                                                                                      \
    }
    GDN_SK_ISSUE(r0, 0)
    GDN_SK_ISSUE(r1, 1)
    GDN_SK_ISSUE(r2, 2)
    GDN_SK_ISSUE(r3, 3)
    if constexpr (D == 8) {
        GDN_SK_ISSUE(r4, 4)
        GDN_SK_ISSUE(r5, 5)
        GDN_SK_ISSUE(r6, 6)
        GDN_SK_ISSUE(r7, 7)
    }

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one chunk: store the ring slot to LDS buffer BUF, refill the slot D
    // chunks ahead, meet, and run the chunk's products
#define GDN_SK_STEP(R, BUF, CH)                                                                \
    {                                                                                          \
        _Pragma("unroll") for (int q = 0; q < 2; ++q) {                                        \
            const int o = (prow + 32 * q) * kSkRS + 8 * pc;                                    \
            _Pragma("unroll") for (int part = 0; part < NPART; ++part) {                       \
                if (MT == 4)                                                                   \
                    *reinterpret_cast<u32x4 *>(&sa[BUF][part][o]) = R[q][part];                \
                else if (q == 0)                                                               \
                    *reinterpret_cast<uint2 *>(&sa[BUF][part][arow1 * kSkRS + 4 * ac1]) =      \
                        make_uint2(R[0][part].x, R[0][part].y);                                \
            }                                                                                  \
            *reinterpret_cast<u32x4 *>(&sw[BUF][o]) = R[q][NPART];                             \
        }                                                                                      \
        GDN_SK_ISSUE(R, (CH) + D)                                                              \
        sk_lds_barrier();                                                                      \
        _Pragma("unroll") for (int s = 0; s < kSkKC / 32; ++s) {                               \
            const bf16x8 bw = *reinterpret_cast<const bf16x8 *>(                               \
                &sw[BUF][(16 * wave + col) * kSkRS + 32 * s + 8 * kq]);                        \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                                \
                _Pragma("unroll") for (int part = 0; part < NPART; ++part) {                   \
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(                        \
                        &sa[BUF][part][(16 * mt + col) * kSkRS + 32 * s + 8 * kq]);            \
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw, acc[mt], 0, 0, 0); \
                }                                                                              \
            }                                                                                  \
        }                                                                                      \
    }
    // (every wave has finished reading a buffer before it is refilled: it
    // passed the barrier of the chunk in between after computing on it)
#pragma unroll
    for (int c0 = 0; c0 < nch; c0 += D) {
        GDN_SK_STEP(r0, 0, c0)
        GDN_SK_STEP(r1, 1, c0 + 1)
        GDN_SK_STEP(r2, 0, c0 + 2)
        GDN_SK_STEP(r3, 1, c0 + 3)
        if constexpr (D == 8) {
            GDN_SK_STEP(r4, 0, c0 + 4)
            GDN_SK_STEP(r5, 1, c0 + 5)
            GDN_SK_STEP(r6, 0, c0 + 6)
            GDN_SK_STEP(r7, 1, c0 + 7)
        }
    }
#undef GDN_SK_STEP
#undef GDN_SK_ISSUE

    // lane (col, kq) holds rows 16 mt + 4 kq + r of column n
    const int n = n0 + 16 * wave + col;
    if (EPI) {
        // The in_proj epilogue of rows 4 kq + r of column n (the direct path
        // carries at most 16 rows: row tile 0).  The column's block comes from
        // the block starts compared at constant indices (kernel arguments, no
        // lookup through memory), and every tap and history value is loaded
        // unconditionally from a clamped address before any is used, so the
        // lane's loads are in flight together (a load under a per-lane branch
        // is waited for where it is issued).
        int blk = 0, st = 0, en = e.start[1];
        float *dstb = e.dst[0];
#pragma unroll
        for (int b = 1; b < 4; ++b)
            if (n >= e.start[b]) {
                blk = b;
                st = e.start[b];
                en = e.start[b + 1];
                dstb = e.dst[b];
            }
        const int cols = en - st, j = n - st;
        const int K = e.conv_k, c0 = e.start[1];
        const int jc = min(max(n, 0), c0 - 1); // a conv channel whatever the block
        float w[4], hist[4][3];
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = e.conv_w[(size_t)jc * K + min(t, K - 1)];
        if (K > 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mc = min(4 * kq + r, e.M - 1);
                const float *h = e.conv_state + (size_t)mc * (K - 1) * c0 + jc;
#pragma unroll
                for (int t = 0; t < 3; ++t) hist[r][t] = h[(size_t)min(t, K - 2) * c0];
            }
        }
        // x is the newest raw input of channel j; history slot 0 is the
        // oldest, and the newest input meets the last tap.  All results
        // first, then the stores (stores count against the same load
        // counter, so a store issued before a wait would be waited for too).
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float a = 0.0f;
#pragma unroll
            for (int t = 0; t < 3; ++t)
                if (t < K - 1) a = fmaf(w[t], hist[r][t], a);
            a = fmaf(w[K - 1], acc[0][r], a);
            y[r] = blk == 0 ? a * sigmoid_hw(a) : acc[0][r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * kq + r;
            if (m < e.M && n < e.N) {
                if (blk == 0) {
                    float *h = e.conv_state + (size_t)m * (K - 1) * c0 + j;
#pragma unroll
                    for (int t = 0; t < 3; ++t)
                        if (t < K - 1) h[(size_t)t * c0] = t + 1 < K - 1 ? hist[r][t + 1] : acc[0][r];
                }
                dstb[(size_t)m * cols + j] = y[r];
            }
        }
        return;
    }
    float *dst = p.part + (size_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * mt + 4 * kq + r;
            if (m < p.M && n < p.N) dst[(size_t)m * p.N + n] = acc[mt][r];
        }
}

// in_proj epilogue: each thread takes four consecutive columns of one row
// (every block's start is a multiple of four: launch_proj_epilogue checks).
__global__ void __launch_bounds__(256) proj_epilogue_kernel(const ProjEpilogue p)
{
    const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i4 * 4 >= (size_t)p.M * p.N) return;
    const size_t i = 4 * i4;
    const int m = (int)(i / p.N), n = (int)(i % p.N);
    f32x4 v[kSkinnyMaxSplit];
#pragma unroll
    for (int s = 0; s < kSkinnyMaxSplit; ++s)
        v[s] = s < p.ksplit ? *reinterpret_cast<const f32x4 *>(p.part + (size_t)s * p.M * p.N + i)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 x = v[0];
#pragma unroll
    for (int s = 1; s < kSkinnyMaxSplit; ++s)
        if (s < p.ksplit) x += v[s];
    int blk = 0;
#pragma unroll
    for (int b = 1; b < 4; ++b)
        if (n >= p.start[b]) blk = b;
    const int j = n - p.start[blk];
    const int cols = p.start[blk + 1] - p.start[blk];
    if (blk == 0) {
        // x holds the newest raw inputs of channels j..j+3; history slot 0 is
        // the oldest, and the newest input meets the last tap
        const int K = p.conv_k;
        float *h = p.conv_state + (size_t)m * (K - 1) * cols + j;
        f32x4 hist[3];
        float w[4][4]; // [channel][tap]
        if (K == 4) { // four 16-byte rows
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x4 t4 = *reinterpret_cast<const f32x4 *>(p.conv_w + (size_t)(j + e) * 4);
#pragma unroll
                for (int t = 0; t < 4; ++t) w[e][t] = t4[t];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int t = 0; t < 4; ++t) w[e][t] = t < K ? p.conv_w[(size_t)(j + e) * K + t] : 0.0f;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 3; ++s)
            if (s < K - 1) {
                hist[s] = *reinterpret_cast<const f32x4 *>(h + (size_t)s * cols);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[e][s], hist[s][e], acc[e]);
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[e][K - 1], x[e], acc[e]);
#pragma unroll
        for (int s = 0; s < 3; ++s)
            if (s < K - 1)
                *reinterpret_cast<f32x4 *>(h + (size_t)s * cols) = s + 1 < K - 1 ? hist[s + 1] : x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[e] * sigmoid_hw(acc[e]);
    }
    *reinterpret_cast<f32x4 *>(p.dst[blk] + (size_t)m * cols + j) = x;
}

// out_proj epilogue: the slices' partial sums, four outputs per thread.
__global__ void __launch_bounds__(256) out_epilogue_kernel(const float *__restrict__ part,
                                                           int ksplit, size_t n4, void *out,
                                                           int out_bf16)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 *p4 = reinterpret_cast<const float4 *>(part);
    float4 v[kSkinnyMaxSplit];
#pragma unroll
    for (int s = 0; s < kSkinnyMaxSplit; ++s)
        v[s] = s < ksplit ? p4[(size_t)s * n4 + i] : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 acc = v[0];
#pragma unroll
    for (int s = 1; s < kSkinnyMaxSplit; ++s)
        if (s < ksplit) acc = acc + v[s];
    store_out4(out, 4 * i, acc, out_bf16);
}

static bool sk_slice_ok(int sl) { return sl == 256 || sl == 512 || sl == 1024 || sl == 2048; }

// Contraction slices: the fewest that give slices of 256, 512 or 1024 (at
// most 512 with two A parts, so that there are enough workgroups); 0 when K
// does not split into such slices.
int skinny_ksplit(int K, int nparts)
{
    const int cap = nparts == 1 ? 1024 : 512;
    if (K <= 0 || K % 256 != 0) return 0;
    for (int ks = 1; ks <= kSkinnyMaxSplit; ++ks) {
        const int sl = K % ks == 0 ? K / ks : 0;
        if (sl <= cap && sk_slice_ok(sl)) return ks;
    }
    return 0;
}

bool skinny_direct_ok(int K) { return sk_slice_ok(K); }

template <int NPART, bool EPI>
static hipError_t launch_skinny_t(const SkinnyGemm &g, const ProjEpilogue &e, int ksl, dim3 grid,
                                  hipStream_t s)
{
    switch (ksl) {
    case 256: hipLaunchKernelGGL((skinny_gemm_kernel<NPART, 256, EPI>), grid, dim3(256), 0, s, g, e); break;
    case 512: hipLaunchKernelGGL((skinny_gemm_kernel<NPART, 512, EPI>), grid, dim3(256), 0, s, g, e); break;
    case 1024: hipLaunchKernelGGL((skinny_gemm_kernel<NPART, 1024, EPI>), grid, dim3(256), 0, s, g, e); break;
    case 2048: hipLaunchKernelGGL((skinny_gemm_kernel<NPART, 2048, EPI>), grid, dim3(256), 0, s, g, e); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_skinny_gemm(SkinnyGemm g, int nparts, const ProjEpilogue *epi, hipStream_t s)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    const int ks = epi ? (nparts == 1 && skinny_direct_ok(g.K) ? 1 : 0) : skinny_ksplit(g.K, nparts);
    // the epilogue inside the product covers row tile 0 only
    if (ks == 0 || (epi && g.M > kSkinnyDirectRows)) return hipErrorInvalidValue;
    g.kslice = g.K / ks;
    const dim3 grid((g.N + kSkinnyCols - 1) / kSkinnyCols, ks);
    const ProjEpilogue none{};
    if (nparts == 2) return launch_skinny_t<2, false>(g, none, g.kslice, grid, s);
    if (epi) return launch_skinny_t<1, true>(g, *epi, g.kslice, grid, s);
    return launch_skinny_t<1, false>(g, none, g.kslice, grid, s);
}

hipError_t launch_proj_epilogue(const ProjEpilogue &e, hipStream_t s)
{
    for (int b = 0; b < 5; ++b)
        if (e.start[b] % 4 != 0) return hipErrorInvalidValue; // four columns per thread
    const size_t n4 = (size_t)e.M * e.N / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(proj_epilogue_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, e);
    return hipGetLastError();
}

hipError_t launch_out_epilogue(const float *part, int ksplit, size_t n, void *out, int out_bf16,
                               hipStream_t s)
{
    const size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(out_epilogue_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       part, ksplit, n4, out, out_bf16);
    return hipGetLastError();
}

} // namespace gdn
