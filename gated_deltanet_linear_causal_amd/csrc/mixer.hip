// The GDN mixer with its projections: in_proj (qkv, z, b, a) from the
// model's hidden states, the mixer core, and out_proj back to the hidden
// size ("oxinfer 0.0.5 src/qwen.rs", Gdn struct and gdn_forward;
// "cherenkov qwen4_exp/cpu.rs", fn deltanet).
//
// The projections are plain dense GEMMs and run on hipBLASLt (bf16
// operands, fp32 accumulation), apart from the two narrow gate projections
// of a decode step, which a small kernel does.  The projected activations
// stay fp32, so the core runs on fp32 inputs.  The core writes its output
// as a bf16 hi part and a bf16 lo part (hi = bf16(o), lo = bf16(o - hi)),
// stacked as [hi rows; lo rows], and out_proj is one GEMM over the stacked
// rows whose two halves are then added: rounding the core output to one
// bf16 alone would cost about as much as the whole error budget of the
// layer.

#include "gdn_device.h"
#include "gdn_internal.h"

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

namespace gdn {

// ---------------------------------------------------------------------------
// element-wise kernels
// ---------------------------------------------------------------------------

// v -> (hi, lo) with hi = bf16(v), lo = bf16(v - hi), four per thread.
__global__ void __launch_bounds__(256) split_bf16_kernel(const float *__restrict__ v,
                                                         bf16_t *__restrict__ hi,
                                                         bf16_t *__restrict__ lo, size_t n4)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 x = reinterpret_cast<const float4 *>(v)[i];
    const float xs[4] = {x.x, x.y, x.z, x.w};
    bf16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = f32_to_bf16(xs[e]);
        l[e] = f32_to_bf16(xs[e] - bf16_bits_to_f32(h[e]));
    }
    reinterpret_cast<uint2 *>(hi)[i] = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
    reinterpret_cast<uint2 *>(lo)[i] = make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16));
}

// b = x W_b^T and a = x W_a^T for a few rows of x (the decode step), where a
// library GEMM with this few output columns costs more in launch and tiling
// than in work.  A wave per (output column, 8 rows of x): its lanes run over
// the hidden size 8 elements at a time, with the weight row and all 8 rows
// of x loaded before the sums so that the loads overlap.
constexpr int kGateRows = 8;

__global__ void __launch_bounds__(256) gates_proj_kernel(const bf16_t *__restrict__ x,
                                                         const bf16_t *__restrict__ wb,
                                                         const bf16_t *__restrict__ wa,
                                                         float *__restrict__ b,
                                                         float *__restrict__ a, int T, int H, int nb)
{
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= 2 * nb) return; // whole waves; no barrier below
    const int t0 = blockIdx.y * kGateRows;
    const bf16_t *w = j < nb ? wb + (size_t)j * H : wa + (size_t)(j - nb) * H;
    const bf16_t *xr[kGateRows];
#pragma unroll
    for (int r = 0; r < kGateRows; ++r) xr[r] = x + (size_t)min(t0 + r, T - 1) * H;
    float acc[kGateRows] = {};
    for (int k = lane * 8; k < H; k += 512) {
        const uint4 wv = *reinterpret_cast<const uint4 *>(w + k);
        uint4 xv[kGateRows];
#pragma unroll
        for (int r = 0; r < kGateRows; ++r) xv[r] = *reinterpret_cast<const uint4 *>(xr[r] + k);
        const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int r = 0; r < kGateRows; ++r) {
            const uint32_t xs[4] = {xv[r].x, xv[r].y, xv[r].z, xv[r].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[r] = fmaf(__uint_as_float(xs[e] << 16), __uint_as_float(ws[e] << 16), acc[r]);
                acc[r] = fmaf(__uint_as_float(xs[e] & 0xffff0000u),
                              __uint_as_float(ws[e] & 0xffff0000u), acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kGateRows; ++r) acc[r] = group_sum<64>(acc[r]);
    float *dst = j < nb ? b + j : a + (j - nb);
#pragma unroll
    for (int r = 0; r < kGateRows; ++r)
        if (lane == r && t0 + r < T) dst[(size_t)(t0 + r) * nb] = acc[r];
}

// y = p[i] + p[n + i]: the products of the hi and lo parts, stacked as
// rows 0..T-1 and T..2T-1 of one GEMM, added and stored as fp32 or bf16
// (round to nearest even), four per thread.
__global__ void __launch_bounds__(256) add_halves_kernel(const float *__restrict__ v, void *out,
                                                         size_t n4, int out_bf16)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 *v4 = reinterpret_cast<const float4 *>(v);
    store_out4(out, 4 * i, v4[i] + v4[n4 + i], out_bf16);
}

// ---------------------------------------------------------------------------
// hipBLASLt: one handle per device, algorithms cached per GEMM shape
// ---------------------------------------------------------------------------
namespace {

// Everything a GEMM shape needs, made once and kept for the process.
struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulAlgo_t algo;
};

struct Blas {
    hipblasLtHandle_t handle = nullptr;
    std::map<std::tuple<int64_t, int64_t, int64_t, size_t>, GemmPlan> plans;
};

std::mutex g_blas_mu;
Blas g_blas[64];

hipError_t blas_error(hipblasStatus_t st)
{
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

// The plan of D[m][n] = X[m][k] . W[n][k]^T: in column-major terms
// D^T (n x m) = W (k x n)^T . X^T (k x m); bf16 operands, fp32 D.
hipblasStatus_t make_plan(hipblasLtHandle_t h, int64_t m, int64_t n, int64_t k, size_t ws_bytes,
                          GemmPlan &g)
{
    hipblasStatus_t st = hipblasLtMatmulDescCreate(&g.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT));
    if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN));
    if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&g.la, HIP_R_16BF, k, n, k);
    if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&g.lb, HIP_R_16BF, k, m, k);
    if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&g.lc, HIP_R_32F, n, m, n);
    hipblasLtMatmulPreference_t pref = nullptr;
    if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatmulPreferenceCreate(&pref);
    const uint64_t cap = ws_bytes;
    if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                   &cap, sizeof(cap));
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulAlgoGetHeuristic(h, g.desc, g.la, g.lb, g.lc, g.lc, pref, 1, res, &found);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (st == HIPBLAS_STATUS_SUCCESS && found < 1) st = HIPBLAS_STATUS_NOT_SUPPORTED;
    if (st == HIPBLAS_STATUS_SUCCESS) g.algo = res[0].algo;
    return st;
}

// The plan of D[m][n] = X[m][k] . W[n][k]^T on the current device: the
// device's handle and the shape's plan are made on first use (under the
// lock) and kept for the process; the returned plan is never modified or
// freed afterwards, so it is used without the lock.
hipError_t get_plan(int64_t m, int64_t n, int64_t k, size_t ws_bytes, hipblasLtHandle_t &handle,
                    const GemmPlan *&plan)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    Blas &b = g_blas[dev];
    if (!b.handle && hipblasLtCreate(&b.handle) != HIPBLAS_STATUS_SUCCESS) {
        b.handle = nullptr;
        return hipErrorLaunchFailure;
    }
    const auto key = std::make_tuple(m, n, k, ws_bytes);
    auto it = b.plans.find(key);
    if (it == b.plans.end()) {
        GemmPlan g;
        const hipblasStatus_t st = make_plan(b.handle, m, n, k, ws_bytes, g);
        if (st != HIPBLAS_STATUS_SUCCESS) {
            if (g.lc) hipblasLtMatrixLayoutDestroy(g.lc);
            if (g.lb) hipblasLtMatrixLayoutDestroy(g.lb);
            if (g.la) hipblasLtMatrixLayoutDestroy(g.la);
            if (g.desc) hipblasLtMatmulDescDestroy(g.desc);
            return blas_error(st);
        }
        it = b.plans.emplace(key, g).first; // std::map nodes never move
    }
    handle = b.handle;
    plan = &it->second;
    return hipSuccess;
}

// One GEMM of a call, with its plan resolved before the call's first launch.
struct Gemm {
    int64_t m = 0, n = 0, k = 0;
    hipblasLtHandle_t handle = nullptr;
    const GemmPlan *plan = nullptr;
    hipError_t prepare(int64_t m_, int64_t n_, int64_t k_, size_t ws_bytes)
    {
        m = m_, n = n_, k = k_;
        if (m == 0 || n == 0) return hipSuccess;
        return get_plan(m, n, k, ws_bytes, handle, plan);
    }
    // D[m][n] (fp32, row-major) = X[m][k] . W[n][k]^T, X and W bf16 row-major.
    hipError_t run(const void *X, const void *W, float *D, void *ws, size_t ws_bytes,
                   hipStream_t s) const
    {
        if (m == 0 || n == 0) return hipSuccess;
        const float alpha = 1.0f, beta = 0.0f;
        return blas_error(hipblasLtMatmul(handle, plan->desc, &alpha, W, plan->la, X, plan->lb,
                                          &beta, D, plan->lc, D, plan->lc, &plan->algo, ws,
                                          ws_bytes, s));
    }
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr size_t kBlasWorkspace = size_t(32) << 20;

struct MixerWs {
    size_t qkv, z, b, a, core, hl, acc, blas, prefill, part_in, part_out, total;
};

// The core runs on fp32 activations and writes its output as bf16 hi and
// lo parts (the operands of out_proj): the dims it sees.
Dims core_dims(const Dims &d, bool split)
{
    Dims c = d;
    c.act_bf16 = 0;
    c.out_bf16 = 0;
    c.out_split = split;
    return c;
}

MixerWs mixer_ws(const Dims &d, int hidden, int n_seq, int t_total, bool prefill)
{
    MixerWs w;
    const size_t T = (size_t)t_total, gw = d.chan_decay ? d.d_k : 1;
    size_t off = 0;
    w.qkv = off;
    off = align256(off + T * d.conv_dim * 4);
    w.z = off;
    off = align256(off + T * d.value_dim * 4);
    w.b = off;
    off = align256(off + T * d.h_v * 4);
    w.a = off;
    off = align256(off + T * d.h_v * gw * 4);
    w.core = off; // fp32 core output, only where the core cannot split it itself
    off = align256(off + T * d.value_dim * 4);
    w.hl = off;   // [hi parts][lo parts]
    off = align256(off + T * d.value_dim * 2 * 2);
    w.acc = off;  // the two stacked out_proj products
    off = align256(off + 2 * T * hidden * 4);
    w.blas = off;
    off = align256(off + kBlasWorkspace);
    w.prefill = off;
    off = align256(off + (prefill ? prefill_workspace_bytes(core_dims(d, true), n_seq, t_total) : 0));
    // the decode step's matrix-core projections: partial products of the
    // contraction slices of in_proj and out_proj
    const size_t n_in = (size_t)d.conv_dim + d.value_dim + d.h_v + (size_t)d.h_v * gw;
    w.part_in = off;
    off = align256(off + (prefill ? 0 : (size_t)skinny_ksplit(hidden, 1) * T * n_in * 4));
    w.part_out = off;
    off = align256(off + (prefill ? 0 : (size_t)skinny_ksplit(d.value_dim, 2) * T * hidden * 4));
    w.total = off;
    return w;
}

// The GEMMs of one mixer call: in_proj (qkv, z and, unless the small gate
// kernel takes them, b and a) and the stacked out_proj.
struct MixerGemms {
    Gemm qkv, z, b, a, out;
    bool gate_kernel = false;
};

// Resolves every GEMM plan the call needs, so that a failure is reported
// before anything is enqueued (the call then has written nothing).
hipError_t prepare_gemms(const Dims &d, const Proj &pj, int T, const void *x, MixerGemms &g)
{
    const int64_t H = pj.hidden, gw = d.chan_decay ? d.d_k : 1;
    const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(pj.w_b) |
                           reinterpret_cast<uintptr_t>(pj.w_a)) & 15) == 0;
    g.gate_kernel = gw == 1 && T > 0 && T <= 256 && aligned;
    hipError_t e;
    if ((e = g.qkv.prepare(T, d.conv_dim, H, kBlasWorkspace)) != hipSuccess) return e;
    if ((e = g.z.prepare(T, d.value_dim, H, kBlasWorkspace)) != hipSuccess) return e;
    if (!g.gate_kernel) {
        if ((e = g.b.prepare(T, d.h_v, H, kBlasWorkspace)) != hipSuccess) return e;
        if ((e = g.a.prepare(T, d.h_v * gw, H, kBlasWorkspace)) != hipSuccess) return e;
    }
    return g.out.prepare(2 * (int64_t)T, pj.hidden, d.value_dim, kBlasWorkspace);
}

// in_proj: the four projections of x [T][H] into fp32 qkv, z, b, a.
hipError_t in_proj(const Dims &d, const Proj &pj, const MixerGemms &g, int T, const void *x,
                   char *base, const MixerWs &w, hipStream_t s)
{
    void *bw = base + w.blas;
    hipError_t e;
    if ((e = g.qkv.run(x, pj.w_qkv, reinterpret_cast<float *>(base + w.qkv), bw, kBlasWorkspace,
                       s)) != hipSuccess)
        return e;
    if ((e = g.z.run(x, pj.w_z, reinterpret_cast<float *>(base + w.z), bw, kBlasWorkspace, s)) !=
        hipSuccess)
        return e;
    if (g.gate_kernel) {
        const dim3 grid((2 * d.h_v + 3) / 4, (T + kGateRows - 1) / kGateRows);
        hipLaunchKernelGGL(gates_proj_kernel, grid, dim3(256), 0, s,
                           static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(pj.w_b),
                           static_cast<const bf16_t *>(pj.w_a), reinterpret_cast<float *>(base + w.b),
                           reinterpret_cast<float *>(base + w.a), T, pj.hidden, d.h_v);
        return hipGetLastError();
    }
    if ((e = g.b.run(x, pj.w_b, reinterpret_cast<float *>(base + w.b), bw, kBlasWorkspace, s)) !=
        hipSuccess)
        return e;
    return g.a.run(x, pj.w_a, reinterpret_cast<float *>(base + w.a), bw, kBlasWorkspace, s);
}

// out_proj of the core output split into bf16 parts: y = hi . W_out^T +
// lo . W_out^T, one GEMM over the stacked [hi; lo] rows and a pass that adds
// the halves (split here from the fp32 core output when `split_here`).
hipError_t out_proj(const Dims &d, const Proj &pj, const MixerGemms &g, int T, char *base,
                    const MixerWs &w, void *y, bool split_here, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const size_t n4 = (size_t)T * d.value_dim / 4;
    bf16_t *hi = reinterpret_cast<bf16_t *>(base + w.hl), *lo = hi + (size_t)T * d.value_dim;
    hipError_t e;
    if (split_here) {
        hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           reinterpret_cast<const float *>(base + w.core), hi, lo, n4);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    float *acc = reinterpret_cast<float *>(base + w.acc);
    if ((e = g.out.run(hi, pj.w_out, acc, base + w.blas, kBlasWorkspace, s)) != hipSuccess)
        return e;
    const size_t m4 = (size_t)T * pj.hidden / 4;
    hipLaunchKernelGGL(add_halves_kernel, dim3((unsigned)((m4 + 255) / 256)), dim3(256), 0, s, acc, y,
                       m4, d.out_bf16);
    return hipGetLastError();
}

} // namespace

size_t mixer_workspace_bytes(const Dims &d, int hidden, int n_seq, int t_total, bool prefill)
{
    const size_t dec = mixer_ws(d, hidden, t_total, t_total, false).total;
    if (!prefill) return dec;
    // (the prefill size also covers a decode step of up to t_total sequences)
    const size_t pre = mixer_ws(d, hidden, n_seq, t_total, true).total;
    return pre > dec ? pre : dec;
}

hipError_t launch_mixer_prefill(const Dims &d, const Params &p, const Proj &pj, int n_seq,
                                int t_total, int max_len, const int32_t *cu_host,
                                const int32_t *cu_dev, const void *x,
                                const float *state_in, float *state_out, const float *conv_in,
                                float *conv_out, void *y, void *ws, hipStream_t s)
{
    const MixerWs w = mixer_ws(d, pj.hidden, n_seq, t_total, true);
    char *base = static_cast<char *>(ws);
    MixerGemms g;
    hipError_t e;
    if ((e = prepare_gemms(d, pj, t_total, x, g)) != hipSuccess) return e;
    if ((e = in_proj(d, pj, g, t_total, x, base, w, s)) != hipSuccess) return e;
    if ((e = launch_prefill(core_dims(d, true), p, n_seq, t_total, max_len, cu_host, cu_dev,
                            base + w.qkv,
                            base + w.z, base + w.a, base + w.b, state_in, state_out, conv_in,
                            conv_out, base + w.hl, base + w.prefill, s)) != hipSuccess)
        return e;
    return out_proj(d, pj, g, t_total, base, w, y, false, s);
}

// The decode step with its projections on the matrix cores (skinny.hip):
// possible for up to 64 sequences, a hidden size and value_dim that split
// into contraction slices (multiples of 256), 16-byte aligned x and
// weights, and a core that takes the one-token path.
static bool fused_decode_ok(const Dims &d, const Proj &pj, int batch, const void *x)
{
    const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(pj.w_qkv) |
                         reinterpret_cast<uintptr_t>(pj.w_z) | reinterpret_cast<uintptr_t>(pj.w_b) |
                         reinterpret_cast<uintptr_t>(pj.w_a) | reinterpret_cast<uintptr_t>(pj.w_out);
    return batch <= kSkinnyRows && (al & 15) == 0 && skinny_ksplit(pj.hidden, 1) > 0 &&
           skinny_ksplit(d.value_dim, 2) > 0 && d.h_v % 4 == 0 && // (epilogue: column quads)
           decode_multi_lds_bytes(core_dims(d, true), 1) <= kDecodeMultiMaxLds;
}

// in_proj (one skinny product over the four weights, then the conv epilogue
// into fp32 activations), the core on convolved activations writing bf16 hi
// and lo parts, and out_proj over both parts with its epilogue.
static hipError_t mixer_decode_fused(const Dims &d, const Params &p, const Proj &pj, int batch,
                                     const void *x, float *conv_state, float *state, void *y,
                                     char *base, const MixerWs &w, hipStream_t s)
{
    const int gw = d.chan_decay ? d.d_k : 1;
    const int s1 = d.conv_dim, s2 = s1 + d.value_dim, s3 = s2 + d.h_v, n_in = s3 + d.h_v * gw;
    SkinnyGemm g{};
    g.a[0] = static_cast<const bf16_t *>(x);
    g.a[1] = nullptr;
    g.M = batch;
    g.K = pj.hidden;
    g.N = n_in;
    g.w[0] = static_cast<const bf16_t *>(pj.w_qkv);
    g.w[1] = static_cast<const bf16_t *>(pj.w_z);
    g.w[2] = static_cast<const bf16_t *>(pj.w_b);
    g.w[3] = static_cast<const bf16_t *>(pj.w_a);
    g.wstart[0] = 0, g.wstart[1] = s1, g.wstart[2] = s2, g.wstart[3] = s3;
    g.part = reinterpret_cast<float *>(base + w.part_in);
    hipError_t e;
    ProjEpilogue pe{};
    pe.part = g.part;
    pe.ksplit = skinny_ksplit(g.K, 1);
    pe.M = batch;
    pe.N = n_in;
    pe.start[0] = 0, pe.start[1] = s1, pe.start[2] = s2, pe.start[3] = s3, pe.start[4] = n_in;
    pe.dst[0] = reinterpret_cast<float *>(base + w.qkv);
    pe.dst[1] = reinterpret_cast<float *>(base + w.z);
    pe.dst[2] = reinterpret_cast<float *>(base + w.b);
    pe.dst[3] = reinterpret_cast<float *>(base + w.a);
    pe.conv_w = p.conv_w;
    pe.conv_state = conv_state;
    pe.conv_k = d.conv_k;
    // A few rows: one contraction slice, the product kernel applies the
    // epilogue (B=1: 30.6 against 34.1 us per mixer step at hidden 2048).
    // More rows: split slices (B=64: the product with its epilogue took
    // 37 us, the split product 13.6 us).  With two slices at d_k = d_v = 128
    // the core sums them as it loads its inputs and runs the conv itself
    // (B=64: saves the separate epilogue launch, 6.8 us); otherwise a
    // separate, vectorised epilogue writes the convolved activations.
    Dims c = core_dims(d, true);
    bf16_t *hi = reinterpret_cast<bf16_t *>(base + w.hl);
    const bool direct = batch <= kSkinnyDirectRows && skinny_direct_ok(g.K);
    const bool core_sums = !direct && pe.ksplit == 2 && !d.chan_decay && d.d_k == 128 && d.d_v == 128;
    if (direct) {
        if ((e = launch_skinny_gemm(g, 1, &pe, s)) != hipSuccess) return e;
    } else {
        if ((e = launch_skinny_gemm(g, 1, nullptr, s)) != hipSuccess) return e;
        if (!core_sums && (e = launch_proj_epilogue(pe, s)) != hipSuccess) return e;
    }
    if (core_sums) {
        c.in_split = 2;
        c.in_ld = n_in;
        c.in_split_stride = (size_t)batch * n_in;
        const float *part = g.part;
        e = launch_decode_multi(c, p, batch, 1, nullptr, part, part + s1, part + s3, part + s2,
                                conv_state, conv_state, state, state, nullptr, hi, s);
    } else {
        c.preconv = 1;
        e = launch_decode_multi(c, p, batch, 1, nullptr, base + w.qkv, base + w.z, base + w.a,
                                base + w.b, conv_state, conv_state, state, state, nullptr, hi, s);
    }
    if (e != hipSuccess) return e;
    SkinnyGemm o{};
    o.a[0] = hi;
    o.a[1] = hi + (size_t)batch * d.value_dim;
    o.M = batch;
    o.K = d.value_dim;
    o.N = pj.hidden;
    o.w[0] = o.w[1] = o.w[2] = o.w[3] = static_cast<const bf16_t *>(pj.w_out);
    o.wstart[0] = 0, o.wstart[1] = o.wstart[2] = o.wstart[3] = pj.hidden;
    o.part = reinterpret_cast<float *>(base + w.part_out);
    if ((e = launch_skinny_gemm(o, 2, nullptr, s)) != hipSuccess) return e;
    return launch_out_epilogue(o.part, skinny_ksplit(o.K, 2), (size_t)batch * pj.hidden, y,
                               d.out_bf16, s);
}

hipError_t launch_mixer_decode(const Dims &d, const Params &p, const Proj &pj, int batch,
                               const void *x, float *conv_state, float *state, void *y, void *ws,
                               hipStream_t s)
{
    const MixerWs w = mixer_ws(d, pj.hidden, batch, batch, false);
    char *base = static_cast<char *>(ws);
    if (fused_decode_ok(d, pj, batch, x))
        return mixer_decode_fused(d, p, pj, batch, x, conv_state, state, y, base, w, s);
    MixerGemms g;
    hipError_t e;
    if ((e = prepare_gemms(d, pj, batch, x, g)) != hipSuccess) return e;
    if ((e = in_proj(d, pj, g, batch, x, base, w, s)) != hipSuccess) return e;
    const Dims c = core_dims(d, true);
    const bool multi = decode_multi_lds_bytes(c, 1) <= kDecodeMultiMaxLds;
    if (multi)
        e = launch_decode_multi(c, p, batch, 1, nullptr, base + w.qkv, base + w.z, base + w.a,
                                base + w.b, conv_state, conv_state, state, state, nullptr,
                                base + w.hl, s);
    else // the persistent kernel (very wide groups) writes fp32
        e = launch_decode(core_dims(d, false), p, batch, base + w.qkv, base + w.z, base + w.a,
                          base + w.b, conv_state, state, base + w.core, s);
    if (e != hipSuccess) return e;
    return out_proj(d, pj, g, batch, base, w, y, !multi, s);
}

} // namespace gdn
