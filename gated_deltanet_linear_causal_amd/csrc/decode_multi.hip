// Multi-token decode of the Gated DeltaNet mixer core on gfx950: a few new
// tokens per sequence (speculative verification), and the replay that
// rewinds a sequence to a position inside such a span.
//
// Unlike a KV cache the recurrent state cannot be truncated, so a rewind
// restarts from the state saved before the span and replays the delta rule
// over the kept tokens ("oxinfer 0.0.5 src/qwen.rs", GdnRecord and
// QwenSession::rewind).  Both operations are this one kernel: the replay is
// the forward with no outputs, so the state it reaches is bit-identical to
// the one the forward reached after the same tokens.
//
// A workgroup owns one (sequence, key head): the q/k channels of the key
// head and the v channels of its value heads.  It
//   1. runs the causal conv + SiLU of every owned channel over the n new
//      tokens (one thread per channel, the K-1 history in registers) into
//      LDS and writes the new history (last K-1 raw inputs);
//   2. forms the q/k L2 scales of every token;
//   3. per value head: loads the [d_k][d_v] fp32 state into registers once,
//      steps it through the n tokens (per token one LDS reduction for
//      S^T k^ and S^T q^, then the rank-one update and the gated RMSNorm),
//      and stores it once.
// The state, the dominant traffic, therefore crosses HBM once per call
// however many tokens the call carries.
//
// Thread layout per value head (as in the single-token kernel): 2*d_v
// threads = (d_v/4 column quads) x (8 row groups); thread (c4, rg) holds rows
// rg, rg+8, ... of columns 4*c4 .. 4*c4+3.

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct MultiArgs {
    const void *qkv, *z, *a, *b;
    const float *conv_w, *a_log, *decay_coef, *dt_bias, *norm_w;
    const float *conv_in;
    float *conv_out;
    const float *state_in;
    float *state_out;
    float *ckpt;         // [batch][t_new][H_v][d_k][d_v] or NULL
    void *out;           // [batch][t_new][value_dim] or NULL
    const int32_t *n_tok; // [batch] tokens to run per sequence, or NULL (= t_new)
    int t_new;
    int h_k, h_v, group, conv_k, conv_dim, value_dim;
    int gate, out_bf16, tiled;
    float norm_eps, l2_eps;
};

__device__ __forceinline__ void lds_sync_m()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float pick3(const float (&w)[3], int i)
{
    return i == 0 ? w[0] : (i == 1 ? w[1] : w[2]);
}

template <typename TIn, int DK, int DV, int NSLOT>
__global__ void __launch_bounds__(2 * DV * NSLOT)
decode_multi_kernel(const MultiArgs p)
{
    constexpr int TPH = 2 * DV;     // threads per value head
    constexpr int NT = TPH * NSLOT; // threads per workgroup
    constexpr int NW = NT / 64;     // waves
    constexpr int C4 = DV / 4;      // column quads
    constexpr int RG = TPH / C4;    // row groups (8)
    constexpr int RPT = DK / RG;    // state rows per thread
    constexpr int RPW = 64 / C4;    // row groups per wave (summed by lane shuffles)
    constexpr int NPART = RG / RPW; // partial sums per column quad left for LDS
    static_assert(RG == 8 && DK % RG == 0 && NT % 64 == 0 && RPW >= 1, "layout");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = __builtin_amdgcn_readfirstlane(tid / TPH); // TPH is a multiple of 64
    const int lt = tid % TPH;
    const int c4 = lt % C4;
    const int rg = lt / C4;
    const int group = p.group, K = p.conv_k, CD = p.conv_dim, T = p.t_new;
    const int u = blockIdx.x, bs = u / p.h_k, hk = u % p.h_k;
    const int nch = 2 * DK + group * DV;
    int n = T;
    if (p.n_tok) n = min(max(p.n_tok[bs], 0), T);
    n = __builtin_amdgcn_readfirstlane(n);

    extern __shared__ __attribute__((aligned(16))) float smem[];
    float *cb = smem;                                      // [T][nch]
    float *scal = cb + (size_t)T * nch;                    // [T][4]
    float *sgate = scal + 4 * T;                           // [T][group][2] beta, alpha
    f32x4 *red = reinterpret_cast<f32x4 *>(sgate + 2 * ((T * group + 1) & ~1)); // [2][NSLOT][NPART][C4][2]

    // ---- 1. causal conv + SiLU of the owned channels, new history --------
    // The window holds the last three raw inputs, oldest first, and the taps
    // are right-aligned to four (zero taps in front when K < 4), so one code
    // path serves every K <= 4.
    const TIn *qkv = static_cast<const TIn *>(p.qkv);
    for (int l = tid; l < nch; l += NT) {
        int ch;
        if (l < DK) ch = hk * DK + l;
        else if (l < 2 * DK) ch = p.h_k * DK + hk * DK + (l - DK);
        else {
            const int lv = l - 2 * DK;
            ch = 2 * p.h_k * DK + value_head_of(hk, lv / DV, p.h_k, group, p.tiled) * DV + lv % DV;
        }
        float win[3] = {0.f, 0.f, 0.f}, tap[4] = {0.f, 0.f, 0.f, 0.f};
        const float *hin = p.conv_in + (size_t)bs * (K - 1) * CD + ch;
#pragma unroll
        for (int pos = 0; pos < 3; ++pos) {
            const int j = pos - 4 + K; // history slot feeding window position pos
            if (j >= 0) win[pos] = hin[(size_t)j * CD];
        }
#pragma unroll
        for (int pos = 0; pos < 4; ++pos) {
            const int j = pos - 4 + K;
            if (j >= 0) tap[pos] = p.conv_w[(size_t)ch * K + j];
        }
        float xs[kDecodeMultiMaxTokens];
#pragma unroll
        for (int t = 0; t < kDecodeMultiMaxTokens; ++t)
            xs[t] = t < n ? load_act(qkv, ((size_t)bs * T + t) * CD + ch) : 0.0f;
#pragma unroll
        for (int t = 0; t < kDecodeMultiMaxTokens; ++t) {
            if (t < n) {
                float acc = 0.0f;
                acc = fmaf(tap[0], win[0], acc);
                acc = fmaf(tap[1], win[1], acc);
                acc = fmaf(tap[2], win[2], acc);
                acc = fmaf(tap[3], xs[t], acc);
                cb[(size_t)t * nch + l] = siluf_(acc);
                win[0] = win[1];
                win[1] = win[2];
                win[2] = xs[t];
            }
        }
        float *hout = p.conv_out + (size_t)bs * (K - 1) * CD + ch;
        for (int j = 0; j < K - 1; ++j) hout[(size_t)j * CD] = pick3(win, 3 - (K - 1) + j);
    }
    lds_sync_m();

    // ---- 2. L2 scales of q and k and q^.k^ per token (a wave per token),
    // and the gates of every (token, value head) ("cherenkov
    // qwen4_exp/cpu.rs" fn deltanet) ------------------------------------
    {
        const TIn *pa = static_cast<const TIn *>(p.a), *pb = static_cast<const TIn *>(p.b);
        for (int i = tid; i < n * group; i += NT) {
            const int t = i / group, hl = i % group;
            const int hv = value_head_of(hk, hl, p.h_k, group, p.tiled);
            const size_t gi = ((size_t)bs * T + t) * p.h_v + hv;
            const float g = decay_coef_of(p.a_log, p.decay_coef, hv) *
                            softplusf_(load_act(pa, gi) + p.dt_bias[hv]);
            sgate[2 * i + 0] = sigmoidf_(load_act(pb, gi));
            sgate[2 * i + 1] = expf(g);
        }
    }
    for (int t = wave; t < n; t += NW) {
        const float *ct = cb + (size_t)t * nch;
        float ssq = 0.f, ssk = 0.f, dqk = 0.f;
        for (int i = lane; i < DK; i += 64) {
            const float qv = ct[i], kv = ct[DK + i];
            ssq = fmaf(qv, qv, ssq);
            ssk = fmaf(kv, kv, ssk);
            dqk = fmaf(qv, kv, dqk);
        }
        ssq = group_sum<64>(ssq);
        ssk = group_sum<64>(ssk);
        dqk = group_sum<64>(dqk);
        if (lane == 0) {
            const float qs = rsqrtf(ssq + p.l2_eps) * rsqrtf((float)DK);
            const float ks = rsqrtf(ssk + p.l2_eps);
            scal[4 * t + 0] = qs;
            scal[4 * t + 1] = ks;
            scal[4 * t + 2] = dqk * qs * ks; // q^ . k^
        }
    }
    lds_sync_m();

    // ---- 3. the delta rule over the tokens, per value head ---------------
    const TIn *pz = static_cast<const TIn *>(p.z);
    const float4 w4 = *reinterpret_cast<const float4 *>(p.norm_w + 4 * c4);
    const int npass = group / NSLOT;
    for (int pass = 0; pass < npass; ++pass) {
        const int hl = pass * NSLOT + slot;
        const int hv = value_head_of(hk, hl, p.h_k, group, p.tiled);
        // Uniform head base plus a 32-bit lane offset, so that row addresses
        // are not kept as 64-bit per-lane pairs.
        const size_t head = ((size_t)bs * p.h_v + hv) * DK * DV;
        const int toff = rg * DV + 4 * c4;
        const float *Sin = p.state_in + head;
        f32x4 s[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = *reinterpret_cast<const f32x4 *>(Sin + toff + r * RG * DV);
#pragma unroll 1
        for (int t = 0; t < n; ++t) {
            const float *ct = cb + (size_t)t * nch;
            const float qs = scal[4 * t + 0], ks = scal[4 * t + 1], qk = scal[4 * t + 2];
            float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
            const size_t obase = ((size_t)bs * T + t) * p.value_dim + (size_t)hv * DV + 4 * c4;
            if (p.out) z4 = load_act4(pz, obase); // (uniform branch: the load stays in flight)
            const float beta = sgate[2 * (t * group + hl) + 0];
            const float alpha = sgate[2 * (t * group + hl) + 1];

            float kk[RPT]; // k^ of this thread's rows, for S^T k^ and the update
            f32x4 mk = {0.f, 0.f, 0.f, 0.f}, mq = mk;
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rg + RG * r;
                kk[r] = ct[DK + i] * ks;
                mk += kk[r] * s[r];
                mq += (ct[i] * qs) * s[r];
            }
            // Sum over the row groups: those of one wave by lane shuffles,
            // the waves' partials through LDS (double-buffered by token
            // parity, so one barrier per token).
#pragma unroll
            for (int off = C4; off < 64; off <<= 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mk[e] += __shfl_xor(mk[e], off, 64);
                    mq[e] += __shfl_xor(mq[e], off, 64);
                }
            }
            f32x4 *rd = red + ((size_t)(t & 1) * NSLOT + slot) * NPART * C4 * 2;
            if (rg % RPW == 0) {
                rd[((rg / RPW) * C4 + c4) * 2 + 0] = mk;
                rd[((rg / RPW) * C4 + c4) * 2 + 1] = mq;
            }
            lds_sync_m();
            f32x4 MK = rd[c4 * 2 + 0], MQ = rd[c4 * 2 + 1];
#pragma unroll
            for (int g2 = 1; g2 < NPART; ++g2) {
                MK += rd[(g2 * C4 + c4) * 2 + 0];
                MQ += rd[(g2 * C4 + c4) * 2 + 1];
            }
            const f32x4 v4 = *reinterpret_cast<const f32x4 *>(ct + 2 * DK + hl * DV + 4 * c4);
            f32x4 delta, o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                delta[e] = beta * (v4[e] - alpha * MK[e]);
                o[e] = fmaf(alpha, MQ[e], qk * delta[e]); // = S_new^T q^
            }
            // (one row at a time: the scheduler would otherwise form all
            // the k delta^T products first and double the live registers)
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s[r][e] = fmaf(alpha, s[r][e], kk[r] * delta[e]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (p.ckpt) {
                float *cp = p.ckpt + (((size_t)bs * T + t) * p.h_v + hv) * DK * DV;
#pragma unroll
                for (int r = 0; r < RPT; ++r)
                    *reinterpret_cast<f32x4 *>(cp + toff + r * RG * DV) = s[r];
            }
            if (p.out) {
                // Gated RMSNorm over the d_v lanes of this head.
                float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
                ss = group_sum<C4>(ss);
                if (rg == 0) {
                    const float rn = rsqrtf(ss / DV + p.norm_eps);
                    float4 y;
                    y.x = o[0] * rn * w4.x * gatef_(z4.x, p.gate);
                    y.y = o[1] * rn * w4.y * gatef_(z4.y, p.gate);
                    y.z = o[2] * rn * w4.z * gatef_(z4.z, p.gate);
                    y.w = o[3] * rn * w4.w * gatef_(z4.w, p.gate);
                    store_out4(p.out, obase, y, p.out_bf16);
                }
            }
        }
        float *Sout = p.state_out + head;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            *reinterpret_cast<f32x4 *>(Sout + toff + r * RG * DV) = s[r];
        if (pass + 1 < npass) lds_sync_m(); // the reduction buffers are reused
    }
}

// LDS of one workgroup: [T][nch] conv outputs, [T][4] q/k scales,
// [T][group][2] gates (padded to 16 bytes) and [2][NSLOT][NPART][d_v/4][2]
// f32x4 reduction partials.
size_t decode_multi_lds_bytes(const Dims &d, int t_new)
{
    const int nch = 2 * d.d_k + d.group * d.d_v;
    const int nslot = d.group % 2 == 0 ? 2 : 1;
    const int c4 = d.d_v / 4, npart = 8 / (64 / c4 < 8 ? 64 / c4 : 8);
    const size_t gates = 2 * (((size_t)t_new * d.group + 1) & ~(size_t)1);
    return sizeof(float) * ((size_t)t_new * nch + 4 * (size_t)t_new + gates) +
           sizeof(f32x4) * 2 * nslot * npart * c4 * 2;
}

template <typename TIn, int DK, int DV, int NSLOT>
static hipError_t launch_multi_t(const MultiArgs &a, int batch, hipStream_t s)
{
    constexpr int NT = 2 * DV * NSLOT;
    Dims d;
    d.d_k = DK;
    d.d_v = DV;
    d.group = a.group;
    const size_t shmem = decode_multi_lds_bytes(d, a.t_new); // <= 64 KiB, checked by the caller
    hipLaunchKernelGGL((decode_multi_kernel<TIn, DK, DV, NSLOT>), dim3(batch * a.h_k), dim3(NT),
                       shmem, s, a);
    return hipGetLastError();
}

template <typename TIn, int DK, int DV>
static hipError_t launch_multi_slots(const MultiArgs &a, int batch, hipStream_t s)
{
    if (a.group % 2 == 0) return launch_multi_t<TIn, DK, DV, 2>(a, batch, s);
    return launch_multi_t<TIn, DK, DV, 1>(a, batch, s);
}

template <typename TIn>
static hipError_t launch_multi_dims(const MultiArgs &a, int dk, int dv, int batch, hipStream_t s)
{
#define GDN_MULTI_CASE(K_, V_)                                                                \
    if (dk == K_ && dv == V_) return launch_multi_slots<TIn, K_, V_>(a, batch, s);
    GDN_MULTI_CASE(32, 32) GDN_MULTI_CASE(32, 64) GDN_MULTI_CASE(32, 128)
    GDN_MULTI_CASE(64, 32) GDN_MULTI_CASE(64, 64) GDN_MULTI_CASE(64, 128)
    GDN_MULTI_CASE(128, 32) GDN_MULTI_CASE(128, 64) GDN_MULTI_CASE(128, 128)
#undef GDN_MULTI_CASE
    return hipErrorInvalidValue;
}


hipError_t launch_decode_multi(const Dims &d, const Params &p, int batch, int t_new,
                               const int32_t *n_tok, const void *qkv, const void *z,
                               const void *a, const void *b, const float *conv_in,
                               float *conv_out, const float *state_in, float *state_out,
                               float *ckpt, void *out, hipStream_t s)
{
    if (batch <= 0) return hipSuccess;
    MultiArgs args;
    args.qkv = qkv;
    args.z = z;
    args.a = a;
    args.b = b;
    args.conv_w = p.conv_w;
    args.a_log = p.a_log;
    args.decay_coef = p.decay_coef;
    args.dt_bias = p.dt_bias;
    args.norm_w = p.norm_w;
    args.conv_in = conv_in;
    args.conv_out = conv_out;
    args.state_in = state_in;
    args.state_out = state_out;
    args.ckpt = ckpt;
    args.out = out;
    args.n_tok = n_tok;
    args.t_new = t_new;
    args.h_k = d.h_k;
    args.h_v = d.h_v;
    args.group = d.group;
    args.conv_k = d.conv_k;
    args.conv_dim = d.conv_dim;
    args.value_dim = d.value_dim;
    args.gate = d.gate;
    args.out_bf16 = d.out_bf16;
    args.tiled = d.tiled;
    args.norm_eps = d.norm_eps;
    args.l2_eps = d.l2_eps;
    if (d.act_bf16) return launch_multi_dims<bf16_t>(args, d.d_k, d.d_v, batch, s);
    return launch_multi_dims<float>(args, d.d_k, d.d_v, batch, s);
}

} // namespace gdn
