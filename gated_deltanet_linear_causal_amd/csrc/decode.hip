// Fused single-token decode step of the Gated DeltaNet mixer core on gfx950.
//
// One workgroup owns one (sequence, key head): the q/k conv channels of that
// key head and the v channels of every value head in its group, so the
// in-place conv-history update has exactly one writer per channel.  For
// each value head hv (processed NSLOT at a time) the [d_k][d_v] fp32 state
// is streamed HBM -> VGPR once and written back once:
//
//   m = S_old^T k^,  r = S_old^T q^          (one pass over S_old)
//   delta = beta (v - alpha m)               (S is decayed first)
//   o = alpha r + (q^.k^) delta              (= S_new^T q^)
//   S_new = alpha S_old + k^ delta^T
//
// which is the per-token recurrence of "cherenkov qwen4_exp/cpu.rs"
// fn deltanet with the two state reads fused.  The path is bound by HBM:
// every other step (conv, norms, gates, gated RMSNorm) is register / LDS
// work hidden under the state stream.
//
// Thread layout for one value head: 2*d_v threads = (d_v/4 column quads) x
// (8 row groups); thread (c4, rg) holds rows rg, rg+8, ... of columns
// 4*c4 .. 4*c4+3 as float4.  A wavefront load instruction therefore reads
// two adjacent 512-byte state rows (d_v = 128).

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct DecodeArgs {
    const void *qkv, *z, *a, *b;
    const float *conv_w, *a_log, *dt_bias, *norm_w;
    float *conv_state, *state;
    void *out;
    int h_k, h_v, group, conv_k, conv_dim, value_dim;
    int gate, out_bf16;
    float norm_eps, l2_eps;
};

template <typename TIn, int DK, int DV, int NSLOT>
__global__ void __launch_bounds__(2 * DV * NSLOT)
decode_kernel(const DecodeArgs p)
{
    constexpr int TPH = 2 * DV;     // threads per value head
    constexpr int NT = TPH * NSLOT; // threads per workgroup
    constexpr int C4 = DV / 4;      // column quads
    constexpr int RG = TPH / C4;    // row groups (8)
    constexpr int RPT = DK / RG;    // state rows per thread
    static_assert(RG == 8 && DK % RG == 0, "layout");

    const int tid = threadIdx.x;
    const int hk = blockIdx.x;
    const int bs = blockIdx.y;
    const int slot = tid / TPH;
    const int lt = tid % TPH;
    const int c4 = lt % C4;
    const int rg = lt / C4;
    const int group = p.group;
    const int K = p.conv_k;
    const int CD = p.conv_dim;

    extern __shared__ float smem[];
    float *sq = smem;                      // [DK] conv(q) of key head hk
    float *sk = sq + DK;                   // [DK] conv(k)
    float *sv = sk + DK;                   // [group][DV] conv(v)
    float4 *red = reinterpret_cast<float4 *>(sv + group * DV); // [NSLOT][RG][C4][2]
    float *scal = reinterpret_cast<float *>(red + NSLOT * RG * C4 * 2); // [4]

    // Issue the first state loads before anything else: they do not depend
    // on the conv and dominate the runtime.
    float4 s[RPT];
    {
        const int hv = hk * group + slot;
        const float *Sp = p.state + ((size_t)bs * p.h_v + hv) * DK * DV;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = *reinterpret_cast<const float4 *>(Sp + (size_t)(rg + RG * r) * DV + 4 * c4);
    }

    // Causal conv + SiLU of this workgroup's channels, history update in
    // place (each channel has exactly one reader/writer: this thread).
    const TIn *qkv = static_cast<const TIn *>(p.qkv);
    const int nch = 2 * DK + group * DV;
    for (int l = tid; l < nch; l += NT) {
        int ch;
        if (l < DK)
            ch = hk * DK + l;
        else if (l < 2 * DK)
            ch = p.h_k * DK + hk * DK + (l - DK);
        else
            ch = 2 * p.h_k * DK + hk * group * DV + (l - 2 * DK);
        const float x = load_act(qkv, (size_t)bs * CD + ch);
        const float *w = p.conv_w + (size_t)ch * K;
        float *hist = p.conv_state + (size_t)bs * (K - 1) * CD + ch;
        float prev[3];
        float acc = 0.0f;
        for (int j = 0; j < K - 1; ++j) {
            prev[j] = hist[(size_t)j * CD];
            acc = fmaf(w[j], prev[j], acc);
        }
        acc = fmaf(w[K - 1], x, acc);
        for (int j = 0; j + 1 < K - 1; ++j) hist[(size_t)j * CD] = prev[j + 1];
        if (K > 1) hist[(size_t)(K - 2) * CD] = x;
        smem[l] = siluf_(acc);
    }
    __syncthreads();

    // L2 norms of q and k and their raw dot product (wave 0).
    if (tid < 64) {
        float ssq = 0.f, ssk = 0.f, dqk = 0.f;
        for (int i = tid; i < DK; i += 64) {
            const float qv = sq[i], kv = sk[i];
            ssq = fmaf(qv, qv, ssq);
            ssk = fmaf(kv, kv, ssk);
            dqk = fmaf(qv, kv, dqk);
        }
        ssq = group_sum<64>(ssq);
        ssk = group_sum<64>(ssk);
        dqk = group_sum<64>(dqk);
        if (tid == 0) {
            const float qs = rsqrtf(ssq + p.l2_eps) * rsqrtf((float)DK);
            const float ks = rsqrtf(ssk + p.l2_eps);
            scal[0] = qs;
            scal[1] = ks;
            scal[2] = dqk * qs * ks; // q^ . k^
        }
    }
    __syncthreads();
    const float qs = scal[0], ks = scal[1], qk = scal[2];

    const int npass = group / NSLOT;
    for (int pass = 0; pass < npass; ++pass) {
        const int hl = pass * NSLOT + slot; // value head within the group
        const int hv = hk * group + hl;
        float *Sp = p.state + ((size_t)bs * p.h_v + hv) * DK * DV;
        if (pass > 0) {
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                s[r] = *reinterpret_cast<const float4 *>(Sp + (size_t)(rg + RG * r) * DV + 4 * c4);
        }
        // Gates ("cherenkov qwen4_exp/cpu.rs" fn deltanet).
        const float beta = sigmoidf_(load_act(static_cast<const TIn *>(p.b), (size_t)bs * p.h_v + hv));
        const float araw = load_act(static_cast<const TIn *>(p.a), (size_t)bs * p.h_v + hv);
        const float g = -expf(p.a_log[hv]) * softplusf_(araw + p.dt_bias[hv]);
        const float alpha = expf(g);

        float4 mk = make_float4(0.f, 0.f, 0.f, 0.f), mq = mk;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + RG * r;
            mk = fma4(sk[i] * ks, s[r], mk);
            mq = fma4(sq[i] * qs, s[r], mq);
        }
        float4 *rd = red + (size_t)slot * RG * C4 * 2;
        rd[(rg * C4 + c4) * 2 + 0] = mk;
        rd[(rg * C4 + c4) * 2 + 1] = mq;
        __syncthreads();
        float4 MK = rd[c4 * 2 + 0], MQ = rd[c4 * 2 + 1];
#pragma unroll
        for (int g2 = 1; g2 < RG; ++g2) {
            MK = MK + rd[(g2 * C4 + c4) * 2 + 0];
            MQ = MQ + rd[(g2 * C4 + c4) * 2 + 1];
        }
        const float4 v4 = *reinterpret_cast<const float4 *>(sv + hl * DV + 4 * c4);
        float4 delta, o;
        delta.x = beta * (v4.x - alpha * MK.x);
        delta.y = beta * (v4.y - alpha * MK.y);
        delta.z = beta * (v4.z - alpha * MK.z);
        delta.w = beta * (v4.w - alpha * MK.w);
        o.x = fmaf(alpha, MQ.x, qk * delta.x);
        o.y = fmaf(alpha, MQ.y, qk * delta.y);
        o.z = fmaf(alpha, MQ.z, qk * delta.z);
        o.w = fmaf(alpha, MQ.w, qk * delta.w);

#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int i = rg + RG * r;
            const float kv = sk[i] * ks;
            float4 sn;
            sn.x = fmaf(alpha, s[r].x, kv * delta.x);
            sn.y = fmaf(alpha, s[r].y, kv * delta.y);
            sn.z = fmaf(alpha, s[r].z, kv * delta.z);
            sn.w = fmaf(alpha, s[r].w, kv * delta.w);
            *reinterpret_cast<float4 *>(Sp + (size_t)i * DV + 4 * c4) = sn;
        }

        // Gated RMSNorm over the d_v lanes of this head.
        float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
        ss = group_sum<C4>(ss);
        if (rg == 0) {
            const float rn = rsqrtf(ss / DV + p.norm_eps);
            const size_t base = (size_t)bs * p.value_dim + (size_t)hv * DV + 4 * c4;
            const float4 z4 = load_act4(static_cast<const TIn *>(p.z), base);
            const float4 w4 = *reinterpret_cast<const float4 *>(p.norm_w + 4 * c4);
            float4 y;
            y.x = o.x * rn * w4.x * gatef_(z4.x, p.gate);
            y.y = o.y * rn * w4.y * gatef_(z4.y, p.gate);
            y.z = o.z * rn * w4.z * gatef_(z4.z, p.gate);
            y.w = o.w * rn * w4.w * gatef_(z4.w, p.gate);
            store_out4(p.out, base, y, p.out_bf16);
        }
        if (pass + 1 < npass) __syncthreads();
    }
}

template <typename TIn, int DK, int DV, int NSLOT>
static hipError_t launch_t(const DecodeArgs &a, int batch, hipStream_t s)
{
    constexpr int NT = 2 * DV * NSLOT;
    const size_t shmem = sizeof(float) * (2 * DK + a.group * DV) +
                         sizeof(float4) * NSLOT * 8 * (DV / 4) * 2 + 4 * sizeof(float);
    hipLaunchKernelGGL((decode_kernel<TIn, DK, DV, NSLOT>), dim3(a.h_k, batch), dim3(NT),
                       shmem, s, a);
    return hipGetLastError();
}

template <typename TIn, int DK, int DV>
static hipError_t launch_slots(const DecodeArgs &a, int batch, hipStream_t s)
{
    // Value heads of a group processed side by side (at most 4, so at most
    // 1024 threads per workgroup for d_v <= 128).
    if (a.group % 4 == 0) return launch_t<TIn, DK, DV, 4>(a, batch, s);
    if (a.group % 2 == 0) return launch_t<TIn, DK, DV, 2>(a, batch, s);
    return launch_t<TIn, DK, DV, 1>(a, batch, s);
}

template <typename TIn>
static hipError_t launch_dims(const DecodeArgs &a, int dk, int dv, int batch, hipStream_t s)
{
#define GDN_DEC_CASE(K_, V_)                                                                  \
    if (dk == K_ && dv == V_) return launch_slots<TIn, K_, V_>(a, batch, s);
    GDN_DEC_CASE(32, 32) GDN_DEC_CASE(32, 64) GDN_DEC_CASE(32, 128)
    GDN_DEC_CASE(64, 32) GDN_DEC_CASE(64, 64) GDN_DEC_CASE(64, 128)
    GDN_DEC_CASE(128, 32) GDN_DEC_CASE(128, 64) GDN_DEC_CASE(128, 128)
#undef GDN_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const Dims &d, const Params &p, int batch, const void *qkv,
                         const void *z, const void *a, const void *b, float *conv_state,
                         float *state, void *out, hipStream_t s)
{
    DecodeArgs args;
    args.qkv = qkv;
    args.z = z;
    args.a = a;
    args.b = b;
    args.conv_w = p.conv_w;
    args.a_log = p.a_log;
    args.dt_bias = p.dt_bias;
    args.norm_w = p.norm_w;
    args.conv_state = conv_state;
    args.state = state;
    args.out = out;
    args.h_k = d.h_k;
    args.h_v = d.h_v;
    args.group = d.group;
    args.conv_k = d.conv_k;
    args.conv_dim = d.conv_dim;
    args.value_dim = d.value_dim;
    args.gate = d.gate;
    args.out_bf16 = d.out_bf16;
    args.norm_eps = d.norm_eps;
    args.l2_eps = d.l2_eps;
    if (d.act_bf16) return launch_dims<bf16_t>(args, d.d_k, d.d_v, batch, s);
    return launch_dims<float>(args, d.d_k, d.d_v, batch, s);
}

} // namespace gdn
