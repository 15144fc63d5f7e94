// Fused single-token decode step of the Gated DeltaNet mixer core on gfx950.
//
// A unit of work is one (sequence, key head): the q/k conv channels of that
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
// The grid is persistent (at most one workgroup per CU): each workgroup
// walks its units and, while it updates and writes back one unit's state,
// already has the next unit's state in flight in a second register set, so
// HBM sees a steady mix of reads and writes instead of a read wave followed
// by a write wave.
//
// Thread layout for one value head: 2*d_v threads = (d_v/4 column quads) x
// (8 row groups); thread (c4, rg) holds rows rg, rg+8, ... of columns
// 4*c4 .. 4*c4+3.  A wavefront load instruction therefore reads two adjacent
// 512-byte state rows (d_v = 128).

#include <atomic>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct DecodeArgs {
    const void *qkv, *z, *a, *b;
    const float *conv_w, *a_log, *dt_bias, *norm_w;
    const float *decay_coef; // when not NULL, the log-decay coefficient itself (a_log NULL)
    float *conv_state, *state;
    void *out;
    int h_k, h_v, group, conv_k, conv_dim, value_dim;
    int gate, out_bf16, tiled;
    float norm_eps, l2_eps;
    int units; // batch * h_k
};

// Barrier for LDS traffic only (the waves of a workgroup exchange nothing
// through global memory), so that state loads in flight for the next unit
// are not drained at every barrier.
__device__ __forceinline__ void lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

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
    const int slot = tid / TPH;
    const int lt = tid % TPH;
    const int c4 = lt % C4;
    const int rg = lt / C4;
    const int group = p.group;
    const int K = p.conv_k;
    const int CD = p.conv_dim;
    const int G = gridDim.x;

    extern __shared__ float smem[];
    float *sq = smem;                      // [DK] conv(q) of key head hk
    float *sk = sq + DK;                   // [DK] conv(k)
    float *sv = sk + DK;                   // [group][DV] conv(v)
    f32x4 *red = reinterpret_cast<f32x4 *>(sv + group * DV); // [NSLOT][RG][C4][2]
    float *scal = reinterpret_cast<float *>(red + NSLOT * RG * C4 * 2); // [4]

    // Value head of member hl of unit u's group.
    auto vhead = [&](int u, int hl) { return value_head_of(u % p.h_k, hl, p.h_k, group, p.tiled); };
    auto state_ptr = [&](int u, int hl) {
        const int bs = u / p.h_k;
        return p.state + ((size_t)bs * p.h_v + vhead(u, hl)) * DK * DV;
    };
    auto load_state = [&](f32x4 (&s)[RPT], int u, int hl) {
        const float *Sp = state_ptr(u, hl);
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            s[r] = *reinterpret_cast<const f32x4 *>(Sp + (size_t)(rg + RG * r) * DV + 4 * c4);
    };

    // One unit.  s holds its first pass's state slab (loaded during the
    // previous unit).  Every other global load of the unit is issued first;
    // only then is the next unit's first slab put in flight into s_next, so
    // that (loads complete in issue order) no wait of this unit covers it.
    // Conv channel l of unit u (q, then k, then the group's v channels).
    const TIn *qkv = static_cast<const TIn *>(p.qkv);
    const int nch = 2 * DK + group * DV;
    auto channel = [&](int u, int l) {
        const int hk = u % p.h_k;
        if (l < DK) return hk * DK + l;
        if (l < 2 * DK) return p.h_k * DK + hk * DK + (l - DK);
        const int lv = l - 2 * DK;
        return 2 * p.h_k * DK + vhead(u, lv / DV) * DV + lv % DV;
    };
    // Raw input and history of this thread's first channel of a unit, loaded
    // one unit ahead (further channels, when a unit has more than NT, are
    // loaded when used).
    float cx = 0.0f, ch0 = 0.0f, ch1 = 0.0f, ch2 = 0.0f;
    float cw[4] = {0.f, 0.f, 0.f, 0.f};
    const float4 w4 = *reinterpret_cast<const float4 *>(p.norm_w + 4 * c4); // same for every head
    // The first pass's gate inputs and z of a unit, also loaded one unit
    // ahead and kept as raw values until used (the decay coefficient as
    // stored: A_log, or the coefficient itself).
    const float *coef_src = p.decay_coef ? p.decay_coef : p.a_log;
    auto coef_of = [&](float raw) { return p.decay_coef ? raw : -expf(raw); };
    const TIn *pa = static_cast<const TIn *>(p.a), *pb = static_cast<const TIn *>(p.b);
    const TIn *pz = static_cast<const TIn *>(p.z);
    TIn nb = TIn(0), na = TIn(0);
    float nalog = 0.0f, ndtb = 0.0f;
    RawQuad<TIn> nz;
    auto load_gates = [&](int u) {
        const int bs = u / p.h_k, hv = vhead(u, slot);
        nb = pb[(size_t)bs * p.h_v + hv];
        na = pa[(size_t)bs * p.h_v + hv];
        nalog = coef_src[hv];
        ndtb = p.dt_bias[hv];
        if (rg == 0) nz.load(pz + (size_t)bs * p.value_dim + (size_t)hv * DV + 4 * c4);
    };
    auto load_conv = [&](int u) {
        if (tid < nch) {
            const int bs = u / p.h_k, ch = channel(u, tid);
            cx = load_act(qkv, (size_t)bs * CD + ch);
            const float *hist = p.conv_state + (size_t)bs * (K - 1) * CD + ch;
            if (K > 1) ch0 = hist[0];
            if (K > 2) ch1 = hist[(size_t)CD];
            if (K > 3) ch2 = hist[(size_t)2 * CD];
            const float *w = p.conv_w + (size_t)ch * K;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < K) cw[j] = w[j];
        }
    };
    // silu(conv) of one channel from its raw input x, history prev[] and
    // taps w[], and the history shifted in place.
    auto conv_one = [&](int u, int l, float x, const float (&prev)[3], const float (&w)[4]) {
        const int bs = u / p.h_k, ch = channel(u, l);
        float *hist = p.conv_state + (size_t)bs * (K - 1) * CD + ch;
        float acc = 0.0f;
        for (int j = 0; j < K - 1; ++j) acc = fmaf(w[j], prev[j], acc);
        acc = fmaf(w[K - 1], x, acc);
        for (int j = 0; j + 1 < K - 1; ++j) hist[(size_t)j * CD] = prev[j + 1];
        if (K > 1) hist[(size_t)(K - 2) * CD] = x;
        smem[l] = siluf_(acc);
    };

    auto run_unit = [&](int u, f32x4 (&s)[RPT], f32x4 (&s_next)[RPT]) {
        const int bs = u / p.h_k;
        lds_sync(); // the previous unit's LDS reads are done

        // Causal conv + SiLU of this unit's channels, history update in
        // place (each channel has exactly one reader/writer: this thread).
        if (tid < nch) {
            const float prev[3] = {ch0, ch1, ch2};
            conv_one(u, tid, cx, prev, cw);
        }
        for (int l = tid + NT; l < nch; l += NT) {
            const int ch = channel(u, l);
            const float *hist = p.conv_state + (size_t)bs * (K - 1) * CD + ch;
            float prev[3] = {0.f, 0.f, 0.f}, w[4] = {0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < K - 1; ++j) prev[j] = hist[(size_t)j * CD];
            for (int j = 0; j < K; ++j) w[j] = p.conv_w[(size_t)ch * K + j];
            conv_one(u, l, load_act(qkv, (size_t)bs * CD + ch), prev, w);
        }
        // Gates and z of the first pass (prefetched), of later passes loaded
        // when used.
        float g_b = act_to_f32(nb), g_a = act_to_f32(na), g_alog = nalog, g_dtb = ndtb;
        float4 z4 = nz.to_f32();
        auto load_pass = [&](int hv) {
            g_b = load_act(pb, (size_t)bs * p.h_v + hv);
            g_a = load_act(pa, (size_t)bs * p.h_v + hv);
            g_alog = coef_src[hv];
            g_dtb = p.dt_bias[hv];
            if (rg == 0) z4 = load_act4(pz, (size_t)bs * p.value_dim + (size_t)hv * DV + 4 * c4);
        };
        asm volatile("" ::: "memory");
        if (u + G < p.units) {
            load_gates(u + G);
            load_conv(u + G);
            load_state(s_next, u + G, slot);
        }
        lds_sync();

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
        lds_sync();
        const float qs = scal[0], ks = scal[1], qk = scal[2];

        const int npass = group / NSLOT;
        for (int pass = 0; pass < npass; ++pass) {
            const int hl = pass * NSLOT + slot; // value head within the group
            const int hv = vhead(u, hl);
            float *Sp = state_ptr(u, hl);
            if (pass > 0) {
                load_state(s, u, hl);
                load_pass(hv);
            }
            // Gates ("cherenkov qwen4_exp/cpu.rs" fn deltanet).
            const float beta = sigmoidf_(g_b);
            const float g = coef_of(g_alog) * softplusf_(g_a + g_dtb);
            const float alpha = expf(g);

            f32x4 mk = {0.f, 0.f, 0.f, 0.f}, mq = mk;
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rg + RG * r;
                mk += (sk[i] * ks) * s[r];
                mq += (sq[i] * qs) * s[r];
            }
            f32x4 *rd = red + (size_t)slot * RG * C4 * 2;
            rd[(rg * C4 + c4) * 2 + 0] = mk;
            rd[(rg * C4 + c4) * 2 + 1] = mq;
            lds_sync();
            f32x4 MK = rd[c4 * 2 + 0], MQ = rd[c4 * 2 + 1];
#pragma unroll
            for (int g2 = 1; g2 < RG; ++g2) {
                MK += rd[(g2 * C4 + c4) * 2 + 0];
                MQ += rd[(g2 * C4 + c4) * 2 + 1];
            }
            const f32x4 v4 = *reinterpret_cast<const f32x4 *>(sv + hl * DV + 4 * c4);
            f32x4 delta, o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                delta[e] = beta * (v4[e] - alpha * MK[e]);
                o[e] = fmaf(alpha, MQ[e], qk * delta[e]);
            }
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rg + RG * r;
                const float kv = sk[i] * ks;
                f32x4 sn;
#pragma unroll
                for (int e = 0; e < 4; ++e) sn[e] = fmaf(alpha, s[r][e], kv * delta[e]);
                *reinterpret_cast<f32x4 *>(Sp + (size_t)i * DV + 4 * c4) = sn;
            }

            // Gated RMSNorm over the d_v lanes of this head.
            float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
            ss = group_sum<C4>(ss);
            if (rg == 0) {
                const float rn = rsqrtf(ss / DV + p.norm_eps);
                const size_t base = (size_t)bs * p.value_dim + (size_t)hv * DV + 4 * c4;
                float4 y;
                y.x = o[0] * rn * w4.x * gatef_(z4.x, p.gate);
                y.y = o[1] * rn * w4.y * gatef_(z4.y, p.gate);
                y.z = o[2] * rn * w4.z * gatef_(z4.z, p.gate);
                y.w = o[3] * rn * w4.w * gatef_(z4.w, p.gate);
                store_out4(p.out, base, y, p.out_bf16);
            }
            if (pass + 1 < npass) lds_sync();
        }
    };

    // Units u = blockIdx.x + k G, alternating between the two register sets.
    f32x4 sa[RPT], sb[RPT];
    int u = blockIdx.x;
    if (u < p.units) {
        load_gates(u);
        load_conv(u);
        load_state(sa, u, slot);
    }
    for (; u < p.units; u += 2 * G) {
        run_unit(u, sa, sb);
        if (u + G < p.units) run_unit(u + G, sb, sa);
    }
}

// Compute units per device, queried on first use.  Concurrent first calls
// may both query; they store the same value, and the atomics make the
// cache safe to read from any thread.
hipError_t device_cu_count(int *n)
{
    static std::atomic<int> ncu[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int c = ncu[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        c = c > 0 ? c : 1;
        ncu[dev].store(c, std::memory_order_relaxed);
    }
    *n = c;
    return hipSuccess;
}

template <typename TIn, int DK, int DV, int NSLOT>
static hipError_t launch_t(const DecodeArgs &a, int batch, hipStream_t s)
{
    constexpr int NT = 2 * DV * NSLOT;
    const size_t shmem = sizeof(float) * (2 * DK + a.group * DV) +
                         sizeof(f32x4) * NSLOT * 8 * (DV / 4) * 2 + 4 * sizeof(float);
    // One workgroup per CU at most (each holds two state slabs in registers).
    int ncu = 0;
    const hipError_t e = device_cu_count(&ncu);
    if (e != hipSuccess) return e;
    DecodeArgs args = a;
    args.units = batch * a.h_k;
    const int grid = args.units < ncu ? args.units : ncu;
    hipLaunchKernelGGL((decode_kernel<TIn, DK, DV, NSLOT>), dim3(grid), dim3(NT), shmem, s, args);
    return hipGetLastError();
}

template <typename TIn, int DK, int DV>
static hipError_t launch_slots(const DecodeArgs &a, int batch, hipStream_t s)
{
    // Two value heads of a group side by side when the group allows it.
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
    if (batch <= 0) return hipSuccess;
    DecodeArgs args;
    args.qkv = qkv;
    args.z = z;
    args.a = a;
    args.b = b;
    args.conv_w = p.conv_w;
    args.a_log = p.a_log;
    args.decay_coef = p.decay_coef;
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
    args.tiled = d.tiled;
    args.out_bf16 = d.out_bf16;
    args.norm_eps = d.norm_eps;
    args.l2_eps = d.l2_eps;
    args.units = 0;
    if (d.act_bf16) return launch_dims<bf16_t>(args, d.d_k, d.d_v, batch, s);
    return launch_dims<float>(args, d.d_k, d.d_v, batch, s);
}

} // namespace gdn
