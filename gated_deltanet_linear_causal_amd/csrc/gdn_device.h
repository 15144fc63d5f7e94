// Device helpers shared by the gfx950 kernels of the GDN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bf16 lives in memory as its 16 raw bits.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h)
{
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ bf16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> __device__ __forceinline__ float load_act(const T *p, size_t i);
template <> __device__ __forceinline__ float load_act<float>(const float *p, size_t i)
{
    return p[i];
}
template <> __device__ __forceinline__ float load_act<bf16_t>(const bf16_t *p, size_t i)
{
    return bf16_bits_to_f32(p[i]);
}

// Four consecutive activations starting at a multiple of 4.
template <typename T> __device__ __forceinline__ float4 load_act4(const T *p, size_t i);
template <> __device__ __forceinline__ float4 load_act4<float>(const float *p, size_t i)
{
    return *reinterpret_cast<const float4 *>(p + i);
}
template <> __device__ __forceinline__ float4 load_act4<bf16_t>(const bf16_t *p, size_t i)
{
    const uint2 u = *reinterpret_cast<const uint2 *>(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// Raw activation values, converted to fp32 only where they are used (a
// conversion right after the load would wait for it).
__device__ __forceinline__ float act_to_f32(float v) { return v; }
__device__ __forceinline__ float act_to_f32(bf16_t v) { return bf16_bits_to_f32(v); }
template <typename T> struct RawQuad;
template <> struct RawQuad<float> {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    __device__ __forceinline__ void load(const float *p) { v = *reinterpret_cast<const float4 *>(p); }
    __device__ __forceinline__ float4 to_f32() const { return v; }
};
template <> struct RawQuad<bf16_t> {
    uint2 v = make_uint2(0u, 0u);
    __device__ __forceinline__ void load(const bf16_t *p) { v = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ float4 to_f32() const
    {
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
};

// Store four consecutive outputs as fp32 or bf16.
__device__ __forceinline__ void store_out4(void *out, size_t i, float4 v, bool bf16)
{
    if (bf16) {
        const uint32_t lo = f32_to_bf16(v.x) | (uint32_t(f32_to_bf16(v.y)) << 16);
        const uint32_t hi = f32_to_bf16(v.z) | (uint32_t(f32_to_bf16(v.w)) << 16);
        *reinterpret_cast<uint2 *>(static_cast<bf16_t *>(out) + i) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(out) + i) = v;
    }
}

// Four fp32 outputs as two bf16 parts, hi = bf16(v) at out[i] and
// lo = bf16(v - hi) at out[lo_off + i] (the operands of a split-bf16
// product).
__device__ __forceinline__ void store_split4(void *out, size_t i, size_t lo_off, float4 v)
{
    const float x[4] = {v.x, v.y, v.z, v.w};
    bf16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = f32_to_bf16(x[e]);
        l[e] = f32_to_bf16(x[e] - bf16_bits_to_f32(h[e]));
    }
    bf16_t *o = static_cast<bf16_t *>(out);
    *reinterpret_cast<uint2 *>(o + i) =
        make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
    *reinterpret_cast<uint2 *>(o + lo_off + i) =
        make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16));
}

__device__ __forceinline__ void store_out1(void *out, size_t i, float v, bool bf16)
{
    if (bf16)
        static_cast<bf16_t *>(out)[i] = f32_to_bf16(v);
    else
        static_cast<float *>(out)[i] = v;
}

// Nonlinearities of the mixer ("cortiq-engine 0.6.5 src/qwen4_exp.rs"
// fn sigmoid / fn silu; softplus with threshold 20 as in "oxinfer 0.0.5
// src/qwen.rs" DeltaRule::run).  Full-precision expf/log1pf.
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * sigmoidf_(x); }
__device__ __forceinline__ float softplusf_(float x) { return x > 20.0f ? x : log1pf(expf(x)); }
// The same softplus with the hardware exponential and logarithm, for the
// per-channel decays (d_k of them per token and value head): x above 20,
// below it max(x, 0) + log(1 + e^{-|x|}), absolute error about 1e-7.
__device__ __forceinline__ float softplus_hw(float x)
{
    return x > 20.0f ? x : fmaxf(x, 0.0f) + __logf(1.0f + __expf(-fabsf(x)));
}
// σ and the output gate with the hardware exponential and reciprocal (a few
// ulp), for the decode kernel's conv, gates and output, where a handful of
// threads per value head compute them while the rest of the workgroup waits.
__device__ __forceinline__ float sigmoid_hw(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float gate_hw(float z, int sigmoid_gate)
{
    return sigmoid_gate ? sigmoid_hw(z) : z * sigmoid_hw(z);
}
__device__ __forceinline__ float gatef_(float z, int sigmoid_gate)
{
    return sigmoid_gate ? sigmoidf_(z) : siluf_(z);
}

// Key head read by value head hv: contiguous groups of H_v/H_k value heads
// per key head, or the tiled order hv mod H_k of GGUF conversions ("oxinfer
// 0.0.5 src/qwen.rs", DeltaRule::run).
__device__ __forceinline__ int key_head_of(int hv, int h_k, int group, int tiled)
{
    return tiled ? hv % h_k : hv / group;
}

// Value head of the hl-th member (0 <= hl < H_v/H_k) of key head hk's group.
__device__ __forceinline__ int value_head_of(int hk, int hl, int h_k, int group, int tiled)
{
    return tiled ? hl * h_k + hk : hk * group + hl;
}

// Coefficient of softplus in the log-decay g of value head hv: -exp(A_log),
// or the coefficient itself when a layer stores it directly (GGUF ssm_a;
// "oxinfer 0.0.5 src/qwen.rs", weight loading).
// (one load from whichever array is given, so that the load is not under a
// branch; the hardware exponential, ~1e-7 relative)
__device__ __forceinline__ float decay_coef_of(const float *a_log, const float *decay_coef, int hv)
{
    const float raw = (decay_coef ? decay_coef : a_log)[hv];
    return decay_coef ? raw : -__expf(raw);
}

// Sum over the lanes of an aligned group of W lanes (W a power of two <= 64).
template <int W> __device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float4 operator+(float4 a, float4 b)
{
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 operator*(float s, float4 a)
{
    return make_float4(s * a.x, s * a.y, s * a.z, s * a.w);
}
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c)
{
    return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z),
                       fmaf(s, a.w, c.w));
}

// ---- split-bf16 matrix-core products --------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> (hi, lo) bf16 pair with hi + lo = v to ~16 significant bits.
__device__ __forceinline__ void split1(float v, __bf16 &h, __bf16 &l)
{
    h = static_cast<__bf16>(v);
    l = static_cast<__bf16>(v - static_cast<float>(h));
}

// D += A B on one 16x16x16 tile, split-bf16 with three MFMAs (the lo.lo
// product dropped).  Lane l holds A[l%16][4*(l/16) + e], B[4*(l/16) + e][l%16]
// and D[4*(l/16) + e][l%16] (e < 4), so an accumulator tile is directly the
// B operand of the next product.
typedef short s16x4 __attribute__((ext_vector_type(4)));
struct Frag4 {
    s16x4 hi, lo;
};
__device__ __forceinline__ Frag4 split4(const f32x4 &v)
{
    Frag4 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        __bf16 h, l;
        split1(v[e], h, l);
        f.hi[e] = __builtin_bit_cast(short, h);
        f.lo[e] = __builtin_bit_cast(short, l);
    }
    return f;
}
__device__ __forceinline__ f32x4 mma3k16(const Frag4 &A, const Frag4 &B, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A.lo, B.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A.hi, B.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A.hi, B.hi, c, 0, 0, 0);
    return c;
}

} // namespace gdn
