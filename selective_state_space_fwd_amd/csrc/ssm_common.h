// ssm_common.h -- device helpers shared by the libssm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;       // CDNA wavefront
constexpr int kGroup = 16;      // states per group in the chunk-operator rows

// ---------------------------------------------------------------- I/O types
// float32 or bfloat16 (raw bits); arithmetic is always float32.
struct F32 {
    using T = float;
    static __device__ __forceinline__ float load(const T *p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void store(T *p, size_t i, float v) { p[i] = v; }
};
struct BF16 {
    using T = uint16_t;
    static __device__ __forceinline__ float load(const T *p, size_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
    // Round to nearest, ties to even (gfx950 v_cvt_pk_bf16_f32).
    static __device__ __forceinline__ void store(T *p, size_t i, float v) {
        __hip_bfloat16 b = __float2bfloat16(v);
        p[i] = *reinterpret_cast<uint16_t *>(&b);
    }
};

// ---------------------------------------------------------------- constant view
// Read-only view of global memory in the constant address space: loads whose
// address is uniform across the wavefront become scalar (s_load) loads.  Only
// for buffers that no kernel writes while the reading kernel runs.
using cfloat = __attribute__((address_space(4))) const float;
__device__ __forceinline__ cfloat *as_constant(const float *p) {
    return (cfloat *)(p);
}

// ---------------------------------------------------------------- buffer views
// Raw buffer views (a gfx9 buffer resource: base address, byte range, 32-bit
// data format, no stride).  A load at or past the range returns 0 and a store
// there is dropped.  Ranges are below 2^31 bytes, so kDrop lies past every
// one of them.
constexpr int kRsrcFormat = 0x00020000;
constexpr uint32_t kDrop = 0x80000000u;
using Rsrc = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ Rsrc view(const void *p, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes),
                                             kRsrcFormat);
}

// ---------------------------------------------------------------- scheduling
// Wavefronts that share a SIMD get its issue slots oldest first, so of two
// wavefronts with equal work the younger runs its last tiles alone, at the
// issue rate of a single wavefront.  Here the priority falls as the
// wavefront's own tiles are done (3 in the first quarter, then 2, 1, 0): the
// wavefront that is behind issues first, and those on a SIMD finish close
// together.
__device__ __forceinline__ void fair_prio(int64_t done, int64_t total) {
    const int64_t p = 3 - (4 * done) / total;
    if (p >= 3) __builtin_amdgcn_s_setprio(3);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}).
// log1p(e) is taken as log(1 + e) plus the exact rounding error of 1 + e,
// c = (1 - fl(1 + e)) + e: log1p(e) = log(fl(1+e)) + log(1 + c / fl(1+e)),
// and |c| <= 2^-24 makes the last term equal to c within 2^-24 relative.
__device__ __forceinline__ float softplus_f32(float x) {
    const float e = exp2_hw(-fabsf(x) * kLog2e);
    const float s = 1.0f + e;
    const float c = (1.0f - s) + e;
    return fmaxf(x, 0.0f) + __builtin_fmaf(log2_hw(s), kLn2, c);
}

// silu(z) = z / (1 + e^{-z}); e^{-z} = inf for very negative z gives -0.
__device__ __forceinline__ float silu_f32(float z) {
    return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// Zero-order-hold input factor (SSM engineering essay, §1.2: B_bar =
// (dt A)^-1 (exp(dt A) - 1) dt B), per unit of dt: phi(x) = (e^x - 1) / x at
// x = dt A, given e = e^x; (exp(dt A) - 1) / A = dt phi(dt A), and phi(0) = 1
// (the Euler factor).  Near 0 the difference e - 1 loses about 2^-24 / |x|
// relative, so below |x| = 1/8 phi is its Taylor polynomial; above, (e - 1) / x.
__device__ __forceinline__ float zoh_phi(float x, float e) {
    // |x| < 1/8: the series to x^4 (the first omitted term, x^5 / 720, is
    // below 4.3e-8 relative there); otherwise the quotient, whose relative
    // error, that of e - 1, is at most about 7.5 times that of e at |x| = 1/8
    float p = 1.0f / 120.0f;
    p = __builtin_fmaf(p, x, 1.0f / 24.0f);
    p = __builtin_fmaf(p, x, 1.0f / 6.0f);
    p = __builtin_fmaf(p, x, 0.5f);
    p = __builtin_fmaf(p, x, 1.0f);
    const float q = (e - 1.0f) * rcp_hw(x);
    return fabsf(x) < 0.125f ? p : q;
}

template <class IO>
struct Seg;   // one 16-byte piece of a row: VW consecutive tokens

template <>
struct Seg<F32> {
    static constexpr int VW = 4;
    using V = float4;
    static __device__ __forceinline__ void unpack(const V &v, float (&o)[VW]) {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    static __device__ __forceinline__ V pack(const float (&o)[VW]) {
        return make_float4(o[0], o[1], o[2], o[3]);
    }
};

template <>
struct Seg<BF16> {
    static constexpr int VW = 8;
    using V = uint4;
    static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
    static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
    static __device__ __forceinline__ void unpack(const V &v, float (&o)[VW]) {
        o[0] = lo(v.x); o[1] = hi(v.x); o[2] = lo(v.y); o[3] = hi(v.y);
        o[4] = lo(v.z); o[5] = hi(v.z); o[6] = lo(v.w); o[7] = hi(v.w);
    }
    static __device__ __forceinline__ uint32_t pk(float a, float b) {
        const __hip_bfloat162 h = __float22bfloat162_rn(make_float2(a, b));
        return *reinterpret_cast<const uint32_t *>(&h);
    }
    static __device__ __forceinline__ V pack(const float (&o)[VW]) {
        return make_uint4(pk(o[0], o[1]), pk(o[2], o[3]), pk(o[4], o[5]), pk(o[6], o[7]));
    }
};

// psi(x) = (x e^x - e^x + 1) / x^2, x = dt A, e = e^x: the derivative of the
// zero-order-hold factor (e^{dt A} - 1) / A with respect to A is dt^2 psi(dt A)
// (backward pass).  Its power series is sum_{m >= 2} (m - 1) x^(m-2) / m!;
// below |x| = 1/2 the closed form loses digits to cancellation, so there it is
// that series to x^7 (truncation below 1e-8 relative); above, the closed form.
__device__ __forceinline__ float zoh_psi(float x, float e) {
    float p = 1.0f / 45360.0f;
    p = __builtin_fmaf(p, x, 1.0f / 5760.0f);
    p = __builtin_fmaf(p, x, 1.0f / 840.0f);
    p = __builtin_fmaf(p, x, 1.0f / 144.0f);
    p = __builtin_fmaf(p, x, 1.0f / 30.0f);
    p = __builtin_fmaf(p, x, 1.0f / 8.0f);
    p = __builtin_fmaf(p, x, 1.0f / 3.0f);
    p = __builtin_fmaf(p, x, 0.5f);
    const float q = __builtin_fmaf(x, e, -(e - 1.0f)) * rcp_hw(x * x);
    return fabsf(x) < 0.5f ? p : q;
}

}  // namespace ssm
