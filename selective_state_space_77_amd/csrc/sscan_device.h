// Device helpers shared by the forward, decode-step and backward kernels.
// Private to the library; included by the .hip translation units only.
#pragma once

#include <math.h>

#include "sscan_internal.h"

namespace sscan {
namespace dev {

constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

// Debug build (SSCAN_LDS_POISON=1, libsscan_poison.so): every kernel that uses LDS
// first fills it with a NaN pattern (0x7FC07FC0: a quiet NaN as fp32 and as each of
// its two bf16 halves) and waits at a barrier, so a read of LDS that nothing wrote
// turns into NaN outputs instead of a stale value from an earlier workgroup.  Called
// by every thread of the workgroup, before any early exit.  No-op otherwise.
#ifndef SSCAN_LDS_POISON
#define SSCAN_LDS_POISON 0
#endif
template <class... Ts>
__device__ __forceinline__ void lds_poison(Ts &...arrays) {
    if constexpr (SSCAN_LDS_POISON != 0) {
        auto fill = [](void *p, size_t bytes) {
            uint32_t *w = static_cast<uint32_t *>(p);
            for (size_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0x7FC07FC0u;
        };
        (fill(static_cast<void *>(&arrays), sizeof(arrays)), ...);
        __syncthreads();
    }
}

// s_waitcnt lgkmcnt(0) alone (gfx9 encoding: vmcnt and expcnt fields left at
// their "no wait" maxima).  Scalar loads return out of order, so the only wait
// for one is lgkmcnt(0); issuing it before the next token's loads makes that
// wait cover only the loads issued one token earlier.
__device__ __forceinline__ void wait_scalar_loads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ZOH input gain g = (exp(z) - 1)/A with z = dt*A (dt when A == 0), given
// abar = exp(z).  For |z| < 1/4 it uses dt * expm1(z)/z as the Taylor
// polynomial 1 + z/2 + ... + z^6/7! (truncation below 2e-9 relative), which
// avoids the cancellation in abar - 1 and needs no division; otherwise
// (abar - 1)/A has no cancellation.
__device__ __forceinline__ float zoh_gain(float dt, float a, float z, float abar) {
    if (fabsf(z) < 0.25f) {
        float p = 1.f / 5040.f;
        p = fmaf(p, z, 1.f / 720.f);
        p = fmaf(p, z, 1.f / 120.f);
        p = fmaf(p, z, 1.f / 24.f);
        p = fmaf(p, z, 1.f / 6.f);
        p = fmaf(p, z, 0.5f);
        p = fmaf(p, z, 1.f);
        return dt * p;
    }
    return (abar - 1.f) / a;
}

// The same gain without a branch or an IEEE division, for kernels that hold many
// states per lane: both forms are evaluated and one selected, and (Abar - 1)/A
// uses the hardware reciprocal (1 ulp), so the result is within a few ulp of the
// form above.
__device__ __forceinline__ float zoh_gain_nb(float dt, float a, float z, float abar) {
    float p = 1.f / 5040.f;
    p = fmaf(p, z, 1.f / 720.f);
    p = fmaf(p, z, 1.f / 120.f);
    p = fmaf(p, z, 1.f / 24.f);
    p = fmaf(p, z, 1.f / 6.f);
    p = fmaf(p, z, 0.5f);
    p = fmaf(p, z, 1.f);
    const float big = (abar - 1.f) * __builtin_amdgcn_rcpf(a);
    return fabsf(z) < 0.25f ? dt * p : big;
}

// 1 - exp(z) given r = exp(z), without the cancellation of 1 - r near z = 0:
// -z (1 + z/2 + z^2/6 + ... + z^5/720) for |z| < 1/8 (truncation below 1e-9
// relative), 1 - r otherwise (there the cancellation costs at most a factor
// 1/(1 - exp(-1/8)) < 9 on the rounding of r).  Both are evaluated and one
// selected.
__device__ __forceinline__ float one_minus_exp(float z, float r) {
    float p = 1.f / 720.f;
    p = fmaf(p, z, 1.f / 120.f);
    p = fmaf(p, z, 1.f / 24.f);
    p = fmaf(p, z, 1.f / 6.f);
    p = fmaf(p, z, 0.5f);
    p = fmaf(p, z, 1.f);
    return fabsf(z) < 0.125f ? -z * p : 1.f - r;
}

// 1 - 2^u given r = 2^u (hardware exp2, within 1 ulp), in five operations and
// without a branch or a compare: the smaller of
//   * the series -u ln2 (1 + u ln2/2 + (u ln2)^2/6), which for u <= 0 is never
//     below the true value and exceeds it by (u ln2)^4/24 at most, and
//   * (1 + 2^-22) - r, which is never below the true value either (2^-22 is twice
//     the largest error of r next to 1) and exceeds it by at most 3 * 2^-24.
// For small |u| the series is the smaller (it is the accurate one there, where
// 1 - r cancels); from |u ln2| ~ 0.05 on, 1 - r is, with a relative error below
// 1e-5.  The same ordering holds for u > 0 (negative step sizes), where both
// underestimate the magnitude of a negative value.  u = 0 gives -0 (a zero step
// leaves the state exactly unchanged); NaN propagates.
__device__ __forceinline__ float one_minus_exp2(float u, float r) {
    constexpr float c0 = -0.69314718055994530942f;   // -ln2
    constexpr float c1 = -0.24022650695910071233f;   // -ln2^2/2
    constexpr float c2 = -0.05550410866482157995f;   // -ln2^3/6
    const float p = fmaf(fmaf(u, c2, c1), u, c0);
    return fminf(p * u, (1.f + 0x1p-22f) - r);
}

// Structured-real state update shared by the scan kernels.  With A[d,n] =
// (n+1) A[d,0], r = exp(delta A[d,0]), the state kept scaled, k = -A[d,0] h, and
// w_n = (B_n/(n+1)) x, the zero-order-hold step is
//     k_n <- k_n + (1 - r^(n+1)) (w_n - k_n).
// 1 - r^(n+1) runs as q_0 = 1 - r, q_n = r q_{n-1} + q_0: terms of one sign,
// no cancellation.  Each rounding is relative to the state and to the change
// written into it, never to w_n alone, so small delta*A (a slowly moving
// state) keeps full precision.  Three VALU operations per state.
template <int NT, class F>
__device__ __forceinline__ void sr_update(float r, float q, float xv, const float *brow, float *k,
                                          F &&after) {
    float qn = q;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float e = fmaf(brow[n], xv, -k[n]);
        k[n] = fmaf(qn, e, k[n]);
        after(n);
        qn = fmaf(qn, r, q);
    }
}

// ---------------------------------------------------------------------------
// Front end of the fused entry points, one channel per lane.
constexpr float kLn2 = 0.69314718055994530942f;

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e), e = e^-|v| in (0, 1] from the
// hardware exp2.  log1p(e) is the series e - e^2/2 + e^3/3 - e^4/4 for e < 1/64
// (truncation below e^4/5 relative, 2e-8) and log2(1 + e) ln 2 otherwise (the
// rounding of 1 + e then costs at most 2^-24/e <= 2^-18 relative).  Both are
// evaluated and one selected.
__device__ __forceinline__ float softplus_f(float v) {
    const float e = exp2_hw(-fabsf(v) * kLog2e);
    float p = fmaf(e, -0.25f, 1.f / 3.f);
    p = fmaf(e, p, -0.5f);
    p = fmaf(e, p, 1.f);
    const float lg = __builtin_amdgcn_logf(1.f + e) * kLn2;  // hardware log2
    return fmaxf(v, 0.f) + (e < 0.015625f ? e * p : lg);
}

// Per-lane front-end coefficients: the K taps right-aligned in a window of
// kMaxConv inputs (w3 multiplies the current token, w0 the token 3 before;
// taps beyond K are 0), the convolution bias and the step-size bias.
struct FeLane {
    float w0, w1, w2, w3, cb, db;
    float silu;  // 1 for SiLU, 0 for none (a blend factor: no branch on it)

    __device__ void init(const FeArgs &fe, int64_t d) {
        const int K = fe.K;
        auto tap = [&](int j) {  // window position j (0: t-3 ... 3: t)
            const int k = j - (kMaxConv - K);
            return k >= 0 ? fe.conv_w[d * K + k] : 0.f;
        };
        w0 = tap(0);
        w1 = tap(1);
        w2 = tap(2);
        w3 = tap(3);
        cb = fe.conv_b ? fe.conv_b[d] : 0.f;
        db = fe.delta_bias ? fe.delta_bias[d] : 0.f;
        silu = fe.act == 1 ? 1.f : 0.f;
    }
    // scan input of a token from its raw input x and the raw inputs 1, 2 and 3
    // tokens before it (sum in the order oldest tap first, bias first)
    __device__ __forceinline__ float u(float p3, float p2, float p1, float x) const {
        const float c = fmaf(w3, x, fmaf(w2, p1, fmaf(w1, p2, fmaf(w0, p3, cb))));
        const float sig = __builtin_amdgcn_rcpf(1.f + exp2_hw(-c * kLog2e));  // sigmoid(c)
        return c * fmaf(silu, sig - 1.f, 1.f);  // c * sigmoid(c), or c
    }
    __device__ __forceinline__ float delta(float raw) const { return softplus_f(raw + db); }
};

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    // round to nearest even (the gfx950 conversion instruction)
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

using rsrc_t = __amdgpu_buffer_rsrc_t;

// Raw buffer descriptor over `bytes` bytes from `base` (stride 0).  Accesses at
// or past `bytes` read 0 and drop stores; the hardware range check is what
// keeps loads of tokens past the end of the sequence in bounds.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), short(0), int(n), 0x00020000);
}

struct IoF32 {
    using T = float;
    static constexpr int kBytes = 4;
    __device__ static float ld(const T *p, int64_t i) { return p[i]; }
    __device__ static float cvt(T v) { return v; }
    __device__ static T enc(float v) { return v; }
    __device__ static T bld(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
    __device__ static void bst(T v, rsrc_t r, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
    }
};

struct IoBF16 {
    using T = uint16_t;
    static constexpr int kBytes = 2;
    __device__ static float ld(const T *p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
    __device__ static float cvt(T v) { return __uint_as_float(uint32_t(v) << 16); }
    __device__ static T enc(float v) { return f32_to_bf16(v); }
    __device__ static T bld(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
    }
    __device__ static void bst(T v, rsrc_t r, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
    }
};

}  // namespace dev
}  // namespace sscan
