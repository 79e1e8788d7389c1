// gfx950 backward pass of the selective scan (S6): gradients of a scalar loss
// through the forward pass, given dLoss/dy and dLoss/d(final state).
//
// With Abar = exp(delta*A), gain = (exp(delta*A) - 1)/A (delta when A = 0),
// h_t = Abar_t h_{t-1} + gain_t B_t x_t and y_t = C_t.h_t + D x_t, the adjoint
// lam_t = dLoss/dh_t runs backwards in time,
//     lam_t = C_t dy_t + Abar_{t+1} lam_{t+1},
// and, per token and state,
//     dx      += lam * gain * B            (plus D*dy)
//     ddelta  += lam * (A h_t + B x)        (dh_t/ddelta = A h_t + B x exactly)
//     dA      += lam * (delta Abar h_{t-1} + dgain/dA B x)
//     dB      += lam * gain * x             (summed over channels)
//     dC      += dy * h_t                   (summed over channels)
// with dgain/dA = (delta Abar - gain)/A = delta^2 psi(delta A),
// psi(z) = (z exp(z) - exp(z) + 1)/z^2 (delta^2/2 at A = 0), and
// dh0 = Abar_0 lam_0.  This is the chain rule through the definition of the
// forward pass ("The loop that beats attention", eqs. (1)-(2)); the pages name
// the backward pass and its recomputation of the states ("Mamba and State
// Space Models", the hardware-aware implementation; "Mamba matches the
// Transformer...", "Fuse the kernel and recompute") without spelling it out.
//
// Mapping.  Each pass takes one 64-channel tile per workgroup (lane = channel,
// B/C wave-uniform in SGPRs, as in the forward kernels) for the whole
// sequence, in chunks of BCH = BW * BT tokens:
//   pass 1 (k_bwd_ckpt), chunks in order, CW = 16 waves of one chunk each:
//     each run is scanned from zero (run 0 from the carried state), the runs
//     are composed through LDS with the associative combine, and the state
//     entering every chunk is saved;
//   pass 2 (k_bwd), chunks in reverse, BW waves of BT tokens per chunk: each
//     run scans its tokens forward from zero
//     (run 0: from the chunk's entering state), keeping the BT states in
//     VGPRs, and backward (adjoint from zero at its right end); the forward
//     aggregates are folded left to right (state entering each run) and the
//     reverse ones right to left (adjoint entering each run from the right);
//     every run then adds (decay since its start) x (entering state) to its
//     kept states, which makes them exact, and walks them backwards with its
//     exact adjoint.
// dB/dC are summed over the 64 lanes through LDS and written as one partial
// per tile; dA/dDskip as one partial per batch row; k_bwd_reduce adds the
// partials in a fixed order, so the result is deterministic.

#include <type_traits>

#include "sscan_device.h"

namespace sscan {
namespace {

using namespace dev;

constexpr int BW = 8;   // waves per tile
constexpr int BT = 4;   // tokens per run
constexpr int BCH = BW * BT;

// Orders one wave's LDS accesses around a cross-lane exchange: the wave's LDS
// writes before it are complete and visible to all its lanes after it, and no
// access moves across it.
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A copy of v that the compiler cannot prove equal to v: per-token
// coefficients are recomputed in each phase instead of being kept live
// across phases.
__device__ __forceinline__ float opaque(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Polynomial (expm1(z)/z - 1)/z = 1/2 + z/6 + ... + z^5/7! for |z| < 1/4
// (truncation below 2e-9 relative).
__device__ __forceinline__ float phi1m1_over_z(float z) {
    float p = 1.f / 5040.f;
    p = fmaf(p, z, 1.f / 720.f);
    p = fmaf(p, z, 1.f / 120.f);
    p = fmaf(p, z, 1.f / 24.f);
    p = fmaf(p, z, 1.f / 6.f);
    return fmaf(p, z, 0.5f);
}

// ZOH gain (exp(z) - 1)/A for z = dt*A, given abar = exp(z) and 1/A: the
// Taylor polynomial dt*(1 + z/2 + ... + z^6/7!) for |z| < 1/4 (no
// cancellation in abar - 1), the closed form otherwise.  Both are evaluated
// and one selected: no divergent branch.
__device__ __forceinline__ float gain_of(float dt, float z, float abar, float a_inv) {
    const float series = dt * fmaf(z, phi1m1_over_z(z), 1.f);
    const float direct = (abar - 1.f) * a_inv;
    return fabsf(z) < 0.25f ? series : direct;
}

// dgain/dA = (dt*abar - gain)/A for one state, given z = dt*A, abar = exp(z),
// the gain and 1/A.  For |z| < 1/2 the difference cancels, so it is evaluated
// as dt^2 psi(z) with psi(z) = sum_j (j+1)/(j+2)! z^j (the series of
// (z e^z - e^z + 1)/z^2) up to z^7: truncation below 1e-8 relative.  Both
// forms are evaluated and one selected.
__device__ __forceinline__ float dgain_da(float dt, float z, float abar, float gain, float a_inv) {
    float p = 1.f / 45360.f;
    p = fmaf(p, z, 1.f / 5760.f);
    p = fmaf(p, z, 1.f / 840.f);
    p = fmaf(p, z, 1.f / 144.f);
    p = fmaf(p, z, 1.f / 30.f);
    p = fmaf(p, z, 1.f / 8.f);
    p = fmaf(p, z, 1.f / 3.f);
    p = fmaf(p, z, 0.5f);
    const float direct = fmaf(dt, abar, -gain) * a_inv;
    return fabsf(z) < 0.5f ? (dt * dt) * p : direct;
}

// ---------------------------------------------------------------------------
// Per-token arithmetic, in two policies that share the kernel's structure.
// Both keep the state in an internal form (`to_state`), compose it with the
// same run decays, and provide: fwd (one token of the forward update), rev
// (one token of the local reverse adjoint), correct (add decay x entering
// state to a state computed from zero) and walk (one token of the gradient).
//
// GenMath (any A): the state is h itself; every token needs, per state,
// Abar = exp(dt*A), the gain and dgain/dA.
//
// FastMath (structured-real A: A[d,n] = (n+1) A[d,0], A[d,0] < 0): as in the
// forward kernels the state is kept scaled, k = alpha*h with alpha = -A[d,0],
// so that with r = exp(dt*A[d,0]) and w_n = (B_n/(n+1)) x
//     k_n <- k_n + (1 - r^(n+1)) (w_n - k_n)   (sr_update),
// and gain_n = g0 s_n/(n+1) with g0 = (1 - r)/alpha, s_n = 1 + r + ... + r^n.
// The gradient with respect to A uses the identity
//     A dh/dA = delta dh/ddelta - gain B x
// (both sides equal delta A Abar h_{t-1} + (delta Abar - gain) B x), which in
// the scaled variables reads
//     alpha dh_n/dA_n = (gain_n - delta) w_n + delta k_n,
// with gain_n - delta = E_n/(n+1),
//     E_n = sum_{j<=n} (g0 r^j - delta) = E_{n-1} + (g0 - delta) - g0 (1 - r) s_{n-1}:
// terms of one sign (z < 0 makes g0 < delta and r < 1), so there is no
// cancellation for any delta and no per-state series.  Likewise
//     ddelta = sum_n (n+1) lam_n (w_n - k_n),
//     dx     = D dy + g0 sum_n lam_n s_n B_n/(n+1),
//     dB_n   = sum over lanes of lam_n g0 s_n x, times 1/(n+1),
//     dC_n   = sum over lanes of (dy/alpha) k_n,
//     dA_n   = (sum over tokens of lam_n alpha dh_n/dA_n)/alpha.

// Per-lane view of one wave's [value][lane] reduction buffer.
struct RedRow {
    float *p;  // &buf[0][lane]
    __device__ __forceinline__ void put(int j, float v) const { p[j * kWave] = v; }
};

template <int NT>
struct FastMath {
    float a0, alpha, inv_alpha, a2, inv_a0;

    __device__ void init(const float *A, int64_t d, int N) {
        a0 = A[d * N];
        alpha = -a0;
        inv_alpha = 1.f / alpha;
        inv_a0 = -inv_alpha;
        a2 = a0 * kLog2e;
    }
    __device__ float to_state(float h) const { return h * alpha; }
    __device__ float run_decay(int n, float s) const { return exp2_hw(s * (a2 * float(n + 1))); }
    // scale of the dB partial of state j after the lane sum, and of dA at the end
    __device__ static float b_scale(int j) { return 1.f / float(j + 1); }
    __device__ float a_scale() const { return inv_alpha; }

    __device__ __forceinline__ void fwd(float dv, float xv, const float *row, float *k) const {
        const float r = exp2_hw(dv * a2);
        sr_update<NT>(r, one_minus_exp(dv * a0, r), xv, row, k, [](int) {});
    }
    __device__ __forceinline__ void rev(float dv, float gv, const float *row, float *l) const {
        const float r = exp2_hw(dv * a2);
        float pw = r;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            l[n] = pw * fmaf(row[NT + n], gv, l[n]);
            pw *= r;
        }
    }
    // k += (decay over deltas summing to dsum) * P
    __device__ __forceinline__ void correct(float dsum, const float *P, float *k) const {
        const float rho = exp2_hw(dsum * a2);
        float pw = rho;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            k[n] = fmaf(pw, P[n], k[n]);
            pw *= rho;
        }
    }
    // One token of the walk: kt = state after the token (kp, the state before,
    // is not needed here); lc = adjoint carried in from the right, updated to
    // the one carried further left; dA accumulates; returns dx without D*dy.
    __device__ __forceinline__ float walk(float dv, float xv, float gv, const float *row,
                                          const float *kt, const float * /*kp*/, float *lc,
                                          float *dA, float &ddv, RedRow red) const {
        const float r = exp2_hw(dv * a2);
        const float z0 = dv * a0;
        const float p = phi1m1_over_z(z0);
        const bool small = fabsf(z0) < 0.25f;
        const float g0 = small ? dv * fmaf(z0, p, 1.f) : (r - 1.f) * inv_a0;  // (1 - r)/alpha
        const float d0 = small ? (dv * z0) * p : g0 - dv;                       // g0 - delta
        const float ngq = -g0 * (g0 * alpha);                                  // -g0 (1 - r)
        const float qx = g0 * xv, gva = gv * inv_alpha;
        // Ep = E_n - (n+1) d0 = g0 sum_{j<=n} (r^j - 1), one-signed like E_n, so that
        // u = E_n/(n+1) = Ep/(n+1) + d0 = gain_n - delta is one fma; then
        //     alpha dh_n/dA_n = u w_n + delta k_n = u (w_n - k_n) + (u + delta) k_n,
        // which reuses w_n - k_n from the delta gradient
        float pw = r, s = 1.f, sprev = 0.f, Ep = 0.f, dxa = 0.f, dda = 0.f;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            Ep = fmaf(ngq, sprev, Ep);
            const float l = fmaf(row[NT + n], gv, lc[n]);
            lc[n] = pw * l;
            const float ls = l * s;
            dxa = fmaf(ls, row[n], dxa);
            red.put(n, ls * qx);
            red.put(NT + n, gva * kt[n]);
            const float wk = fmaf(row[n], xv, -kt[n]);  // w_n - k_n
            dda = fmaf(l * wk, float(n + 1), dda);
            const float u = fmaf(Ep, 1.f / float(n + 1), d0);
            dA[n] = fmaf(l, fmaf(u, wk, (u + dv) * kt[n]), dA[n]);
            sprev = s;
            s += pw;
            pw *= r;
        }
        ddv = dda;
        return g0 * dxa;
    }
};

template <int NT>
struct GenMath {
    float a[NT];      // A[d, n] (0 for padded states)
    float a_inv[NT];  // 1/A[d, n] (0 for A = 0, where the series forms are used)

    __device__ void init(const float *A, int64_t d, int N) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            a[n] = (n < N) ? A[d * N + n] : 0.f;
            a_inv[n] = a[n] != 0.f ? 1.f / a[n] : 0.f;
        }
    }
    __device__ float to_state(float h) const { return h; }
    __device__ float run_decay(int n, float s) const { return exp2_hw(s * (a[n] * kLog2e)); }
    __device__ static float b_scale(int) { return 1.f; }
    __device__ float a_scale() const { return 1.f; }

    __device__ __forceinline__ void fwd(float dv, float xv, const float *row, float *k) const {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const float z = dv * a[n];
            const float abar = exp2_hw(dv * (a[n] * kLog2e));
            const float g = gain_of(dv, z, abar, a_inv[n]);
            k[n] = fmaf(abar, k[n], g * (row[n] * float(n + 1) * xv));
        }
    }
    __device__ __forceinline__ void rev(float dv, float gv, const float *row, float *l) const {
#pragma unroll
        for (int n = 0; n < NT; ++n)
            l[n] = exp2_hw(dv * (a[n] * kLog2e)) * fmaf(row[NT + n], gv, l[n]);
    }
    __device__ __forceinline__ void correct(float dsum, const float *P, float *k) const {
#pragma unroll
        for (int n = 0; n < NT; ++n) k[n] = fmaf(run_decay(n, dsum), P[n], k[n]);
    }
    __device__ __forceinline__ float walk(float dv, float xv, float gv, const float *row,
                                          const float *kt, const float *kp, float *lc, float *dA,
                                          float &ddv, RedRow red) const {
        float dxa = 0.f, dda = 0.f;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const float z = dv * a[n];
            const float abar = exp2_hw(dv * (a[n] * kLog2e));
            const float g = gain_of(dv, z, abar, a_inv[n]);
            const float dg = dgain_da(dv, z, abar, g, a_inv[n]);
            const float bn = row[n] * float(n + 1);
            const float bxn = bn * xv;
            const float l = fmaf(row[NT + n], gv, lc[n]);
            const float lg = l * g;
            dxa = fmaf(lg, bn, dxa);
            dda = fmaf(l, fmaf(a[n], kt[n], bxn), dda);
            dA[n] = fmaf(l, fmaf(dv * abar, kp[n], dg * bxn), dA[n]);
            red.put(n, lg * xv);
            red.put(NT + n, gv * kt[n]);
            lc[n] = abar * l;
        }
        ddv = dda;
        return dxa;
    }
};

// Pass 1 of the backward: the state entering every BCH-token chunk, saved for the
// reverse pass (ckpt, (chunks, batch, NT, dim), in the Math's state form).  One
// workgroup of CW waves per tile (lane = channel), over the sequence in steps of
// CW chunks: wave w scans chunk c*CW + w from zero -- wave 0 from the state
// carried in -- and the CW runs are composed through LDS with the associative
// combine, which gives the state entering each of them (the same fold as the
// forward kernels).  Only states: no readout and no correction, so a token costs
// the update's 3 operations per state, and a workgroup holds CW = 16 waves where
// the reverse pass, short of registers, holds BW = 8.
constexpr int CW = 16;   // waves (runs of one chunk each) per workgroup of the checkpoint pass
constexpr int CU8 = 8;   // tokens per load group

template <class IO, int NT, bool kFast>
__global__ __launch_bounds__(CW *kWave) void k_bwd_ckpt(
    const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ delta,
    const float *__restrict__ A, const float *__restrict__ bc, const float *__restrict__ h0,
    float *__restrict__ ckpt, const int *__restrict__ tile_fast, int64_t batch, int64_t L, int64_t dim,
    int N, int64_t tiles_per_batch) {
    using T = typename IO::T;
    using Math = std::conditional_t<kFast, FastMath<NT>, GenMath<NT>>;
    constexpr int NPW = (NT + CW - 1) / CW;  // states each wave folds
    constexpr int ES = IO::kBytes;
    static_assert(BCH % CU8 == 0, "a chunk is a whole number of load groups");
    __shared__ float s_sum[CW][kWave];
    __shared__ float s_k[CW][NT][kWave];    // run end states (from the run's start state)
    __shared__ float s_pre[CW][NT][kWave];  // [0]: state carried into the next step; [j]: entering run j
    lds_poison(s_sum, s_k, s_pre);

    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
    const int lane = int(threadIdx.x) % kWave;
    const int64_t tile = blockIdx.x;
    const int64_t b = tile / tiles_per_batch;
    const int64_t dt_ = tile - b * tiles_per_batch;
    if ((tile_fast[dt_] != 0) != kFast) return;  // whole workgroup
    const int64_t dbase = dt_ * kWave;
    const bool active = dbase + lane < dim;
    const int64_t d = active ? dbase + lane : dim - 1;
    Math m;
    m.init(A, d, N);
    // inactive lanes read channel dim-1 with x = 0 and store nothing
    const float amask = active ? 1.f : 0.f;
    const uint32_t voff = uint32_t(d * ES);
    const uint32_t rowb = uint32_t(dim * ES);
    const float *bcrow = bc + (b * L) * (2 * NT);
    const int64_t ncb = (L + BCH - 1) / BCH;  // chunks of the reverse pass
    const int64_t nst = (ncb + CW - 1) / CW;  // steps of CW chunks
    auto ck = [&](int64_t cb, int n) -> float & { return ckpt[((cb * batch + b) * NT + n) * dim + d]; };
    // CU8 tokens from token tg on (a descriptor per group keeps every offset small;
    // tokens at or past L read 0, which leaves the state unchanged)
    auto load = [&](int64_t tg, T *xo, T *dq) {
        const int64_t tc = tg < L ? tg : L;
        const int64_t bytes = (L - tc) * dim * ES;
        const rsrc_t rx = make_rsrc(x + (b * L + tc) * dim, bytes), rd = make_rsrc(delta + (b * L + tc) * dim, bytes);
#pragma unroll
        for (int u = 0; u < CU8; ++u) {
            xo[u] = IO::bld(rx, voff, uint32_t(u) * rowb);
            dq[u] = IO::bld(rd, voff, uint32_t(u) * rowb);
        }
    };

    if (w == 0) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
            s_pre[0][n][lane] = (h0 && n < N) ? m.to_state(h0[(b * dim + d) * N + n]) : 0.f;
    }
    __syncthreads();
    float k[NT];
    T xr[CU8], dr[CU8];
    load(int64_t(w) * BCH, xr, dr);
    for (int64_t c = 0; c < nst; ++c) {
        const int64_t cb = c * CW + w;  // this wave's chunk
        const int64_t t0 = cb * BCH;
        if (w == 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n) k[n] = s_pre[0][n][lane];
            if (active && cb < ncb) {
#pragma unroll
                for (int n = 0; n < NT; ++n) ck(cb, n) = k[n];
            }
        } else {
#pragma unroll
            for (int n = 0; n < NT; ++n) k[n] = 0.f;
        }
        const float *bc0 = bcrow + (t0 < L ? t0 : L - 1) * (2 * NT);
        const int last = int(max<int64_t>(0, min<int64_t>(BCH, L - t0) - 1));
        float dsum = 0.f;
#pragma unroll
        for (int g = 0; g < BCH / CU8; ++g) {
            float xv[CU8], dv[CU8];
#pragma unroll
            for (int u = 0; u < CU8; ++u) {
                xv[u] = amask * IO::cvt(xr[u]);
                dv[u] = IO::cvt(dr[u]);
            }
            // the next group: the rest of this chunk, then this wave's chunk of the next step
            load(g + 1 < BCH / CU8 ? t0 + (g + 1) * CU8 : t0 + int64_t(CW) * BCH, xr, dr);
#pragma unroll
            for (int u = 0; u < CU8; ++u) {
                m.fwd(dv[u], xv[u], bc0 + min(g * CU8 + u, last) * (2 * NT), k);
                dsum += dv[u];
            }
        }
        s_sum[w][lane] = dsum;
#pragma unroll
        for (int n = 0; n < NT; ++n) s_k[w][n][lane] = k[n];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            if (n < NT) {
                float dec[CW], kv[CW];
#pragma unroll
                for (int j = 0; j < CW; ++j) {
                    dec[j] = m.run_decay(n, s_sum[j][lane]);
                    kv[j] = s_k[j][n][lane];
                }
                float P = kv[0];  // run 0 started from the carried state
#pragma unroll
                for (int j = 1; j < CW; ++j) {
                    s_pre[j][n][lane] = P;
                    P = fmaf(dec[j], P, kv[j]);
                }
                s_pre[0][n][lane] = P;
            }
        }
        __syncthreads();
        if (w != 0 && active && cb < ncb) {
#pragma unroll
            for (int n = 0; n < NT; ++n) ck(cb, n) = s_pre[w][n][lane];
        }
    }
}

template <class IO, int NT, bool kFast>
__global__ __launch_bounds__(BW *kWave) void k_bwd(
    const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ delta,
    const float *__restrict__ A, const float *__restrict__ bc, const float *__restrict__ Dskip,
    const typename IO::T *__restrict__ dy,
    const float *__restrict__ dhT, typename IO::T *__restrict__ dx,
    typename IO::T *__restrict__ ddelta, float *__restrict__ part_bc,
    float *__restrict__ part_ad, float *__restrict__ dh0, float *__restrict__ ckpt,
    const int *__restrict__ tile_fast, int64_t batch, int64_t L, int64_t dim, int N,
    int64_t tiles_per_batch) {
    using T = typename IO::T;
    using Math = std::conditional_t<kFast, FastMath<NT>, GenMath<NT>>;
    constexpr int NPW = (NT + BW - 1) / BW;  // states each wave folds
    constexpr int ES = IO::kBytes;
    __shared__ float s_sum[BW][kWave];
    __shared__ float s_k[BW][NT][kWave];   // run end states (forward, from zero)
    __shared__ float s_q[BW][NT][kWave];   // run adjoint contributions to the token before
    // s_pm[0]: state entering each run ([0][0]: the chunk's carry-out);
    // s_pm[1]: adjoint entering each run from the right
    __shared__ float s_pm[2][BW][NT][kWave];
    float(*s_pre)[NT][kWave] = s_pm[0];
    float(*s_mu)[NT][kWave] = s_pm[1];
    // lane partials of dB/dC for the 64-lane sums, [wave][value][lane]: the same
    // memory as s_pm, which every wave has read into registers, and passed a
    // barrier, before any wave writes it
    float(*s_red)[2 * NT][kWave] = reinterpret_cast<float(*)[2 * NT][kWave]>(&s_pm[0][0][0][0]);
    static_assert(sizeof(s_pm) == sizeof(float) * BW * 2 * NT * kWave, "reduction buffer");
    lds_poison(s_sum, s_k, s_q, s_pm);

    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
    const int lane = int(threadIdx.x) % kWave;
    const int64_t tile = blockIdx.x;
    const int64_t b = tile / tiles_per_batch;
    const int64_t dt_ = tile - b * tiles_per_batch;
    if ((tile_fast[dt_] != 0) != kFast) return;  // whole workgroup
    const int64_t dbase = dt_ * kWave;
    const bool active = dbase + lane < dim;
    const int64_t d = active ? dbase + lane : dim - 1;
    Math m;
    m.init(A, d, N);
    const float dsk = Dskip ? Dskip[d] : 0.f;
    const float *bcrow = bc + (b * L) * (2 * NT);
    const int64_t nchunks = (L + BCH - 1) / BCH;
    // inactive lanes (channels past dim) read channel dim-1 and use x = dy = 0,
    // so they add nothing to the dB/dC lane sums; their stores are dropped
    const uint32_t voff = uint32_t(d * ES);
    const uint32_t voff_st = active ? voff : 0x80000000u;  // past every range
    const float amask = active ? 1.f : 0.f;
    const uint32_t rowb = uint32_t(dim * ES);
    auto rsrc_at = [&](const T *base, int64_t t0) {
        return make_rsrc(base + (b * L + t0) * dim, (L - t0) * dim * ES);
    };
    // inputs of chunk c (c < 0: an empty descriptor, whose loads read 0): the next
    // chunk's loads are issued unconditionally and stay in flight while the current
    // chunk computes
    auto rsrc_chunk = [&](const T *base, int64_t c) {
        const int64_t t0 = (c < 0 ? 0 : c) * BCH + int64_t(w) * BT;
        return make_rsrc(base + (b * L + t0) * dim, c < 0 ? 0 : (L - t0) * dim * ES);
    };
    const RedRow red{&s_red[w][0][lane]};

    // (pass 1, the state entering every chunk, is k_bwd_ckpt's: read from ckpt)
    float k[NT];
    T cx[BT], cd[BT];  // raw x and delta of the chunk, loaded one chunk ahead

    // ---------------- pass 2: chunks in reverse
    float mu[NPW];  // adjoint entering the current chunk from the right (states this wave folds)
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int n = w * NPW + i;
        mu[i] = (dhT && n < N) ? dhT[(b * dim + d) * N + n] : 0.f;
    }
    float dA_acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) dA_acc[n] = 0.f;
    float dD_acc = 0.f;

    // raw x, delta, dy and (wave 0) the entering-state checkpoint of the chunk,
    // loaded one chunk ahead (chunk c - 1 while chunk c computes); the general-A
    // path, short of registers, loads them at the top of its chunk
    T cg[BT];
    float cck[NT];
    auto load_ck = [&](int64_t c, float *kr) {
        const int64_t cc = c < 0 ? 0 : c;
        const rsrc_t rk = make_rsrc(ckpt + (cc * batch + b) * NT * dim, (c < 0 || w != 0) ? 0 : NT * dim * 4);
#pragma unroll
        for (int n = 0; n < NT; ++n)
            kr[n] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rk, uint32_t((n * dim + d) * 4), 0, 0));
    };
    auto load2 = [&](int64_t c, T *xr, T *dr, T *gr, float *kr) {
        const rsrc_t rx = rsrc_chunk(x, c), rd = rsrc_chunk(delta, c), rg = rsrc_chunk(dy, c);
#pragma unroll
        for (int tau = 0; tau < BT; ++tau) {
            xr[tau] = IO::bld(rx, voff, uint32_t(tau) * rowb);
            dr[tau] = IO::bld(rd, voff, uint32_t(tau) * rowb);
            gr[tau] = IO::bld(rg, voff, uint32_t(tau) * rowb);
        }
        if constexpr (kFast) load_ck(c, kr);
    };
    if constexpr (kFast) load2(nchunks - 1, cx, cd, cg, cck);
    for (int64_t c = nchunks - 1; c >= 0; --c) {
        const int64_t t0 = c * BCH + int64_t(w) * BT;
        T nx[BT], nd[BT], ng[BT];
        float nck[NT];
        if constexpr (kFast) load2(c - 1, nx, nd, ng, nck);
        else load2(c, cx, cd, cg, cck);
        const rsrc_t rdx = rsrc_at(dx, t0), rdd = rsrc_at(ddelta, t0);
        const float *bc0 = bcrow + min(t0, L - 1) * (2 * NT);
        const int last = int(max<int64_t>(0, min<int64_t>(BT, L - t0) - 1));
        // tokens of this run (past the end of the sequence: x = delta = dy = 0,
        // which leaves both the state and the adjoint unchanged)
        float xs[BT], ds[BT], gs[BT];
#pragma unroll
        for (int tau = 0; tau < BT; ++tau) {
            xs[tau] = amask * IO::cvt(cx[tau]);
            ds[tau] = IO::cvt(cd[tau]);
            gs[tau] = amask * IO::cvt(cg[tau]);
        }

        // phase A: the run's states from its entering state (run 0: the chunk's,
        // exact; other runs: zero, corrected below) and its adjoint from zero
        float hist[BT + 1][NT];  // hist[0]: entering state, hist[tau+1]: after token tau
        float dcum[BT];          // delta summed from the run start through token tau
        if constexpr (!kFast) load_ck(c, cck);  // (load2 leaves it to this point)
#pragma unroll
        for (int n = 0; n < NT; ++n) hist[0][n] = cck[n];  // 0 for waves other than 0
        float dsum = 0.f;
#pragma unroll
        for (int tau = 0; tau < BT; ++tau) {
#pragma unroll
            for (int n = 0; n < NT; ++n) hist[tau + 1][n] = hist[tau][n];
            m.fwd(opaque(ds[tau]), xs[tau], bc0 + min(tau, last) * (2 * NT), hist[tau + 1]);
            dsum += ds[tau];
            dcum[tau] = dsum;
        }
        s_sum[w][lane] = dsum;
#pragma unroll
        for (int n = 0; n < NT; ++n) s_k[w][n][lane] = hist[BT][n];
#pragma unroll
        for (int n = 0; n < NT; ++n) k[n] = 0.f;  // the run's adjoint from zero
#pragma unroll
        for (int tau = BT - 1; tau >= 0; --tau)
            m.rev(opaque(ds[tau]), gs[tau], bc0 + min(tau, last) * (2 * NT), k);
#pragma unroll
        for (int n = 0; n < NT; ++n) s_q[w][n][lane] = k[n];
        __syncthreads();
        // folds: states entering each run (left to right), adjoints entering each
        // run from the right (right to left), and the adjoint leaving the chunk
        // (the runs' values and decays are read and formed first, independently, so
        // that only the short fma chains are serial)
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            if (n < NT) {
                float dec[BW], kv[BW], qv[BW];
#pragma unroll
                for (int j = 0; j < BW; ++j) {
                    dec[j] = m.run_decay(n, s_sum[j][lane]);
                    kv[j] = s_k[j][n][lane];
                    qv[j] = s_q[j][n][lane];
                }
                float P = kv[0];  // run 0 started from the chunk's entering state
#pragma unroll
                for (int j = 1; j < BW; ++j) {
                    s_pre[j][n][lane] = P;
                    P = fmaf(dec[j], P, kv[j]);
                }
                float M = mu[i];
#pragma unroll
                for (int j = BW - 1; j >= 1; --j) {
                    s_mu[j][n][lane] = M;
                    M = fmaf(dec[j], M, qv[j]);
                }
                s_mu[0][n][lane] = M;
                mu[i] = fmaf(dec[0], M, qv[0]);
            }
        }
        __syncthreads();
        float lc[NT];  // adjoint carried into the token being walked
#pragma unroll
        for (int n = 0; n < NT; ++n) lc[n] = s_mu[w][n][lane];
        if (w != 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n) hist[0][n] = s_pre[w][n][lane];
#pragma unroll
            for (int tau = 0; tau < BT; ++tau) m.correct(dcum[tau], hist[0], hist[tau + 1]);
        }
        __syncthreads();  // s_pre/s_mu become the reduction buffer

        // phase B: walk the run backwards
#pragma unroll
        for (int tau = BT - 1; tau >= 0; --tau) {
            const float *row = bc0 + min(tau, last) * (2 * NT);
            const float xv = xs[tau], gv = gs[tau];
            float ddv;
            const float dxv = fmaf(dsk, gv, m.walk(opaque(ds[tau]), xv, gv, row, hist[tau + 1],
                                                   hist[tau], lc, dA_acc, ddv, red));
            dD_acc = fmaf(gv, xv, dD_acc);
            IO::bst(IO::enc(dxv), rdx, voff_st, uint32_t(tau) * rowb);
            IO::bst(IO::enc(ddv), rdd, voff_st, uint32_t(tau) * rowb);
            // sum the 64 lanes' partials of the 2*NT values of this token: lanes
            // j and j+32 (j < 2*NT) add value j over channels 0..31 and 32..63,
            // in a rotated order that keeps the LDS reads on distinct banks
            wave_sync_lds();
            float acc = 0.f;
            const int j = lane & 31;
            if (j < 2 * NT) {
                const int i0 = lane & 32;
#pragma unroll 8
                for (int i = 0; i < 32; ++i) acc += s_red[w][j][i0 + ((i + j) & 31)];
            }
            acc += __shfl_xor(acc, 32);
            if (lane < 2 * NT && t0 + tau < L)
                part_bc[((dt_ * batch + b) * L + t0 + tau) * (2 * NT) + lane] =
                    lane < NT ? acc * Math::b_scale(lane) : acc;
            wave_sync_lds();
        }
        if constexpr (kFast) {
#pragma unroll
            for (int tau = 0; tau < BT; ++tau) {
                cx[tau] = nx[tau];
                cd[tau] = nd[tau];
                cg[tau] = ng[tau];
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) cck[n] = nck[n];
        }
    }
    // adjoint leaving chunk 0 = dLoss/d(initial state)
    if (dh0 && active) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            if (n < N) dh0[(b * dim + d) * N + n] = mu[i];
        }
    }
    // dA and dDskip partials of this batch row: the waves hold disjoint runs, so
    // they add their accumulators in LDS first (wave order, deterministic)
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NT; ++n) s_k[w][n][lane] = dA_acc[n];
    s_sum[w][lane] = dD_acc;
    __syncthreads();
    if (w == 0 && active) {
        const float as = m.a_scale();
        for (int n = 0; n < NT; ++n) {
            float sacc = 0.f;
            for (int j = 0; j < BW; ++j) sacc += s_k[j][n][lane];
            part_ad[(b * dim + d) * (NT + 1) + n] = sacc * as;
        }
        float sd = 0.f;
        for (int j = 0; j < BW; ++j) sd += s_sum[j][lane];
        part_ad[(b * dim + d) * (NT + 1) + NT] = sd;
    }
}

// dB, dC: sum of the per-tile partials; dA, dDskip: sum over batch rows.
template <int NT>
__global__ __launch_bounds__(256) void k_bwd_reduce(const float *__restrict__ part_bc,
                                                    const float *__restrict__ part_ad,
                                                    float *__restrict__ dB, float *__restrict__ dC,
                                                    float *__restrict__ dA, float *__restrict__ dD,
                                                    int64_t batch, int64_t L, int64_t dim, int N,
                                                    int64_t tiles_per_batch) {
    const int64_t nbc = batch * L * (2 * NT);
    // the blocks stride over both ranges, so the launch stays within the 32-bit
    // work-item count
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nbc + dim * (NT + 1);
         i += int64_t(gridDim.x) * blockDim.x) {
        if (i < nbc) {
            float s = 0.f;
            for (int64_t t = 0; t < tiles_per_batch; ++t) s += part_bc[t * nbc + i];
            const int64_t row = i / (2 * NT);
            const int j = int(i - row * (2 * NT));
            if (j < NT) {
                if (j < N) dB[row * N + j] = s;
            } else if (j - NT < N) {
                dC[row * N + (j - NT)] = s;
            }
            continue;
        }
        const int64_t k = i - nbc;
        const int64_t dd = k / (NT + 1);
        const int n = int(k - dd * (NT + 1));
        float s = 0.f;
        for (int64_t bb = 0; bb < batch; ++bb) s += part_ad[(bb * dim + dd) * (NT + 1) + n];
        if (n == NT) {
            if (dD) dD[dd] = s;
        } else if (n < N) {
            dA[dd * N + n] = s;
        }
    }
}

template <class IO, int NT>
hipError_t backward_t(const BwdArgs &a, const BwdPlan &p, void *ws, hipStream_t s) {
    using T = typename IO::T;
    char *base = static_cast<char *>(ws);
    float *bc = reinterpret_cast<float *>(base + p.off_bc);
    int *flags = reinterpret_cast<int *>(base + p.off_flags);
    float *ckpt = reinterpret_cast<float *>(base + p.off_ckpt);
    float *part_bc = reinterpret_cast<float *>(base + p.off_pbc);
    float *part_ad = reinterpret_cast<float *>(base + p.off_pad);
    hipError_t e = launch_prep(a.B, a.C, a.A, bc, flags, a.batch * a.L, a.dim, a.N, NT, a.io, s);
    if (e != hipSuccess) return e;
#define SSCAN_CKPT(FAST)                                                                               \
    hipLaunchKernelGGL((k_bwd_ckpt<IO, NT, FAST>), dim3(unsigned(p.tiles)), dim3(CW * kWave), 0, s,     \
                       static_cast<const T *>(a.x), static_cast<const T *>(a.delta), a.A, bc, a.h0, ckpt, \
                       flags, a.batch, a.L, a.dim, a.N, p.tiles_per_batch)
    SSCAN_CKPT(true);
    SSCAN_CKPT(false);
#undef SSCAN_CKPT
#define SSCAN_BWD(FAST)                                                                                \
    hipLaunchKernelGGL((k_bwd<IO, NT, FAST>), dim3(unsigned(p.tiles)), dim3(BW * kWave), 0, s,          \
                       static_cast<const T *>(a.x), static_cast<const T *>(a.delta), a.A, bc, a.Dskip,  \
                       static_cast<const T *>(a.dy), a.dhT, static_cast<T *>(a.dx),                     \
                       static_cast<T *>(a.ddelta), part_bc, part_ad, a.dh0, ckpt, flags, a.batch, a.L,   \
                       a.dim, a.N, p.tiles_per_batch)
    SSCAN_BWD(true);
    SSCAN_BWD(false);
#undef SSCAN_BWD
    const int64_t n = a.batch * a.L * 2 * NT + a.dim * (NT + 1);
    hipLaunchKernelGGL((k_bwd_reduce<NT>), dim3(unsigned(std::min<int64_t>((n + 255) / 256, int64_t(1) << 20))),
                       dim3(256), 0, s, part_bc,
                       part_ad, a.dB, a.dC, a.dA, a.dD, a.batch, a.L, a.dim, a.N, p.tiles_per_batch);
    return hipGetLastError();
}

template <class IO>
hipError_t backward_io(const BwdArgs &a, const BwdPlan &p, void *ws, hipStream_t s) {
    switch (p.nt) {
        case 1: return backward_t<IO, 1>(a, p, ws, s);
        case 2: return backward_t<IO, 2>(a, p, ws, s);
        case 4: return backward_t<IO, 4>(a, p, ws, s);
        case 8: return backward_t<IO, 8>(a, p, ws, s);
        default: return backward_t<IO, 16>(a, p, ws, s);
    }
}

size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

BwdPlan plan_backward(int64_t batch, int64_t L, int64_t dim, int64_t N) {
    BwdPlan p{};
    p.nt = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16;
    p.tiles_per_batch = (dim + kWave - 1) / kWave;
    p.tiles = batch * p.tiles_per_batch;
    if (p.tiles > kMaxWorkItems / (BW * kWave)) p.reject = "batch * dim too large for one backward launch";
    const int64_t nchunks = (L + BCH - 1) / BCH;
    size_t off = 0;
    p.off_bc = off;
    off += al256(size_t(batch) * L * 2 * p.nt * sizeof(float));
    p.off_flags = off;
    off += al256(size_t(p.tiles_per_batch) * sizeof(int));
    p.off_ckpt = off;
    off += al256(size_t(nchunks) * batch * p.nt * dim * sizeof(float));
    p.off_pbc = off;
    off += al256(size_t(p.tiles_per_batch) * batch * L * 2 * p.nt * sizeof(float));
    p.off_pad = off;
    off += al256(size_t(batch) * dim * (p.nt + 1) * sizeof(float));
    p.ws_bytes = off;
    return p;
}

hipError_t launch_backward(const BwdArgs &a, const BwdPlan &p, void *ws, hipStream_t s) {
    return a.io == 1 ? backward_io<dev::IoBF16>(a, p, ws, s) : backward_io<dev::IoF32>(a, p, ws, s);
}

}  // namespace sscan
