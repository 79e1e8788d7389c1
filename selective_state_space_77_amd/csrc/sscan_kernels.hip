// gfx950 kernels of the selective scan (S6): forward pass over a whole
// sequence and the single-token decode step.
//
// Method (pages: "The loop that beats attention" eqs. (1)-(2); "Mamba and
// State Space Models", selective pseudocode; "State space models and Mamba",
// continuous form with D):  Abar = exp(delta*A), Bbar = (exp(delta*A)-1)/A*B,
// h = Abar*h + Bbar*x, y = C.h + Dskip*x.  The fused-kernel idea (parameters
// read from HBM once, discretisation and scan on chip, only y written, the
// (batch, L, dim, N) tensor never materialised) follows "Mamba matches the
// Transformer...", "The scan that pays for selection".
//
// Mapping on CDNA4.  One lane owns one channel d and keeps its N fp32 states
// in VGPRs; the 64 lanes of a wave are 64 consecutive channels of one batch
// row, so every lane of a wave works on the same token t:
//   * x[b,t,d..d+63] and delta[...] are one contiguous 128 B (bf16) / 256 B
//     (fp32) row per load instruction -- fully coalesced without LDS staging;
//   * B[b,t,:] and C[b,t,:] are wave-uniform, so they come in through scalar
//     loads into SGPRs and feed the VALU as scalar operands (no per-lane
//     traffic, no cross-lane exchange).
// Time is split so the chip has enough waves, and the pieces are composed with
// the associative combine (a1,b1) o (a2,b2) = (a1*a2, a2*b1 + b2) ("Mamba and
// State Space Models", the parallel scan).  The decay of a run of tokens needs
// no per-token product: the Abar of a diagonal mode multiply to exp(A*sum(delta)).
//   k_lockstep: one workgroup of W waves per 64-channel tile; runs of a chunk
//               are scanned locally, composed through LDS, and corrected.
//   k_seg:      one wave per (tile, time segment) scans its segment from
//               zero; k_carry chains the segment end states into the state
//               each segment really started from; k_segfix adds that state's
//               decayed contribution to the segment's outputs.
//
// Structured-real fast path.  When every A row of a tile is
// A[d,n] = (n+1)*A[d,0] with A[d,0] < 0, Abar_n = r^(n+1) with
// r = exp(delta*A[d,0]): one exp per (t,d) instead of N.  The state is kept
// scaled, k_n = -A[d,0]*h_n, which turns the ZOH update into
//     k_n <- k_n + (1 - Abar_n)*(w_n - k_n),   w_n = (B[t,n]/(n+1)) * x
// with 1 - Abar_n built by a positive recurrence from 1 - r (sr_update: two
// FMAs per state plus one for the recurrence), and the readout into
// y = (sum_n C_n k_n) / (-A[d,0]) + Dskip*x.  B/(n+1) is staged once per
// token by k_prep, which also classifies each tile; any other A takes the
// general path (exp2 and the ZOH gain per state).

#include <math.h>
#include <cstdlib>
#include <type_traits>

#include "sscan_device.h"

namespace sscan {
namespace {

using namespace dev;

// ----------------------------------------------------------------------------
// Prologue of every forward pass, one launch with two roles:
//  * blocks [0, prep_blocks): stage B/(n+1) and C of every token as fp32 rows
//    of 2*NT floats, so a scan wave reads one token's parameters with two
//    scalar loads.  States n >= N (padding up to NT) get B = C = 0 and stay 0.
//    The blocks stride over the rows, so the launch stays within the 32-bit
//    work-item count however many tokens there are.
//  * the remaining blocks: one wave per 64-channel tile decides whether every
//    A row of the tile has the structured-real form A[d,n] = (n+1)*A[d,0],
//    A[d,0] < 0 (tile_fast = 1) or not (0).  Later launches read the flag and
//    take the matching path; A is never copied to the host.
template <class IO, int NT>
__global__ __launch_bounds__(256) void k_prep(const typename IO::T *__restrict__ B,
                                              const typename IO::T *__restrict__ C,
                                              float *__restrict__ bc, int64_t rows, int N,
                                              const float *__restrict__ A, int64_t dim,
                                              int *__restrict__ tile_fast, int64_t tiles_per_batch,
                                              int64_t prep_blocks) {
    if (blockIdx.x < prep_blocks) {
        for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < rows * NT;
             i += prep_blocks * blockDim.x) {
            const int64_t r = i / NT;
            const int n = int(i - r * NT);
            float bv = 0.f, cv = 0.f;
            if (n < N) {
                bv = IO::ld(B, r * N + n);
                cv = IO::ld(C, r * N + n);
            }
            bc[r * (2 * NT) + n] = bv / float(n + 1);
            bc[r * (2 * NT) + NT + n] = cv;
        }
        return;
    }
    const int64_t dt = (int64_t(blockIdx.x) - prep_blocks) * 4 + threadIdx.x / kWave;
    if (dt >= tiles_per_batch) return;  // whole wave
    const int lane = threadIdx.x % kWave;
    const int64_t d = min(dt * kWave + lane, dim - 1);
    const float a0 = A[d * N];
    bool ok = (a0 < 0.f) && (a0 > -INFINITY);
    for (int n = 1; n < N; ++n) ok = ok && (A[d * N + n] == a0 * float(n + 1));
    const bool all_ok = __all(ok);
    if (lane == 0) tile_fast[dt] = all_ok ? 1 : 0;
}

// Elementwise launches stride over their range with at most this many blocks.
constexpr int64_t kMaxStrideBlocks = int64_t(1) << 20;

__global__ __launch_bounds__(256) void k_copy_or_zero(float *__restrict__ dst,
                                                      const float *__restrict__ src, int64_t count) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += int64_t(gridDim.x) * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

// ----------------------------------------------------------------------------
// Front end: raw inputs of the three tokens before token ts of batch row b,
// channel d -- from x for tokens >= 0, from the carried inputs for tokens < 0
// (row K-1+t of conv_state; zero when it is absent or the row does not exist).
template <class IO>
__device__ void fe_prefix(const typename IO::T *x, const FeArgs &fe, int64_t b, int64_t L,
                          int64_t dim, int64_t d, int64_t ts, float &p3, float &p2, float &p1) {
    using T = typename IO::T;
    const T *cs = static_cast<const T *>(fe.conv_state);
    auto raw = [&](int64_t t) -> float {
        if (t >= 0) return t < L ? IO::ld(x, (b * L + t) * dim + d) : 0.f;
        const int64_t r = fe.K - 1 + t;
        return (cs && r >= 0) ? IO::ld(cs, (b * (fe.K - 1) + r) * dim + d) : 0.f;
    };
    p3 = raw(ts - 3);
    p2 = raw(ts - 2);
    p1 = raw(ts - 1);
}

// conv_state_out[b, j, d] = raw input of token L-(K-1)+j: from x, or, for
// sequences shorter than K-1, from the carried inputs (zero when absent).
template <class IO>
__global__ __launch_bounds__(256) void k_conv_tail(const typename IO::T *__restrict__ x,
                                                   FeArgs fe, typename IO::T *__restrict__ out,
                                                   int64_t batch, int64_t L, int64_t dim) {
    using T = typename IO::T;
    const int64_t rows = fe.K - 1;
    const T *cs = static_cast<const T *>(fe.conv_state);
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < batch * rows * dim;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t d = i % dim;
        const int64_t j = (i / dim) % rows;
        const int64_t b = i / (dim * rows);
        const int64_t t = L - rows + j;
        T v = T(0);
        if (t >= 0)
            v = x[(b * L + t) * dim + d];
        else if (cs)
            v = cs[(b * rows + (t + rows)) * dim + d];
        out[i] = v;
    }
}

// ----------------------------------------------------------------------------
// Segment kernels (shapes with too few 64-channel tiles to fill the chip with
// the lockstep kernel): the sequence is cut into time segments and
//   k_seg:    one wave per (tile, segment) scans its segment -- segment 0 from
//             the state before token 0, every other one from zero -- stores
//             its outputs and writes its aggregate (sum of delta, end state);
//   k_carry:  per (batch row, state, channel), folds the aggregates in segment
//             order with the associative combine (groups of segments composed
//             through LDS), overwriting each with the state that enters the
//             next segment, and writes the final state;
//   k_segfix: one wave per (tile, segment >= 1) reads the state k_in its
//             segment really started from and adds its contribution
//             sum_n C_n Abar_n(segment start..t) k_in[n] to the stored outputs
//             (2 operations per state and token, against 3 for a second pass
//             over the recurrence).
// The contribution decays with exp(A * (sum of delta since the segment start)):
// on the structured-real path, once that decay is exactly 0 in every lane (and
// k_in is finite) every later term is exactly 0 and the wave stops.
constexpr int kUnroll = 8;  // tokens of x/delta prefetched ahead

// Workgroups are handed to the 8 XCDs in turn (workgroup i to XCD i mod 8), and
// each XCD has its own L2.  The forward kernels renumber them so that XCD x
// takes the x-th eighth of the logical order, in order: the tiles of one segment
// (segment kernels) or of one batch row (lockstep kernel) run on one XCD at
// about the same time and read the B/C rows they share from that XCD's L2
// instead of each fetching them.  (Launches not a multiple of 8 keep the plain
// order.)  Measured on the lockstep kernel: 416 -> 408-411 us on the
// 4 x 8192 x 4096 workload; the same renumbering made the backward and the
// scalar-A scan 3-4% slower, and they keep the plain order.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_order(int64_t wid, int64_t n) {
    return n % kXcds == 0 ? (wid % kXcds) * (n / kXcds) + wid / kXcds : wid;
}

template <class IO, int NT, bool kFast, bool FE>
__device__ __forceinline__ void seg_scan(
    const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ delta,
    const float *__restrict__ A, const float *__restrict__ bc, const float *__restrict__ Dskip,
    const float *__restrict__ h0, typename IO::T *__restrict__ y, float *__restrict__ final_state,
    float *__restrict__ agg_sum, float *__restrict__ agg_h, int64_t batch, int64_t L, int64_t dim, int N,
    int64_t seg_len, int segments, int seg, int64_t b, int64_t dbase, int lane, const FeArgs &fe) {
    using T = typename IO::T;
    const bool active = dbase + lane < dim;
    const int lo = active ? lane : int(dim - 1 - dbase);  // clamped lane offset
    const int64_t d = dbase + lo;
    const int64_t t0 = int64_t(seg) * seg_len;
    const int64_t t1 = min(L, t0 + seg_len);

    float a[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) a[n] = (n < N) ? A[d * N + n] : 0.f;

    // segment 0 starts from the state before token 0, the others from zero
    float h[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) h[n] = (seg == 0 && h0 && n < N) ? h0[(b * dim + d) * N + n] : 0.f;

    // Descriptors cover exactly this segment: tokens past its end read x = delta
    // = 0 (the state is left unchanged) and their stores are dropped, so the
    // token loop has no per-token branches.
    constexpr int ES = IO::kBytes;
    constexpr int U = kUnroll;
    const int nseg = int(t1 - t0);
    const int last = nseg - 1;
    const uint32_t voff = uint32_t((dbase + lane) * ES);
    const uint32_t rowb = uint32_t(dim * ES);
    const int64_t seg_bytes = int64_t(nseg) * dim * ES;
    const rsrc_t rx = make_rsrc(x + (b * L + t0) * dim, seg_bytes);
    const rsrc_t rd = make_rsrc(delta + (b * L + t0) * dim, seg_bytes);
    const rsrc_t ry = make_rsrc(y + (b * L + t0) * dim, seg_bytes);
    const float *bc0 = bc + (b * L + t0) * (2 * NT);
    float dsum = 0.f;

    T xr[U], dr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        xr[u] = IO::bld(rx, voff, uint32_t(u) * rowb);
        dr[u] = IO::bld(rd, voff, uint32_t(u) * rowb);
    }
    float rowA[2 * NT], rowB[2 * NT];
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) rowA[i] = bc0[i];

    const float alpha = -a[0];
    const float inv_alpha = 1.f / alpha;
    const float a2 = a[0] * kLog2e;
    // the structured-real state is held scaled, k = alpha h
    const float dska = (Dskip ? Dskip[d] : 0.f) * (kFast ? alpha : 1.f);
    float k[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) k[n] = kFast ? h[n] * alpha : h[n];
    // front end: per-lane coefficients and the raw inputs of the 3 tokens before
    // the segment (the convolution window, carried through the token loop)
    FeLane fl{};
    float p3 = 0.f, p2 = 0.f, p1 = 0.f;
    if constexpr (FE) {
        fl.init(fe, d);
        fe_prefix<IO>(x, fe, b, L, dim, d, t0, p3, p2, p1);
    }

    // one token: structured-real update on the scaled state, or the general one;
    // sto is the token's output offset in the row stream
    auto token = [&](float xv, float dv, const float *row, uint32_t sto) {
        float yacc = dska * xv;
        dsum += dv;
        if constexpr (kFast) {
            const float u = dv * a2;
            const float r = exp2_hw(u);
            sr_update<NT>(r, one_minus_exp2(u, r), xv, row, k,
                          [&](int n) { yacc = fmaf(row[NT + n], k[n], yacc); });
        } else {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float an = a[n];
                const float abar = exp2_hw(dv * (an * kLog2e));
                const float g = zoh_gain(dv, an, dv * an, abar);
                k[n] = fmaf(abar, k[n], g * ((row[n] * float(n + 1)) * xv));
                yacc = fmaf(row[NT + n], k[n], yacc);
            }
        }
        if (active) IO::bst(IO::enc(kFast ? yacc * inv_alpha : yacc), ry, voff, sto);
    };
    for (int g0 = 0; g0 < nseg; g0 += U) {
        float xv[U], dv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (FE) {
                // tokens past the segment would not be neutral after the front end
                // (softplus(bias) > 0): they are zeroed explicitly
                // (a 0/1 factor rather than a select, so nothing is branched around)
                const float xr0 = IO::cvt(xr[u]);
                const float vm = g0 + u < nseg ? 1.f : 0.f;
                const float uu = fl.u(p3, p2, p1, xr0);
                p3 = p2;
                p2 = p1;
                p1 = xr0;
                xv[u] = uu * vm;
                dv[u] = fl.delta(IO::cvt(dr[u])) * vm;
            } else {
                xv[u] = IO::cvt(xr[u]);
                dv[u] = IO::cvt(dr[u]);
            }
        }
        // token offsets formed here, one add per token, rather than kept live
        // across the loop as a set of scalar registers
        uint32_t sl = uint32_t(g0 + U) * rowb, sto = uint32_t(g0) * rowb;
        asm volatile("" : "+s"(sl), "+s"(sto));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xr[u] = IO::bld(rx, voff, sl);
            dr[u] = IO::bld(rd, voff, sl);
            sl += rowb;
        }
#pragma unroll
        for (int u = 0; u < U; u += 2) {
            const int tau = g0 + u;
            __builtin_amdgcn_sched_barrier(0);
            wait_scalar_loads();
            {
                const float *rn = bc0 + min(tau + 1, last) * (2 * NT);
#pragma unroll
                for (int i = 0; i < 2 * NT; ++i) rowB[i] = rn[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            token(xv[u], dv[u], rowA, sto);
            sto += rowb;
            __builtin_amdgcn_sched_barrier(0);
            wait_scalar_loads();
            {
                const float *rn = bc0 + min(tau + 2, last) * (2 * NT);
#pragma unroll
                for (int i = 0; i < 2 * NT; ++i) rowA[i] = rn[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            token(xv[u + 1], dv[u + 1], rowB, sto);
            sto += rowb;
        }
    }
    if (!active) return;
    if (segments == 1) {
        // one segment: its end state is the final state
        if (final_state) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                if (n < N) final_state[(b * dim + d) * N + n] = kFast ? k[n] * inv_alpha : k[n];
        }
        return;
    }
    const int64_t cs = int64_t(seg) * batch + b;
    agg_sum[cs * dim + d] = dsum;
#pragma unroll
    for (int n = 0; n < NT; ++n) agg_h[(cs * NT + n) * dim + d] = kFast ? k[n] * inv_alpha : k[n];
}

// one launch per A path (a wave of a tile of the other kind returns at once):
// the general path's registers would otherwise set the fast path's occupancy
template <class IO, int NT, bool kFast, bool FE>
__global__ __launch_bounds__(kWave) void k_seg(
    const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ delta,
    const float *__restrict__ A, const float *__restrict__ bc, const float *__restrict__ Dskip,
    const float *__restrict__ h0, typename IO::T *__restrict__ y, float *__restrict__ final_state,
    float *__restrict__ agg_sum, float *__restrict__ agg_h, const int *__restrict__ tile_fast,
    int64_t batch, int64_t L, int64_t dim, int N, int64_t seg_len, int segments,
    int64_t tiles_per_batch, int64_t tiles, FeArgs fe) {
    const int lane = threadIdx.x;
    const int64_t wid = xcd_order(blockIdx.x, gridDim.x);
    const int seg = int(wid / tiles);
    const int64_t tile = wid - int64_t(seg) * tiles;
    const int64_t b = tile / tiles_per_batch;
    const int64_t dt = tile - b * tiles_per_batch;
    if ((tile_fast[dt] != 0) != kFast) return;
    seg_scan<IO, NT, kFast, FE>(x, delta, A, bc, Dskip, h0, y, final_state, agg_sum, agg_h, batch, L, dim, N,
                                seg_len, segments, seg, b, dt * kWave, lane, fe);
}

// Carry pass: the aggregates of segment j (sum of delta, end state from zero,
// unscaled) are folded in order, H <- exp(A[d,n] * sum_j) H + h_j, starting
// from zero (segment 0 started from the state before token 0, so its end state
// already holds it); aggregate j is overwritten with H, the state that enters
// segment j+1, and the last H is the final state.
// A workgroup takes 64 channels of one (batch row, state) and splits the
// segments into kCarryG consecutive groups, one wave each: every wave folds its
// group from zero, the group results are composed through LDS into the state
// entering each group, and every wave walks its group again from that state,
// storing the entering states (the second walk reads what the first brought
// into L2).  The loads of kCarryU segments are issued ahead of their fold.
constexpr int kCarryU = 8;
constexpr int kCarryG = 16;

__global__ __launch_bounds__(kCarryG *kWave) void k_carry(const float *__restrict__ A,
                                                          const float *__restrict__ agg_sum,
                                                          float *__restrict__ agg_h, float *__restrict__ final_state,
                                                          int64_t batch, int64_t dim, int N, int nt, int segments) {
    __shared__ float lsum[kCarryG][kWave], lh[kCarryG][kWave];
    lds_poison(lsum, lh);
    const int lane = threadIdx.x % kWave, g = threadIdx.x / kWave;
    const int64_t tpb = (dim + kWave - 1) / kWave;
    const int64_t blocks = batch * nt * tpb;
    const int per = (segments + kCarryG - 1) / kCarryG;
    const int j0 = min(segments, g * per), j1 = min(segments, j0 + per);
    for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x) {
        const int64_t dt = blk % tpb;
        const int64_t bn = blk / tpb;
        const int n = int(bn % nt);
        const int64_t b = bn / nt;
        const bool active = dt * kWave + lane < dim;
        const int64_t d = active ? dt * kWave + lane : dim - 1;
        const float an = n < N ? A[d * N + n] * kLog2e : 0.f;  // padded states: sums of zeros
        // walk this wave's group from H; `store` writes each entering state
        auto walk = [&](float H, float &ssum, bool store) {
            for (int j = j0; j < j1; j += kCarryU) {
                float sv[kCarryU], hv[kCarryU];
#pragma unroll
                for (int u = 0; u < kCarryU; ++u) {
                    const int64_t cj = int64_t(min(j + u, j1 - 1)) * batch + b;
                    sv[u] = agg_sum[cj * dim + d];
                    hv[u] = agg_h[(cj * nt + n) * dim + d];
                }
#pragma unroll
                for (int u = 0; u < kCarryU; ++u) {
                    if (j + u < j1) {
                        ssum += sv[u];
                        H = fmaf(exp2_hw(an * sv[u]), H, hv[u]);
                        if (store && active) agg_h[((int64_t(j + u) * batch + b) * nt + n) * dim + d] = H;
                    }
                }
            }
            return H;
        };
        float ssum = 0.f;
        const float Hg = walk(0.f, ssum, false);
        lsum[g][lane] = ssum;
        lh[g][lane] = Hg;
        __syncthreads();
        float E = 0.f;  // the state entering this wave's group
        for (int q = 0; q < g; ++q) E = fmaf(exp2_hw(an * lsum[q][lane]), E, lh[q][lane]);
        float unused = 0.f;
        const float H = walk(E, unused, true);
        // the last group ends at the last segment (an empty group: E is the total)
        if (g == kCarryG - 1 && active && n < N && final_state) final_state[(b * dim + d) * N + n] = H;
        __syncthreads();  // LDS reused by the next block of the loop
    }
}

template <class IO, int NT, bool kFast, bool FE>
__device__ __forceinline__ void seg_fix(
    const typename IO::T *__restrict__ delta, const float *__restrict__ A, const float *__restrict__ bc,
    typename IO::T *__restrict__ y, const float *__restrict__ carried, int64_t batch, int64_t L,
    int64_t dim, int N, int64_t seg_len, int seg, int64_t b, int64_t dbase, int lane, const FeArgs &fe) {
    using T = typename IO::T;
    const bool active = dbase + lane < dim;
    const int lo = active ? lane : int(dim - 1 - dbase);
    const int64_t d = dbase + lo;
    float a[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) a[n] = (n < N) ? A[d * N + n] : 0.f;
    // the state entering this segment (unscaled), from the carry pass
    const int64_t cs = int64_t(seg - 1) * batch + b;
    float kin[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) kin[n] = carried[(cs * NT + n) * dim + d];
    // early exit needs k_in finite in every lane (an infinite or NaN entering
    // state keeps adding to the outputs however small the decay)
    bool fin = true;
#pragma unroll
    for (int n = 0; n < NT; ++n) fin = fin && (fabsf(kin[n]) <= 3.402823466e38f);
    const bool may_stop = kFast && __all(fin);

    constexpr int ES = IO::kBytes;
    constexpr int U = kUnroll;
    const int64_t t0 = int64_t(seg) * seg_len;
    const int nseg = int(min(L, t0 + seg_len) - t0);
    const int last = nseg - 1;
    const uint32_t voff = uint32_t((dbase + lane) * ES);
    const uint32_t voff_st = active ? voff : 0x80000000u;  // lanes past dim: beyond every range
    const uint32_t rowb = uint32_t(dim * ES);
    const int64_t seg_bytes = int64_t(nseg) * dim * ES;
    const rsrc_t rd = make_rsrc(delta + (b * L + t0) * dim, seg_bytes);
    const rsrc_t ry = make_rsrc(y + (b * L + t0) * dim, seg_bytes);
    const float *cc0 = bc + (b * L + t0) * (2 * NT) + NT;
    const float a2 = a[0] * kLog2e;
    float db = 0.f;
    if constexpr (FE) db = fe.delta_bias ? fe.delta_bias[d] : 0.f;
    float rho = 1.f, cum = 0.f;  // decay / sum of delta since the segment start

    // the step sizes and stored outputs of a group of U tokens are loaded one group
    // ahead of their use
    T dr[U], yr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        dr[u] = IO::bld(rd, voff, uint32_t(u) * rowb);
        yr[u] = IO::bld(ry, voff, uint32_t(u) * rowb);
    }
    float cA[NT], cB[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) cA[n] = cc0[n];
    auto fix = [&](float dv, float yl, const float *crow, uint32_t sto) {
        float corr;
        if constexpr (kFast) {
            rho *= exp2_hw(dv * a2);
            float acc = crow[NT - 1] * kin[NT - 1];
#pragma unroll
            for (int n = NT - 2; n >= 0; --n) acc = fmaf(acc, rho, crow[n] * kin[n]);
            corr = acc * rho;
        } else {
            cum += dv;
            corr = 0.f;
#pragma unroll
            for (int n = 0; n < NT; ++n) corr = fmaf(crow[n] * kin[n], exp2_hw((a[n] * kLog2e) * cum), corr);
        }
        IO::bst(IO::enc(yl + corr), ry, voff_st, sto);
    };
    for (int g0 = 0; g0 < nseg; g0 += U) {
        uint32_t sy = uint32_t(g0) * rowb, sl = uint32_t(g0 + U) * rowb;
        asm volatile("" : "+s"(sy), "+s"(sl));
        float dv[U], yv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (FE)
                dv[u] = softplus_f(IO::cvt(dr[u]) + db);  // tokens past the end: never stored
            else
                dv[u] = IO::cvt(dr[u]);
            yv[u] = IO::cvt(yr[u]);
        }
        // the next group's loads
#pragma unroll
        for (int u = 0; u < U; ++u) {
            dr[u] = IO::bld(rd, voff, sl);
            yr[u] = IO::bld(ry, voff, sl);
            sl += rowb;
        }
        uint32_t sto = sy;
#pragma unroll
        for (int u = 0; u < U; u += 2) {
            const int tau = g0 + u;
            __builtin_amdgcn_sched_barrier(0);
            wait_scalar_loads();
            {
                const float *rn = cc0 + min(tau + 1, last) * (2 * NT);
#pragma unroll
                for (int n = 0; n < NT; ++n) cB[n] = rn[n];
            }
            __builtin_amdgcn_sched_barrier(0);
            fix(dv[u], yv[u], cA, sto);
            sto += rowb;
            __builtin_amdgcn_sched_barrier(0);
            wait_scalar_loads();
            {
                const float *rn = cc0 + min(tau + 2, last) * (2 * NT);
#pragma unroll
                for (int n = 0; n < NT; ++n) cA[n] = rn[n];
            }
            __builtin_amdgcn_sched_barrier(0);
            fix(dv[u + 1], yv[u + 1], cB, sto);
            sto += rowb;
        }
        // every later contribution is exactly zero once the decay is
        if (may_stop && !__any(rho != 0.f)) break;
    }
}

template <class IO, int NT, bool kFast, bool FE>
__global__ __launch_bounds__(kWave) void k_segfix(
    const typename IO::T *__restrict__ delta, const float *__restrict__ A, const float *__restrict__ bc,
    typename IO::T *__restrict__ y, const float *__restrict__ carried, const int *__restrict__ tile_fast, int64_t batch, int64_t L,
    int64_t dim, int N, int64_t seg_len, int64_t tiles_per_batch, int64_t tiles, FeArgs fe) {
    const int lane = threadIdx.x;
    const int64_t wid = xcd_order(blockIdx.x, gridDim.x);
    const int seg = 1 + int(wid / tiles);  // segments 1 .. segments-1
    const int64_t tile = wid - int64_t(seg - 1) * tiles;
    const int64_t b = tile / tiles_per_batch;
    const int64_t dt = tile - b * tiles_per_batch;
    if ((tile_fast[dt] != 0) != kFast) return;
    seg_fix<IO, NT, kFast, FE>(delta, A, bc, y, carried, batch, L, dim, N, seg_len, seg, b, dt * kWave, lane,
                               fe);
}

// ----------------------------------------------------------------------------
// Lockstep chunked scan (one launch, no aggregate pass).  A workgroup of W waves
// owns one 64-channel tile for the whole sequence, processed in chunks of W*TS
// tokens; wave w takes the w-th run of TS tokens of every chunk:
//   1. local pass: wave 0 starts from the chunk's carried state, the others
//      from zero; each keeps its TS outputs and what it needs to rebuild the
//      decay since its run start in VGPRs;
//   2. every wave publishes (sum of delta, local end state) in LDS; after a
//      barrier the states are split across the waves (NT/W each) and every
//      wave folds the W aggregates of its states in order with the
//      associative combine -- the decay of a run is exp(A sum(delta)) -- writing
//      the state entering each wave's run and the chunk's carry-out to LDS;
//   3. after a second barrier waves 1..W-1 add the contribution of the state
//      they entered with, sum_n C_n Abar_n(run start..t) k_in[n], and store y.
// A tile whose A rows all have the structured-real form takes the fast path:
// one exp per token, the scaled state k = -A[d,0] h, and the step-3 sum as a
// Horner polynomial in rho = prod r (2 VALU per state).  Any other tile takes
// the general path in the same launch: an exp and the ZOH gain per state, and
// the step-3 decays exp(A[d,n] * (sum of delta since the run start)).
template <int NT, int W>
struct LockLds {
    float sum[W][kWave];      // sum of delta over each run
    float k[W][NT][kWave];    // each run's end state from its starting state
    float pre[W][NT][kWave];  // [0]: the chunk's carry-out; [j]: state entering run j
    float zero[NT][kWave];    // the (zero) state runs 1.. start from
    float arow[NT][kWave];    // general path: each lane's A row (kept out of VGPRs)
};

template <class IO, int NT, int W, int TS, bool FE, bool kFast>
__device__ __forceinline__ void lockstep_tile(
    LockLds<NT, W> &sh, const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ delta,
    const float *__restrict__ A, const float *__restrict__ bc, const float *__restrict__ Dskip,
    const float *__restrict__ h0, typename IO::T *__restrict__ y, float *__restrict__ final_state, int L,
    int64_t dim, int N, int64_t b, int64_t dbase, int w, int lane, const FeArgs &fe) {
    using T = typename IO::T;
    constexpr int U = kUnroll;
    static_assert(TS % U == 0 && U % 2 == 0, "TS must be a multiple of the prefetch group");
    static_assert(W >= 3, "waves 0, 1 and 2 each initialise a part of the LDS");
    constexpr int NPW = (NT + W - 1) / W;  // states each wave folds
    constexpr int CH = W * TS;             // tokens per chunk
    constexpr int ES = IO::kBytes;

    const bool active = dbase + lane < dim;
    const int64_t d = active ? dbase + lane : dim - 1;
    const float a0 = A[d * N];
    // structured-real: the state is held scaled, k = alpha h with alpha = -A[d,0] > 0
    const float alpha = kFast ? -a0 : 1.f;
    const float inv_alpha = kFast ? 1.f / alpha : 1.f;
    const float a2 = a0 * kLog2e;
    const float dska = (Dskip ? Dskip[d] : 0.f) * alpha;  // the skip in the state's scale
    // the states this wave folds: their decay exponent (log2) per unit of delta
    float afold[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int n = w * NPW + i;
        afold[i] = (n < N ? A[d * N + n] : 0.f) * kLog2e;
    }
    const float *bcrow = bc + (b * L) * (2 * NT);
    const int nchunks = (L + CH - 1) / CH;
    // per-lane byte offset inside a token row; per-token row stride (uniform).
    // Stores of lanes past dim go to an offset beyond every descriptor's range.
    const uint32_t voff = uint32_t((dbase + lane) * ES);
    const uint32_t voff_st = active ? voff : 0x80000000u;
    const uint32_t rowb = uint32_t(dim * ES);

    // descriptors over [token t0, end of the sequence) of this batch row
    auto rsrc_at = [&](const T *base, int t0) {
        return make_rsrc(base + (b * L + t0) * dim, int64_t(L - t0) * dim * ES);
    };

    T xr[U], dr[U];
    {
        const rsrc_t rx = rsrc_at(x, w * TS), rd = rsrc_at(delta, w * TS);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xr[u] = IO::bld(rx, voff, uint32_t(u) * rowb);
            dr[u] = IO::bld(rd, voff, uint32_t(u) * rowb);
        }
    }
    // Every run starts from a state read from LDS: run 0 from pre[0] (the state
    // before token 0 for the first chunk, the carry-out of the previous chunk
    // after it), the others from zeros.  One code path for every wave, so the
    // reads land in the state registers without copies.
    if (w == 0) {
#pragma unroll
        for (int n = 0; n < NT; ++n) sh.pre[0][n][lane] = (h0 && n < N) ? h0[(b * dim + d) * N + n] * alpha : 0.f;
    } else if (w == 1) {
#pragma unroll
        for (int n = 0; n < NT; ++n) sh.zero[n][lane] = 0.f;
    } else if (!kFast && w == 2) {
#pragma unroll
        for (int n = 0; n < NT; ++n) sh.arow[n][lane] = n < N ? A[d * N + n] : 0.f;
    }
    __syncthreads();
    const float(*kstart)[kWave] = w == 0 ? sh.pre[0] : sh.zero;
    float k[NT];
    // front end: per-lane coefficients; the convolution window (raw inputs of
    // the 3 tokens before the current one) starts from the tokens before this
    // wave's first run, and the 3 tokens before its next run are prefetched with
    // that run's first group
    FeLane fl{};
    float p3 = 0.f, p2 = 0.f, p1 = 0.f;
    T pr[3] = {T(0), T(0), T(0)};
    if constexpr (FE) {
        fl.init(fe, d);
        fe_prefix<IO>(x, fe, b, L, dim, d, int64_t(w) * TS, p3, p2, p1);
    }

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * CH + w * TS;  // below 2^31 (launch condition)
        const int nv = __builtin_amdgcn_readfirstlane(max(0, min(TS, L - t0)));  // uniform
        const rsrc_t rx = rsrc_at(x, t0), rd = rsrc_at(delta, t0), ry = rsrc_at(y, t0);
        const float *bc0 = bcrow + int64_t(min(t0, L - 1)) * (2 * NT);
#pragma unroll
        for (int n = 0; n < NT; ++n) k[n] = kstart[n][lane];
        if constexpr (FE) {
            if (c > 0) {
                p3 = IO::cvt(pr[0]);
                p2 = IO::cvt(pr[1]);
                p1 = IO::cvt(pr[2]);
            }
        }
        // yl: the run's outputs from its starting state (fast path: in the state's
        // scale); tk: fast path r of each token (rho = their running product),
        // general path the running sum of delta after each token
        float yl[TS], tk[TS];
        float dsum = 0.f;
        // The run is processed branch-free even when it is ragged: tokens past
        // the end of the sequence read x = delta = 0 through the descriptor's
        // range check, which leaves the state exactly unchanged, and their stores
        // fall outside the range and are dropped.  Only the B/C row index is
        // clamped.  uniform: kept in a scalar register, so the per-token B/C row
        // offsets below are scalar arithmetic
        const int last = __builtin_amdgcn_readfirstlane(max(nv - 1, 0));
        int nvs = nv;  // the valid-token count as an opaque 32-bit scalar
        if constexpr (FE) asm volatile("" : "+s"(nvs));
        // B/(n+1) and C rows of two consecutive tokens (ping-pong): the scalar
        // loads of token tau+1 are issued, after waiting for those of tau,
        // before tau computes, so they have a whole token to arrive.
        float rowA[2 * NT], rowB[2 * NT];
#pragma unroll
        for (int i = 0; i < 2 * NT; ++i) rowA[i] = bc0[i];
        auto token = [&](int tau, float xv, float dv, const float *row) {
            dsum += dv;
            float yacc = dska * xv;
            if constexpr (kFast) {
                const float u = dv * a2;
                const float r = exp2_hw(u);
                tk[tau] = r;
                sr_update<NT>(r, one_minus_exp2(u, r), xv, row, k,
                              [&](int n) { yacc = fmaf(row[NT + n], k[n], yacc); });
            } else {
                tk[tau] = dsum;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const float an = sh.arow[n][lane];
                    const float abar = exp2_hw(dv * (an * kLog2e));
                    const float g = zoh_gain_nb(dv, an, dv * an, abar);
                    k[n] = fmaf(abar, k[n], g * ((row[n] * float(n + 1)) * xv));
                    yacc = fmaf(row[NT + n], k[n], yacc);
                }
            }
            yl[tau] = yacc;
        };
#pragma unroll
        for (int g = 0; g < TS / U; ++g) {
            float xv[U], dv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (FE) {
                    // tokens past the end are not neutral after the front end
                    // (softplus(bias) > 0): their step size is zeroed (a 0/1 factor
                    // rather than a select, so nothing is branched around), which
                    // leaves the state exactly unchanged whatever their input; their
                    // outputs are not stored.  The factor is chosen on the scalar
                    // unit from a 32-bit count.
                    const float xr0 = IO::cvt(xr[u]);
                    int vmb = g * U + u < nvs ? 0x3f800000 : 0;  // 1.0f or 0.0f
                    asm volatile("" : "+s"(vmb));
                    const float vm = __int_as_float(vmb);
                    const float uu = fl.u(p3, p2, p1, xr0);
                    p3 = p2;
                    p2 = p1;
                    p1 = xr0;
                    xv[u] = uu;
                    dv[u] = fl.delta(IO::cvt(dr[u])) * vm;
                } else {
                    xv[u] = IO::cvt(xr[u]);
                    dv[u] = IO::cvt(dr[u]);
                }
            }
            // prefetch the next group of this wave's stream: the rest of this run,
            // then the start of its run in the next chunk
            const uint32_t nxt = (g + 1 < TS / U) ? uint32_t((g + 1) * U) : uint32_t(CH);
            // the token offsets are formed here, one add per token, rather than
            // hoisted out of the chunk loop as 16 live scalar registers
            uint32_t so = nxt * rowb;
            asm volatile("" : "+s"(so));
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xr[u] = IO::bld(rx, voff, so);
                dr[u] = IO::bld(rd, voff, so);
                so += rowb;
            }
            if constexpr (FE) {
                if (g + 1 == TS / U) {
#pragma unroll
                    for (int i = 0; i < 3; ++i) pr[i] = IO::bld(rx, voff, uint32_t(CH - 3 + i) * rowb);
                }
            }
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                const int tau = g * U + u;
                __builtin_amdgcn_sched_barrier(0);
                wait_scalar_loads();
                {
                    const float *rn = bc0 + min(tau + 1, last) * (2 * NT);
#pragma unroll
                    for (int i = 0; i < 2 * NT; ++i) rowB[i] = rn[i];
                }
                __builtin_amdgcn_sched_barrier(0);
                token(tau, xv[u], dv[u], rowA);
                __builtin_amdgcn_sched_barrier(0);
                wait_scalar_loads();
                {
                    const float *rn = bc0 + min(tau + 2, last) * (2 * NT);
#pragma unroll
                    for (int i = 0; i < 2 * NT; ++i) rowA[i] = rn[i];
                }
                __builtin_amdgcn_sched_barrier(0);
                token(tau + 1, xv[u + 1], dv[u + 1], rowB);
            }
        }
        if (w == 0) {
            // run 0 started from the carried state: its outputs are final
            uint32_t sto = 0;
            asm volatile("" : "+s"(sto));
#pragma unroll
            for (int tau = 0; tau < TS; ++tau) {
                IO::bst(IO::enc(yl[tau] * inv_alpha), ry, voff_st, sto);
                sto += rowb;
            }
        }
        sh.sum[w][lane] = dsum;
#pragma unroll
        for (int n = 0; n < NT; ++n) sh.k[w][n][lane] = k[n];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            if (n < NT) {
                float P = sh.k[0][n][lane];  // run 0 started from the carry: its end state is exact
                for (int j = 1; j < W; ++j) {
                    sh.pre[j][n][lane] = P;
                    P = fmaf(exp2_hw(afold[i] * sh.sum[j][lane]), P, sh.k[j][n][lane]);
                }
                sh.pre[0][n][lane] = P;
            }
        }
        __syncthreads();
        if (w != 0 && nv > 0) {
            float kin[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) kin[n] = sh.pre[w][n][lane];
            float cA[NT], cB[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) cA[n] = bc0[NT + n];
            float rho = 1.f;
            auto fix = [&](int tau, const float *crow, uint32_t sto) {
                float yv;
                if constexpr (kFast) {
                    // sum_n C_n rho^(n+1) k_in[n] as a Horner polynomial in rho
                    rho *= tk[tau];
                    float acc = crow[NT - 1] * kin[NT - 1];
#pragma unroll
                    for (int n = NT - 2; n >= 0; --n) acc = fmaf(acc, rho, crow[n] * kin[n]);
                    yv = fmaf(acc, rho, yl[tau]) * inv_alpha;
                } else {
                    float acc = yl[tau];
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        acc = fmaf(crow[n] * kin[n], exp2_hw((sh.arow[n][lane] * kLog2e) * tk[tau]), acc);
                    yv = acc;
                }
                IO::bst(IO::enc(yv), ry, voff_st, sto);
            };
            uint32_t sto = 0;
            asm volatile("" : "+s"(sto));
            // an opaque copy of the run's last index: the C row addresses are formed
            // again here (scalar arithmetic) instead of being kept from the token
            // loop across the barriers, where they would not fit in scalar registers
            int lastf = last;
            if constexpr (!FE) asm volatile("" : "+s"(lastf));
#pragma unroll
            for (int tau = 0; tau < TS; tau += 2) {
                __builtin_amdgcn_sched_barrier(0);
                wait_scalar_loads();
                {
                    const float *rn = bc0 + min(tau + 1, lastf) * (2 * NT) + NT;
#pragma unroll
                    for (int n = 0; n < NT; ++n) cB[n] = rn[n];
                }
                __builtin_amdgcn_sched_barrier(0);
                fix(tau, cA, sto);
                sto += rowb;
                __builtin_amdgcn_sched_barrier(0);
                wait_scalar_loads();
                {
                    const float *rn = bc0 + min(tau + 2, lastf) * (2 * NT) + NT;
#pragma unroll
                    for (int n = 0; n < NT; ++n) cA[n] = rn[n];
                }
                __builtin_amdgcn_sched_barrier(0);
                fix(tau + 1, cB, sto);
                sto += rowb;
            }
        }
    }
    if (final_state && active) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            const int n = w * NPW + i;
            if (n < N) final_state[(b * dim + d) * N + n] = sh.pre[0][n][lane] * inv_alpha;
        }
    }
}

template <class IO, int NT, int W, int TS, bool FE>
__global__ __launch_bounds__(W *kWave) void k_lockstep(
    const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ delta,
    const float *__restrict__ A, const float *__restrict__ bc, const float *__restrict__ Dskip,
    const float *__restrict__ h0, typename IO::T *__restrict__ y, float *__restrict__ final_state,
    const int *__restrict__ tile_fast, int L, int64_t dim, int N, int64_t tiles_per_batch, FeArgs fe) {
    __shared__ LockLds<NT, W> sh;
    lds_poison(sh);
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
    const int lane = int(threadIdx.x) % kWave;
    const int64_t tile = xcd_order(blockIdx.x, gridDim.x);
    const int64_t b = tile / tiles_per_batch;
    const int64_t dt = tile - b * tiles_per_batch;
    // the tile's path is uniform over the workgroup
    if (tile_fast[dt])
        lockstep_tile<IO, NT, W, TS, FE, true>(sh, x, delta, A, bc, Dskip, h0, y, final_state, L, dim, N, b,
                                                dt * kWave, w, lane, fe);
    else
        lockstep_tile<IO, NT, W, TS, FE, false>(sh, x, delta, A, bc, Dskip, h0, y, final_state, L, dim, N, b,
                                                 dt * kWave, w, lane, fe);
}

// 1/(n+1) for state n = q SPL + j of a lane (q < LPC): constants for one or two
// lanes per channel
template <int SPL, int LPC>
__device__ __forceinline__ float inv_np1(int q, int j) {
    if constexpr (LPC == 1) return 1.f / float(j + 1);
    else if constexpr (LPC == 2) return q == 0 ? 1.f / float(j + 1) : 1.f / float(SPL + j + 1);
    else return 1.f / float(q * SPL + j + 1);
}

// S consecutive elements (S a multiple of 4, aligned to 4 elements) as floats,
// in 16-byte loads
template <int S>
__device__ __forceinline__ void ldrow(const float *p, float *o) {
#pragma unroll
    for (int j = 0; j < S; j += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(p + j);
        o[j] = v.x; o[j + 1] = v.y; o[j + 2] = v.z; o[j + 3] = v.w;
    }
}
template <int S>
__device__ __forceinline__ void ldrow(const uint16_t *p, float *o) {
    if constexpr (S % 8 == 0) {
#pragma unroll
        for (int j = 0; j < S; j += 8) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p + j);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                o[j + 2 * u] = __uint_as_float(w[u] << 16);
                o[j + 2 * u + 1] = __uint_as_float(w[u] & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < S; j += 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p + j);
            o[j] = __uint_as_float(v.x << 16);
            o[j + 1] = __uint_as_float(v.x & 0xFFFF0000u);
            o[j + 2] = __uint_as_float(v.y << 16);
            o[j + 3] = __uint_as_float(v.y & 0xFFFF0000u);
        }
    }
}

// One lane's SPL states of one channel (states n = q SPL + j, those >= N padded
// with zeros): the state update, and the lane's part of the readout C.h.
// The per-channel constants (which form the A row has, 1/A[d,0], the 1/(n+1) of
// the lane's states) are formed once by init() and shared by every batch row the
// thread updates.
template <int SPL, int LPC>
struct StepLane {
    bool sr;           // structured-real: A[d,n] = (n+1) A[d,0], A[d,0] < 0 for the lane's states
    float a0, a2, ra;  // A[d,0], A[d,0] log2(e), -1/A[d,0]
    float w[SPL];      // 1/(n+1) of the lane's states
    int n0;            // the lane's first state

    __device__ __forceinline__ void init(int q, int N, float a0_, const float *av) {
        a0 = a0_;
        a2 = a0 * kLog2e;
        ra = -1.f / a0;
        n0 = q * SPL;
        sr = (a0 < 0.f) && (a0 > -INFINITY);
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            w[j] = inv_np1<SPL, LPC>(q, j);
            if (n0 + j < N) sr = sr && (av[j] == a0 * float(n0 + j + 1));
        }
    }

    // structured-real states: one exp per lane, and with r = exp(delta A[d,0]) and
    // q_n = 1 - r^(n+1) = r q_(n-1) + q_0,
    //     h_n <- h_n + q_n (B_n x / ((n+1) alpha) - h_n),  alpha = -A[d,0],
    // the update of the scan kernels on the unscaled state; other states take
    // the general form (an exp and the ZOH gain per state)
    __device__ __forceinline__ float row(float dt, float xv, const float *av, const float *bv,
                                         const float *cv, float *h) const {
        float yacc = 0.f;
        if (sr) {
            const float u = dt * a2;
            const float r = exp2_hw(u);
            const float q0 = one_minus_exp2(u, r);
            // q_(n0-1) = 1 - r^n0 for this lane's first state n0
            const float un = u * float(n0);
            float qn = n0 == 0 ? 0.f : one_minus_exp2(un, exp2_hw(un));
            const float xa = xv * ra;
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                qn = fmaf(qn, r, q0);
                const float e = fmaf(bv[j] * w[j], xa, -h[j]);
                h[j] = fmaf(qn, e, h[j]);
                yacc = fmaf(cv[j], h[j], yacc);
            }
        } else {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const float z = dt * av[j];
                const float abar = exp2_hw(dt * (av[j] * kLog2e));
                const float g = zoh_gain(dt, av[j], z, abar);
                h[j] = fmaf(abar, h[j], g * (bv[j] * xv));
                yacc = fmaf(cv[j], h[j], yacc);
            }
        }
        return yacc;
    }
};

// ----------------------------------------------------------------------------
// Decode step: LPC lanes share one channel, each owning SPL consecutive states,
// so a wave reads and writes one contiguous span of the (batch, dim, N) state
// (SPL x 256 B).  The partial readouts are summed across the LPC lanes.  Memory
// bound: what limits it is the state bytes each CU keeps in flight, hence
// several 16-byte state loads per lane.  Per state one hardware exp2 and the
// gain above.
// With the front end (FE), x and delta are the raw token inputs: the step
// reads the K-1 carried raw inputs of its channel from conv_state, forms the
// convolution and softplus, and shifts conv_state by one token in place.
template <class IO, int NT, int SPL, bool kVec, bool FE, int BT>
__global__ __launch_bounds__(256) void k_step(float *__restrict__ state,
                                              const typename IO::T *__restrict__ x,
                                              const typename IO::T *__restrict__ delta,
                                              const float *__restrict__ A,
                                              const typename IO::T *__restrict__ B,
                                              const typename IO::T *__restrict__ C,
                                              const float *__restrict__ Dskip,
                                              typename IO::T *__restrict__ y, int64_t batch,
                                              int64_t dim, int N, FeArgs fe,
                                              typename IO::T *__restrict__ conv_state) {
    using T = typename IO::T;
    constexpr int LPC = NT / SPL;
    static_assert(!FE || BT == 1, "the front-end step takes one batch row per thread");
    // thread -> (group of BT batch rows, channel d, lane q of the channel); the
    // BT rows of a thread share the A row, Dskip and the channel's constants
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t units = (batch + BT - 1) / BT * dim;
    const int64_t u0 = i / LPC;
    const int q = int(i - u0 * LPC);
    const bool active = u0 < units;
    const int64_t u = active ? u0 : units - 1;
    const int64_t bg = u / dim;
    const int64_t d = u - bg * dim;
    int64_t c[BT];
    bool live[BT];
#pragma unroll
    for (int j = 0; j < BT; ++j) {
        const int64_t b = bg * BT + j;
        live[j] = active && b < batch;
        c[j] = (b < batch ? b : batch - 1) * dim + d;
    }
    // Every load goes out at the start, the state, A, B and C rows first and x and delta
    // last: a wait for x (the swaps below, the front end) then comes after every load
    // has been issued.  (A load issued after that wait, or after the readout, would put
    // a second memory round trip in each wave's lifetime.)
    float h[BT][SPL], av[SPL], bv[BT][SPL], cv[BT][SPL];
    if constexpr (kVec) {
        // N == NT (a multiple of 4), 16-byte aligned state and A, B and C rows
        // aligned to 4 elements: vector accesses
#pragma unroll
        for (int j = 0; j < BT; ++j) ldrow<SPL>(state + c[j] * N + q * SPL, h[j]);
        ldrow<SPL>(A + d * N + q * SPL, av);
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            const int64_t b = c[j] / dim;
            ldrow<SPL>(B + b * N + q * SPL, bv[j]);
            ldrow<SPL>(C + b * N + q * SPL, cv[j]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < SPL; ++k) {
            const int n = q * SPL + k;
            av[k] = n < N ? A[d * N + n] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            const int64_t b = c[j] / dim;
            const float *sp = state + c[j] * N + q * SPL;
#pragma unroll
            for (int k = 0; k < SPL; ++k) {
                const int n = q * SPL + k;
                const bool ok = n < N;
                h[j][k] = ok ? sp[k] : 0.f;
                bv[j][k] = ok ? IO::ld(B, b * N + n) : 0.f;
                cv[j][k] = ok ? IO::ld(C, b * N + n) : 0.f;
            }
        }
    }
    const float a0 = A[d * N];
    const float dsk = Dskip ? Dskip[d] : 0.f;
    // front end: the carried raw inputs of this channel, row r of conv_state being the
    // token K-1-r before this one
    // (rows past K-1 repeat the last one, so the loads take no branch, and with no carried
    // rows, where conv_state may be NULL, they read x; neither is ever used)
    T cr[kMaxConv - 1];
    if constexpr (FE) {
        const int64_t b = c[0] / dim;
        const int rows = fe.K - 1;
        const T *cs = rows > 0 ? conv_state : x;
        const int64_t rb = b * rows;
#pragma unroll
        for (int r = 0; r < kMaxConv - 1; ++r) cr[r] = cs[(rb + min(r, max(rows - 1, 0))) * dim + d];
    }
    __builtin_amdgcn_sched_barrier(0);
    // the two lanes of a channel (adjacent lanes) load x and delta of different batch
    // rows -- lane q rows q, 2+q, ... -- and swap them with a DPP move: one load
    // instruction per two rows
    constexpr bool kPairs = !FE && LPC == 2 && BT % 2 == 0;
    float xv[BT], dt[BT];
    T xraw = T(0);
    if constexpr (kPairs) {
        auto swap = [](float v) {  // the value of the other lane of the pair
            return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
        };
        T xr[BT / 2], dr[BT / 2];  // raw: converted after the barrier, so no load waits for one
#pragma unroll
        for (int j = 0; j < BT; j += 2) {
            const int64_t cq = min(bg * BT + j + q, batch - 1) * dim + d;
            xr[j / 2] = x[cq];
            dr[j / 2] = delta[cq];
        }
        // the swaps wait for these loads: every other load is already in flight
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < BT; j += 2) {
            const float xo = IO::cvt(xr[j / 2]), dto = IO::cvt(dr[j / 2]);
            const float xn = swap(xo), dtn = swap(dto);
            xv[j] = q ? xn : xo;
            xv[j + 1] = q ? xo : xn;
            dt[j] = q ? dtn : dto;
            dt[j + 1] = q ? dto : dtn;
        }
    } else {
        T xr[BT], dr[BT];
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            xr[j] = x[c[j]];
            dr[j] = delta[c[j]];
        }
        __builtin_amdgcn_sched_barrier(0);
        xraw = xr[0];  // the front end carries the raw input
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            xv[j] = IO::cvt(xr[j]);
            dt[j] = IO::cvt(dr[j]);
        }
    }
    if constexpr (FE) {
        const int64_t b = c[0] / dim;
        const int rows = fe.K - 1;
        auto back = [&](int j) {  // raw input of token t-j (selects: no indexed local array)
            const int r = rows - j;
            return r == 0 ? IO::cvt(cr[0]) : r == 1 ? IO::cvt(cr[1]) : r == 2 ? IO::cvt(cr[2]) : 0.f;
        };
        FeLane fl;
        fl.init(fe, d);
        xv[0] = fl.u(back(3), back(2), back(1), xv[0]);
        dt[0] = fl.delta(dt[0]);
        if (active && q == 0) {
#pragma unroll
            for (int r = 0; r < kMaxConv - 1; ++r)
                if (r < rows) conv_state[(b * rows + r) * dim + d] = r + 1 < rows ? cr[r + 1] : xraw;
        }
    }

    StepLane<SPL, LPC> sl;
    sl.init(q, N, a0, av);
    float yrow[BT];
#pragma unroll
    for (int j = 0; j < BT; ++j) {
        float yacc = sl.row(dt[j], xv[j], av, bv[j], cv[j], h[j]);
#pragma unroll
        for (int off = LPC / 2; off >= 1; off /= 2) yacc += __shfl_xor(yacc, off, LPC);
        yrow[j] = fmaf(dsk, xv[j], yacc);
        if (!live[j]) continue;
        float *sp = state + c[j] * N + q * SPL;
        if constexpr (kVec) {
#pragma unroll
            for (int k = 0; k < SPL; k += 4)
                *reinterpret_cast<float4 *>(sp + k) = make_float4(h[j][k], h[j][k + 1], h[j][k + 2], h[j][k + 3]);
        } else {
#pragma unroll
            for (int k = 0; k < SPL; ++k)
                if (q * SPL + k < N) sp[k] = h[j][k];
        }
        if (!kPairs && q == 0) y[c[j]] = IO::enc(yrow[j]);
    }
    if constexpr (kPairs) {
        // both lanes of a channel hold every row's output: lane q stores rows q, 2+q, ...
#pragma unroll
        for (int j = 0; j < BT; j += 2) {
            const int64_t b = bg * BT + j + q;
            const float ya = yrow[j], yb = yrow[j + 1];
            if (active && b < batch) y[b * dim + d] = IO::enc(q ? yb : ya);
        }
    }
}


// states per lane of the decode step (N above it: several lanes per channel)
#ifndef SSCAN_STEP_SPL
#define SSCAN_STEP_SPL 8
#endif
constexpr int kStepSpl = SSCAN_STEP_SPL;
// batch rows per thread of the decode step without the front end (they share the
// channel's A row and Dskip, and a wave keeps that many rows of state in flight)
#ifndef SSCAN_STEP_BT
#define SSCAN_STEP_BT 4
#endif
constexpr int kStepBt = SSCAN_STEP_BT;

int round_nt(int64_t N) { return N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

template <class IO, int NT>
void prep_t(const void *B, const void *C, const float *A, float *bc, int *flags, int64_t rows,
            int64_t dim, int N, hipStream_t s) {
    using T = typename IO::T;
    const int64_t tiles_per_batch = (dim + kWave - 1) / kWave;
    const int64_t prep_blocks = std::min<int64_t>((rows * NT + 255) / 256, kMaxStrideBlocks);
    const int64_t cls_blocks = (tiles_per_batch + 3) / 4;
    hipLaunchKernelGGL((k_prep<IO, NT>), dim3(unsigned(prep_blocks + cls_blocks)), dim3(256), 0, s,
                       static_cast<const T *>(B), static_cast<const T *>(C), bc, rows, N, A, dim,
                       flags, tiles_per_batch, prep_blocks);
}

template <class IO>
void prep_io(const void *B, const void *C, const float *A, float *bc, int *flags, int64_t rows,
             int64_t dim, int N, int nt, hipStream_t s) {
    switch (nt) {
        case 1: return prep_t<IO, 1>(B, C, A, bc, flags, rows, dim, N, s);
        case 2: return prep_t<IO, 2>(B, C, A, bc, flags, rows, dim, N, s);
        case 4: return prep_t<IO, 4>(B, C, A, bc, flags, rows, dim, N, s);
        case 8: return prep_t<IO, 8>(B, C, A, bc, flags, rows, dim, N, s);
        default: return prep_t<IO, 16>(B, C, A, bc, flags, rows, dim, N, s);
    }
}

template <class IO, int NT, bool FE>
hipError_t forward_t(const FwdArgs &a, const FwdPlan &p, void *ws, hipStream_t s) {
    using T = typename IO::T;
    char *base = static_cast<char *>(ws);
    float *bc = reinterpret_cast<float *>(base + p.off_bc);
    int *flags = reinterpret_cast<int *>(base + p.off_flags);
    float *agg_sum = reinterpret_cast<float *>(base + p.off_sum);
    float *agg_h = reinterpret_cast<float *>(base + p.off_h);
    const T *x = static_cast<const T *>(a.x), *dl = static_cast<const T *>(a.delta);
    T *y = static_cast<T *>(a.y);
    prep_t<IO, NT>(a.B, a.C, a.A, bc, flags, a.batch * a.L, a.dim, a.N, s);
    if (p.lockstep) {
        // every tile in one launch (the general-A tiles take their own path in it);
        // the fused variant too: with the token loop free of register copies it fits
        // 128 VGPRs (4 waves per SIMD) without spilling
        hipLaunchKernelGGL((k_lockstep<IO, NT, kLockW, kLockT, FE>), dim3(unsigned(p.tiles)), dim3(kLockW * kWave),
                           0, s, x, dl, a.A, bc, a.Dskip, a.h0, y, a.final_state, flags, int(a.L), a.dim, a.N,
                           p.tiles_per_batch, a.fe);
    } else {
        // every segment from its own start, then the segments after the first
        // corrected for the state they really started from
#define SSCAN_SEG(FAST)                                                                                   \
    hipLaunchKernelGGL((k_seg<IO, NT, FAST, FE>), dim3(unsigned(p.segments * p.tiles)), dim3(kWave), 0, s, x, dl,  \
                       a.A, bc, a.Dskip, a.h0, y, a.final_state, agg_sum, agg_h, flags, a.batch, a.L, a.dim,     \
                       a.N, p.seg_len, p.segments, p.tiles_per_batch, p.tiles, a.fe)
#define SSCAN_SEGFIX(FAST)                                                                                \
    hipLaunchKernelGGL((k_segfix<IO, NT, FAST, FE>), dim3(unsigned((p.segments - 1) * p.tiles)), dim3(kWave),   \
                       0, s, dl, a.A, bc, y, agg_h, flags, a.batch, a.L, a.dim, a.N, p.seg_len,               \
                       p.tiles_per_batch, p.tiles, a.fe)
        SSCAN_SEG(true);
        SSCAN_SEG(false);
        if (p.segments > 1) {
            const int64_t blocks = std::min<int64_t>(a.batch * NT * p.tiles_per_batch, kMaxStrideBlocks / 16);
            hipLaunchKernelGGL(k_carry, dim3(unsigned(blocks)), dim3(kCarryG * kWave), 0, s, a.A, agg_sum, agg_h,
                               a.final_state, a.batch, a.dim, a.N, NT, p.segments);
            SSCAN_SEGFIX(true);
            SSCAN_SEGFIX(false);
        }
#undef SSCAN_SEG
#undef SSCAN_SEGFIX
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && FE && a.conv_state_out)
        e = launch_conv_tail(a.x, a.fe, a.conv_state_out, a.batch, a.L, a.dim, a.io, s);
    return e;
}

template <class IO>
hipError_t forward_io(const FwdArgs &a, const FwdPlan &p, void *ws, hipStream_t s) {
    const bool fe = a.fe.K > 0;
    switch (p.nt) {
        case 1: return fe ? forward_t<IO, 1, true>(a, p, ws, s) : forward_t<IO, 1, false>(a, p, ws, s);
        case 2: return fe ? forward_t<IO, 2, true>(a, p, ws, s) : forward_t<IO, 2, false>(a, p, ws, s);
        case 4: return fe ? forward_t<IO, 4, true>(a, p, ws, s) : forward_t<IO, 4, false>(a, p, ws, s);
        case 8: return fe ? forward_t<IO, 8, true>(a, p, ws, s) : forward_t<IO, 8, false>(a, p, ws, s);
        default: return fe ? forward_t<IO, 16, true>(a, p, ws, s) : forward_t<IO, 16, false>(a, p, ws, s);
    }
}

template <class IO, int NT, bool FE>
hipError_t step_t(const StepArgs &a, hipStream_t s) {
    using T = typename IO::T;
    constexpr int SPL = NT < kStepSpl ? NT : kStepSpl;
    constexpr int LPC = NT / SPL;
    constexpr int BT = FE ? 1 : kStepBt;
    const int64_t threads = (a.batch + BT - 1) / BT * a.dim * LPC;
    const dim3 grid(unsigned((threads + 255) / 256));
    const uintptr_t rb = (sizeof(T) == 2 && SPL % 8 == 0 ? 8 : 4) * sizeof(T);  // one B or C load
    const bool vec = (SPL % 4 == 0) && (a.N == NT) && (reinterpret_cast<uintptr_t>(a.state) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.A) % 16 == 0) && (reinterpret_cast<uintptr_t>(a.B) % rb == 0) &&
                     (reinterpret_cast<uintptr_t>(a.C) % rb == 0);
    if (vec) {
        if constexpr (SPL % 4 == 0)
            hipLaunchKernelGGL((k_step<IO, NT, SPL, true, FE, BT>), grid, dim3(256), 0, s, a.state,
                               static_cast<const T *>(a.x), static_cast<const T *>(a.delta), a.A,
                               static_cast<const T *>(a.B), static_cast<const T *>(a.C), a.Dskip,
                               static_cast<T *>(a.y), a.batch, a.dim, a.N, a.fe,
                               static_cast<T *>(a.conv_state));
    } else {
        hipLaunchKernelGGL((k_step<IO, NT, SPL, false, FE, BT>), grid, dim3(256), 0, s, a.state,
                           static_cast<const T *>(a.x), static_cast<const T *>(a.delta), a.A,
                           static_cast<const T *>(a.B), static_cast<const T *>(a.C), a.Dskip,
                           static_cast<T *>(a.y), a.batch, a.dim, a.N, a.fe,
                           static_cast<T *>(a.conv_state));
    }
    return hipGetLastError();
}

template <class IO>
hipError_t step_io(const StepArgs &a, hipStream_t s) {
    const bool fe = a.fe.K > 0;
    switch (round_nt(a.N)) {
        case 1: return fe ? step_t<IO, 1, true>(a, s) : step_t<IO, 1, false>(a, s);
        case 2: return fe ? step_t<IO, 2, true>(a, s) : step_t<IO, 2, false>(a, s);
        case 4: return fe ? step_t<IO, 4, true>(a, s) : step_t<IO, 4, false>(a, s);
        case 8: return fe ? step_t<IO, 8, true>(a, s) : step_t<IO, 8, false>(a, s);
        default: return fe ? step_t<IO, 16, true>(a, s) : step_t<IO, 16, false>(a, s);
    }
}

}  // namespace

FwdPlan plan_forward(int64_t batch, int64_t L, int64_t dim, int64_t N, int io, size_t max_ws) {
    FwdPlan p{};
    p.nt = round_nt(N);
    p.tiles_per_batch = (dim + kWave - 1) / kWave;
    p.tiles = batch * p.tiles_per_batch;
    const int64_t rowb = dim * (io == 1 ? 2 : 4);  // bytes of one token row of x, delta or y
    // Segment kernels walk a segment's token rows through one buffer descriptor
    // with 32-bit offsets, prefetching up to 2*kUnroll rows past its end: the
    // segment must fit a descriptor (kMaxDescBytes) and those extra rows must fit
    // below 2^31 as well, so no offset reaches 2^32.
    if (rowb * (2 * kUnroll) > kMaxDescBytes) {
        p.reject = "dim too large: one token row of x exceeds 2^27 bytes";
        return p;
    }
    const int64_t seg_max = rowb > 0 ? kMaxDescBytes / rowb : L;  // tokens per segment, at most
    // Enough segments for ~32 waves per SIMD (1024 SIMDs), several rounds of
    // waves, so that waves of uneven speed even out before the launch ends (a
    // segment costs one aggregate in the carry pass), with segments of >= 64
    // tokens, and at least as many as the descriptor span needs.
    const int64_t target_waves = kTargetWaves;
    int64_t S = p.tiles > 0 ? (target_waves + p.tiles - 1) / p.tiles : 1;
    S = std::min<int64_t>(S, std::max<int64_t>(1, L / 64));
    S = std::max<int64_t>(1, std::min<int64_t>(S, 4096));
    // Test hook: SSCAN_FORCE_SEGMENTS=n (n > 0) sends every shape down the segment path
    // with n segments (at most one per token, and at least as many as the descriptor
    // bound below needs), so that one shape can be scanned through differently cut
    // decompositions and the results compared with each other.
    int64_t force = 0;
    if (const char *e = std::getenv("SSCAN_FORCE_SEGMENTS")) force = std::max<long long>(0, std::atoll(e));
    if (force > 0) S = std::min<int64_t>(force, std::max<int64_t>(1, L));
    const int64_t s_min = seg_max > 0 ? (L + seg_max - 1) / seg_max : 1;  // the descriptor bound
    S = std::max<int64_t>(S, s_min);
    // Lockstep kernel when the tiles alone give at least one wave per SIMD.
    // Its buffer offsets reach (W*TS + kUnroll) rows past a run start (keep them
    // below 2^31), its token arithmetic is 32-bit (L < 2^31), and its launch is
    // tiles x W*64 work items.
    const bool lockstep = force == 0 && p.tiles >= kLockMinTiles &&
                          (int64_t(kLockW) * kLockT + kUnroll) * rowb <= kMaxDescBytes && L < (int64_t(1) << 31) &&
                          p.tiles <= kMaxWorkItems / (kLockW * kWave);
    // A fixed scratch budget (the no-allocation entry point): on the segment path,
    // fewer segments when their aggregates would not fit beside the staged B/C rows,
    // never fewer than the descriptor bound needs (a shape that still does not fit is
    // refused by the caller).
    if (max_ws > 0 && !lockstep) {
        const size_t fixed = align256(size_t(batch) * L * 2 * p.nt * sizeof(float)) +
                             align256(size_t(p.tiles_per_batch) * sizeof(int)) + 512;  // + the aggregates' alignment
        const size_t per_seg = size_t(batch) * dim * (1 + p.nt) * sizeof(float);
        if (fixed < max_ws && per_seg > 0) {
            const int64_t fit = int64_t(std::min<size_t>((max_ws - fixed) / per_seg, size_t(1) << 40));
            S = std::max<int64_t>(s_min, std::min<int64_t>(S, std::max<int64_t>(fit, 1)));
        }
    }
    p.seg_len = L > 0 ? (L + S - 1) / S : 1;
    p.segments = L > 0 ? int(std::min<int64_t>((L + p.seg_len - 1) / p.seg_len, 0x7FFFFFFF)) : 1;
    if (p.seg_len > seg_max || p.tiles > kMaxWorkItems / (int64_t(p.segments) * kWave)) {
        p.reject = "shape too large for the segment kernels' launch";
        return p;
    }
    p.lockstep = lockstep;
    size_t off = 0;
    p.off_bc = off;
    off += align256(size_t(batch) * L * 2 * p.nt * sizeof(float));
    p.off_flags = off;
    off += align256(size_t(p.tiles_per_batch) * sizeof(int));
    // segment aggregates: the segment path only (the lockstep kernel takes every tile)
    const size_t nagg = p.lockstep ? 0 : size_t(p.segments) * batch * dim;
    p.off_sum = off;
    off += align256(nagg * sizeof(float));
    p.off_h = off;
    off += align256(nagg * p.nt * sizeof(float));
    p.ws_bytes = off;
    return p;
}

hipError_t launch_forward(const FwdArgs &a, const FwdPlan &p, void *ws, hipStream_t s) {
    return a.io == 1 ? forward_io<IoBF16>(a, p, ws, s) : forward_io<IoF32>(a, p, ws, s);
}

hipError_t launch_prep(const void *B, const void *C, const float *A, float *bc, int *tile_fast,
                       int64_t rows, int64_t dim, int N, int nt, int io, hipStream_t s) {
    if (io == 1)
        prep_io<IoBF16>(B, C, A, bc, tile_fast, rows, dim, N, nt, s);
    else
        prep_io<IoF32>(B, C, A, bc, tile_fast, rows, dim, N, nt, s);
    return hipGetLastError();
}

hipError_t launch_conv_tail(const void *x, const FeArgs &fe, void *conv_state_out, int64_t batch,
                            int64_t seqlen, int64_t dim, int io, hipStream_t s) {
    const int64_t n = batch * (fe.K - 1) * dim;
    if (n <= 0) return hipSuccess;
    const dim3 grid(unsigned(std::min<int64_t>((n + 255) / 256, kMaxStrideBlocks)));
    if (io == 1)
        hipLaunchKernelGGL((k_conv_tail<IoBF16>), grid, dim3(256), 0, s, static_cast<const uint16_t *>(x), fe,
                           static_cast<uint16_t *>(conv_state_out), batch, seqlen, dim);
    else
        hipLaunchKernelGGL((k_conv_tail<IoF32>), grid, dim3(256), 0, s, static_cast<const float *>(x), fe,
                           static_cast<float *>(conv_state_out), batch, seqlen, dim);
    return hipGetLastError();
}

hipError_t launch_copy_or_zero(float *dst, const float *src, int64_t count, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_copy_or_zero, dim3(unsigned(std::min<int64_t>((count + 255) / 256, kMaxStrideBlocks))),
                       dim3(256), 0, s, dst, src, count);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    return a.io == 1 ? step_io<IoBF16>(a, s) : step_io<IoF32>(a, s);
}

int64_t step_work_items(int64_t batch, int64_t dim, int64_t N, bool front_end) {
    const int nt = round_nt(N);
    const int64_t lpc = nt < kStepSpl ? 1 : nt / kStepSpl;
    const int64_t bt = front_end ? 1 : kStepBt;
    return ((batch + bt - 1) / bt * dim * lpc + 255) / 256 * 256;
}

}  // namespace sscan
