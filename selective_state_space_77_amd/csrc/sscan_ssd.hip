// gfx950 kernel of the scalar-A-per-head selective scan (Mamba-2's SSM) in its
// chunked matrix form, with the dense block products on MFMA.
//
// Per head h (scalar A_h), channel p < P, state n < N, with B, C shared by the
// heads of a group:  h_t = exp(delta_t A) h_{t-1} + gain_t B_t x_t,
// y_t = C_t . h_t + D x_t, gain = (exp(delta A) - 1)/A (delta at A = 0) -- the
// same zero-order hold as the per-channel scan ("The loop that beats
// attention", eqs. (1)-(2)).  With A a scalar per head the map x -> y is a
// lower-triangular structured matrix ("Mamba and State Space Models";
// "Mamba matches the Transformer...", the state space duality):
//     y_t = sum_{s<=t} (C_t . B_s) exp(A (cum_t - cum_s)) gain_s x_s + D x_t,
// cum the running sum of delta.  Cut into chunks of Q tokens this is
//     Y = (L o C B^T) X + diag(e) C S_in + D X       (inside the chunk / from before it)
//     S_out = exp(A sum delta) S_in + B^T diag(w) X   (state carried to the next chunk)
// with L[t,s] = exp(A (cum_t - cum_s)) gain_s (s <= t), e_t = exp(A cum_t),
// w_s = exp(A (cum_Q - cum_s)) gain_s: three dense products per chunk.
//
// Mapping.  One workgroup of 4 waves per (batch row, head) walks the chunks in
// order; the P x N state stays on chip (MFMA accumulators, plus a copy in LDS
// that feeds the next chunk's C S_in).  Wave w computes the outputs of tokens
// 16w..16w+15 of each chunk and updates state channels 16w..16w+15.  Products
// are 16x16 tiles accumulated over K in slabs of 16: v_mfma_f32_16x16x16_bf16
// for bf16 inputs (computed operands split into two bf16 parts), four
// v_mfma_f32_16x16x4_f32 for fp32 inputs.  G^T = B C^T is
// computed rather than C B^T because its accumulator layout (lane = column t,
// 4 consecutive rows s) is exactly the A-operand layout (lane = row t, 4
// consecutive k = s) of the next product, so the masked scores feed it
// without a shuffle.  x and B of a chunk are staged transposed in LDS, where
// the operands that need "4 consecutive tokens of one channel" read them.

#include <type_traits>

#include "sscan_device.h"

namespace sscan {
namespace {

using namespace dev;

constexpr int SQ = 64;          // tokens per chunk
constexpr int SP = 64;          // channels per head
constexpr int SWV = 4;          // waves per workgroup
constexpr int SPITCH = SQ + 4;  // LDS row pitch of the transposed staging (bank spread)

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// acc += A * B for one 16x16 tile and a K slab of 16.  Lane l (r = l % 16,
// q = l / 16) holds a[j] = A[r][4q + j] and b[j] = B[4q + j][r]; acc[j] is
// D[4q + j][r].
//
// bf16 inputs: an operand that is an input (x, B, C: already bf16 values) goes
// to the matrix core as it is; an operand computed in fp32 (scores, weighted
// x, the state; kSplitA / kSplitB) is split into a bf16 high part and the bf16
// rounding of its remainder, and both parts are multiplied: about 2^-17
// relative error per product instead of 2^-9, for a second matrix instruction.
__device__ __forceinline__ void split_bf16(const float (&v)[4], v4s &hi, v4s &lo) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint16_t hb = f32_to_bf16(v[j]);
        hi[j] = short(hb);
        lo[j] = short(f32_to_bf16(v[j] - __uint_as_float(uint32_t(hb) << 16)));
    }
}

template <bool kBF16, bool kSplitA = false, bool kSplitB = false>
__device__ __forceinline__ v4f mma16(v4f acc, const float (&a)[4], const float (&b)[4]) {
    static_assert(!(kSplitA && kSplitB), "at most one computed operand");
    if constexpr (kBF16) {
        v4s ah, al, bh, bl;
        if constexpr (kSplitA) {
            split_bf16(a, ah, al);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) ah[j] = short(f32_to_bf16(a[j]));
        }
        if constexpr (kSplitB) {
            split_bf16(b, bh, bl);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) bh[j] = short(f32_to_bf16(b[j]));
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
        if constexpr (kSplitA) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
        if constexpr (kSplitB) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
        return acc;
    } else {
        // four K=4 products; product j takes k = 4q + j in lane group q (any
        // order of the K sum gives the same result)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
        return acc;
    }
}

template <class IO, int NS>
__global__ __launch_bounds__(SWV *kWave) void k_ssd(
    const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ delta,
    const float *__restrict__ A, const typename IO::T *__restrict__ Bm,
    const typename IO::T *__restrict__ Cm, const float *__restrict__ Dskip,
    const float *__restrict__ h0, typename IO::T *__restrict__ y, float *__restrict__ hT,
    int64_t L, int64_t H, int64_t G) {
    constexpr int NB = NS / 16;
    constexpr bool kBF = std::is_same<IO, IoBF16>::value;
    __shared__ float sX[SP][SPITCH];    // x of the chunk, [channel][token]
    __shared__ float sBt[NS][SPITCH];   // B of the chunk, [state][token]
    __shared__ float sS[SP][NS + 4];    // state entering the chunk, [channel][state]
    __shared__ float sCum[SQ], sGain[SQ], sW[SQ], sE[SQ];
    __shared__ float sDec;

    const int tid = int(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave, r = lane % 16, q = lane / 16;
    const int64_t b = int64_t(blockIdx.x) / H;
    const int64_t h = int64_t(blockIdx.x) - b * H;
    const int64_t g = h / (H / G);
    const float a = A[h];
    const float a2 = a * kLog2e;
    const float dsk = Dskip ? Dskip[h] : 0.f;
    auto xidx = [&](int64_t t, int p) { return ((b * L + t) * H + h) * SP + p; };
    auto bcidx = [&](int64_t t, int n) { return ((b * L + t) * G + g) * NS + n; };

    // state: wave w owns channels 16w..16w+15; S[nb][j] = S[n = 16nb + 4q + j][p = 16w + r]
    v4f S[NB];
    const int64_t srow = ((b * H + h) * SP + 16 * w + r) * NS;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[nb][j] = h0 ? h0[srow + 16 * nb + 4 * q + j] : 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) sS[16 * w + r][16 * nb + 4 * q + j] = S[nb][j];

    const int64_t nchunks = (L + SQ - 1) / SQ;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * SQ;
        // ---- per-token scalars of the chunk (wave 0): running sum of delta
        // (inclusive), gain, state weight w_s, output decay e_t, chunk decay.
        // Tokens past the end have delta = 0: gain 0, decay 1 -- no effect.
        if (w == 0) {
            const int64_t t = t0 + lane;
            const float dv = t < L ? IO::ld(delta, (b * L + t) * H + h) : 0.f;
            float cum = dv;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float v = __shfl_up(cum, off);
                if (lane >= off) cum += v;
            }
            const float total = __shfl(cum, kWave - 1);
            const float z = dv * a;
            const float abar = exp2_hw(dv * a2);
            const float gain = zoh_gain(dv, a, z, abar);  // delta when A = 0
            sCum[lane] = cum;
            sGain[lane] = gain;
            sW[lane] = exp2_hw(a2 * (total - cum)) * gain;
            sE[lane] = exp2_hw(a2 * cum);
            if (lane == 0) sDec = exp2_hw(a2 * total);
        }
        // ---- stage x and B of the chunk transposed (tokens past the end: 0)
        {
            const int s = tid / 4;
            const int64_t t = t0 + s;
            const int p0 = 16 * (tid % 4);
#pragma unroll
            for (int k = 0; k < 16; ++k) sX[p0 + k][s] = t < L ? IO::ld(x, xidx(t, p0 + k)) : 0.f;
            constexpr int NPT = NS / 4;
            const int n0 = NPT * (tid % 4);
#pragma unroll
            for (int k = 0; k < NPT; ++k) sBt[n0 + k][s] = t < L ? IO::ld(Bm, bcidx(t, n0 + k)) : 0.f;
        }
        __syncthreads();

        // ---- C fragments of this wave's tokens: cf[nb][j] = C[t = 16w + r][n = 16nb + 4q + j]
        const int tl = 16 * w + r;
        const int64_t tt = t0 + tl;
        float cf[NB][4];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) cf[nb][j] = tt < L ? IO::ld(Cm, bcidx(tt, 16 * nb + 4 * q + j)) : 0.f;

        // ---- masked scores: G^T tile (s-block sb, t-block w) = B[sb] C[w]^T, scaled
        // by exp(A (cum_t - cum_s)) gain_s where s <= t, zero above the diagonal.
        // gm[sb][j] = score(t = 16w + r, s = 16sb + 4q + j): the A operand of (scores) X.
        const float cum_t = sCum[tl];
        float gm[SQ / 16][4];
#pragma unroll
        for (int sb = 0; sb < SQ / 16; ++sb) {
            if (sb > w) break;  // uniform: blocks above the diagonal are zero
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float bf[4];  // A operand: B[s = 16sb + r][n = 16nb + 4q + j]
#pragma unroll
                for (int j = 0; j < 4; ++j) bf[j] = sBt[16 * nb + 4 * q + j][16 * sb + r];
                acc = mma16<kBF>(acc, bf, cf[nb]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sl = 16 * sb + 4 * q + j;
                const float v = acc[j] * exp2_hw(a2 * (cum_t - sCum[sl])) * sGain[sl];
                gm[sb][j] = sl <= tl ? v : 0.f;
            }
        }

        // ---- outputs of tokens 16w..16w+15: Y = scores X + diag(e) (C S_in) + D x;
        // the decay e_t is applied to C S_in in fp32, after the product
        float et[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) et[j] = sE[16 * w + 4 * q + j];
#pragma unroll
        for (int pb = 0; pb < SP / 16; ++pb) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < SQ / 16; ++sb) {
                if (sb > w) break;
                float xf[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) xf[j] = sX[16 * pb + r][16 * sb + 4 * q + j];
                acc = mma16<kBF, true, false>(acc, gm[sb], xf);
            }
            v4f off = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float sf[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) sf[j] = sS[16 * pb + r][16 * nb + 4 * q + j];
                off = mma16<kBF, false, true>(off, cf[nb], sf);
            }
            // acc[j], off[j] = (scores X), (C S_in) at [t = 16w + 4q + j][p = 16pb + r]
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tj = 16 * w + 4 * q + j;
                const int64_t t = t0 + tj;
                const float v = fmaf(et[j], off[j], fmaf(dsk, sX[16 * pb + r][tj], acc[j]));
                if (t < L) y[xidx(t, 16 * pb + r)] = IO::enc(v);
            }
        }
        __syncthreads();  // every wave has read the entering state

        // ---- state update of channels 16w..16w+15: S = exp(A sum delta) S + B^T diag(w) X
        const float dec = sDec;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) S[nb] *= dec;
#pragma unroll
        for (int sb = 0; sb < SQ / 16; ++sb) {
            float xw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sl = 16 * sb + 4 * q + j;
                xw[j] = sX[16 * w + r][sl] * sW[sl];
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float bt[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) bt[j] = sBt[16 * nb + r][16 * sb + 4 * q + j];
                S[nb] = mma16<kBF, false, true>(S[nb], bt, xw);
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) sS[16 * w + r][16 * nb + 4 * q + j] = S[nb][j];
        __syncthreads();  // the next chunk restages x, B and reads the new state
    }
    if (hT) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) hT[srow + 16 * nb + 4 * q + j] = S[nb][j];
    }
}

// ---------------------------------------------------------------------------
// bf16 kernel.  8 waves per (batch row, head); each chunk of x, B, C and delta
// is fetched with 16-byte loads one chunk ahead (into registers, while the
// current chunk computes) and staged in LDS as bf16, in the layouts the
// matrix operands read with single 8- or 16-byte LDS reads: x and B transposed
// ([channel][token], [state][token]), B and C row-major ([token][state]), the
// entering state as a bf16 high part and remainder ([channel][state]).
// A chunk is three phases between barriers: staging (with the state
// carried in from the previous chunk); the 10 causal 16x16 score tiles, spread
// over the 8 waves and shared through LDS, beside the state update (wave v
// owns channel block v % 4 and half of the state blocks: equal work); the
// outputs, wave v taking channel block v % 4 of token blocks {0, 3} or {1, 2}
// (equal causal work).  The scores, C S_in and the update use the K = 32
// matrix instruction (v_mfma_f32_16x16x32_bf16); (scores) X, whose K is a
// 16-token block of the causal triangle, the K = 16 one.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int BWV = 8;            // waves per workgroup
constexpr int BTH = BWV * kWave;  // threads per workgroup
constexpr int XPB = SQ + 8;       // pitch (bf16) of the [channel][token] and [state][token] tiles

__device__ __forceinline__ float bfv(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }

__device__ __forceinline__ v4f mfma16(v4f acc, v4s a, v4s b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
// K slab of 32: lane l holds a[j] = A[r][8q + j], b[j] = B[8q + j][r], j < 8
__device__ __forceinline__ v4f mfma32(v4f acc, v8bf a, v8bf b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void split8(const float (&v)[8], v8bf &hi, v8bf &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 hb = static_cast<__bf16>(v[j]);
        hi[j] = hb;
        lo[j] = static_cast<__bf16>(v[j] - static_cast<float>(hb));
    }
}

template <int NS>
__global__ __launch_bounds__(BTH) void k_ssd_bf(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ delta, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dskip,
    const float *__restrict__ h0, uint16_t *__restrict__ y, float *__restrict__ hT, int64_t L,
    int64_t H, int64_t G) {
    constexpr int NB = NS / 16;        // 16-wide state blocks
    constexpr int NK = NS / 32;        // 32-wide K steps over the states
    constexpr int RP = NS + 8;         // pitch (bf16) of the [token][state] and [channel][state] tiles
    constexpr int NBW = NB / 2;        // state tiles per wave in the update
    constexpr int BE = NS * SQ / BTH;  // bf16 elements of B (and of C) staged per thread
    constexpr int NG = 10;             // causal 16x16 score tiles of a 64-token chunk
    static_assert(BE % 8 == 0 && SP * SQ / BTH == 8, "staging split");
    __shared__ __align__(16) uint16_t sXt[SP][XPB];
    __shared__ __align__(16) uint16_t sBt[NS][XPB];
    __shared__ __align__(16) uint16_t sB[SQ][RP];
    __shared__ __align__(16) uint16_t sC[SQ][RP];
    __shared__ __align__(16) uint16_t sSh[SP][RP];
    __shared__ __align__(16) uint16_t sSl[SP][RP];
    __shared__ __align__(16) uint16_t sGh[NG][16][16];  // masked scores, A-operand layout [tile][t][s]
    __shared__ __align__(16) uint16_t sGl[NG][16][16];
    __shared__ __align__(16) uint16_t sY[BWV][2][16][16];  // each wave's two output tiles
    __shared__ float sCum[SQ], sGain[SQ], sW[SQ], sE[SQ];
    __shared__ float sDec;

    const int tid = int(threadIdx.x);
    const int v = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave, r = lane % 16, q = lane / 16;
    const int64_t b = int64_t(blockIdx.x) / H;
    const int64_t h = int64_t(blockIdx.x) - b * H;
    const int64_t g = h / (H / G);
    const float a = A[h];
    const float a2 = a * kLog2e;
    const float dsk = Dskip ? Dskip[h] : 0.f;
    // row t of this (batch row, head): x and y at xb/yb + t*rx, B/C at Bb/Cb + t*rbc,
    // delta at db + t*H (elements).  Each chunk reads and writes through buffer
    // descriptors over [t0, L): 32-bit offsets, and tokens past the end read 0
    // and drop their stores in the hardware range check.
    const int64_t rx = H * SP, rbc = G * NS;
    const uint16_t *xb = x + (b * L * H + h) * SP;
    uint16_t *yb = y + (b * L * H + h) * SP;
    const uint16_t *Bb = Bm + (b * L * G + g) * NS;
    const uint16_t *Cb = Cm + (b * L * G + g) * NS;
    const uint16_t *db = delta + b * L * H + h;

    // ---- chunk fetch (registers) and staging (LDS).  Thread roles: token
    // st = lane, x channels 8v..8v+7, B and C states BE*v..BE*v+BE-1 (v = wave):
    // the transposed LDS writes of a wave then fill consecutive tokens of one
    // row (no bank conflicts); the 16-byte global reads of a wave hit 64 rows,
    // whose other bytes the other waves read from the same cache lines.
    const int st = lane, c8 = v;
    const uint32_t ox = uint32_t(st * rx * 2 + 16 * c8);  // byte offsets of this thread
    const uint32_t obc = uint32_t(st * rbc * 2 + 2 * BE * c8);
    const uint32_t od = uint32_t(lane * H * 2);
    v4u px, pb[BE / 8], pc[BE / 8];
    uint16_t pd = 0;
    auto fetch = [&](int64_t t0) {
        const rsrc_t rxs = make_rsrc(xb + t0 * rx, (L - t0) * rx * 2);
        const rsrc_t rbs = make_rsrc(Bb + t0 * rbc, (L - t0) * rbc * 2);
        const rsrc_t rcs = make_rsrc(Cb + t0 * rbc, (L - t0) * rbc * 2);
        px = __builtin_amdgcn_raw_buffer_load_b128(rxs, ox, 0, 0);
#pragma unroll
        for (int i = 0; i < BE / 8; ++i) {
            pb[i] = __builtin_amdgcn_raw_buffer_load_b128(rbs, obc + 16 * i, 0, 0);
            pc[i] = __builtin_amdgcn_raw_buffer_load_b128(rcs, obc + 16 * i, 0, 0);
        }
        if (v == 0) pd = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(db + t0 * H, (L - t0) * H * 2), od, 0, 0);
    };
    auto stage = [&]() {
        const uint16_t *xv = reinterpret_cast<const uint16_t *>(&px);
#pragma unroll
        for (int k = 0; k < 8; ++k) sXt[8 * c8 + k][st] = xv[k];
#pragma unroll
        for (int i = 0; i < BE / 8; ++i) {
            *reinterpret_cast<v4u *>(&sB[st][BE * c8 + 8 * i]) = pb[i];
            *reinterpret_cast<v4u *>(&sC[st][BE * c8 + 8 * i]) = pc[i];
            const uint16_t *bv = reinterpret_cast<const uint16_t *>(&pb[i]);
#pragma unroll
            for (int k = 0; k < 8; ++k) sBt[BE * c8 + 8 * i + k][st] = bv[k];
        }
        // per-token scalars (wave 0, lane = token): running sum of delta
        // (inclusive), gain, state weight, output decay; chunk decay.  Tokens
        // past the end have delta = 0: gain 0, decay 1.
        if (v == 0) {
            const float dv = bfv(pd);
            float cum = dv;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float u = __shfl_up(cum, off);
                if (lane >= off) cum += u;
            }
            const float total = __shfl(cum, kWave - 1);
            const float gain = zoh_gain(dv, a, dv * a, exp2_hw(dv * a2));  // delta when A = 0
            sCum[lane] = cum;
            sGain[lane] = gain;
            sW[lane] = exp2_hw(a2 * (total - cum)) * gain;
            sE[lane] = exp2_hw(a2 * cum);
            if (lane == 0) sDec = exp2_hw(a2 * total);
        }
    };

    // ---- state tiles of this wave: channel block pbs, state blocks nb0..nb0+NBW-1;
    // S[i][j] = S[n = 16(nb0 + i) + 4q + j][p = 16 pbs + r]
    const int pbs = v % 4, nb0 = NBW * (v / 4);
    v4f S[NBW];
    const int64_t srow = ((b * H + h) * SP + 16 * pbs + r) * NS;
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[i][j] = h0 ? h0[srow + 16 * (nb0 + i) + 4 * q + j] : 0.f;
    auto publish_state = [&]() {
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            v4s hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint16_t hb = f32_to_bf16(S[i][j]);
                hi[j] = short(hb);
                lo[j] = short(f32_to_bf16(S[i][j] - bfv(hb)));
            }
            *reinterpret_cast<v4s *>(&sSh[16 * pbs + r][16 * (nb0 + i) + 4 * q]) = hi;
            *reinterpret_cast<v4s *>(&sSl[16 * pbs + r][16 * (nb0 + i) + 4 * q]) = lo;
        }
    };

    // causal score tile k (0..9) = (token block tb, source block sb <= tb), row-major
    // over the triangle; tile_of(tb, sb) = tb (tb + 1) / 2 + sb
    // outputs of this wave: channel block pbo, token blocks tbo[0] + tbo[1] = 3 (equal work)
    const int pbo = v % 4;
    const int tbo0 = v < 4 ? 0 : 1, tbo1 = 3 - tbo0;

    fetch(0);
    const int64_t nchunks = (L + SQ - 1) / SQ;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * SQ;
        publish_state();  // the state entering this chunk
        stage();
        __syncthreads();
        if (c + 1 < nchunks) fetch(t0 + SQ);  // next chunk, in flight during this one

        // ---- phase 2a: causal score tiles, spread over the waves (k = v, v + 8):
        // G^T tile (s-block sb, t-block tb) = B C^T, times exp(A (cum_t - cum_s)) gain_s
        // where s <= t, split into bf16 parts and stored in the A-operand layout
        // of (scores) X: lane (t = r, k = s = 4q + j)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int k = v + 8 * kk;
            if (k >= NG) break;
            const int tb = k >= 6 ? 3 : k >= 3 ? 2 : k >= 1 ? 1 : 0;
            const int sb = k - tb * (tb + 1) / 2;
            const int tl = 16 * tb + r;
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NK; ++kb) {
                const v8bf bf = *reinterpret_cast<const v8bf *>(&sB[16 * sb + r][32 * kb + 8 * q]);
                const v8bf cf = *reinterpret_cast<const v8bf *>(&sC[tl][32 * kb + 8 * q]);
                acc = mfma32(acc, bf, cf);
            }
            const float cum_t = sCum[tl];
            v4s hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sl = 16 * sb + 4 * q + j;
                const float m = acc[j] * exp2_hw(a2 * (cum_t - sCum[sl])) * sGain[sl];
                const float gv = sl <= tl ? m : 0.f;
                const uint16_t hb = f32_to_bf16(gv);
                hi[j] = short(hb);
                lo[j] = short(f32_to_bf16(gv - bfv(hb)));
            }
            *reinterpret_cast<v4s *>(&sGh[k][r][4 * q]) = hi;
            *reinterpret_cast<v4s *>(&sGl[k][r][4 * q]) = lo;
        }
        // ---- phase 2b: state update (registers): S = exp(A sum delta) S + B^T diag(w) X
        const float dec = sDec;
#pragma unroll
        for (int i = 0; i < NBW; ++i) S[i] *= dec;
#pragma unroll
        for (int kb = 0; kb < SQ / 32; ++kb) {
            float xw[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sl = 32 * kb + 8 * q + j;
                xw[j] = bfv(sXt[16 * pbs + r][sl]) * sW[sl];
            }
            v8bf xh, xl;
            split8(xw, xh, xl);
#pragma unroll
            for (int i = 0; i < NBW; ++i) {
                const v8bf bt = *reinterpret_cast<const v8bf *>(&sBt[16 * (nb0 + i) + r][32 * kb + 8 * q]);
                S[i] = mfma32(S[i], bt, xh);
                S[i] = mfma32(S[i], bt, xl);
            }
        }
        __syncthreads();  // scores in LDS

        // ---- phase 3: outputs Y = scores X + diag(e) (C S_in) + D x for
        // (token block tbo[u], channel block pbo), u = 0, 1
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tb = u == 0 ? tbo0 : tbo1;
            const int tl = 16 * tb + r;
            v4f acc = {0.f, 0.f, 0.f, 0.f}, off = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < SQ / 16; ++sb) {
                if (sb > tb) break;
                const int k = tb * (tb + 1) / 2 + sb;
                const v4s gh = *reinterpret_cast<const v4s *>(&sGh[k][r][4 * q]);
                const v4s gl = *reinterpret_cast<const v4s *>(&sGl[k][r][4 * q]);
                const v4s xf = *reinterpret_cast<const v4s *>(&sXt[16 * pbo + r][16 * sb + 4 * q]);
                acc = mfma16(acc, gh, xf);
                acc = mfma16(acc, gl, xf);
            }
#pragma unroll
            for (int kb = 0; kb < NK; ++kb) {
                const v8bf ca = *reinterpret_cast<const v8bf *>(&sC[tl][32 * kb + 8 * q]);
                const v8bf sh = *reinterpret_cast<const v8bf *>(&sSh[16 * pbo + r][32 * kb + 8 * q]);
                const v8bf sl = *reinterpret_cast<const v8bf *>(&sSl[16 * pbo + r][32 * kb + 8 * q]);
                off = mfma32(off, ca, sh);
                off = mfma32(off, ca, sl);
            }
            // acc[j], off[j] at [t = 16 tb + 4q + j][p = 16 pbo + r]
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tj = 16 * tb + 4 * q + j;
                const float val = fmaf(sE[tj], off[j], fmaf(dsk, bfv(sXt[16 * pbo + r][tj]), acc[j]));
                sY[v][u][4 * q + j][r] = f32_to_bf16(val);
            }
        }
        // the wave's two 16 x 16 output tiles leave as one 16-byte store per lane:
        // lane -> tile u = lane / 32, token row (lane % 32) / 2, channels 8 (lane % 2)..+7
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            const int u = lane / 32, row = (lane % 32) / 2, seg = lane % 2;
            const int tb = u == 0 ? tbo0 : tbo1;
            const v4u yv = *reinterpret_cast<const v4u *>(&sY[v][u][row][8 * seg]);
            const rsrc_t rys = make_rsrc(yb + t0 * rx, (L - t0) * rx * 2);
            __builtin_amdgcn_raw_buffer_store_b128(
                yv, rys, uint32_t(((16 * tb + row) * rx + 16 * pbo + 8 * seg) * 2), 0, 0);
        }
        __syncthreads();  // every wave is done with this chunk's staged data and state
    }
    if (hT) {
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) hT[srow + 16 * (nb0 + i) + 4 * q + j] = S[i][j];
    }
}

template <class IO, int NS>
hipError_t ssd_t(const SsdArgs &a, hipStream_t s) {
    using T = typename IO::T;
    hipLaunchKernelGGL((k_ssd<IO, NS>), dim3(unsigned(a.batch * a.H)), dim3(SWV * kWave), 0, s,
                       static_cast<const T *>(a.x), static_cast<const T *>(a.delta), a.A,
                       static_cast<const T *>(a.B), static_cast<const T *>(a.C), a.Dskip, a.h0,
                       static_cast<T *>(a.y), a.final_state, a.L, a.H, a.G);
    return hipGetLastError();
}

template <int NS>
hipError_t ssd_bf_t(const SsdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((k_ssd_bf<NS>), dim3(unsigned(a.batch * a.H)), dim3(BTH), 0, s,
                       static_cast<const uint16_t *>(a.x), static_cast<const uint16_t *>(a.delta), a.A,
                       static_cast<const uint16_t *>(a.B), static_cast<const uint16_t *>(a.C), a.Dskip, a.h0,
                       static_cast<uint16_t *>(a.y), a.final_state, a.L, a.H, a.G);
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <class IO>
hipError_t ssd_io(const SsdArgs &a, hipStream_t s) {
    // the bf16 kernel's 16-byte loads need 16-byte aligned x, B and C; other
    // bf16 arguments take the 4-wave kernel, which reads element by element
    if constexpr (std::is_same<IO, IoBF16>::value) {
        if (aligned16(a.x) && aligned16(a.B) && aligned16(a.C))
            return a.N == 64 ? ssd_bf_t<64>(a, s) : ssd_bf_t<128>(a, s);
    }
    return a.N == 64 ? ssd_t<IO, 64>(a, s) : ssd_t<IO, 128>(a, s);
}

}  // namespace

hipError_t launch_ssd(const SsdArgs &a, hipStream_t s) {
    return a.io == 1 ? ssd_io<dev::IoBF16>(a, s) : ssd_io<dev::IoF32>(a, s);
}

}  // namespace sscan
