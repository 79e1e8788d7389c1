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
    lds_poison(sX, sBt, sS, sCum, sGain, sW, sE, sDec);

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
// is fetched two chunks ahead (into registers, while the chunks before it
// compute) with coalesced 16-byte loads, 8 or 16 lanes to a token's row, and
// staged in LDS row-major ([token][channel], [token][state]) with 16-byte
// writes.  Operands whose K runs over tokens (x and B, transposed) are read
// with gfx950's transposing LDS read (ds_read_b64_tr_b16: each group of 16
// lanes reads a 4 x 16 block and lane i receives its column i), from tiles
// whose pitch keeps the four rows of a read in different banks; the state
// entering the chunk is kept as a bf16 high part and remainder.
// A chunk is three phases between barriers: staging (with the state
// carried in from the previous chunk); the 10 causal 16x16 score tiles, spread
// over the 8 waves and shared through LDS, beside the state update (wave v
// owns channel block v % 4 and half of the state blocks: equal work); the
// outputs, wave v taking channel block v % 4 of token blocks {0, 3} or {1, 2}
// (equal causal work).  Every product uses the K = 32 matrix instruction
// (v_mfma_f32_16x16x32_bf16); the outputs are formed transposed
// (channels x tokens), so that each lane holds 4 adjacent channels of one
// token and stores them directly.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4bf lds_v4bf_t;

// raw buffer descriptor over `bytes` (< 2^31) bytes from `base`
__device__ __forceinline__ rsrc_t make_rsrc32(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), short(0), int(bytes), 0x00020000);
}

__device__ __forceinline__ lds_v4bf_t *lds_v4bf(const uint16_t *p) {
    return (lds_v4bf_t *)(p);
}

constexpr int BWV = 16;           // waves per workgroup
constexpr int BTH = BWV * kWave;  // threads per workgroup

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

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, kRowMask, 0xF, false));
}

// inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each row
// of 16 lanes (lanes without a source add 0), then the running total at the
// end of row 0 added into row 1 and that of row 2 into row 3 (row_bcast:15),
// then the one at lane 31 into rows 2 and 3 (row_bcast:31)
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v += dpp_or_zero<0x111, 0xF>(v);
    v += dpp_or_zero<0x112, 0xF>(v);
    v += dpp_or_zero<0x114, 0xF>(v);
    v += dpp_or_zero<0x118, 0xF>(v);
    v += dpp_or_zero<0x142, 0xA>(v);
    v += dpp_or_zero<0x143, 0xC>(v);
    return v;
}

template <int NS>
__global__ __launch_bounds__(BTH) void k_ssd_bf(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ delta, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dskip,
    const float *__restrict__ h0, uint16_t *__restrict__ y, float *__restrict__ hT, int64_t L,
    int64_t H, int64_t G) {
    constexpr int NK = NS / 32;        // 32-wide K steps over the states
    // LDS pitches (bf16).  A 16-byte read of rows r = 0..15 at one column is
    // conflict-free on gfx950's 64 banks when the pitch is 8 (mod 16) dwords, so
    // tiles read by rows take NS + 16 (72 or 40 dwords); transposing reads run at
    // one 4 x 16 block per group for any of these pitches, so B serves both ways.
    constexpr int RP = NS + 16;        // [token or channel][state] tiles
    constexpr int XP = SP + 16;        // x read transposed
    constexpr int NBW = NS / 32;       // 16x16 state tiles per state wave (8 waves: 4 channel blocks x 2 halves)
    constexpr int BPL = NS / 16;       // bf16 of a B (or C) row per lane: 16 lanes to a row
    constexpr int NG = 10;             // causal 16x16 score tiles of a 64-token chunk
    constexpr int NM = 6;              // 16 x 32 tiles they are stored in
    constexpr int GP = 48;             // row pitch (bf16) of the stored score tiles (24 dwords)
    constexpr int kScalarWave = 7;    // an output wave: it forms the next chunk's scalars after its score tile
    static_assert(BWV == 16 && SQ == 64 && SP == 64, "work split");
    using VB = typename std::conditional<BPL == 8, v4u, v2u>::type;
    // a chunk's x (two sets: chunk c in set c % 2, as the outputs of chunk c read it
    // while chunk c + 1 is staged), w x, B and C (read before the scores barrier only)
    __shared__ __align__(16) uint16_t sX[2][SQ][XP];  // x, [token][channel]
    __shared__ __align__(16) uint16_t sXWh[SQ][XP];   // w_s x, bf16 high part
    __shared__ __align__(16) uint16_t sXWl[SQ][XP];   // and remainder
    __shared__ __align__(16) uint16_t sB[SQ][RP];     // B, [token][state], read by rows and transposed
    __shared__ __align__(16) uint16_t sC[SQ][RP];     // C, [token][state]
    __shared__ __align__(16) uint16_t sSh[SP][RP];   // entering state, [channel][state], bf16
    __shared__ __align__(16) uint16_t sSl[SP][RP];   // and its remainder
    // masked scores as 16 x 32 tiles [t][s] (B operand of the transposed causal product):
    // tile m(tb, sp) holds tokens 16 tb.. and sources 32 sp..; rows padded to 48
    __shared__ __align__(16) uint16_t sGh[NM][16][GP];
    __shared__ __align__(16) uint16_t sGl[NM][16][GP];
    // per-token scalars, two sets: those of chunk c + 1 are formed during chunk c
    __shared__ __align__(16) float sCum[2][SQ], sGain[2][SQ], sW[2][SQ], sE[2][SQ];
    __shared__ float sDec[2];
    lds_poison(sX, sXWh, sXWl, sB, sC, sSh, sSl, sGh, sGl, sCum, sGain, sW, sE, sDec);

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
    // descriptors over its tokens inside the sequence: 32-bit offsets, and tokens
    // past the end read 0 and drop their stores in the hardware range check.
    const int64_t rx = H * SP, rbc = G * NS;
    const uint16_t *xb = x + (b * L * H + h) * SP;
    uint16_t *yb = y + (b * L * H + h) * SP;
    const uint16_t *Bb = Bm + (b * L * G + g) * NS;
    const uint16_t *Cb = Cm + (b * L * G + g) * NS;
    const uint16_t *db = delta + b * L * H + h;

    // ---- chunk fetch (registers) and staging (LDS), coalesced: 16 lanes to a
    // token's row (8 bytes of x, BPL states of B and C each), wave v taking tokens
    // 4v..4v+3; staged row-major.
    const int srow = 4 * v + lane / 16;
    const int xc = 4 * (lane % 16), bc = BPL * (lane % 16);
    const uint32_t ox = uint32_t((srow * rx + xc) * 2), ob = uint32_t((srow * rbc + bc) * 2);
    const uint32_t od = uint32_t(lane * H * 2);
    struct Chunk {  // one chunk's loads, in flight in registers
        v2u px;
        VB pb, pc;
        uint16_t pd;
    };
    // tokens of chunk c inside the sequence (64, the tail, or 0 past the end); a
    // chunk's bytes fit in 32 bits and the chunk count in 31 (checked at launch)
    const int nfull = int(L / SQ), tail = int(L % SQ);
    auto toks = [&](int c) { return uint32_t(c < nfull ? SQ : c == nfull ? tail : 0); };
    auto ldb = [&](rsrc_t rs, uint32_t o) {
        if constexpr (BPL == 8) return __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
        else return __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
    };
    auto fetch = [&](int c, Chunk &P) {
        // the loads of one fetch stay together and in order (no scheduling across
        // these points): the compiler's wait before a stage then counts only the
        // operations issued after that chunk's loads
        __builtin_amdgcn_sched_barrier(0);
        const int64_t t0 = int64_t(c) * SQ;
        const uint32_t n = toks(c);
        P.px = __builtin_amdgcn_raw_buffer_load_b64(make_rsrc32(xb + t0 * rx, n * uint32_t(rx) * 2), ox, 0, 0);
        P.pb = ldb(make_rsrc32(Bb + t0 * rbc, n * uint32_t(rbc) * 2), ob);
        P.pc = ldb(make_rsrc32(Cb + t0 * rbc, n * uint32_t(rbc) * 2), ob);
        // delta: the scalar wave only (the other waves' descriptor is empty, so their
        // load reads 0 without a memory access and without a branch around it)
        P.pd = __builtin_amdgcn_raw_buffer_load_b16(
            make_rsrc32(db + t0 * H, v == kScalarWave ? n * uint32_t(H) * 2 : 0), od, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // per-token scalars of a chunk (the scalar wave, lane = token): running sum of
    // delta (inclusive), gain, state weight, output decay; chunk decay.  Tokens
    // past the end have delta = 0: gain 0, decay 1.
    auto scalars = [&](const Chunk &P, int par) {
        const float dv = bfv(P.pd);
        const float cum = wave_prefix_sum(dv);
        const float total = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), kWave - 1));
        const float gain = zoh_gain(dv, a, dv * a, exp2_hw(dv * a2));  // delta when A = 0
        sCum[par][lane] = cum;
        sGain[par][lane] = gain;
        sW[par][lane] = exp2_hw(a2 * (total - cum)) * gain;
        sE[par][lane] = exp2_hw(a2 * cum);
        if (lane == 0) sDec[par] = exp2_hw(a2 * total);
    };
    // staging of the chunk with scalar set par; x also as w_s x split into bf16 parts
    // (the update's operand, formed once here rather than by the waves that share a
    // channel block)
    auto stage = [&](const Chunk &P, int par) {
        *reinterpret_cast<v2u *>(&sX[par][srow][xc]) = P.px;
        {
            const float w = sW[par][srow];
            const uint16_t *xv = reinterpret_cast<const uint16_t *>(&P.px);
            v4s hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float xw = bfv(xv[j]) * w;
                const uint16_t hb = f32_to_bf16(xw);
                hi[j] = short(hb);
                lo[j] = short(f32_to_bf16(xw - bfv(hb)));
            }
            *reinterpret_cast<v4s *>(&sXWh[srow][xc]) = hi;
            *reinterpret_cast<v4s *>(&sXWl[srow][xc]) = lo;
        }
        *reinterpret_cast<VB *>(&sB[srow][bc]) = P.pb;
        *reinterpret_cast<VB *>(&sC[srow][bc]) = P.pc;
    };
    // K = 32 operand from a [k][column] tile: lane (r, q) gets rows k0 + 8q .. k0 + 8q + 7
    // of column c0 + r, as two transposing 8-byte reads (each 16-lane group reads a
    // 4 x 16 block, lane i of the group the 4 elements at row i / 4, column 4 (i % 4))
    auto ld_t = [&](const uint16_t *tile, int pitch, int k0, int c0) {
        const int row = k0 + 8 * q + r / 4, col = c0 + 4 * (r % 4);
        const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_v4bf(tile + row * pitch + col));
        const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_v4bf(tile + (row + 4) * pitch + col));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // ---- wave roles.  Output waves (v < 8) form C S_in for two output tiles and a
    // score tile before the scores barrier, and (scores) X after; state waves (v >= 8)
    // update a quarter of the state before (waves 8 and 9 also take a score tile) and
    // publish it after.  (The older waves of a SIMD get its issue slots first: with
    // the state waves first the output products after the barrier ran last.)
    // State tiles of state wave v: channel block pbs, state blocks nb0..nb0+NBW-1;
    // S[i][j] = S[n = 16(nb0 + i) + 4q + j][p = 16 pbs + r]
    const bool outw = v < 8;
    const int pbs = v % 4, nb0 = NBW * ((v / 4) % 2);
    v4f S[NBW];
    const int64_t hrow = ((b * H + h) * SP + 16 * pbs + r) * NS;
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

    // output wave v: channel block pbo, token blocks tbo0 and 3 - tbo0, whose causal
    // work sums to the same for every output wave; the two tiles share the state operand
    const int pbo = v % 4, tbo0 = (v / 4) % 2;
    // score tiles: k = v on output waves 0..7 and state waves 8, 9
    const int ktile = v < 10 ? v : -1;

    // the two 16 x 16 halves of the stored tiles above the diagonal blocks,
    // (tb 0, sb 1) and (tb 2, sb 3), are never written and stay zero
    auto tile32 = [](int tb, int sp) { return tb < 2 ? tb : 2 * tb - 2 + sp; };
    if (v == 12) *reinterpret_cast<v4s *>(&sGh[tile32(0, 0)][r][16 + 4 * q]) = v4s{0, 0, 0, 0};
    if (v == 13) *reinterpret_cast<v4s *>(&sGl[tile32(0, 0)][r][16 + 4 * q]) = v4s{0, 0, 0, 0};
    if (v == 14) *reinterpret_cast<v4s *>(&sGh[tile32(2, 1)][r][16 + 4 * q]) = v4s{0, 0, 0, 0};
    if (v == 15) *reinterpret_cast<v4s *>(&sGl[tile32(2, 1)][r][16 + 4 * q]) = v4s{0, 0, 0, 0};

    // causal score tile k (token block tb, source block sb <= tb, row-major over the
    // triangle): G^T tile (s-block sb, t-block tb) = B C^T, times exp(A (cum_t - cum_s))
    // gain_s where s <= t, plus the skip D on the diagonal (D x is then part of the
    // causal product), split into bf16 parts and stored as rows t, columns s
    auto score_tile = [&](int k, int par) {
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
        const float cum_t = sCum[par][tl];
        v4s hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int sl = 16 * sb + 4 * q + j;
            const float m = acc[j] * exp2_hw(a2 * (cum_t - sCum[par][sl])) * sGain[par][sl];
            const float gv = sl < tl ? m : sl == tl ? m + dsk : 0.f;
            const uint16_t hb = f32_to_bf16(gv);
            hi[j] = short(hb);
            lo[j] = short(f32_to_bf16(gv - bfv(hb)));
        }
        *reinterpret_cast<v4s *>(&sGh[tile32(tb, sb / 2)][r][16 * (sb % 2) + 4 * q]) = hi;
        *reinterpret_cast<v4s *>(&sGl[tile32(tb, sb / 2)][r][16 * (sb % 2) + 4 * q]) = lo;
    };

    // Chunk c is fetched into registers during chunk c - 2 and staged into LDS during
    // chunk c - 1, after the scores barrier (its scalars are formed before it), so a
    // chunk has two barriers: scores ready, and chunk done.  Chunks go in pairs, so an
    // odd count ends with one past the end of the sequence: its loads read 0 (delta
    // 0: decay 1, gain 0, the state unchanged) and its stores are dropped.  Fetches
    // past the end are likewise unconditional: with no branch around them the
    // compiler waits only for the loads a stage needs.  The two roles run loops of
    // their own with the same barriers, so that each loop issues one fixed sequence of
    // loads, and prologues of their own: a load issued before the split whose result
    // one role never uses would leave its registers pending into that role's loop,
    // where the compiler then waits for every load at the loop head.
    const int nchunks = nfull + (tail > 0);
    Chunk P0, P1;
    if (outw) {
        fetch(0, P0);
        fetch(1, P1);
        if (v == kScalarWave) scalars(P0, 0);
        __syncthreads();  // scalars of chunk 0
        stage(P0, 0);
        fetch(2, P0);
        __syncthreads();  // chunk 0 staged
        // chunk c with its x in LDS set par; Pn holds chunk c + 1 in registers
        auto chunk = [&](int c, int par, Chunk &Pn) {
            const int64_t t0 = int64_t(c) * SQ;

            // ---- phase A: S_in C^T for both tiles (the state operand's K steps serve
            // both), kept in registers across the barrier, score tile v, and on the
            // scalar wave chunk c + 1's scalars
            v4f off[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) off[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NK; ++kb) {
                const v8bf sh = *reinterpret_cast<const v8bf *>(&sSh[16 * pbo + r][32 * kb + 8 * q]);
                const v8bf sl = *reinterpret_cast<const v8bf *>(&sSl[16 * pbo + r][32 * kb + 8 * q]);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int tb = u == 0 ? tbo0 : 3 - tbo0;
                    const v8bf cb = *reinterpret_cast<const v8bf *>(&sC[16 * tb + r][32 * kb + 8 * q]);
                    off[u] = mfma32(off[u], sh, cb);
                    off[u] = mfma32(off[u], sl, cb);
                }
            }
            // the score tiles gate every wave's next phase: their waves take a raised issue
            // priority while they compute them, so that their matrix and LDS work goes first
            __builtin_amdgcn_s_setprio(2);
            score_tile(ktile, par);
            __builtin_amdgcn_s_setprio(0);
            if (v == kScalarWave) scalars(Pn, par ^ 1);
            __syncthreads();  // scores and scalars in LDS; every read of S_in, B, C, w x done

            // ---- phase B: Y^T = X^T G'^T + (S_in C^T) diag(e), transposed: lane (r, q)
            // ends with channels 16 pbo + 4q .. + 3 of token 16 tb + r and stores them
            // as 8 bytes; then chunk c + 1 staged and chunk c + 3 fetched
            const rsrc_t rys = make_rsrc32(yb + t0 * rx, toks(c) * uint32_t(rx) * 2);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tb = u == 0 ? tbo0 : 3 - tbo0;
                const int tl = 16 * tb + r;
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    if (32 * sp > 16 * tb + 15) break;
                    const int m = tile32(tb, sp);
                    const v8bf xa = ld_t(&sX[par][0][0], XP, 32 * sp, 16 * pbo);  // x[s = 32sp + 8q + j][16 pbo + r]
                    const v8bf gh = *reinterpret_cast<const v8bf *>(&sGh[m][r][8 * q]);
                    const v8bf gl = *reinterpret_cast<const v8bf *>(&sGl[m][r][8 * q]);
                    acc = mfma32(acc, xa, gh);
                    acc = mfma32(acc, xa, gl);
                }
                const float e = sE[par][tl];
                v4s yv;
#pragma unroll
                for (int j = 0; j < 4; ++j) yv[j] = short(f32_to_bf16(fmaf(e, off[u][j], acc[j])));
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, yv), rys,
                                                      uint32_t((tl * rx + 16 * pbo + 4 * q) * 2), 0, 0);
            }
            stage(Pn, par ^ 1);
            fetch(c + 3, Pn);
            __syncthreads();  // chunk c done; chunk c + 1 staged
        };
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, 0, P1);
            chunk(c + 1, 1, P0);
        }
    } else {
        {
            // the initial state through a descriptor of 0 bytes when there is none
            // (reads 0), with no branch around these loads
            const rsrc_t rh = make_rsrc32(h0 ? h0 + (b * H + h) * SP * NS : nullptr, h0 ? SP * NS * 4 : 0);
#pragma unroll
            for (int i = 0; i < NBW; ++i)
                S[i] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rh, uint32_t(((16 * pbs + r) * NS + 16 * (nb0 + i) + 4 * q) * 4), 0, 0));
        }
        fetch(0, P0);
        fetch(1, P1);
        __syncthreads();  // scalars of chunk 0
        stage(P0, 0);
        fetch(2, P0);
        publish_state();  // the initial state
        __syncthreads();  // chunk 0 staged
        auto chunk = [&](int c, int par, Chunk &Pn) {
            // ---- phase A: waves 8 and 9 a score tile, then S = exp(A sum delta) S +
            // B^T diag(w) X
            if (ktile >= 0) {
                __builtin_amdgcn_s_setprio(2);  // as on the output waves
                score_tile(ktile, par);
                __builtin_amdgcn_s_setprio(0);
            }
            const float dec = sDec[par];
#pragma unroll
            for (int i = 0; i < NBW; ++i) S[i] *= dec;
#pragma unroll
            for (int kb = 0; kb < SQ / 32; ++kb) {
                // (w x)[s = 32kb + 8q + j][16 pbs + r], both parts
                const v8bf xh = ld_t(&sXWh[0][0], XP, 32 * kb, 16 * pbs);
                const v8bf xl = ld_t(&sXWl[0][0], XP, 32 * kb, 16 * pbs);
#pragma unroll
                for (int i = 0; i < NBW; ++i) {
                    const v8bf bt = ld_t(&sB[0][0], RP, 32 * kb, 16 * (nb0 + i));  // B[s][16(nb0 + i) + r]
                    S[i] = mfma32(S[i], bt, xh);
                    S[i] = mfma32(S[i], bt, xl);
                }
            }
            __syncthreads();  // scores and scalars in LDS; every read of S_in, B, C, w x done

            // ---- phase B: the state entering chunk c + 1, then chunk c + 1 staged and
            // chunk c + 3 fetched
            publish_state();
            stage(Pn, par ^ 1);
            fetch(c + 3, Pn);
            __syncthreads();  // chunk c done; chunk c + 1 staged
        };
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, 0, P1);
            chunk(c + 1, 1, P0);
        }
        if (hT) {
#pragma unroll
            for (int i = 0; i < NBW; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) hT[hrow + 16 * (nb0 + i) + 4 * q + j] = S[i][j];
        }
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
        // its chunk offsets are 32-bit: a 64-token chunk of x, B, C or delta below
        // 2^31 bytes, and the chunk count (plus the two fetched ahead) below 2^31
        const bool fits = a.H < (int64_t(1) << 18) && a.G * a.N < (int64_t(1) << 23) &&
                          a.L / SQ < (int64_t(1) << 31) - 4;
        if (fits && aligned16(a.x) && aligned16(a.B) && aligned16(a.C))
            return a.N == 64 ? ssd_bf_t<64>(a, s) : ssd_bf_t<128>(a, s);
    }
    return a.N == 64 ? ssd_t<IO, 64>(a, s) : ssd_t<IO, 128>(a, s);
}

}  // namespace

hipError_t launch_ssd(const SsdArgs &a, hipStream_t s) {
    return a.io == 1 ? ssd_io<dev::IoBF16>(a, s) : ssd_io<dev::IoF32>(a, s);
}

namespace {

// One decode step of the scalar-A-per-head recurrence (the chunk form with one
// token): per (batch row, head, channel p) the state row h[p][0..N) becomes
//     h[p][n] = exp(delta A) h[p][n] + gain B[n] x[p],   y[p] = C . h[p] + D x[p].
// Thread = SPT consecutive states of one row (SPT/4 16-byte state accesses); the
// NS/SPT threads of a row sum their partial readouts with lane shuffles.
// Memory-bound: the state is read and written once, B and C rows are shared by the
// heads of a group (cache hits).  kVec: the state is 16-byte aligned (else element
// accesses).
template <class IO, int NS, bool kVec, int SPT>
__global__ __launch_bounds__(256) void k_ssd_step(float *__restrict__ state, const typename IO::T *__restrict__ x,
                                                  const typename IO::T *__restrict__ delta,
                                                  const float *__restrict__ A, const typename IO::T *__restrict__ B,
                                                  const typename IO::T *__restrict__ C,
                                                  const float *__restrict__ Dskip, typename IO::T *__restrict__ y,
                                                  int64_t rows, int64_t H, int64_t G) {
    constexpr int TPR = NS / SPT;  // threads per state row
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t row0 = i / TPR;
    const int j = int(i % TPR);
    const bool active = row0 < rows;
    const int64_t row = active ? row0 : rows - 1;  // (b H + h) P + p
    const int64_t bh = row / SP;
    const int64_t b = bh / H, h = bh - b * H;
    const int64_t g = h / (H / G);
    const float xv = IO::ld(x, row);
    const float dv = IO::ld(delta, bh);
    const float a = A[h];
    const float dsk = Dskip ? Dskip[h] : 0.f;
    const int64_t bc = (b * G + g) * NS + SPT * j;
    float bv[SPT], cv[SPT], hv[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        bv[k] = IO::ld(B, bc + k);
        cv[k] = IO::ld(C, bc + k);
    }
    float *sp = state + row * NS + SPT * j;
    if constexpr (kVec) {
#pragma unroll
        for (int k = 0; k < SPT; k += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(sp + k);
            hv[k] = v.x; hv[k + 1] = v.y; hv[k + 2] = v.z; hv[k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < SPT; ++k) hv[k] = sp[k];
    }
    const float z = dv * a;
    const float abar = exp2_hw(z * kLog2e);
    const float gx = zoh_gain(dv, a, z, abar) * xv;  // delta x when A = 0
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        hv[k] = fmaf(abar, hv[k], gx * bv[k]);
        part = fmaf(cv[k], hv[k], part);
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off /= 2) part += __shfl_xor(part, off, TPR);
    if (!active) return;
    if constexpr (kVec) {
#pragma unroll
        for (int k = 0; k < SPT; k += 4)
            *reinterpret_cast<float4 *>(sp + k) = make_float4(hv[k], hv[k + 1], hv[k + 2], hv[k + 3]);
    } else {
#pragma unroll
        for (int k = 0; k < SPT; ++k) sp[k] = hv[k];
    }
    if (j == 0) y[row] = IO::enc(fmaf(dsk, xv, part));
}

// states per thread of the decode step: 8 (two 16-byte accesses) measured faster
// than 4 and 16 on the 64 x 64-head, N = 128 decode workload (44.9 vs 47.7 and 52.0 us)
constexpr int kSsdStepSpt = 8;

template <class IO, int NS>
hipError_t ssd_step_t(const SsdStepArgs &a, hipStream_t s) {
    using T = typename IO::T;
    const int64_t rows = a.batch * a.H * a.P;
    const int64_t threads = rows * (NS / kSsdStepSpt);
    const dim3 grid(unsigned((threads + 255) / 256));
    const bool vec = (reinterpret_cast<uintptr_t>(a.state) & 15) == 0;
#define SSCAN_SSD_STEP(V)                                                                                  \
    hipLaunchKernelGGL((k_ssd_step<IO, NS, V, kSsdStepSpt>), grid, dim3(256), 0, s, a.state, static_cast<const T *>(a.x), \
                       static_cast<const T *>(a.delta), a.A, static_cast<const T *>(a.B),                  \
                       static_cast<const T *>(a.C), a.Dskip, static_cast<T *>(a.y), rows, a.H, a.G)
    if (vec) SSCAN_SSD_STEP(true);
    else SSCAN_SSD_STEP(false);
#undef SSCAN_SSD_STEP
    return hipGetLastError();
}

template <class IO>
hipError_t ssd_step_io(const SsdStepArgs &a, hipStream_t s) {
    return a.N == 64 ? ssd_step_t<IO, 64>(a, s) : ssd_step_t<IO, 128>(a, s);
}

}  // namespace

hipError_t launch_ssd_step(const SsdStepArgs &a, hipStream_t s) {
    return a.io == 1 ? ssd_step_io<dev::IoBF16>(a, s) : ssd_step_io<dev::IoF32>(a, s);
}

int64_t ssd_work_items(const SsdArgs &a) {
    // either kernel: one workgroup per (batch row, head), the larger of the two shapes
    return a.batch * a.H * std::max<int64_t>(BTH, SWV * kWave);
}

int64_t ssd_step_work_items(int64_t batch, int64_t H, int64_t P, int64_t N) {
    return (batch * H * P * (N / kSsdStepSpt) + 255) / 256 * 256;
}

}  // namespace sscan
