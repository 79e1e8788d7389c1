// Private interface between the C-ABI layer (sscan_api.hip) and the kernels
// (sscan_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sscan {

constexpr int kWave = 64;  // CDNA wavefront width: one lane per channel

// Launch shape of the lockstep kernel: kLockW waves per 64-channel tile, each
// taking runs of kLockT tokens.  A tile's workgroup fills one CU, so the kernel
// is used when there are at least kLockMinTiles tiles (MI355X has 256 CUs);
// fewer tiles go to the segment kernels, which spread over every CU.
#ifndef SSCAN_LOCK_W
#define SSCAN_LOCK_W 16
#endif
#ifndef SSCAN_LOCK_T
#define SSCAN_LOCK_T 16
#endif
#ifndef SSCAN_TARGET_WAVES
#define SSCAN_TARGET_WAVES 32768
#endif
constexpr int kLockW = SSCAN_LOCK_W;
constexpr int kLockT = SSCAN_LOCK_T;
#ifndef SSCAN_LOCK_MIN_TILES
#define SSCAN_LOCK_MIN_TILES 192
#endif
constexpr int64_t kLockMinTiles = SSCAN_LOCK_MIN_TILES;
constexpr int64_t kTargetWaves = SSCAN_TARGET_WAVES;  // segment kernels: waves to aim for

// Front end of the fused entry points: the scan input is the causal depthwise
// convolution (width K, optional bias, optional SiLU) of x, and the step size
// is softplus(delta_raw + delta_bias).  K == 0: no front end (x and delta are
// the scan's inputs as given).
constexpr int kMaxConv = 4;
struct FeArgs {
    const float *conv_w;      // (dim, K) fp32; tap k multiplies x[t - K + 1 + k]
    const float *conv_b;      // (dim) fp32, or NULL
    const float *delta_bias;  // (dim) fp32, or NULL
    const void *conv_state;   // (batch, K-1, dim) I/O dtype: inputs before token 0, or NULL (zero)
    int K;                    // 0 (no front end) or 1..kMaxConv
    int act;                  // 0 none, 1 SiLU
};

// Limits every launch is planned against.  A raw buffer descriptor covers at
// most kMaxDescBytes bytes (its record count is kept below 2^31), and the byte
// offsets added to it are 32-bit: a kernel that walks a span through one
// descriptor needs the span, plus whatever it prefetches past its end, below
// 2^32 so that no offset wraps.  A dispatch's total work-item count in x is a
// 32-bit quantity (kMaxWorkItems).
constexpr int64_t kMaxDescBytes = 0x7FFFFFFF;
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;

// Work split of one forward pass.  Segment kernels cut the sequence into
// `segments` time segments of `seg_len` tokens (the last may be shorter); each
// wave scans one segment of 64 channels of one batch row.  The lockstep kernel
// gives each 64-channel tile one workgroup for the whole sequence.
// `reject` is non-NULL when the shape cannot be run within the limits above
// (then nothing may be launched); it names the reason.
struct FwdPlan {
    const char *reject;
    int64_t tiles_per_batch;  // ceil(dim / 64)
    int64_t tiles;            // batch * tiles_per_batch
    int64_t seg_len;
    int segments;
    int nt;                   // dstate rounded up to 1, 2, 4, 8 or 16
    bool lockstep;            // structured-real tiles use the lockstep kernel
    size_t off_bc, off_flags, off_sum, off_h;  // scratch layout
    size_t ws_bytes;          // scratch: [B/(n+1), C] rows, tile flags, segment aggregates
};

// io: 0 fp32, 1 bf16 (the element size of x, delta and y sets the segment spans);
// max_ws > 0: a scratch budget the segment path is fitted to where it can be
FwdPlan plan_forward(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io, size_t max_ws = 0);

struct FwdArgs {
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *Dskip;
    const float *h0;  // state before token 0, (batch, dim, N); NULL = zero
    void *y;
    float *final_state;
    int64_t batch, L, dim;
    int N;
    int io;  // 0 fp32, 1 bf16
    FeArgs fe;             // front end (fe.K == 0: none)
    void *conv_state_out;  // (batch, K-1, dim) I/O dtype, or NULL; front end only
};

// Enqueue the forward pass; `ws` points at plan.ws_bytes of device scratch.
hipError_t launch_forward(const FwdArgs &a, const FwdPlan &plan, void *ws, hipStream_t s);

// Enqueue the prologue shared by the forward and backward passes: B/(n+1) and C
// of each of `rows` tokens as fp32 rows of 2*nt floats into `bc`, and one flag
// per 64-channel tile into `tile_fast` (1 when every A row of the tile is
// A[d,n] = (n+1)*A[d,0] with A[d,0] < 0).
hipError_t launch_prep(const void *B, const void *C, const float *A, float *bc, int *tile_fast,
                       int64_t rows, int64_t dim, int N, int nt, int io, hipStream_t s);

// Backward pass: one workgroup per (batch row, 64-channel tile) walks the whole
// sequence; scratch holds the staged B/C rows, tile flags, the state entering
// every chunk, per-tile dB/dC partials and per-batch-row dA/dDskip partials.
struct BwdPlan {
    const char *reject;  // non-NULL: the shape exceeds a launch limit (reason)
    int64_t tiles_per_batch, tiles;
    int nt;
    size_t off_bc, off_flags, off_ckpt, off_pbc, off_pad;
    size_t ws_bytes;
};

BwdPlan plan_backward(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

struct BwdArgs {
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *Dskip;
    const float *h0;   // NULL = zero
    const void *dy;
    const float *dhT;  // NULL = zero
    void *dx, *ddelta;
    float *dA, *dB, *dC, *dD, *dh0;  // dD, dh0 may be NULL
    int64_t batch, L, dim;
    int N;
    int io;
};

hipError_t launch_backward(const BwdArgs &a, const BwdPlan &plan, void *ws, hipStream_t s);

// Enqueue conv_state_out[b, j, d] = raw input of token seqlen-(K-1)+j (from x, or
// from fe.conv_state for tokens before 0, zero when absent); fe.K >= 2.
hipError_t launch_conv_tail(const void *x, const FeArgs &fe, void *conv_state_out, int64_t batch,
                            int64_t seqlen, int64_t dim, int io, hipStream_t s);

// Scalar-A-per-head scan (Mamba-2's SSM) in its chunked matrix form.
struct SsdArgs {
    const void *x, *delta;  // (batch, L, H, P), (batch, L, H)
    const float *A;         // (H)
    const void *B, *C;      // (batch, L, G, N)
    const float *Dskip;     // (H) or NULL
    const float *h0;        // (batch, H, P, N) or NULL
    void *y;                // (batch, L, H, P)
    float *final_state;     // (batch, H, P, N) or NULL
    int64_t batch, L, H, P, G;
    int N;
    int io;
};
constexpr int kSsdHeadDim = 64;  // supported P

hipError_t launch_ssd(const SsdArgs &a, hipStream_t s);

// One decode step of the scalar-A-per-head scan, state updated in place.
struct SsdStepArgs {
    float *state;           // (batch, H, P, N)
    const void *x, *delta;  // (batch, H, P), (batch, H)
    const float *A;         // (H)
    const void *B, *C;      // (batch, G, N)
    const float *Dskip;     // (H) or NULL
    void *y;                // (batch, H, P)
    int64_t batch, H, P, G;
    int N;
    int io;
};
hipError_t launch_ssd_step(const SsdStepArgs &a, hipStream_t s);

// Enqueue dst[i] = src ? src[i] : 0 for `count` floats (final_state at seqlen 0).
hipError_t launch_copy_or_zero(float *dst, const float *src, int64_t count, hipStream_t s);

struct StepArgs {
    float *state;
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *Dskip;
    void *y;
    int64_t batch, dim;
    int N;
    int io;
    FeArgs fe;         // front end (fe.K == 0: none); fe.conv_state is read and
    void *conv_state;  // updated in place through this pointer (same buffer)
};

hipError_t launch_step(const StepArgs &a, hipStream_t s);

// Total work items of the decode step's launch (checked against kMaxWorkItems
// before launching).
int64_t step_work_items(int64_t batch, int64_t dim, int64_t N, bool front_end);
// Workgroups x threads of the scalar-A-per-head launches.
int64_t ssd_work_items(const SsdArgs &a);
int64_t ssd_step_work_items(int64_t batch, int64_t H, int64_t P, int64_t N);

}  // namespace sscan
