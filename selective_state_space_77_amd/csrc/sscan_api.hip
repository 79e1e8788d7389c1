// C-ABI entry points of libsscan.so: argument validation, scratch memory and
// dispatch to the gfx950 kernels.  Declarations and contracts: include/sscan.h.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/sscan.h"
#include "sscan_internal.h"

namespace {

thread_local char g_last_error[512];

int fail(int status, const char *fmt, const char *a = "", const char *b = "") {
    snprintf(g_last_error, sizeof g_last_error, fmt, a, b);
    return status;
}

int fail_hip(const char *what, hipError_t e) {
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), int(e));
    return SSCAN_ERR_HIP;
}

// bytes = product of sizes * elem; false on overflow or negative size
bool nbytes(int64_t *out, int64_t elem, int64_t a, int64_t b = 1, int64_t c = 1) {
    if (a < 0 || b < 0 || c < 0) return false;
    int64_t v = elem;
    if (__builtin_mul_overflow(v, a, &v) || __builtin_mul_overflow(v, b, &v) ||
        __builtin_mul_overflow(v, c, &v))
        return false;
    *out = v;
    return true;
}

struct Span {
    const void *p;
    int64_t bytes;
    const char *name;
};

bool overlap(const Span &u, const Span &v) {
    if (!u.p || !v.p || u.bytes == 0 || v.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(u.p), a1 = a0 + uintptr_t(u.bytes);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(v.p), b1 = b0 + uintptr_t(v.bytes);
    return a0 < b1 && b0 < a1;
}

// every output must be disjoint from every other span
int check_alias(const Span *outs, int nout, const Span *ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], ins[j]))
                return fail(SSCAN_ERR_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(SSCAN_ERR_ALIAS, "outputs %s and %s overlap", outs[i].name, outs[j].name);
    }
    return SSCAN_OK;
}

int check_ptrs(const Span *s, int n) {
    for (int i = 0; i < n; ++i)
        if (!s[i].p && s[i].bytes > 0) return fail(SSCAN_ERR_NULL, "required pointer %s is NULL", s[i].name);
    return SSCAN_OK;
}

// Scratch of sscan_forward_noalloc, for callers that cannot allocate: a file-scope
// device array (every GPU the library runs on holds its own copy until the process
// ends).  In host code `scratch` only names the symbol: kernels receive the
// per-device address that hipGetSymbolAddress returns for it, looked up once per
// device with that device current and kept in g_scratch_dev.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];

// The address of `scratch` on the device of `stream` (NULL stream: the current
// device), or NULL with the status in *rc.
void *noalloc_scratch(hipStream_t stream, int *rc) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) {
        *rc = fail_hip("device of the stream", e);
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *rc = fail(SSCAN_ERR_UNSUPPORTED, "device ordinal beyond the library's table");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) {
            *rc = fail_hip("hipSetDevice", e);
            return nullptr;
        }
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess || !p) {
            *rc = fail_hip("hipGetSymbolAddress (static scratch)", e);
            return nullptr;
        }
        g_scratch_dev[dev] = p;
    }
    return g_scratch_dev[dev];
}

}  // namespace

extern "C" {

int sscan_version(void) { return SSCAN_ABI_VERSION; }

const char *sscan_last_error(void) { return g_last_error; }

const char *sscan_status_string(int status) {
    switch (status) {
        case SSCAN_OK: return "ok";
        case SSCAN_ERR_NULL: return "required pointer is NULL";
        case SSCAN_ERR_SHAPE: return "invalid shape (negative size or int64 overflow)";
        case SSCAN_ERR_UNSUPPORTED: return "unsupported dstate, io_dtype or size";
        case SSCAN_ERR_ALIAS: return "output overlaps another argument";
        case SSCAN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int sscan_forward_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                       sscan_plan_info *out) {
    g_last_error[0] = '\0';
    if (!out) return fail(SSCAN_ERR_NULL, "required pointer %s is NULL", "out");
    memset(out, 0, sizeof *out);
    if (io_dtype != SSCAN_F32 && io_dtype != SSCAN_BF16)
        return fail(SSCAN_ERR_UNSUPPORTED, "io_dtype must be SSCAN_F32 or SSCAN_BF16");
    if (dstate < 1 || dstate > SSCAN_MAX_DSTATE)
        return fail(SSCAN_ERR_UNSUPPORTED, "dstate must be in 1..16");
    int64_t bx;
    if (!nbytes(&bx, io_dtype == SSCAN_BF16 ? 2 : 4, batch, seqlen, dim))
        return fail(SSCAN_ERR_SHAPE, "negative size or byte size overflows int64");
    const sscan::FwdPlan p = sscan::plan_forward(batch, seqlen, dim, dstate, io_dtype);
    if (p.reject) return fail(SSCAN_ERR_UNSUPPORTED, "%s", p.reject);
    out->kernel = p.lockstep ? SSCAN_PLAN_LOCKSTEP : SSCAN_PLAN_SEGMENT;
    out->segments = p.lockstep ? 1 : p.segments;
    out->seg_len = p.lockstep ? seqlen : p.seg_len;
    out->tiles = p.tiles;
    out->chunk_tokens = p.lockstep ? int64_t(sscan::kLockW) * sscan::kLockT : 0;
    out->scratch_bytes = int64_t(p.ws_bytes);
    return SSCAN_OK;
}

// Front end of the fused entry points (d_conv == 0: none).
struct FrontEnd {
    const float *conv_weight = nullptr, *conv_bias = nullptr, *delta_bias = nullptr;
    const void *conv_state_in = nullptr;
    void *conv_state_out = nullptr;
    int d_conv = 0, activation = 0;
};

static int forward_impl(const void *x, const void *delta, const float *A, const void *B,
                        const void *C, const float *Dskip, const float *initial_state, void *y,
                        float *final_state, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                        int io_dtype, void *stream, const FrontEnd &fe = FrontEnd(),
                        bool static_scratch = false) {
    g_last_error[0] = '\0';
    if (io_dtype != SSCAN_F32 && io_dtype != SSCAN_BF16)
        return fail(SSCAN_ERR_UNSUPPORTED, "io_dtype must be SSCAN_F32 or SSCAN_BF16");
    if (dstate < 1 || dstate > SSCAN_MAX_DSTATE)
        return fail(SSCAN_ERR_UNSUPPORTED, "dstate must be in 1..16");
    const bool fused = fe.d_conv > 0;
    if (fused && fe.d_conv > SSCAN_MAX_DCONV)
        return fail(SSCAN_ERR_UNSUPPORTED, "d_conv must be in 1..4");
    if (fused && fe.activation != SSCAN_ACT_NONE && fe.activation != SSCAN_ACT_SILU)
        return fail(SSCAN_ERR_UNSUPPORTED, "activation must be SSCAN_ACT_NONE or SSCAN_ACT_SILU");
    const int64_t es = io_dtype == SSCAN_BF16 ? 2 : 4;
    int64_t bx, bbc, ba, bd, bs, ws_guard, bw = 0, bcs = 0;
    if (!nbytes(&bx, es, batch, seqlen, dim) || !nbytes(&bbc, es, batch, seqlen, dstate) ||
        !nbytes(&ba, 4, dim, dstate) || !nbytes(&bd, 4, dim) || !nbytes(&bs, 4, batch, dim, dstate) ||
        !nbytes(&ws_guard, 2 * 16 * 4, batch, seqlen) ||
        (fused && (!nbytes(&bw, 4, dim, fe.d_conv) || !nbytes(&bcs, es, batch, fe.d_conv - 1, dim))))
        return fail(SSCAN_ERR_SHAPE, "negative size or byte size overflows int64");
    const Span ins[] = {{x, bx, "x"}, {delta, bx, fused ? "delta_raw" : "delta"}, {A, ba, "A"}, {B, bbc, "B"},
                        {C, bbc, "C"}, {Dskip, Dskip ? bd : 0, "Dskip"},
                        {initial_state, initial_state ? bs : 0, "initial_state"},
                        {fe.conv_weight, bw, "conv_weight"},
                        {fe.conv_bias, fe.conv_bias ? bd : 0, "conv_bias"},
                        {fe.delta_bias, fe.delta_bias ? bd : 0, "delta_bias"},
                        {fe.conv_state_in, fe.conv_state_in ? bcs : 0, "conv_state_in"}};
    const Span outs[] = {{y, bx, "y"}, {final_state, final_state ? bs : 0, "final_state"},
                         {fe.conv_state_out, fe.conv_state_out ? bcs : 0, "conv_state_out"}};
    const Span req[] = {ins[0], ins[1], ins[2], ins[3], ins[4], outs[0], ins[7]};
    int rc = check_ptrs(req, fused ? 7 : 6);
    if (rc) return rc;
    rc = check_alias(outs, 3, ins, 11);
    if (rc) return rc;

    hipStream_t s = static_cast<hipStream_t>(stream);
    sscan::FeArgs fa{};
    if (fused) fa = {fe.conv_weight, fe.conv_bias, fe.delta_bias, fe.conv_state_in, fe.d_conv, fe.activation};
    if (batch == 0 || dim == 0) return SSCAN_OK;
    if (seqlen == 0) {
        hipError_t e = hipSuccess;
        if (final_state) e = sscan::launch_copy_or_zero(final_state, initial_state, batch * dim * dstate, s);
        if (e == hipSuccess && fused && fe.conv_state_out)
            e = sscan::launch_conv_tail(x, fa, fe.conv_state_out, batch, 0, dim, io_dtype, s);
        return e == hipSuccess ? SSCAN_OK : fail_hip("state copy launch", e);
    }

    const sscan::FwdPlan plan =
        sscan::plan_forward(batch, seqlen, dim, dstate, io_dtype, static_scratch ? kNoAllocScratchBytes : 0);
    if (plan.reject) return fail(SSCAN_ERR_UNSUPPORTED, "%s", plan.reject);
    sscan::FwdArgs a{x,   delta,  A,           B,      C,   Dskip,         initial_state,
                     y,   final_state, batch, seqlen, dim, int(dstate), io_dtype,
                     fa,  fe.conv_state_out};
    if (static_scratch) {
        // no allocation: the library's per-device scratch array (every byte a launch
        // reads from it is written earlier in the same call, so nothing is cleared)
        if (plan.ws_bytes > kNoAllocScratchBytes) {
            char need[64];
            snprintf(need, sizeof need, "%zu", plan.ws_bytes);
            return fail(SSCAN_ERR_UNSUPPORTED, "needs %s bytes of scratch, above the static %s",
                        need, "64 MiB");
        }
        void *ws = noalloc_scratch(s, &rc);
        if (!ws) return rc;
        const hipError_t el = sscan::launch_forward(a, plan, ws, s);
        return el == hipSuccess ? SSCAN_OK : fail_hip("forward launch", el);
    }
    void *ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, plan.ws_bytes, s);
    if (e != hipSuccess) return fail_hip("hipMallocAsync (scratch)", e);
    e = sscan::launch_forward(a, plan, ws, s);
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e != hipSuccess) return fail_hip("forward launch", e);
    if (ef != hipSuccess) return fail_hip("hipFreeAsync (scratch)", ef);
    return SSCAN_OK;
}

int sscan_forward(const void *x, const void *delta, const float *A, const void *B, const void *C,
                  const float *Dskip, void *y, float *final_state, int64_t batch, int64_t seqlen,
                  int64_t dim, int64_t dstate, int io_dtype, void *stream) {
    return forward_impl(x, delta, A, B, C, Dskip, nullptr, y, final_state, batch, seqlen, dim, dstate,
                        io_dtype, stream);
}

int sscan_forward_from_state(const void *x, const void *delta, const float *A, const void *B,
                             const void *C, const float *Dskip, const float *initial_state, void *y,
                             float *final_state, int64_t batch, int64_t seqlen, int64_t dim,
                             int64_t dstate, int io_dtype, void *stream) {
    return forward_impl(x, delta, A, B, C, Dskip, initial_state, y, final_state, batch, seqlen, dim,
                        dstate, io_dtype, stream);
}

int sscan_forward_noalloc(const void *x, const void *delta, const float *A, const void *B,
                          const void *C, const float *Dskip, const float *initial_state, void *y,
                          float *final_state, int64_t batch, int64_t seqlen, int64_t dim,
                          int64_t dstate, int io_dtype, void *stream) {
    return forward_impl(x, delta, A, B, C, Dskip, initial_state, y, final_state, batch, seqlen, dim,
                        dstate, io_dtype, stream, FrontEnd(), true);
}

int sscan_backward(const void *x, const void *delta, const float *A, const void *B, const void *C,
                   const float *Dskip, const float *initial_state, const void *dy,
                   const float *dfinal_state, void *dx, void *ddelta, float *dA, float *dB,
                   float *dC, float *dDskip, float *dinitial_state, int64_t batch, int64_t seqlen,
                   int64_t dim, int64_t dstate, int io_dtype, void *stream) {
    g_last_error[0] = '\0';
    if (io_dtype != SSCAN_F32 && io_dtype != SSCAN_BF16)
        return fail(SSCAN_ERR_UNSUPPORTED, "io_dtype must be SSCAN_F32 or SSCAN_BF16");
    if (dstate < 1 || dstate > SSCAN_MAX_DSTATE)
        return fail(SSCAN_ERR_UNSUPPORTED, "dstate must be in 1..16");
    if (dim > (int64_t(1) << 24))
        return fail(SSCAN_ERR_UNSUPPORTED, "backward: dim above 2^24 is not supported");
    const int64_t es = io_dtype == SSCAN_BF16 ? 2 : 4;
    int64_t bx, bbc, bbc32, ba, bd, bs, ws_guard;
    if (!nbytes(&bx, es, batch, seqlen, dim) || !nbytes(&bbc, es, batch, seqlen, dstate) ||
        !nbytes(&bbc32, 4, batch, seqlen, dstate) || !nbytes(&ba, 4, dim, dstate) ||
        !nbytes(&bd, 4, dim) || !nbytes(&bs, 4, batch, dim, dstate) ||
        !nbytes(&ws_guard, 2 * 16 * 4, batch, seqlen, dim / 64 + 1))
        return fail(SSCAN_ERR_SHAPE, "negative size or byte size overflows int64");
    const Span ins[] = {{x, bx, "x"}, {delta, bx, "delta"}, {A, ba, "A"}, {B, bbc, "B"},
                        {C, bbc, "C"}, {Dskip, Dskip ? bd : 0, "Dskip"},
                        {initial_state, initial_state ? bs : 0, "initial_state"}, {dy, bx, "dy"},
                        {dfinal_state, dfinal_state ? bs : 0, "dfinal_state"}};
    const Span outs[] = {{dx, bx, "dx"}, {ddelta, bx, "ddelta"}, {dA, ba, "dA"}, {dB, bbc32, "dB"},
                         {dC, bbc32, "dC"}, {dDskip, dDskip ? bd : 0, "dDskip"},
                         {dinitial_state, dinitial_state ? bs : 0, "dinitial_state"}};
    const Span req[] = {ins[0], ins[1], ins[2], ins[3], ins[4], ins[7], outs[0], outs[1], outs[2],
                        outs[3], outs[4]};
    int rc = check_ptrs(req, 11);
    if (rc) return rc;
    rc = check_alias(outs, 7, ins, 9);
    if (rc) return rc;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (batch == 0 || dim == 0 || seqlen == 0) {
        // sums over an empty set: dA, dDskip (and dB, dC when dim == 0) are zero;
        // with no tokens the gradient passes through to the initial state
        hipError_t e = sscan::launch_copy_or_zero(dA, nullptr, dim * dstate, s);
        if (e == hipSuccess && dDskip) e = sscan::launch_copy_or_zero(dDskip, nullptr, dim, s);
        if (e == hipSuccess) e = sscan::launch_copy_or_zero(dB, nullptr, batch * seqlen * dstate, s);
        if (e == hipSuccess) e = sscan::launch_copy_or_zero(dC, nullptr, batch * seqlen * dstate, s);
        if (e == hipSuccess && dinitial_state)
            e = sscan::launch_copy_or_zero(dinitial_state, seqlen == 0 ? dfinal_state : nullptr,
                                           batch * dim * dstate, s);
        return e == hipSuccess ? SSCAN_OK : fail_hip("zero-fill launch", e);
    }

    const sscan::BwdPlan plan = sscan::plan_backward(batch, seqlen, dim, dstate);
    if (plan.reject) return fail(SSCAN_ERR_UNSUPPORTED, "%s", plan.reject);
    void *ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, plan.ws_bytes, s);
    if (e != hipSuccess) return fail_hip("hipMallocAsync (scratch)", e);
    sscan::BwdArgs a{x,  delta, A,  B,  C,  Dskip,  initial_state,  dy, dfinal_state, dx, ddelta, dA,
                     dB, dC,    dDskip, dinitial_state, batch, seqlen, dim, int(dstate), io_dtype};
    e = sscan::launch_backward(a, plan, ws, s);
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e != hipSuccess) return fail_hip("backward launch", e);
    if (ef != hipSuccess) return fail_hip("hipFreeAsync (scratch)", ef);
    return SSCAN_OK;
}

int sscan_forward_fused(const void *x, const float *conv_weight, const float *conv_bias, int d_conv,
                        int activation, const void *conv_state_in, const void *delta_raw,
                        const float *delta_bias, const float *A, const void *B, const void *C,
                        const float *Dskip, const float *initial_state, void *y, float *final_state,
                        void *conv_state_out, int64_t batch, int64_t seqlen, int64_t dim,
                        int64_t dstate, int io_dtype, void *stream) {
    g_last_error[0] = '\0';
    if (d_conv < 1) return fail(SSCAN_ERR_UNSUPPORTED, "d_conv must be in 1..4");
    FrontEnd fe;
    fe.conv_weight = conv_weight;
    fe.conv_bias = conv_bias;
    fe.delta_bias = delta_bias;
    fe.conv_state_in = conv_state_in;
    fe.conv_state_out = conv_state_out;
    fe.d_conv = d_conv;
    fe.activation = activation;
    return forward_impl(x, delta_raw, A, B, C, Dskip, initial_state, y, final_state, batch, seqlen, dim,
                        dstate, io_dtype, stream, fe);
}

int sscan_ssd_forward(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *Dskip, const float *initial_state, void *y, float *final_state,
                      int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                      int64_t dstate, int io_dtype, void *stream) {
    g_last_error[0] = '\0';
    if (io_dtype != SSCAN_F32 && io_dtype != SSCAN_BF16)
        return fail(SSCAN_ERR_UNSUPPORTED, "io_dtype must be SSCAN_F32 or SSCAN_BF16");
    if (headdim != sscan::kSsdHeadDim) return fail(SSCAN_ERR_UNSUPPORTED, "headdim must be 64");
    if (dstate != 64 && dstate != 128) return fail(SSCAN_ERR_UNSUPPORTED, "dstate must be 64 or 128");
    if (nheads < 1 || ngroups < 1 || nheads % ngroups != 0)
        return fail(SSCAN_ERR_SHAPE, "nheads and ngroups must be positive, nheads a multiple of ngroups");
    const int64_t es = io_dtype == SSCAN_BF16 ? 2 : 4;
    int64_t bx, bd, bbc, bh, bs, tmp;
    if (!nbytes(&bx, es, batch, seqlen, nheads * headdim) || !nbytes(&bd, es, batch, seqlen, nheads) ||
        !nbytes(&bbc, es, batch, seqlen, ngroups * dstate) || !nbytes(&bh, 4, nheads) ||
        !nbytes(&bs, 4, batch, nheads, headdim * dstate) || !nbytes(&tmp, 1, batch, nheads))
        return fail(SSCAN_ERR_SHAPE, "negative size or byte size overflows int64");
    {
        const sscan::SsdArgs probe{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, batch, seqlen, nheads, headdim, ngroups, int(dstate), io_dtype};
        if (batch > 0 && sscan::ssd_work_items(probe) > sscan::kMaxWorkItems)
            return fail(SSCAN_ERR_UNSUPPORTED, "batch * nheads too large for one launch");
    }
    const Span ins[] = {{x, bx, "x"}, {delta, bd, "delta"}, {A, bh, "A"}, {B, bbc, "B"}, {C, bbc, "C"},
                        {Dskip, Dskip ? bh : 0, "Dskip"},
                        {initial_state, initial_state ? bs : 0, "initial_state"}};
    const Span outs[] = {{y, bx, "y"}, {final_state, final_state ? bs : 0, "final_state"}};
    const Span req[] = {ins[0], ins[1], ins[2], ins[3], ins[4], outs[0]};
    int rc = check_ptrs(req, 6);
    if (rc) return rc;
    rc = check_alias(outs, 2, ins, 7);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (batch == 0) return SSCAN_OK;
    if (seqlen == 0) {
        if (!final_state) return SSCAN_OK;
        const hipError_t e = sscan::launch_copy_or_zero(final_state, initial_state, bs / 4, s);
        return e == hipSuccess ? SSCAN_OK : fail_hip("state copy launch", e);
    }
    sscan::SsdArgs a{x, delta, A, B, C, Dskip, initial_state, y, final_state, batch, seqlen, nheads,
                     headdim, ngroups, int(dstate), io_dtype};
    const hipError_t e = sscan::launch_ssd(a, s);
    return e == hipSuccess ? SSCAN_OK : fail_hip("ssd launch", e);
}

int sscan_ssd_step(float *state, const void *x_t, const void *delta_t, const float *A, const void *B_t,
                   const void *C_t, const float *Dskip, void *y_t, int64_t batch, int64_t nheads,
                   int64_t headdim, int64_t ngroups, int64_t dstate, int io_dtype, void *stream) {
    g_last_error[0] = '\0';
    if (io_dtype != SSCAN_F32 && io_dtype != SSCAN_BF16)
        return fail(SSCAN_ERR_UNSUPPORTED, "io_dtype must be SSCAN_F32 or SSCAN_BF16");
    if (headdim != sscan::kSsdHeadDim) return fail(SSCAN_ERR_UNSUPPORTED, "headdim must be 64");
    if (dstate != 64 && dstate != 128) return fail(SSCAN_ERR_UNSUPPORTED, "dstate must be 64 or 128");
    if (nheads < 1 || ngroups < 1 || nheads % ngroups != 0)
        return fail(SSCAN_ERR_SHAPE, "nheads and ngroups must be positive, nheads a multiple of ngroups");
    const int64_t es = io_dtype == SSCAN_BF16 ? 2 : 4;
    int64_t bx, bd, bbc, bh, bs;
    if (!nbytes(&bx, es, batch, nheads * headdim) || !nbytes(&bd, es, batch, nheads) ||
        !nbytes(&bbc, es, batch, ngroups * dstate) || !nbytes(&bh, 4, nheads) ||
        !nbytes(&bs, 4, batch, nheads, headdim * dstate))
        return fail(SSCAN_ERR_SHAPE, "negative size or byte size overflows int64");
    if (sscan::ssd_step_work_items(batch, nheads, headdim, dstate) > sscan::kMaxWorkItems)
        return fail(SSCAN_ERR_UNSUPPORTED, "state too large for one launch");
    const Span ins[] = {{x_t, bx, "x_t"}, {delta_t, bd, "delta_t"}, {A, bh, "A"}, {B_t, bbc, "B_t"},
                        {C_t, bbc, "C_t"}, {Dskip, Dskip ? bh : 0, "Dskip"}};
    const Span outs[] = {{state, bs, "state"}, {y_t, bx, "y_t"}};
    const Span req[] = {ins[0], ins[1], ins[2], ins[3], ins[4], outs[0], outs[1]};
    int rc = check_ptrs(req, 7);
    if (rc) return rc;
    rc = check_alias(outs, 2, ins, 6);
    if (rc) return rc;
    if (batch == 0) return SSCAN_OK;
    sscan::SsdStepArgs a{state, x_t, delta_t, A, B_t, C_t, Dskip, y_t, batch, nheads, headdim, ngroups,
                         int(dstate), io_dtype};
    const hipError_t e = sscan::launch_ssd_step(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSCAN_OK : fail_hip("ssd step launch", e);
}

static int step_impl(float *state, const void *x_t, const void *delta_t, const float *A,
                     const void *B_t, const void *C_t, const float *Dskip, void *y_t, int64_t batch,
                     int64_t dim, int64_t dstate, int io_dtype, void *stream, const FrontEnd &fe,
                     void *conv_state) {
    g_last_error[0] = '\0';
    if (io_dtype != SSCAN_F32 && io_dtype != SSCAN_BF16)
        return fail(SSCAN_ERR_UNSUPPORTED, "io_dtype must be SSCAN_F32 or SSCAN_BF16");
    if (dstate < 1 || dstate > SSCAN_MAX_DSTATE)
        return fail(SSCAN_ERR_UNSUPPORTED, "dstate must be in 1..16");
    const bool fused = fe.d_conv > 0;
    if (fused && fe.d_conv > SSCAN_MAX_DCONV)
        return fail(SSCAN_ERR_UNSUPPORTED, "d_conv must be in 1..4");
    if (fused && fe.activation != SSCAN_ACT_NONE && fe.activation != SSCAN_ACT_SILU)
        return fail(SSCAN_ERR_UNSUPPORTED, "activation must be SSCAN_ACT_NONE or SSCAN_ACT_SILU");
    const int64_t es = io_dtype == SSCAN_BF16 ? 2 : 4;
    int64_t bx, bbc, ba, bd, bs, bw = 0, bcs = 0;
    if (!nbytes(&bx, es, batch, dim) || !nbytes(&bbc, es, batch, dstate) || !nbytes(&ba, 4, dim, dstate) ||
        !nbytes(&bd, 4, dim) || !nbytes(&bs, 4, batch, dim, dstate) ||
        (fused && (!nbytes(&bw, 4, dim, fe.d_conv) || !nbytes(&bcs, es, batch, fe.d_conv - 1, dim))))
        return fail(SSCAN_ERR_SHAPE, "negative size or byte size overflows int64");
    const Span ins[] = {{x_t, bx, "x_t"}, {delta_t, bx, fused ? "delta_raw_t" : "delta_t"}, {A, ba, "A"},
                        {B_t, bbc, "B_t"}, {C_t, bbc, "C_t"}, {Dskip, Dskip ? bd : 0, "Dskip"},
                        {fe.conv_weight, bw, "conv_weight"},
                        {fe.conv_bias, fe.conv_bias ? bd : 0, "conv_bias"},
                        {fe.delta_bias, fe.delta_bias ? bd : 0, "delta_bias"}};
    const Span outs[] = {{state, bs, "state"}, {y_t, bx, "y_t"}, {conv_state, bcs, "conv_state"}};
    const Span req[] = {ins[0], ins[1], ins[2], ins[3], ins[4], outs[0], outs[1], ins[6], outs[2]};
    int rc = check_ptrs(req, fused ? 9 : 7);
    if (rc) return rc;
    rc = check_alias(outs, 3, ins, 9);
    if (rc) return rc;
    if (batch == 0 || dim == 0) return SSCAN_OK;
    if (sscan::step_work_items(batch, dim, dstate, fused) > sscan::kMaxWorkItems)
        return fail(SSCAN_ERR_UNSUPPORTED, "batch * dim too large for one decode-step launch");
    sscan::StepArgs a{state, x_t, delta_t, A, B_t, C_t, Dskip, y_t, batch, dim, int(dstate), io_dtype};
    if (fused) {
        a.fe = {fe.conv_weight, fe.conv_bias, fe.delta_bias, conv_state, fe.d_conv, fe.activation};
        a.conv_state = conv_state;
    }
    const hipError_t e = sscan::launch_step(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSCAN_OK : fail_hip("step launch", e);
}

int sscan_step_fused(float *state, void *conv_state, const void *x_t, const float *conv_weight,
                     const float *conv_bias, int d_conv, int activation, const void *delta_raw_t,
                     const float *delta_bias, const float *A, const void *B_t, const void *C_t,
                     const float *Dskip, void *y_t, int64_t batch, int64_t dim, int64_t dstate,
                     int io_dtype, void *stream) {
    g_last_error[0] = '\0';
    if (d_conv < 1) return fail(SSCAN_ERR_UNSUPPORTED, "d_conv must be in 1..4");
    FrontEnd fe;
    fe.conv_weight = conv_weight;
    fe.conv_bias = conv_bias;
    fe.delta_bias = delta_bias;
    fe.d_conv = d_conv;
    fe.activation = activation;
    return step_impl(state, x_t, delta_raw_t, A, B_t, C_t, Dskip, y_t, batch, dim, dstate, io_dtype, stream,
                     fe, conv_state);
}

int sscan_step(float *state, const void *x_t, const void *delta_t, const float *A,
               const void *B_t, const void *C_t, const float *Dskip, void *y_t, int64_t batch,
               int64_t dim, int64_t dstate, int io_dtype, void *stream) {
    return step_impl(state, x_t, delta_t, A, B_t, C_t, Dskip, y_t, batch, dim, dstate, io_dtype, stream,
                     FrontEnd(), nullptr);
}

}  // extern "C"
