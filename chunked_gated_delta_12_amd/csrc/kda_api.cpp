// kda_api.cpp -- the C ABI of libkda (declared in include/kda.h).
//
// Every entry point validates all of its arguments on the host first (sizes,
// dtype, NULL pointers, 16-byte alignment, overlaps, workspace size) and only
// then touches HIP, so a rejected call enqueues nothing.  Problems are
// reported as kda_status codes plus a thread-local message.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "kda.h"
#include "kda_launch.hpp"

// Device scratch of kda_chunk_fwd_noalloc: the workspace of a segmented
// prefill (segment maps, segment start states, every chunk's T') for callers
// that cannot allocate.  Each device holds its own copy from the first call on
// it until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: kernels and copies get the per-device
// address that hipGetSymbolAddress returns (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device addresses of `scratch`, one per device, resolved once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return KDA_OK;
}

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Range {
    const char* name;
    uintptr_t lo, hi;   // [lo, hi); empty when the pointer is NULL
};

Range rng(const char* name, const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{name, a, p ? a + bytes : a};
}

bool overlap(const Range& a, const Range& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Product of sizes must stay far inside int64 for the kernels' index math.
bool sizes_fit(int64_t a, int64_t b, int64_t c, int64_t d) {
    const double x = (double)a * (double)b * (double)c * (double)d;
    return x < 4.0e18;
}

// The size limits every entry point and size query applies (after check_common).
int check_sizes(int B, int T, int H, int dk) {
    if (T < 1) return fail(KDA_ERR_SHAPE, "T=%d must be >= 1", T);
    if (!sizes_fit(B, T, H, dk)) return fail(KDA_ERR_SHAPE, "B*T*H*d too large");
    // a chunk of one fp32 [B, T, H, d] tensor, 16*H*d*4 bytes, is addressed with
    // 32-bit offsets
    if ((int64_t)H * dk * KDA_CHUNK * 4 >= (1LL << 32))
        return fail(KDA_ERR_SHAPE, "H*d=%lld too large (64*H*d must stay below 2^32)", (long long)H * dk);
    return KDA_OK;
}

int check_common(int dtype, int B, int H, int dk, int dv) {
    if (dtype != KDA_BF16 && dtype != KDA_F32) return fail(KDA_ERR_DTYPE, "unknown dtype %d", dtype);
    if (B < 1 || H < 1) return fail(KDA_ERR_SHAPE, "B=%d H=%d must be >= 1", B, H);
    if (!supported_d(dk) || dk != dv)
        return fail(KDA_ERR_SHAPE, "dk=%d dv=%d: need dk == dv in {16, 32, 64, 128}", dk, dv);
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "unsupported or inconsistent sizes";
        case KDA_ERR_DTYPE: return "unknown dtype";
        case KDA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_ALIAS: return "output overlaps an input";
        case KDA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* kda_last_error(void) { return g_last_error; }

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int kda_chunk_fwd_auto_segments(int B, int T, int H, int dk, int dv) {
    if (B < 1 || T < 1 || H < 1 || !supported_d(dk) || dk != dv) return 0;
    if (check_sizes(B, T, H, dk) != KDA_OK) return 0;
    // The map and output passes run one workgroup per compute unit: aim for one
    // resident round of 256 workgroups (every head of a run of segments at once;
    // at least two segments below 512 sequences, where the single-segment kernel,
    // two workgroups per compute unit, would leave the chip half empty), keeping
    // every segment at least 16 chunks long.
    const int64_t bh = (int64_t)B * H;
    const int64_t nchunks = ((int64_t)T + KDA_CHUNK - 1) / KDA_CHUNK;
    if (bh >= 512) return 1;
    int64_t want = (256 + bh - 1) / bh;
    if (want < 2) want = 2;
    int64_t cap = nchunks / 16;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    return (int)kda::plan_segments(T, (int)want).nseg;
}

int kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int segments, size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_NULL, "bytes is NULL");
    int st = check_common(KDA_BF16, B, H, dk, dv);
    if (st) return st;
    if ((st = check_sizes(B, T, H, dk))) return st;
    const int nchunks = (int)(((int64_t)T + KDA_CHUNK - 1) / KDA_CHUNK);
    if (segments < 0 || segments > nchunks)
        return fail(KDA_ERR_SHAPE, "segments=%d outside [0, %d]", segments, nchunks);
    const int req = segments ? segments : kda_chunk_fwd_auto_segments(B, T, H, dk, dv);
    const kda::SegPlan p = kda::plan_segments(T, req);
    *bytes = kda::chunk_workspace_bytes(B, H, dk, dv, p.nseg, p.nchunks);
    return ok();
}

// The address of `scratch` on the calling thread's current device (resolved
// with that device current on its first use there).
static int scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_HIP, "device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

// kda_chunk_fwd, kda_chunk_fwd_gated, kda_chunk_fwd_unbounded and
// kda_chunk_fwd_noalloc; z (the output gate's pre-activation) is NULL but for
// the gated call.  noalloc: the workspace is the current device's static
// scratch instead of the caller's (workspace is then NULL and workspace_bytes 0).
static int chunk_fwd_impl(int dtype, int B, int T, int H, int dk, int dv, int segments, const void* q,
                          const void* k, const void* v, const float* theta, const float* beta,
                          const float* S0, const void* z, void* o, float* S_T, void* workspace,
                          size_t workspace_bytes, void* stream, bool unbounded = false,
                          bool noalloc = false) {
    int st = check_common(dtype, B, H, dk, dv);
    if (st) return st;
    if ((st = check_sizes(B, T, H, dk))) return st;
    const int nchunks = (int)(((int64_t)T + KDA_CHUNK - 1) / KDA_CHUNK);
    if (segments < 0 || segments > nchunks)
        return fail(KDA_ERR_SHAPE, "segments=%d outside [0, %d]", segments, nchunks);
    if (!q || !k || !v || !theta || !beta || !o)
        return fail(KDA_ERR_NULL, "q, k, v, theta, beta and o must be non-NULL");
    const void* all[] = {q, k, v, theta, beta, S0, o, S_T, workspace, z};
    const char* names[] = {"q", "k", "v", "theta", "beta", "S0", "o", "S_T", "workspace", "z"};
    for (int i = 0; i < 10; ++i)
        if (all[i] && !aligned16(all[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);

    const int req = segments ? segments : kda_chunk_fwd_auto_segments(B, T, H, dk, dv);
    const kda::SegPlan plan = kda::plan_segments(T, req);
    const size_t need = kda::chunk_workspace_bytes(B, H, dk, dv, plan.nseg, plan.nchunks);
    if (noalloc) {
        if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
            return fail(KDA_ERR_WORKSPACE,
                        "%d segments need %zu bytes of scratch, more than the static %zu; pass fewer "
                        "segments (1 needs none) or call kda_chunk_fwd with a workspace",
                        plan.nseg, need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need,
                    workspace_bytes, workspace ? "" : " (NULL)");
    }

    const size_t es = dtype == KDA_BF16 ? 2 : 4;
    const size_t tok = (size_t)B * T * H;
    const size_t st_bytes = (size_t)B * H * dk * dv * 4;
    const Range in[] = {rng("q", q, tok * dk * es), rng("k", k, tok * dk * es), rng("v", v, tok * dv * es),
                        rng("theta", theta, tok * dk * 4), rng("beta", beta, tok * 4),
                        rng("S0", S0, S0 ? st_bytes : 0), rng("z", z, z ? tok * dv * es : 0)};
    const Range r_o = rng("o", o, tok * dv * es);
    const Range r_st = rng("S_T", S_T, S_T ? st_bytes : 0);
    const Range r_ws = rng("workspace", workspace, need);
    for (const Range& x : in) {
        if (overlap(r_o, x)) return fail(KDA_ERR_ALIAS, "o overlaps %s", x.name);
        if (overlap(r_ws, x)) return fail(KDA_ERR_ALIAS, "workspace overlaps %s", x.name);
        if (overlap(r_st, x) && !(x.name[0] == 'S' && (const void*)S0 == (const void*)S_T))
            return fail(KDA_ERR_ALIAS, "S_T overlaps %s (only S_T == S0 is allowed)", x.name);
    }
    if (overlap(r_o, r_st)) return fail(KDA_ERR_ALIAS, "o overlaps S_T");
    if (overlap(r_o, r_ws)) return fail(KDA_ERR_ALIAS, "o overlaps workspace");
    if (overlap(r_st, r_ws)) return fail(KDA_ERR_ALIAS, "S_T overlaps workspace");

    if (noalloc && need > 0) {   // every argument check is done: now the first HIP call
        st = scratch_on_current_device(&workspace);
        if (st) return st;
    }
    hipError_t e = kda::launch_chunk_fwd(dtype == KDA_F32, B, T, H, dk, plan, q, k, v, theta, beta, S0,
                                         z, o, S_T, need ? workspace : nullptr,
                                         reinterpret_cast<hipStream_t>(stream), unbounded);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int kda_chunk_fwd(int dtype, int B, int T, int H, int dk, int dv, int segments, const void* q,
                  const void* k, const void* v, const float* theta, const float* beta,
                  const float* S0, void* o, float* S_T, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return chunk_fwd_impl(dtype, B, T, H, dk, dv, segments, q, k, v, theta, beta, S0, nullptr, o, S_T,
                          workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_noalloc(int dtype, int B, int T, int H, int dk, int dv, int segments, const void* q,
                          const void* k, const void* v, const float* theta, const float* beta,
                          const float* S0, void* o, float* S_T, void* stream) {
    return chunk_fwd_impl(dtype, B, T, H, dk, dv, segments, q, k, v, theta, beta, S0, nullptr, o, S_T,
                          nullptr, 0, stream, false, true);
}

int kda_chunk_fwd_gated(int dtype, int B, int T, int H, int dk, int dv, int segments, const void* q,
                        const void* k, const void* v, const float* theta, const float* beta,
                        const float* S0, const void* z, void* o, float* S_T, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (!z) return fail(KDA_ERR_NULL, "z must be non-NULL");
    return chunk_fwd_impl(dtype, B, T, H, dk, dv, segments, q, k, v, theta, beta, S0, z, o, S_T,
                          workspace, workspace_bytes, stream);
}

int kda_chunk_fwd_unbounded(int dtype, int B, int T, int H, int dk, int dv, const void* q, const void* k,
                            const void* v, const float* theta, const float* beta, const float* S0,
                            void* o, float* S_T, void* stream) {
    return chunk_fwd_impl(dtype, B, T, H, dk, dv, 1, q, k, v, theta, beta, S0, nullptr, o, S_T, nullptr, 0,
                          stream, true);
}

int kda_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_NULL, "bytes is NULL");
    int st = check_common(KDA_BF16, B, H, dk, dv);
    if (st) return st;
    if ((st = check_sizes(B, T, H, dk))) return st;
    *bytes = kda::chunk_bwd_workspace_bytes(B, T, H, dk);
    return ok();
}

int kda_chunk_bwd(int dtype, int B, int T, int H, int dk, int dv, const void* q, const void* k,
                  const void* v, const float* theta, const float* beta, const float* S0, const void* dout,
                  const float* dS_T, float* dq, float* dkk, float* dvv, float* dtheta, float* dbeta,
                  float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_common(dtype, B, H, dk, dv);
    if (st) return st;
    if ((st = check_sizes(B, T, H, dk))) return st;
    if (!q || !k || !v || !theta || !beta || !dout || !dq || !dkk || !dvv || !dtheta || !dbeta)
        return fail(KDA_ERR_NULL, "q, k, v, theta, beta, do and every gradient but dS0 must be non-NULL");
    const void* all[] = {q, k, v, theta, beta, S0, dout, dS_T, dq, dkk, dvv, dtheta, dbeta, dS0, workspace};
    const char* names[] = {"q", "k", "v", "theta", "beta", "S0", "do", "dS_T", "dq", "dk", "dv",
                           "dtheta", "dbeta", "dS0", "workspace"};
    for (int i = 0; i < 15; ++i)
        if (all[i] && !aligned16(all[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const size_t need = kda::chunk_bwd_workspace_bytes(B, T, H, dk);
    if (!workspace || workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    const size_t es = dtype == KDA_BF16 ? 2 : 4;
    const size_t tok = (size_t)B * T * H;
    const size_t st_bytes = (size_t)B * H * dk * dv * 4;
    const Range in[] = {rng("q", q, tok * dk * es), rng("k", k, tok * dk * es), rng("v", v, tok * dv * es),
                        rng("theta", theta, tok * dk * 4), rng("beta", beta, tok * 4),
                        rng("S0", S0, S0 ? st_bytes : 0), rng("do", dout, tok * dv * es),
                        rng("dS_T", dS_T, dS_T ? st_bytes : 0)};
    const Range out[] = {rng("dq", dq, tok * dk * 4), rng("dk", dkk, tok * dk * 4), rng("dv", dvv, tok * dv * 4),
                         rng("dtheta", dtheta, tok * dk * 4), rng("dbeta", dbeta, tok * 4),
                         rng("dS0", dS0, dS0 ? st_bytes : 0), rng("workspace", workspace, need)};
    for (const Range& o : out) {
        for (const Range& x : in)
            if (overlap(o, x)) return fail(KDA_ERR_ALIAS, "%s overlaps %s", o.name, x.name);
        for (const Range& o2 : out)
            if (&o2 != &o && overlap(o, o2)) return fail(KDA_ERR_ALIAS, "%s overlaps %s", o.name, o2.name);
    }
    hipError_t e = kda::launch_chunk_bwd(dtype == KDA_F32, B, T, H, dk, q, k, v, theta, beta, S0, dout, dS_T,
                                         dq, dkk, dvv, dtheta, dbeta, dS0, workspace,
                                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

// kda_decode_step and kda_decode_step_gated; z is NULL for the former.
static int decode_step_impl(int dtype, int B, int H, int dk, int dv, const void* q, const void* k,
                            const void* v, const float* theta, const float* beta, float* S,
                            const void* z, void* o, void* stream) {
    int st = check_common(dtype, B, H, dk, dv);
    if (st) return st;
    if (!sizes_fit(B, H, dk, dv) || (int64_t)B * H > 0x7fffffffLL)
        return fail(KDA_ERR_SHAPE, "B*H too large");
    if (!q || !k || !v || !theta || !beta || !S || !o)
        return fail(KDA_ERR_NULL, "q, k, v, theta, beta, S and o must be non-NULL");
    const void* all[] = {q, k, v, theta, beta, S, o, z};
    const char* names[] = {"q", "k", "v", "theta", "beta", "S", "o", "z"};
    for (int i = 0; i < 8; ++i)
        if (all[i] && !aligned16(all[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const size_t es = dtype == KDA_BF16 ? 2 : 4;
    const size_t bh = (size_t)B * H;
    const Range in[] = {rng("q", q, bh * dk * es), rng("k", k, bh * dk * es), rng("v", v, bh * dv * es),
                        rng("theta", theta, bh * dk * 4), rng("beta", beta, bh * 4),
                        rng("z", z, z ? bh * dv * es : 0)};
    const Range r_s = rng("S", S, bh * dk * dv * 4);
    const Range r_o = rng("o", o, bh * dv * es);
    for (const Range& x : in) {
        if (overlap(r_o, x)) return fail(KDA_ERR_ALIAS, "o overlaps %s", x.name);
        if (overlap(r_s, x)) return fail(KDA_ERR_ALIAS, "S overlaps %s", x.name);
    }
    if (overlap(r_o, r_s)) return fail(KDA_ERR_ALIAS, "o overlaps S");

    hipError_t e = kda::launch_decode(dtype == KDA_F32, B, H, dk, q, k, v, theta, beta, S, z, o,
                                      reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int kda_decode_step(int dtype, int B, int H, int dk, int dv, const void* q, const void* k,
                    const void* v, const float* theta, const float* beta, float* S, void* o,
                    void* stream) {
    return decode_step_impl(dtype, B, H, dk, dv, q, k, v, theta, beta, S, nullptr, o, stream);
}

int kda_decode_step_gated(int dtype, int B, int H, int dk, int dv, const void* q, const void* k,
                          const void* v, const float* theta, const float* beta, float* S,
                          const void* z, void* o, void* stream) {
    if (!z) return fail(KDA_ERR_NULL, "z must be non-NULL");
    return decode_step_impl(dtype, B, H, dk, dv, q, k, v, theta, beta, S, z, o, stream);
}

int kda_gate(int B, int T, int H, int dk, const float* theta, float* g, float* g_cum, void* stream) {
    if (B < 1 || T < 1 || H < 1) return fail(KDA_ERR_SHAPE, "B=%d T=%d H=%d must be >= 1", B, T, H);
    if (!supported_d(dk)) return fail(KDA_ERR_SHAPE, "dk=%d not in {16, 32, 64, 128}", dk);
    if (int st = check_sizes(B, T, H, dk)) return st;
    if (!theta) return fail(KDA_ERR_NULL, "theta is NULL");
    if (!g && !g_cum) return fail(KDA_ERR_NULL, "both g and g_cum are NULL");
    const void* all[] = {theta, g, g_cum};
    const char* names[] = {"theta", "g", "g_cum"};
    for (int i = 0; i < 3; ++i)
        if (all[i] && !aligned16(all[i])) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const size_t n = (size_t)B * T * H * dk * 4;
    const Range rt = rng("theta", theta, n), rg_ = rng("g", g, g ? n : 0), rc = rng("g_cum", g_cum, g_cum ? n : 0);
    if (overlap(rg_, rt) || overlap(rc, rt)) return fail(KDA_ERR_ALIAS, "g or g_cum overlaps theta");
    if (overlap(rg_, rc)) return fail(KDA_ERR_ALIAS, "g overlaps g_cum");

    hipError_t e = kda::launch_gate(B, T, H, dk, theta, g, g_cum, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
