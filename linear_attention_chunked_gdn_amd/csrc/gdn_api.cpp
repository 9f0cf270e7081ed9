// C-ABI entry points of the gated delta-rule library (declared in include/gdn.h):
// argument validation, launch planning and error reporting.  All compute runs in
// the HIP kernels of gdn_prefill.hip, gdn_prefill_pipe.hip, kda_map.hip, kda_chain.hip
// and gdn_decode.hip.
#include "gdn.h"
#include "gdn_launch.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

gdn_status ok() {
    g_last_error.clear();
    return GDN_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    const char *lo, *hi;
    const char *name;
};

Range range(const void *p, size_t bytes, const char *name) {
    const char *c = static_cast<const char *>(p);
    return Range{c, c ? c + bytes : c, name};
}

bool overlap(const Range &a, const Range &b) {
    if (!a.lo || !b.lo || a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

constexpr int kD = 128;
constexpr uint32_t kPrologueAll = GDN_PROLOGUE_QK_L2NORM | GDN_PROLOGUE_BETA_SIGMOID | GDN_PROLOGUE_G_SOFTPLUS;
constexpr int kChunk = 64;

// Kernel choice.  bf16 and fp16 I/O run the software-pipelined kernel (16 value
// channels per workgroup); fp32 I/O runs the phase-by-phase kernel with fp32 MFMAs.
// GDN_KERNEL=v1 selects the phase-by-phase kernel for bf16 too, and GDN_DVS=16|32 its
// slice width (for comparisons and tuning); fp16 I/O has only the pipelined kernel.
struct Plan {
    bool pipe;
    int dvs;
    int lds;
    int threads;
};

bool valid_dtype(gdn_dtype dt) { return dt == GDN_F32 || dt == GDN_BF16 || dt == GDN_F16; }

Plan choose_plan(gdn_dtype dt) {
    const char *kern = std::getenv("GDN_KERNEL");
    const bool force_v1 = kern && std::strcmp(kern, "v1") == 0;
    if (dt == GDN_F16 || (dt == GDN_BF16 && !force_v1))
        return Plan{true, 16, gdn::prefill_pipe_lds_bytes(), gdn::prefill_pipe_threads()};
    int dvs = 16;
    const char *env = std::getenv("GDN_DVS");
    if (env) {
        const int d = std::atoi(env);
        if (gdn::prefill_lds_bytes(dt == GDN_BF16, d) > 0) dvs = d;
    }
    return Plan{false, dvs, gdn::prefill_lds_bytes(dt == GDN_BF16, dvs), gdn::prefill_threads()};
}

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported";
        case GDN_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char *gdn_last_error(void) { return g_last_error.c_str(); }

gdn_status gdn_prefill_plan(int32_t N, int32_t Hv, int32_t Dv, gdn_dtype io_dtype,
                            int32_t *dv_per_workgroup, int32_t *workgroups, int32_t *lds_bytes,
                            int32_t *threads_per_workgroup) {
    if (!valid_dtype(io_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, "io_dtype %d is not GDN_F32, GDN_BF16 or GDN_F16", (int)io_dtype);
    if (N < 1 || Hv < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "N=%d and Hv=%d must be >= 1", N, Hv);
    if (Dv != kD) return fail(GDN_ERR_UNSUPPORTED, "Dv=%d (only 128 is implemented)", Dv);
    const Plan p = choose_plan(io_dtype);
    const long long wg = (long long)N * Hv * (kD / p.dvs);
    if (wg > 0x7fffffffLL) return fail(GDN_ERR_UNSUPPORTED, "%lld workgroups exceed the grid limit", wg);
    if (dv_per_workgroup) *dv_per_workgroup = p.dvs;
    if (workgroups) *workgroups = (int32_t)wg;
    if (lds_bytes) *lds_bytes = p.lds;
    if (threads_per_workgroup) *threads_per_workgroup = p.threads;
    return ok();
}

}  // extern "C"

namespace {

// Chunk lengths of the scalar-gate two-launch prefill.
bool split_chunk_ok(int32_t c) { return c == 32 || c == 64 || c == 128; }

size_t tile_bytes(int32_t c) {
    return c == 32 ? gdn::Tile<32>::BYTES : c == 128 ? gdn::Tile<128>::BYTES : gdn::Tile<64>::BYTES;
}

// GDN_CHECK set to anything but "" or "0" turns on the checks of device-resident
// arguments, which cost a device-to-host copy and a wait on the stream per call.
bool check_enabled() {
    const char *e = std::getenv("GDN_CHECK");
    return e && *e && std::strcmp(e, "0") != 0;
}

// cu_seqlens, read back after the work already queued on `stream` (which may write it),
// must be a packing of T_tot tokens: cu[0] = 0, nondecreasing, cu[N] = T_tot.  The kernels
// index q, k, v, o and the workspace with it unchecked.
gdn_status check_cu_seqlens(const int32_t *cu, int32_t N, int32_t T_tot, void *stream) {
    std::vector<int32_t> h((size_t)N + 1);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    if (e != hipSuccess)
        return fail(GDN_ERR_DEVICE, "GDN_CHECK: reading cu_seqlens back failed: %s", hipGetErrorString(e));
    if (h[0] != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_CHECK: cu_seqlens[0] = %d, not 0", h[0]);
    for (int32_t n = 0; n < N; ++n)
        if (h[n + 1] < h[n])
            return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_CHECK: cu_seqlens decreases at %d (%d, then %d)", n + 1,
                        h[n], h[n + 1]);
    if (h[N] != T_tot)
        return fail(GDN_ERR_INVALID_ARGUMENT, "GDN_CHECK: cu_seqlens[%d] = %d, not T_tot = %d", N, h[N], T_tot);
    return GDN_OK;
}

// Host-side checks shared by the prefill entry points (any_chunk: the chunk lengths of
// split_chunk_ok, else 64 only): g holds g_width values per
// (token, value head) (1, or Dk for a per-key-channel gate); ws / ws_bytes is the
// workspace (none for the scalar gate).
gdn_status check_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         const float *initial_state, const int32_t *cu_seqlens, int32_t N, int32_t T_tot,
                         int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, int32_t chunk_size, bool any_chunk,
                         gdn_dtype io_dtype, const void *o, const float *final_state, size_t g_width,
                         const void *ws, size_t ws_bytes, void *stream) {
    if (!valid_dtype(io_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, "io_dtype %d is not GDN_F32, GDN_BF16 or GDN_F16", (int)io_dtype);
    if (N < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "N=%d must be >= 1", N);
    if (T_tot < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "T_tot=%d must be >= 0", T_tot);
    if (Hk < 1 || Hv < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "Hk=%d, Hv=%d must be >= 1", Hk, Hv);
    if (Hv % Hk != 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "Hv=%d is not a multiple of Hk=%d", Hv, Hk);
    if (Dk != kD || Dv != kD)
        return fail(GDN_ERR_UNSUPPORTED, "Dk=%d, Dv=%d (only 128 is implemented)", Dk, Dv);
    if (any_chunk ? !split_chunk_ok(chunk_size) : chunk_size != kChunk)
        return fail(GDN_ERR_UNSUPPORTED, "chunk_size=%d (%s)", chunk_size,
                    any_chunk ? "32, 64 or 128 are implemented" : "only 64 is implemented");
    if (N > 1 && !cu_seqlens)
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens is required when N=%d > 1", N);
    if (T_tot > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(GDN_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and o must be non-null when T_tot > 0");
    const void *a16[] = {q, k, v, o, initial_state, final_state};
    const char *n16[] = {"q", "k", "v", "o", "initial_state", "final_state"};
    for (int i = 0; i < 6; ++i)
        if (!aligned(a16[i], 16))
            return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n16[i]);
    if (!aligned(g, g_width > 1 ? 16 : 4) || !aligned(beta, 4) || !aligned(cu_seqlens, 4))
        return fail(GDN_ERR_INVALID_ARGUMENT, "g must be %d-byte aligned, beta and cu_seqlens 4-byte",
                    g_width > 1 ? 16 : 4);

    const size_t es = io_dtype == GDN_F32 ? 4 : 2;
    const size_t T = (size_t)T_tot;
    const size_t state_bytes = (size_t)N * Hv * kD * kD * sizeof(float);
    const Range ro = range(o, T * Hv * kD * es, "o");
    const Range ins[] = {range(q, T * Hk * kD * es, "q"), range(k, T * Hk * kD * es, "k"),
                         range(v, T * Hv * kD * es, "v"), range(g, T * Hv * g_width * 4, "g"),
                         range(beta, T * Hv * 4, "beta"),
                         range(initial_state, state_bytes, "initial_state"),
                         range(cu_seqlens, (size_t)(N + 1) * 4, "cu_seqlens")};
    const Range rf = range(final_state, state_bytes, "final_state");
    const Range rw = range(ws, ws_bytes, "workspace");
    for (const Range &r : ins) {
        if (overlap(ro, r)) return fail(GDN_ERR_INVALID_ARGUMENT, "o overlaps %s", r.name);
        if (overlap(rf, r) && !(r.lo == reinterpret_cast<const char *>(initial_state) && rf.lo == r.lo))
            return fail(GDN_ERR_INVALID_ARGUMENT, "final_state overlaps %s", r.name);
        if (overlap(rw, r)) return fail(GDN_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    }
    if (overlap(ro, rf)) return fail(GDN_ERR_INVALID_ARGUMENT, "o overlaps final_state");
    if (overlap(rw, ro) || overlap(rw, rf))
        return fail(GDN_ERR_INVALID_ARGUMENT, "workspace overlaps an output");
    return check_enabled() && cu_seqlens ? check_cu_seqlens(cu_seqlens, N, T_tot, stream) : GDN_OK;
}

// The current device's compute units, 0 if they cannot be read.
int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

// Two 16-channel slices per chain workgroup (chunks of up to 64 tokens) when one slice per
// workgroup would need more than one round of workgroups on the device: half the
// workgroups, each about twice as long per chunk.  One slice otherwise (shorter chunks).
bool wide_chain(int32_t N, int32_t Hv, int32_t chunk) {
    const int cus = device_cus();
    return chunk <= 64 && cus > 0 && (long long)N * Hv * gdn::chain_workgroups_per_head(chunk, false) > cus;
}

// Chunk slots of the per-key-channel prefill: chunk j of sequence n uses slot
// cu[n] / 64 + n + j, and these never exceed T_tot / 64 + N.
size_t kda_slots(int32_t N, int32_t T_tot, int32_t C = kChunk) { return (size_t)T_tot / C + (size_t)N; }

}  // namespace

extern "C" {

gdn_status gdn_prefill(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                       int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                       int32_t chunk_size, gdn_dtype io_dtype, void *o, float *final_state,
                       void *stream) {
    const gdn_status cs = check_prefill(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk,
                                        Dv, chunk_size, false, io_dtype, o, final_state, 1, nullptr, 0, stream);
    if (cs != GDN_OK) return cs;

    int32_t dvs = 0, wg = 0;
    gdn_status ps = gdn_prefill_plan(N, Hv, Dv, io_dtype, &dvs, &wg, nullptr, nullptr);
    if (ps != GDN_OK) return ps;
    if (T_tot == 0 && !final_state) return ok();   // nothing to compute or write

    gdn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu = cu_seqlens; a.o = o; a.sN = final_state;
    a.N = N; a.T_tot = T_tot; a.Hk = Hk; a.Hv = Hv; a.nslices = kD / dvs;
    a.prologue = 0;
    const Plan p = choose_plan(io_dtype);
    (void)hipGetLastError();
    const hipError_t e = p.pipe ? gdn::launch_prefill_pipe(a, io_dtype == GDN_F16, wg,
                                                           static_cast<hipStream_t>(stream))
                                : gdn::launch_prefill(a, io_dtype == GDN_BF16, dvs, wg,
                                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(GDN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

gdn_status gdn_prefill_fused(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                             int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                             int32_t chunk_size, gdn_dtype io_dtype, uint32_t prologue, void *o,
                             float *final_state, void *stream) {
    const gdn_status cs = check_prefill(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk,
                                        Dv, chunk_size, false, io_dtype, o, final_state, 1, nullptr, 0, stream);
    if (cs != GDN_OK) return cs;
    if (prologue & ~kPrologueAll)
        return fail(GDN_ERR_INVALID_ARGUMENT, "prologue flags 0x%x include unknown bits", prologue);
    if (io_dtype == GDN_F32)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill_fused takes bf16 or fp16 q, k, v, o");
    int32_t dvs = 0, wg = 0;
    gdn_status ps = gdn_prefill_plan(N, Hv, Dv, io_dtype, &dvs, &wg, nullptr, nullptr);
    if (ps != GDN_OK) return ps;
    if (T_tot == 0 && !final_state) return ok();

    gdn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu = cu_seqlens; a.o = o; a.sN = final_state;
    a.N = N; a.T_tot = T_tot; a.Hk = Hk; a.Hv = Hv; a.nslices = kD / dvs;
    a.prologue = prologue;
    (void)hipGetLastError();
    const hipError_t e = gdn::launch_prefill_pipe_prologue(a, io_dtype == GDN_F16, wg,
                                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(GDN_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

gdn_status gdn_kda_workspace_size(int32_t N, int32_t T_tot, int32_t Hv, int32_t chunk_size, size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "bytes must be non-null");
    if (N < 1 || T_tot < 0 || Hv < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "N=%d, T_tot=%d, Hv=%d out of range", N, T_tot, Hv);
    if (chunk_size != kChunk)
        return fail(GDN_ERR_UNSUPPORTED, "chunk_size=%d (only 64 is implemented)", chunk_size);
    *bytes = kda_slots(N, T_tot) * (size_t)Hv * gdn::WS_TILE_BYTES;
    return ok();
}

gdn_status gdn_kda_prefill(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                           int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                           int32_t chunk_size, gdn_dtype io_dtype, void *workspace, size_t workspace_bytes,
                           void *o, float *final_state, void *stream) {
    const gdn_status cs = check_prefill(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk,
                                        Dv, chunk_size, false, io_dtype, o, final_state, kD, workspace,
                                        workspace_bytes, stream);
    if (cs != GDN_OK) return cs;
    if (io_dtype == GDN_F32)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_kda_prefill takes bf16 or fp16 q, k, v, o");
    size_t need = 0;
    gdn_kda_workspace_size(N, T_tot, Hv, chunk_size, &need);
    if (T_tot > 0 && (!workspace || workspace_bytes < need))
        return fail(GDN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu required",
                    workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if ((long long)kda_slots(N, T_tot) * Hv > 0x7fffffffLL || (long long)N * Hv * 8 + 64 > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "too many chunks or heads for one launch");
    if (T_tot == 0 && !final_state) return ok();

    gdn::KdaArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu = cu_seqlens; a.o = o; a.sN = final_state;
    a.ws = static_cast<char *>(workspace);
    a.N = N; a.T_tot = T_tot; a.Hk = Hk; a.Hv = Hv;
    a.nslots = (int32_t)kda_slots(N, T_tot);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool f16 = io_dtype == GDN_F16;
    (void)hipGetLastError();
    hipError_t e = T_tot > 0 ? gdn::launch_kda_map(a, f16, hs) : hipSuccess;
    if (e == hipSuccess) e = gdn::launch_kda_chain(a, f16, kChunk, true, wide_chain(N, Hv, kChunk), hs);
    if (e != hipSuccess)
        return fail(GDN_ERR_DEVICE, "kda prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

gdn_status gdn_prefill_split_workspace_size(int32_t N, int32_t T_tot, int32_t Hv, int32_t chunk_size,
                                            size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "bytes must be non-null");
    if (N < 1 || T_tot < 0 || Hv < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "N=%d, T_tot=%d, Hv=%d out of range", N, T_tot, Hv);
    if (!split_chunk_ok(chunk_size))
        return fail(GDN_ERR_UNSUPPORTED, "chunk_size=%d (32, 64 or 128 are implemented)", chunk_size);
    *bytes = kda_slots(N, T_tot, chunk_size) * (size_t)Hv * tile_bytes(chunk_size);
    return ok();
}

}  // extern "C"

namespace {

gdn_status split_impl(const void *q, const void *k, const void *v, const float *g, const float *beta,
                      const float *initial_state, const int32_t *cu_seqlens, int32_t N, int32_t T_tot, int32_t Hk,
                      int32_t Hv, int32_t Dk, int32_t Dv, int32_t chunk_size, gdn_dtype io_dtype,
                      uint32_t prologue, void *workspace, size_t workspace_bytes, void *o, float *final_state,
                      void *stream) {
    if (prologue & ~kPrologueAll)
        return fail(GDN_ERR_INVALID_ARGUMENT, "prologue flags 0x%x include unknown bits", prologue);
    const gdn_status cs = check_prefill(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk,
                                        Dv, chunk_size, true, io_dtype, o, final_state, 1, workspace,
                                        workspace_bytes, stream);
    if (cs != GDN_OK) return cs;
    if (io_dtype == GDN_F32)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill_split takes bf16 or fp16 q, k, v, o");
    size_t need = 0;
    gdn_prefill_split_workspace_size(N, T_tot, Hv, chunk_size, &need);
    if (T_tot > 0 && (!workspace || workspace_bytes < need))
        return fail(GDN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu required",
                    workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if ((long long)kda_slots(N, T_tot, chunk_size) * Hv > 0x7fffffffLL || (long long)N * Hv * 8 + 64 > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "too many chunks or heads for one launch");
    if (T_tot == 0 && !final_state) return ok();

    gdn::KdaArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu = cu_seqlens; a.o = o; a.sN = final_state;
    a.ws = static_cast<char *>(workspace);
    a.N = N; a.T_tot = T_tot; a.Hk = Hk; a.Hv = Hv;
    a.nslots = (int32_t)kda_slots(N, T_tot, chunk_size);
    a.prologue = prologue;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool f16 = io_dtype == GDN_F16;
    (void)hipGetLastError();
    hipError_t e = T_tot > 0 ? gdn::launch_gdn_map(a, f16, chunk_size, hs) : hipSuccess;
    if (e == hipSuccess) e = gdn::launch_kda_chain(a, f16, chunk_size, false, wide_chain(N, Hv, chunk_size), hs);
    if (e != hipSuccess)
        return fail(GDN_ERR_DEVICE, "split prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_split(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                             int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                             int32_t chunk_size, gdn_dtype io_dtype, void *workspace, size_t workspace_bytes,
                             void *o, float *final_state, void *stream) {
    return split_impl(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk, Dv, chunk_size, io_dtype, 0,
                      workspace, workspace_bytes, o, final_state, stream);
}

gdn_status gdn_prefill_split_fused(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                                   int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                   int32_t chunk_size, gdn_dtype io_dtype, uint32_t prologue, void *workspace,
                                   size_t workspace_bytes, void *o, float *final_state, void *stream) {
    return split_impl(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk, Dv, chunk_size, io_dtype,
                      prologue, workspace, workspace_bytes, o, final_state, stream);
}

}  // extern "C"

namespace {

// gdn_prefill_split_noalloc's workspace: a static array in the library's code object, so
// each GPU the library is loaded on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the kernels get the
// device address that hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.  The split kernels write every workspace byte they read, so the
// array needs no clearing between calls.
static __device__ __align__(256) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

gdn_status scratch_on_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GDN_ERR_UNSUPPORTED, "device %d: static scratch is tracked for devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GDN_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_split_noalloc(const void *q, const void *k, const void *v, const float *g,
                                     const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                                     int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                     int32_t chunk_size, gdn_dtype io_dtype, void *o, float *final_state,
                                     void *stream) {
    // every argument is checked before the device is touched
    gdn_status st = check_prefill(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk, Dv,
                                  chunk_size, true, io_dtype, o, final_state, 1, nullptr, 0, stream);
    if (st != GDN_OK) return st;
    if (io_dtype == GDN_F32)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill_split_noalloc takes bf16 or fp16 q, k, v, o");
    size_t need = 0;
    st = gdn_prefill_split_workspace_size(N, T_tot, Hv, chunk_size, &need);
    if (st != GDN_OK) return st;
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
        return fail(GDN_ERR_UNSUPPORTED,
                    "gdn_prefill_split_noalloc: N=%d, T_tot=%d, Hv=%d, chunk_size=%d need %zu workspace bytes, "
                    "more than the %zu of its static scratch (gdn_prefill_split takes a caller workspace)",
                    N, T_tot, Hv, chunk_size, need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    if (T_tot == 0 && !final_state) return ok();
    void *ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != GDN_OK) return st;
    return split_impl(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk, Dv, chunk_size, io_dtype, 0,
                      ws, (size_t)GDN_NOALLOC_SCRATCH_BYTES, o, final_state, stream);
}

// Segmented prefill: the split path's map, the chain in segments, the fix-up.
constexpr int32_t kMaxSegments = 256;

gdn_status gdn_prefill_seg_workspace_size(int32_t N, int32_t T_tot, int32_t Hv, int32_t chunk_size,
                                          int32_t segments, size_t *bytes) {
    if (segments < 1 || segments > kMaxSegments)
        return fail(GDN_ERR_INVALID_ARGUMENT, "segments=%d is outside 1..%d", segments, kMaxSegments);
    size_t tiles = 0;
    const gdn_status st = gdn_prefill_split_workspace_size(N, T_tot, Hv, chunk_size, &tiles);
    if (st != GDN_OK) return st;
    const size_t per_token = (size_t)Hv * kD * 2 * 2;   // o0 and e rows, fp16
    // fp32 end states (S and X^T) and fp16 start states per (sequence, head, segment)
    const size_t states = (size_t)N * Hv * segments * kD * kD * (2 * sizeof(float) + 2);
    *bytes = tiles + (size_t)T_tot * per_token + states;
    return ok();
}

gdn_status gdn_prefill_seg_choose(int32_t N, int32_t T_tot, int32_t Hv, int32_t chunk_size,
                                  int32_t *segments) {
    if (!segments) return fail(GDN_ERR_INVALID_ARGUMENT, "segments must be non-null");
    if (N < 1 || T_tot < 0 || Hv < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "N=%d, T_tot=%d, Hv=%d out of range", N, T_tot, Hv);
    if (!split_chunk_ok(chunk_size))
        return fail(GDN_ERR_UNSUPPORTED, "chunk_size=%d (32, 64 or 128 are implemented)", chunk_size);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(GDN_ERR_DEVICE, "cannot read the current device's compute-unit count");
    // one chain workgroup per compute unit: W (2K - 1) per (sequence, head) for K segments,
    // W the segmented chain's workgroups per head (two slices each up to 64-token chunks)
    const long long pairs = (long long)N * Hv, W = gdn::chain_workgroups_per_head(chunk_size, chunk_size <= 64);
    long long k = ((long long)cus / (W * pairs) + 1) / 2;
    // and at least 4 chunks per segment on average
    const long long chunks = (long long)T_tot / chunk_size / N;
    k = std::min(k, std::max(1LL, chunks / 4));
    *segments = (int32_t)std::max(1LL, std::min<long long>(k, kMaxSegments));
    return ok();
}

}  // extern "C"

namespace {

// The segmented prefill with the scalar gate (g [T_tot, Hv]) or a per-key-channel one
// (g [T_tot, Hv, Dk], 64-token chunks): the two differ only in the map kernel.
gdn_status seg_impl(const char *fn, bool per_channel, const void *q, const void *k, const void *v, const float *g,
                    const float *beta, const float *initial_state, const int32_t *cu_seqlens, int32_t N,
                    int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, int32_t chunk_size,
                    int32_t segments, gdn_dtype io_dtype, void *workspace, size_t workspace_bytes, void *o,
                    float *final_state, void *stream) {
    const gdn_status cs = check_prefill(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk,
                                        Dv, chunk_size, !per_channel, io_dtype, o, final_state,
                                        per_channel ? (size_t)kD : 1, workspace, workspace_bytes, stream);
    if (cs != GDN_OK) return cs;
    if (io_dtype == GDN_F32)
        return fail(GDN_ERR_UNSUPPORTED, "%s takes bf16 or fp16 q, k, v, o", fn);
    size_t need = 0;
    const gdn_status ws_st = gdn_prefill_seg_workspace_size(N, T_tot, Hv, chunk_size, segments, &need);
    if (ws_st != GDN_OK) return ws_st;
    if (T_tot > 0 && (!workspace || workspace_bytes < need))
        return fail(GDN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu required",
                    workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    const long long slots = (long long)kda_slots(N, T_tot, chunk_size);
    if ((slots + N) * Hv * 8 > 0x7fffffffLL || (long long)N * Hv * 16 * (segments + 8) > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "too many chunks, heads or segments for one launch");
    if (T_tot == 0 && !final_state) return ok();

    gdn::KdaArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu = cu_seqlens; a.o = o; a.sN = final_state;
    a.ws = static_cast<char *>(workspace);
    a.N = N; a.T_tot = T_tot; a.Hk = Hk; a.Hv = Hv;
    a.nslots = (int32_t)slots;
    a.nseg = segments;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool f16 = io_dtype == GDN_F16;
    (void)hipGetLastError();
    hipError_t e;
    if (T_tot == 0) {
        // no tokens: the final state is the initial state (the plain chain copies it)
        e = gdn::launch_kda_chain(a, f16, chunk_size, per_channel, chunk_size <= 64, hs);
    } else {
        size_t off = (size_t)slots * Hv * tile_bytes(chunk_size);
        a.o0 = reinterpret_cast<_Float16 *>(a.ws + off);
        off += (size_t)T_tot * Hv * kD * 2;
        a.e = reinterpret_cast<_Float16 *>(a.ws + off);
        off += (size_t)T_tot * Hv * kD * 2;
        a.sseg = reinterpret_cast<float *>(a.ws + off);
        off += (size_t)N * Hv * segments * 2 * kD * kD * sizeof(float);
        a.sin16 = reinterpret_cast<_Float16 *>(a.ws + off);
        e = per_channel ? gdn::launch_kda_map(a, f16, hs) : gdn::launch_gdn_map(a, f16, chunk_size, hs);
        if (e == hipSuccess) e = gdn::launch_seg_chain(a, f16, chunk_size, per_channel, chunk_size <= 64, hs);
        if (e == hipSuccess) e = gdn::launch_seg_join(a, hs);
        if (e == hipSuccess) e = gdn::launch_seg_fix(a, f16, chunk_size, hs);
    }
    if (e != hipSuccess)
        return fail(GDN_ERR_DEVICE, "segmented prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_seg(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                           int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                           int32_t chunk_size, int32_t segments, gdn_dtype io_dtype, void *workspace,
                           size_t workspace_bytes, void *o, float *final_state, void *stream) {
    return seg_impl("gdn_prefill_seg", false, q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk,
                    Dv, chunk_size, segments, io_dtype, workspace, workspace_bytes, o, final_state, stream);
}

gdn_status gdn_kda_prefill_seg(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                               int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                               int32_t chunk_size, int32_t segments, gdn_dtype io_dtype, void *workspace,
                               size_t workspace_bytes, void *o, float *final_state, void *stream) {
    return seg_impl("gdn_kda_prefill_seg", true, q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv,
                    Dk, Dv, chunk_size, segments, io_dtype, workspace, workspace_bytes, o, final_state, stream);
}

}  // extern "C"

namespace {

gdn_status decode_impl(const void *q, const void *k, const void *v, const float *g, const float *beta,
                       float *state, int32_t B, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                       gdn_dtype io_dtype, void *o, void *stream, bool per_channel, uint32_t prologue) {
    if (prologue & ~kPrologueAll)
        return fail(GDN_ERR_INVALID_ARGUMENT, "prologue flags 0x%x include unknown bits", prologue);
    if (!valid_dtype(io_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, "io_dtype %d is not GDN_F32, GDN_BF16 or GDN_F16", (int)io_dtype);
    if (B < 1 || Hk < 1 || Hv < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "B=%d, Hk=%d, Hv=%d must be >= 1", B, Hk, Hv);
    if (Hv % Hk != 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "Hv=%d is not a multiple of Hk=%d", Hv, Hk);
    if (Dk != kD || Dv != kD)
        return fail(GDN_ERR_UNSUPPORTED, "Dk=%d, Dv=%d (only 128 is implemented)", Dk, Dv);
    if (!q || !k || !v || !g || !beta || !state || !o)
        return fail(GDN_ERR_INVALID_ARGUMENT, "all tensor arguments of a decode step are required");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(state, 16) || !aligned(v, 4) || !aligned(o, 4) ||
        !aligned(g, per_channel ? 16 : 4) || !aligned(beta, 4))
        return fail(GDN_ERR_INVALID_ARGUMENT,
                    "q, k and state must be 16-byte aligned (and g for a per-channel gate), the rest 4-byte");
    if ((long long)B * Hv * (kD / 16) > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "B*Hv too large for one launch");
    const size_t es = io_dtype == GDN_F32 ? 4 : 2;
    const Range ro = range(o, (size_t)B * Hv * kD * es, "o");
    const Range rs = range(state, (size_t)B * Hv * kD * kD * 4, "state");
    const Range ins[] = {range(q, (size_t)B * Hk * kD * es, "q"), range(k, (size_t)B * Hk * kD * es, "k"),
                         range(v, (size_t)B * Hv * kD * es, "v"),
                         range(g, (size_t)B * Hv * (per_channel ? kD : 1) * 4, "g"),
                         range(beta, (size_t)B * Hv * 4, "beta")};
    for (const Range &r : ins) {
        if (overlap(ro, r)) return fail(GDN_ERR_INVALID_ARGUMENT, "o overlaps %s", r.name);
        if (overlap(rs, r)) return fail(GDN_ERR_INVALID_ARGUMENT, "state overlaps %s", r.name);
    }
    if (overlap(ro, rs)) return fail(GDN_ERR_INVALID_ARGUMENT, "o overlaps state");

    gdn::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
    a.B = B; a.Hk = Hk; a.Hv = Hv;
    a.prologue = prologue;
    (void)hipGetLastError();
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t e = per_channel ? gdn::launch_kda_decode(a, (int)io_dtype, hs)
                                     : gdn::launch_decode(a, (int)io_dtype, hs);
    if (e != hipSuccess)
        return fail(GDN_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, int32_t B, int32_t Hk, int32_t Hv,
                           int32_t Dk, int32_t Dv, gdn_dtype io_dtype, void *o, void *stream) {
    return decode_impl(q, k, v, g, beta, state, B, Hk, Hv, Dk, Dv, io_dtype, o, stream, false, 0);
}

gdn_status gdn_decode_step_fused(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, float *state, int32_t B, int32_t Hk, int32_t Hv,
                                 int32_t Dk, int32_t Dv, gdn_dtype io_dtype, uint32_t prologue, void *o,
                                 void *stream) {
    return decode_impl(q, k, v, g, beta, state, B, Hk, Hv, Dk, Dv, io_dtype, o, stream, false, prologue);
}

gdn_status gdn_kda_decode_step(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, float *state, int32_t B, int32_t Hk, int32_t Hv,
                               int32_t Dk, int32_t Dv, gdn_dtype io_dtype, void *o, void *stream) {
    return decode_impl(q, k, v, g, beta, state, B, Hk, Hv, Dk, Dv, io_dtype, o, stream, true, 0);
}

}  // extern "C"

namespace {

// The path gdn_prefill_auto takes.  fp32 I/O has only the one-launch path.  With 16-bit
// I/O the two-launch paths win whenever their chain kernel's workgroups (at most one per
// (sequence, head, 32 value channels)) fit the compute units in one round, and for packed
// batches of several sequences: the one-launch kernel's workgroups each redo the
// state-independent products of their chunks on their own critical path, while the
// two-launch map does them once, on the whole chip.  Among the two, the segmented one
// when gdn_prefill_seg_choose gives at least three segments (it has no prologue): its
// chain workgroups hold two slices and take about twice as long per chunk as the split
// path's one-slice workgroups, so two segments only break even.
struct AutoPlan {
    int32_t path, segments;
    size_t workspace;
};

gdn_status auto_plan(int32_t N, int32_t T_tot, int32_t Hv, gdn_dtype io_dtype, uint32_t prologue, AutoPlan *p) {
    if (!valid_dtype(io_dtype))
        return fail(GDN_ERR_INVALID_ARGUMENT, "io_dtype %d is not GDN_F32, GDN_BF16 or GDN_F16", (int)io_dtype);
    if (N < 1 || T_tot < 0 || Hv < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "N=%d, T_tot=%d, Hv=%d out of range", N, T_tot, Hv);
    if (prologue & ~kPrologueAll)
        return fail(GDN_ERR_INVALID_ARGUMENT, "prologue flags 0x%x include unknown bits", prologue);
    *p = AutoPlan{GDN_PATH_ONE_LAUNCH, 1, 0};
    if (io_dtype == GDN_F32) return GDN_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(GDN_ERR_DEVICE, "cannot read the current device's compute-unit count");
    if (!((long long)N * Hv * gdn::chain_workgroups_per_head(kChunk, true) <= cus || N > 1)) return GDN_OK;
    int32_t K = 1;
    if (!prologue) {
        const gdn_status st = gdn_prefill_seg_choose(N, T_tot, Hv, kChunk, &K);
        if (st != GDN_OK) return st;
    }
    if (K >= 3) {
        *p = AutoPlan{GDN_PATH_SEG, K, 0};
        return gdn_prefill_seg_workspace_size(N, T_tot, Hv, kChunk, K, &p->workspace);
    }
    *p = AutoPlan{GDN_PATH_SPLIT, 1, 0};
    return gdn_prefill_split_workspace_size(N, T_tot, Hv, kChunk, &p->workspace);
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_auto_plan(int32_t N, int32_t T_tot, int32_t Hv, gdn_dtype io_dtype, uint32_t prologue,
                                 int32_t *path, int32_t *segments, size_t *workspace_bytes) {
    if (!workspace_bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "workspace_bytes must be non-null");
    AutoPlan p{};
    const gdn_status st = auto_plan(N, T_tot, Hv, io_dtype, prologue, &p);
    if (st != GDN_OK) return st;
    if (path) *path = p.path;
    if (segments) *segments = p.segments;
    *workspace_bytes = p.workspace;
    return ok();
}

gdn_status gdn_prefill_auto(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                            int32_t N, int32_t T_tot, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                            gdn_dtype io_dtype, uint32_t prologue, void *workspace, size_t workspace_bytes,
                            void *o, float *final_state, void *stream) {
    AutoPlan p{};
    const gdn_status st = auto_plan(N, T_tot, Hv, io_dtype, prologue, &p);
    if (st != GDN_OK) return st;
    switch (p.path) {
        case GDN_PATH_SEG:
            return seg_impl("gdn_prefill_auto", false, q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk,
                            Hv, Dk, Dv, kChunk, p.segments, io_dtype, workspace, workspace_bytes, o, final_state,
                            stream);
        case GDN_PATH_SPLIT:
            return split_impl(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk, Dv, kChunk,
                              io_dtype, prologue, workspace, workspace_bytes, o, final_state, stream);
        default:
            return prologue ? gdn_prefill_fused(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk,
                                                Dv, kChunk, io_dtype, prologue, o, final_state, stream)
                            : gdn_prefill(q, k, v, g, beta, initial_state, cu_seqlens, N, T_tot, Hk, Hv, Dk, Dv,
                                          kChunk, io_dtype, o, final_state, stream);
    }
}

}  // extern "C"
