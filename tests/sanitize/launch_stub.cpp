// Launch stubs for the host-only sanitizer build of libgdn's C ABI
// (gdn_host.cpp under AddressSanitizer and UndefinedBehaviorSanitizer, no
// GPU). Instead of launching kernels they check what the host code hands
// them: every workspace region lies inside the caller's workspace, and the
// unit map is consistent with the descriptor. Any violation aborts.
#include <stdio.h>
#include <stdlib.h>

#include "gdn_internal.h"

namespace {
const char* g_lo = nullptr;
const char* g_hi = nullptr;

void fail(const char* what) {
    fprintf(stderr, "launch stub: %s\n", what);
    abort();
}

void region(const void* p, int64_t bytes, const char* what) {
    if (p == nullptr) return;
    const char* c = static_cast<const char*>(p);
    if (g_lo == nullptr || c < g_lo || bytes < 0 || c + bytes > g_hi) fail(what);
    if (reinterpret_cast<uintptr_t>(c) % 256 != 0) fail(what);
}

void check_problem(const gdn::Problem& p, const gdn::Workspace& ws) {
    const int64_t nch = int64_t(p.um.n_chunks) * p.H;
    const int64_t es = p.dtype == 1 ? 2 : 4;
    if (p.H < 1 || p.um.n_units < 0 || p.um.n_chunks < 0) fail("problem");
    region(ws.Tm, nch * 64 * 64 * es, "T region");
    region(ws.P, nch * 64 * 64 * es, "P region");
    region(ws.gam, nch * gdn::GAMR * 64 * 4, "gate rows");
    region(ws.qg, nch * 64 * 128 * es, "q b^G region");
    region(ws.kd, nch * 64 * 128 * es, "k b^G region");
    region(ws.kg, nch * 64 * 128 * es, "k b^(G_L - G) region");
    region(ws.gamL, nch * 128 * 4, "G_L region");
    region(ws.cfh, nch * 1024, "coefficient blocks");
    region(ws.order, int64_t(p.um.n_units) * 4, "unit order");
    if (p.um.dense && int64_t(p.um.n_chunks) != int64_t(p.um.n_units) * p.um.nt_dense) fail("dense chunk count");
}
}  // namespace

// The stream and event calls of the pieced forward: fake handles, success.
extern "C" {
hipError_t hipGetDevice(int* device) {
    *device = 0;
    return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* stream, unsigned int) {
    static int fake_stream;
    *stream = reinterpret_cast<hipStream_t>(&fake_stream);
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned int) {
    static int fake_events[16];
    static int n = 0;
    *event = reinterpret_cast<hipEvent_t>(&fake_events[n++ % 16]);
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
    *device = 0;
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* status) {
    *status = hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t event, hipStream_t) { return event ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t event, unsigned int) {
    return event ? hipSuccess : hipErrorInvalidValue;   // the null stream is the default stream
}
}

void stub_set_workspace(const void* base, size_t bytes) {
    g_lo = static_cast<const char*>(base);
    g_hi = g_lo + bytes;
}

namespace gdn {

hipError_t launch_prep(const Problem& p, const Workspace& ws, const void* k, const void*, const float* g,
                       const void* beta, const PrepSlots&, hipStream_t, bool) {
    check_problem(p, ws);
    if (p.um.total_tokens > 0 && (!k || !g || !beta)) fail("prep inputs");
    return hipSuccess;
}

hipError_t launch_state(const Problem& p, const Workspace& ws, const void*, const void* k, const void*,
                        const void*, const float*, void*, float*, float*, float*, int summary, int want_ext, int want_M,
                        float* S_ext, float* M, const int32_t* units_sel, int n_sel, hipStream_t) {
    check_problem(p, ws);
    if (p.um.total_tokens > 0 && !k) fail("state inputs");
    if (summary && ((want_ext && !S_ext) || (want_M && !M))) fail("summary outputs");
    if (units_sel && (!summary || n_sel < 1 || n_sel > p.um.n_units)) fail("unit selection");
    return hipSuccess;
}

hipError_t launch_merge_adjoint(int B, int H, int n_seg, const float* dS_ext, const float* M, const float*,
                                float* dS_exit, float*, hipStream_t) {
    if (B < 1 || H < 1 || n_seg < 0) fail("adjoint merge sizes");
    if (n_seg > 0 && (!dS_ext || !M || !dS_exit)) fail("adjoint merge buffers");
    return hipSuccess;
}

hipError_t launch_merge_pieces(int n_pieces, int n_docs, int H, const int32_t* piece_doc, const float* S_ext,
                               const float* M, const float*, float* S_in, hipStream_t) {
    if (n_pieces < 0 || n_docs < 1 || H < 1) fail("piece merge sizes");
    if (n_pieces > 0 && (!piece_doc || !S_ext || !M || !S_in)) fail("piece merge buffers");
    return hipSuccess;
}

hipError_t launch_merge(int B, int H, int n_seg, const float* S_ext, const float* M, const float*, float* S_init,
                        float*, hipStream_t) {
    if (B < 1 || H < 1 || n_seg < 0) fail("merge sizes");
    if (n_seg > 0 && (!S_ext || !M || !S_init)) fail("merge buffers");
    return hipSuccess;
}

hipError_t launch_prep_bwd(const Problem& p, const Workspace& ws, const void* k, const void*, const float* g,
                           const void* beta, hipStream_t) {
    check_problem(p, ws);
    if (p.um.total_tokens > 0 && (!k || !g || !beta)) fail("backward prep inputs");
    return hipSuccess;
}

hipError_t launch_bwd(const Problem& p, const Workspace& ws, float* dH, float* dVN, const void* q, const void* k,
                      const void* v, const float* g, const void* beta, const float* h, const void* dout,
                      const float*, float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0, bool dh_only,
                      bool, hipStream_t) {
    gdn::Problem pf = p;
    pf.dtype = 0;                  // the backward's preparation: the fp32 workspace layout
    check_problem(pf, ws);
    const int64_t nch = int64_t(p.um.n_chunks) * p.H;
    region(dH, nch * 128 * 128 * 4, "dH region");
    if (p.per_key) region(dVN, nch * 128 * 128 * 4, "per-key chunk maps A");
    else region(dVN, nch * 64 * 128 * 4, "dvn region");
    if (static_cast<const char*>(static_cast<void*>(dVN)) < static_cast<const char*>(static_cast<void*>(dH)) + nch * 128 * 128 * 4)
        fail("dH and dvn overlap");
    if (p.um.total_tokens > 0 && (!q || !k || !v || !g || !beta || !h || !dout))
        fail("backward inputs");
    if (p.um.total_tokens > 0 && !dh_only && (!dq || !dk || !dv || !dg || !dbeta)) fail("backward pointers");
    if (dh_only && !dh0) fail("gradient summary output");
    return hipSuccess;
}

}  // namespace gdn
