// gdn_chunk_fwd_noalloc: the chunked forward with the library's own scratch
// memory, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace of gdn_chunk_fwd (chunk preparation: T, P, the gated operand
// tiles, the coefficient blocks and the unit order) lives here in a file-scope
// device array. Each GPU holds its own copy from the first call on it until
// the process ends. The array's name is only a host-side stand-in: the device
// address is taken once per device with hipGetSymbolAddress and every launch
// gets that address, exactly as gdn_chunk_fwd gets a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

static_assert(GDN_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch size keeps 256-byte alignment");

__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];   // device address of scratch on every device set up so far

// The scratch address on the current device, looked up on the first call
// there. The stream must belong to the current device: the address is per
// device and the kernels run on the stream's device.
gdn_status scratch_for(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDN_ERR_DEVICE;
    if (dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GDN_ERR_DEVICE;
        if (sdev != dev) return GDN_ERR_INVALID;
    }
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GDN_ERR_DEVICE;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd_noalloc(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                            const float* g, const void* beta, const float* initial_state,
                                            void* o, float* final_state, const gdn_slots* slots, int32_t flags,
                                            hipStream_t stream) {
    // every check and the workspace size, with no HIP call
    gdn::Problem p;
    size_t need = 0;
    gdn_status st = gdn::fwd_preflight(desc, q, k, v, g, beta, o, flags, &p, &need);
    if (st != GDN_OK) return st;
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_CAPACITY;
    void* ws = nullptr;
    st = scratch_for(stream, &ws);
    if (st != GDN_OK) return st;
    size_t bytes = GDN_NOALLOC_SCRATCH_BYTES;
    return gdn::fwd_impl(desc, q, k, v, g, beta, initial_state, o, final_state, slots, flags, ws, &bytes, stream,
                         false);
}
