// gdn_chunk_fwd_noalloc: the chunked prefill for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The workspace of gdn_chunk_fwd comes
// from a file-scope device array instead of the caller; every call on a GPU
// shares that GPU's copy of it, so calls that overlap on one GPU race.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on each device is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// handed to the kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_launch.h"
#include "gdn_validate.h"

namespace {

static_assert(GDN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size keeps the workspace alignment");

// The workspace of the no-allocation prefill, one copy per device for the
// life of the process.  Nothing in it has to start at zero: prep writes every
// intermediate the state kernel reads in the same call.
__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device.
gdn_status scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return gdn::fail(GDN_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return gdn::fail(GDN_ERR_NOT_SUPPORTED, "device %d is beyond the %d devices the no-allocation scratch tracks",
                         dev, kMaxDevices);
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return gdn::fail(GDN_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                             hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return GDN_SUCCESS;
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                           const float* g, const float* beta,
                                           const int32_t* cu_seqlens,
                                           const float* initial_state,
                                           float* out,
                                           float* final_state,
                                           const gdn_dims* dims,
                                           void* stream) {
    size_t need = 0;
    gdn_status s = gdn_chunk_fwd_min_workspace_size(dims, &need);
    if (s != GDN_SUCCESS) return s;
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
        return gdn::fail(GDN_ERR_WORKSPACE,
                         "gdn_chunk_fwd_noalloc: this batch needs %zu bytes of workspace, more than the %zu bytes "
                         "of the fixed scratch (use gdn_chunk_fwd with a caller workspace)",
                         need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    if (dims->n_seqs == 0) return gdn::ok();
    void* ws = nullptr;
    if ((s = scratch_on_current_device(&ws)) != GDN_SUCCESS) return s;
    return gdn::chunk_fwd_impl(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, nullptr, dims, ws,
                               (size_t)GDN_NOALLOC_SCRATCH_BYTES, 3, stream, "gdn_chunk_fwd_noalloc");
}
