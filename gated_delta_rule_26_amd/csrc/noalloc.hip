// gdr_chunk_fwd for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the chunked pass with its workspace in a fixed, file-scope device array
// instead of a caller-provided buffer.  Same kernels, same arithmetic, same
// validation as gdr_chunk_fwd.
//
// The array lives in the library's code object, so every GPU the library runs
// on holds GDR_NOALLOC_SCRATCH_BYTES of it until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in, not a device address): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
#include <mutex>

#include "gdr_internal.h"

namespace {

static_assert(GDR_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch size keeps the 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of the scratch array on the calling thread's current
// device (looked up on the first call on that device).
int scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GDR_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GDR_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDR_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GDR_OK;
}

}  // namespace

extern "C" int gdr_chunk_fwd_noalloc(const gdr_desc *desc, const void *q, const void *k, const void *v,
                                     const float *g, const float *beta_or_eta, const float *s0, void *o,
                                     float *s_final, void *stream) {
    // the size check first: a call that cannot fit fails before any HIP call
    size_t need = 0;
    int rc = gdr_chunk_fwd_workspace_size(desc, &need);
    if (rc != GDR_OK) return rc;
    if (need > GDR_NOALLOC_SCRATCH_BYTES) return GDR_E_WORKSPACE;
    void *ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc != GDR_OK) return rc;
    return gdr_chunk_fwd(desc, q, k, v, g, beta_or_eta, s0, o, s_final, ws, GDR_NOALLOC_SCRATCH_BYTES, stream);
}
