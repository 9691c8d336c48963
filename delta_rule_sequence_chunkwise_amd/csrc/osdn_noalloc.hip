// osdn_chunk_fwd_kda_noalloc: the channel-wise gate forward for callers that cannot allocate
// device memory (HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The bf16 path's workspace (gate-scaled q, k, k~, the chunk planes and G_C) lives in
// `scratch`, a file-scope device array of OSDN_NOALLOC_SCRATCH_BYTES that every GPU the library
// runs on holds until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory, so the kernels never receive it: on the first call on a device (that device
// current) its device address is looked up with hipGetSymbolAddress and kept per device, and
// the kernels take that address as they take a caller's workspace.  The size check runs before
// any HIP call.  Nothing here allocates or frees memory; calls on one GPU share its array, so
// overlapping calls race (the header says so).
#include <mutex>

#include "osdn_internal.h"

namespace {

constexpr int64_t kScratchBytes = OSDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device, looked up once per device
hipError_t scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" osdn_status osdn_chunk_fwd_kda_noalloc(const void *q, const void *k, const void *v,
                                                  const float *beta, const void *d,
                                                  const float *alpha_ch, const float *S0,
                                                  void *o, float *S_T, int64_t B, int64_t H,
                                                  int64_t T, int32_t dk, int32_t dv,
                                                  int32_t chunk, osdn_dtype qkv,
                                                  osdn_dtype d_dtype, void *stream) {
    const int64_t need = osdn_chunk_fwd_kda_workspace(B, H, T, dk, chunk, qkv);
    if (need > kScratchBytes) return OSDN_ERR_SCRATCH;
    void *ws = nullptr;
    // the scratch is only needed when the bf16 path runs over at least one token; an invalid
    // shape (need < 0) is reported by the call below with its own status
    if (need > 0 && B > 0 && H > 0 && T > 0) {
        if (scratch_on_current_device(&ws) != hipSuccess) return OSDN_ERR_LAUNCH;
    }
    return osdn_chunk_fwd_kda(q, k, v, beta, d, alpha_ch, S0, o, S_T, ws, ws ? kScratchBytes : 0,
                              B, H, T, dk, dv, chunk, qkv, d_dtype, stream);
}
