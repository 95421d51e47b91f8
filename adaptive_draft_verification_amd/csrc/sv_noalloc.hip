// sv_verify_noalloc: sv_verify for callers that cannot allocate device memory
// (work recorded under HIP graph capture, serving loops and harnesses that
// forbid allocation).  The per-part statistics that pass 1 hands to pass 2
// live in a static device array instead of a caller's workspace; the kernels
// are sv_verify's own, given that array's device address as their workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "libspecverify.h"
#include "sv_launch.h"

namespace {

// The workspace of sv_verify_noalloc.  The HIP runtime holds one copy per GPU
// (each at its own device address) from the code object's load until the
// process ends.  In host code `scratch` is a host-side stand-in, not a device
// address: kernels only ever receive the address that hipGetSymbolAddress
// returned for the GPU in question.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_WS_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // per device: its copy of scratch, once looked up

// Device address of `dev`'s copy of scratch, looked up once per device with
// that device current (the caller's current device is restored).
hipError_t scratch_address(int dev, void** out) {
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" sv_status sv_verify_noalloc(const void* target_logits, int64_t target_ld,
                                       int64_t target_rows, const void* draft_logits,
                                       int64_t draft_ld, sv_dtype dtype, int32_t vocab,
                                       const int32_t* draft_tokens, const int32_t* cu_rows,
                                       int32_t n_req, int32_t k_max, sv_mode mode,
                                       float temperature, uint64_t seed, uint64_t step,
                                       int32_t* out_tokens, int32_t* out_accepted,
                                       float* out_p_draft, float* out_q_draft,
                                       float* out_residual_mass, float* out_q_entropy,
                                       float* out_q_max, int32_t* dev_error, void* stream) {
    sv::VerifyArgs a{target_logits, target_ld,    target_rows,  draft_logits, draft_ld,
                     dtype,         vocab,        draft_tokens, cu_rows,      n_req,
                     k_max,         mode,         temperature,  seed,         step,
                     out_tokens,    out_accepted, out_p_draft,  out_q_draft,
                     out_residual_mass, out_q_entropy, out_q_max, dev_error,  nullptr,
                     3};
    const sv_status st = sv::check_verify(a);
    if (st != SV_OK || n_req == 0) return st;
    // every part record pass 2 reads is written by pass 1 of the same call, so
    // nothing in the array needs clearing between calls
    if (sv::verify_workspace_bytes(n_req, k_max) > (size_t)SV_NOALLOC_WS_BYTES)
        return SV_ERR_CAPACITY;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    const hipError_t e = s != nullptr ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_LAUNCH;
    if (scratch_address(dev, &a.ws) != hipSuccess) return SV_ERR_LAUNCH;
    return sv::finish_launch(sv::launch_verify(a, s), s);
}
