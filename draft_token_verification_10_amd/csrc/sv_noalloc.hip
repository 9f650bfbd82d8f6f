// sv_noalloc.hip -- stochastic verification for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid hipMalloc): the same call as sv_verify_stochastic, its
// workspace taken from a fixed buffer that the library itself holds on each
// GPU instead of from the caller.
//
// The buffer is a file-scope __device__ array.  Its name is only a host-side
// stand-in for the symbol: host code never passes it to a kernel or a copy.
// On the first call on a device the library asks the runtime for the
// array's address on that device (hipGetSymbolAddress, with the stream's
// device current) and keeps it; every later call on that device passes the
// kept pointer as the workspace.  Nothing is allocated and nothing needs
// clearing: the verification kernels write every workspace word they read
// within the call.  Each GPU keeps its own copy until the process ends;
// calls that overlap in time on one GPU share it and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "specverify.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SV_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

// The device `stream` runs on (the current device for the null stream).
hipError_t stream_device(void* stream, int* dev) {
    if (!stream) return hipGetDevice(dev);
    hipDevice_t d = 0;
    const hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &d);
    *dev = static_cast<int>(d);
    return e;
}

// Device address of `scratch` on device `dev`, looked up once per device.
int scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    DeviceScratch& s = g_scratch[dev];
    std::call_once(s.once, [&s, dev] {
        int cur = -1;
        s.err = hipGetDevice(&cur);
        if (s.err != hipSuccess) return;
        if (cur != dev && (s.err = hipSetDevice(dev)) != hipSuccess) return;
        void* p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        s.ptr = p;
        if (cur != dev) {
            const hipError_t e = hipSetDevice(cur);
            if (s.err == hipSuccess) s.err = e;
        }
    });
    if (s.err != hipSuccess || !s.ptr) return SV_ERR_HIP;
    *out = s.ptr;
    return SV_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" int sv_verify_stochastic_noalloc(const void* target_logits, const void* draft_logits,
                                            const int32_t* draft_tokens, const float* u_accept,
                                            const float* u_sample, int B, int k, int V,
                                            int64_t row_stride, int dtype, float temperature,
                                            int32_t* accept_len, int32_t* tokens,
                                            float* dbg_px_qx, void* stream) {
    // sv_workspace_bytes() is 0 for shapes the call itself refuses, which
    // then fail their own checks below with nothing touched.
    const size_t need = B > 0 ? sv_workspace_bytes(B, 1, k, V) : 0;
    if (need > (size_t)SV_SCRATCH_BYTES) return SV_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        int dev = -1;
        if (stream_device(stream, &dev) != hipSuccess) return SV_ERR_HIP;
        const int st = scratch_on(dev, &ws);
        if (st != SV_OK) return st;
    }
    return sv_verify_stochastic(target_logits, draft_logits, draft_tokens, u_accept, u_sample, B,
                                k, V, row_stride, dtype, temperature, accept_len, tokens,
                                dbg_px_qx, ws, need, stream);
}
#pragma GCC visibility pop
