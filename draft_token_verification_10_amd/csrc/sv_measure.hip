// sv_measure.hip -- a plain streaming read of HBM, the practical ceiling the
// verification kernels are measured against (declared in sv_measure.h).
//
// Each 1024-thread workgroup reads one contiguous share of the buffer with
// 16-byte non-temporal buffer loads, four in flight per lane, exactly the
// access pattern of a sequence-resident verification workgroup streaming its
// rows; the only arithmetic is an XOR that keeps the loads alive, and each
// workgroup stores its own word (a shared atomic would serialise them).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "specverify.h"
#include "sv_measure.h"

namespace {

constexpr int NT = 1024;
constexpr int LOADS = 4;                     // 16-byte loads in flight per lane
constexpr int RSRC_WORD3 = 0x00020000;       // raw buffer resource, gfx9 class
constexpr int POLICY_NT = 2;                 // non-temporal, as the logit loads
constexpr long long kMaxShareBytes = 1LL << 31;

__global__ __launch_bounds__(NT) void k_stream_read(const char* src, long long n16,
                                                    long long share, uint32_t* out) {
    const long long begin = (long long)blockIdx.x * share;
    const long long end = begin + share < n16 ? begin + share : n16;
    const int cnt = (int)(end - begin);  // chunks of this share (host: < 2^27)
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src + begin * 16),
                                                      (short)0, cnt * 16, RSRC_WORD3);
    uint32_t x = 0;
    for (int i = threadIdx.x; i < cnt; i += NT * LOADS) {
        uint32_t w[LOADS][4];
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int c = i + u * NT;
            if (c < cnt) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, POLICY_NT);
                w[u][0] = v[0];
                w[u][1] = v[1];
                w[u][2] = v[2];
                w[u][3] = v[3];
            } else {
                w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < LOADS; ++u) x ^= w[u][0] ^ w[u][1] ^ w[u][2] ^ w[u][3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    __shared__ uint32_t wx[NT / 64];
    if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {  // one plain store per workgroup: no atomic contention
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) t ^= wx[w];
        out[blockIdx.x] = t;
    }
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" int sv_stream_read(const void* src, size_t bytes, int blocks, uint32_t* out,
                              void* stream) {
    if (bytes == 0) return SV_OK;
    if (!src || !out) return SV_ERR_NULL;
    if ((bytes % 16) != 0 || ((uintptr_t)src & 15u) != 0 || blocks < 1 || blocks > 65536)
        return SV_ERR_SHAPE;
    const long long n16 = (long long)(bytes / 16);
    const long long share = (n16 + blocks - 1) / blocks;
    if (share * 16 > kMaxShareBytes - 16) return SV_ERR_SHAPE;
    const long long grid = (n16 + share - 1) / share;  // no empty workgroups
    // The launch's own status (an earlier error of the caller is left alone).
    const char* s = static_cast<const char*>(src);
    void* args[] = {&s, const_cast<long long*>(&n16), const_cast<long long*>(&share), &out};
    return hipLaunchKernel(reinterpret_cast<const void*>(k_stream_read), dim3((unsigned)grid),
                           dim3(NT), args, 0, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SV_OK
               : SV_ERR_HIP;
}
#pragma GCC visibility pop
