// Optional input checking: while the environment variable VQ_CHECK is "1"
// (read at every call), every entry point counts the non-finite values
// (and, for the weight arrays h, hcol and rho, the values with the sign bit
// set) of its floating-point inputs on the device before its own launches,
// and returns VQ_ERR_INVALID naming the array when any is found.  Off by
// default: the arithmetic assumes finite inputs and non-negative weights, and
// the check costs one read of every input plus a synchronization.
#include "vq_internal.h"

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace vq {
namespace {

// One counter per device for the check's result (the device copy lives until
// the process ends; its address is fetched per device before first use).
__device__ __align__(256) unsigned long long g_bad;

__global__ __launch_bounds__(256) void k_zero_u64(unsigned long long* p) { if (threadIdx.x == 0) *p = 0ull; }

// Counts elements that are NaN or +-inf, and with sign_clear also those whose
// sign bit is set (-0 and negative values).
__global__ __launch_bounds__(256) void k_count_bad(const float* __restrict__ a, int64_t n, int sign_clear,
                                                   unsigned long long* __restrict__ out)
{
    unsigned long long c = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
        const uint32_t b = __float_as_uint(a[e]);
        const bool nonfinite = (b & 0x7f800000u) == 0x7f800000u;
        const bool neg = sign_clear && (b >> 31);
        c += (nonfinite || neg) ? 1ull : 0ull;
    }
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if ((threadIdx.x & 63) == 0 && c) atomicAdd(out, c);
}

std::mutex g_mu;
std::vector<unsigned long long*> g_addr;   // per device

vq_status counter_address(unsigned long long** p)
{
    int dev = -1;
    VQ_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_addr.size() <= dev) g_addr.resize(dev + 1, nullptr);
    if (!g_addr[dev]) {
        void* a = nullptr;
        VQ_HIP(hipGetSymbolAddress(&a, HIP_SYMBOL(g_bad)));
        g_addr[dev] = static_cast<unsigned long long*>(a);
    }
    *p = g_addr[dev];
    return VQ_OK;
}

}  // namespace

bool values_check_on()
{
    const char* e = std::getenv("VQ_CHECK");
    return e != nullptr && std::strcmp(e, "1") == 0;
}

vq_status check_values(const float* a, int64_t n, bool sign_clear, const char* call, const char* what,
                       hipStream_t st)
{
    if (!values_check_on() || a == nullptr || n <= 0) return VQ_OK;
    unsigned long long* cnt = nullptr;
    if (vq_status s = counter_address(&cnt); s != VQ_OK) return s;
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, st, cnt);
    VQ_LAUNCHED("k_zero_u64");
    const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_count_bad, dim3(grid), dim3(256), 0, st, a, n, sign_clear ? 1 : 0, cnt);
    VQ_LAUNCHED("k_count_bad");
    unsigned long long bad = 0;
    VQ_HIP(hipMemcpyAsync(&bad, cnt, sizeof(bad), hipMemcpyDeviceToHost, st));
    VQ_HIP(hipStreamSynchronize(st));
    if (bad)
        return fail(VQ_ERR_INVALID, std::string(call) + ": VQ_CHECK: " + what + " holds " + std::to_string(bad) +
                                        (sign_clear ? " non-finite or negative values" : " non-finite values"));
    return VQ_OK;
}

}  // namespace vq
