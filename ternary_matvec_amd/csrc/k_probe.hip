// k_probe.hip -- a plain read of a device buffer, the yardstick the kernels'
// HBM rates are compared with (not part of the method: a measurement aid).
//
// Every byte is read once with 16-byte non-temporal loads (as the weight
// streams read), grid-stride, two loads in flight
// per lane, 16 waves per compute unit (the configuration that read fastest on
// this machine), and folded into one word with xor so that no load can be
// dropped.  The result word is written only by lanes that fold to a value
// nobody asked for, which keeps the write traffic at a few bytes.
#include <algorithm>

#include "qmv_internal.hpp"
#include "unpack.hpp"

namespace qmv {
namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const v4u32* __restrict__ src, int64_t n16,
                                                              uint32_t* __restrict__ out, uint32_t key)
{
    const QMV_GLOBAL v4u32* p = gload_ptr(src);
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + stride < n16; i += 2 * stride) {
        const v4u32 a = __builtin_nontemporal_load(p + i);
        const v4u32 b = __builtin_nontemporal_load(p + i + stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    }
    if (i < n16) {
        const v4u32 a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == key) out[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* data, int64_t bytes, uint32_t* out, int cus, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((int64_t)cus * 4, (n16 + kProbeThreads - 1) / kProbeThreads));
    hipLaunchKernelGGL(k_read_probe, dim3((unsigned)grid), dim3(kProbeThreads), 0, s,
                       reinterpret_cast<const v4u32*>(data), n16, out, 0x9e3779b9u);
    return hipGetLastError();
}

}  // namespace qmv
