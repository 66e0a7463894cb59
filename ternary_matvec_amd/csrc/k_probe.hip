// k_probe.hip -- measurement aids, not part of the method: a plain read of a
// device buffer (the yardstick the kernels' HBM rates are compared with) and a
// register-only stream of int8 matrix instructions (the yardstick of the
// prefill's matrix-core rate).
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

typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef int v16i32 __attribute__((ext_vector_type(16)));

// Independent accumulator chains per wave: with 6 (not 8) chains of the 4-register
// instruction the compiler keeps every accumulator in place (each instruction's
// result registers are its accumulator registers); a test checks the assembly.
constexpr int kProbeChains[2] = {6, 8};

// Every wave issues iters x chains independent int8 matrix instructions on
// register operands (no instruction waits for the one before it), kind 0
// v_mfma_i32_16x16x64_i8, kind 1 v_mfma_i32_32x32x32_i8; the accumulators are
// folded into a word written only if it equals a value nobody asked for.
template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void k_mfma_probe(int iters, uint32_t* __restrict__ out, uint32_t key)
{
    const int t = threadIdx.x;
    const v4i32 a = {t, 3 * t + 1, 5 * t + 2, 7 * t + 3};
    const v4i32 b = {t ^ 5, t + 11, 13 * t, 17};
    uint32_t acc = 0;
    if (KIND == 0) {
        // accumulators start from distinct values of the thread (not constants):
        // every instruction then reads and writes the same four registers
        constexpr int kN = kProbeChains[0];
        v4i32 c[kN];
#pragma unroll
        for (int j = 0; j < kN; ++j) c[j] = v4i32{t + j, t ^ j, 2 * t + j, t - j};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kN; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kN; ++j) acc ^= (uint32_t)(c[j][0] ^ c[j][1] ^ c[j][2] ^ c[j][3]);
    } else {
        constexpr int kN = kProbeChains[1];
        v16i32 c[kN];
#pragma unroll
        for (int j = 0; j < kN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) c[j][q] = t + 16 * j + q;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kN; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc ^= (uint32_t)c[j][q];
    }
    if (acc == key) out[0] = acc;
}

}  // namespace

hipError_t launch_mfma_probe(int kind, int iters, uint32_t* out, int cus, int64_t* ops, hipStream_t s)
{
    // four workgroups of four waves per compute unit: four waves per SIMD
    const int grid = cus * 4;
    const int64_t per_instr = kind == 0 ? 2 * 16 * 16 * 64 : 2 * 32 * 32 * 32;
    *ops = (int64_t)grid * (kProbeThreads / kWave) * iters * kProbeChains[kind] * per_instr;
    if (kind == 0)
        hipLaunchKernelGGL(k_mfma_probe<0>, dim3(grid), dim3(kProbeThreads), 0, s, iters, out, 0x9e3779b9u);
    else
        hipLaunchKernelGGL(k_mfma_probe<1>, dim3(grid), dim3(kProbeThreads), 0, s, iters, out, 0x9e3779b9u);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void* data, int64_t bytes, uint32_t* out, int cus, hipStream_t s)
{
    const int64_t n16 = bytes / 16;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((int64_t)cus * 4, (n16 + kProbeThreads - 1) / kProbeThreads));
    hipLaunchKernelGGL(k_read_probe, dim3((unsigned)grid), dim3(kProbeThreads), 0, s,
                       reinterpret_cast<const v4u32*>(data), n16, out, 0x9e3779b9u);
    return hipGetLastError();
}

}  // namespace qmv
