// k_quant.hip -- activation quantisation and one-time weight packing.
//
// Quantisation formula (cpp20gemma README, "Architecture & implementation"):
// scale = max(max|v|, 1e-9) / 127, code = clip(round(v / scale), -128, 127),
// with one scale per token for activations ("Gemma 3 1B at 114 tokens per
// second on a laptop CPU", "Step 2": every layer's inputs are rounded to int8)
// and one per tensor for int8 weights.  The code is that of an IEEE fp32
// division (the library is built with correctly rounded division) rounded
// half-to-even (v_rndne_f32), the IEEE default; the per-row activation kernels
// reach it with one multiply per value (actq.hpp, quantize_one_r).
//
// Five trits per byte ("Step 1": 3^5 = 243 codes fit in a byte): byte j of a
// row is sum_i (t[5j+i] + 1) * 3^i; columns past k count as trit 0.
#include "qmv_internal.hpp"
#include "actq.hpp"

namespace qmv {
namespace {

// ---------------------------------------------------------------------------
// Per-row quantisation: one workgroup per row.
// ---------------------------------------------------------------------------
// A workgroup of kQuantThreads per row.  Rows of up to 8192 values that are
// 16-byte aligned (in) and 4-byte aligned (out) are read once: the values stay
// in registers between the maximum and the quantisation.  The codes come from
// quantize_one_r, the division's codes with one multiply per value.
constexpr int kQuantThreads = 512;
constexpr int kRegVec = 8192 / (4 * kQuantThreads);

__device__ __forceinline__ void quantize_row(const float* __restrict__ xr, int64_t k, int8_t* __restrict__ qr,
                                             float* __restrict__ sx_out, float* red)
{
    constexpr int BS = kQuantThreads;
    float m = 0.0f;
    const bool vec = ((reinterpret_cast<uintptr_t>(xr) & 15) == 0);
    if (vec && (k & 3) == 0 && k <= 4 * BS * kRegVec && (reinterpret_cast<uintptr_t>(qr) & 3) == 0) {
        const float4* x4 = reinterpret_cast<const float4*>(xr);
        const int n4 = (int)(k >> 2);
        float4 v[kRegVec];
#pragma unroll
        for (int j = 0; j < kRegVec; ++j) {
            const int i = (int)threadIdx.x + BS * j;
            v[j] = i < n4 ? x4[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
        }
        m = block_max<BS>(m, red);
        const float s = scale_from_max(m);
        const float r = 1.0f / s;
        if (threadIdx.x == 0) *sx_out = s;
        uint32_t* q4 = reinterpret_cast<uint32_t*>(qr);
#pragma unroll
        for (int j = 0; j < kRegVec; ++j) {
            const int i = (int)threadIdx.x + BS * j;
            if (i < n4) {
                uint32_t b0 = (uint8_t)quantize_one_r(v[j].x, s, r), b1 = (uint8_t)quantize_one_r(v[j].y, s, r);
                uint32_t b2 = (uint8_t)quantize_one_r(v[j].z, s, r), b3 = (uint8_t)quantize_one_r(v[j].w, s, r);
                q4[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
            }
        }
        return;
    }
    int64_t head = vec ? (k & ~int64_t(3)) : 0;
    if (vec) {
        const float4* x4 = reinterpret_cast<const float4*>(xr);
        for (int64_t i = threadIdx.x; i < head / 4; i += BS) {
            float4 v = x4[i];
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    }
    for (int64_t i = head + threadIdx.x; i < k; i += BS) m = fmaxf(m, fabsf(xr[i]));
    m = block_max<BS>(m, red);
    const float s = scale_from_max(m);
    const float r = 1.0f / s;
    if (threadIdx.x == 0) *sx_out = s;
    const bool vec_out = vec && ((reinterpret_cast<uintptr_t>(qr) & 3) == 0);
    if (vec_out) {
        const float4* x4 = reinterpret_cast<const float4*>(xr);
        uint32_t* q4 = reinterpret_cast<uint32_t*>(qr);
        for (int64_t i = threadIdx.x; i < head / 4; i += BS) {
            float4 v = x4[i];
            uint32_t b0 = (uint8_t)quantize_one_r(v.x, s, r), b1 = (uint8_t)quantize_one_r(v.y, s, r);
            uint32_t b2 = (uint8_t)quantize_one_r(v.z, s, r), b3 = (uint8_t)quantize_one_r(v.w, s, r);
            q4[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
        for (int64_t i = head + threadIdx.x; i < k; i += BS) qr[i] = quantize_one_r(xr[i], s, r);
    } else {
        for (int64_t i = threadIdx.x; i < k; i += BS) qr[i] = quantize_one_r(xr[i], s, r);
    }
}

__global__ __launch_bounds__(kQuantThreads) void k_quantize_rows(const float* __restrict__ x, int64_t k,
                                                                int8_t* __restrict__ x8, float* __restrict__ sx)
{
    __shared__ float red[kQuantThreads / 64];
    const int64_t row = blockIdx.x;
    quantize_row(x + row * k, k, x8 + row * k, sx + row, red);
}

// Several activation sets in one launch: workgroup b quantises row
// b - first[i] of the set i whose rows it falls in.
__global__ __launch_bounds__(kQuantThreads) void k_quantize_many(ActSets sets)
{
    __shared__ float red[kQuantThreads / 64];
    const int64_t b = blockIdx.x;
    int i = 0;
    while (i + 1 < sets.count && b >= sets.first[i + 1]) ++i;
    const ActSet& a = sets.set[i];
    const int64_t row = b - sets.first[i];
    quantize_row(a.x + row * a.k, a.k, a.x8 + row * a.k, a.sx + row, red);
}

// ---------------------------------------------------------------------------
// Fused steps either side of a GEMV (llama2.c tour, "Step 1" / "Step 6":
// RMSNorm; "Step 5": the gated feed-forward; cpp20gemma and gemma.cpp use a
// GeLU gate): the normalised or gated row is quantised as above without a
// round trip through memory.  One workgroup per row.
// ---------------------------------------------------------------------------

// RMSNorm with the sum-of-squares order of rms_reciprocal (actq.hpp), then
// the per-token quantisation; the values and the codes are reproducible
// exactly.
__global__ __launch_bounds__(kBlock) void k_rmsnorm_quantize(const float* __restrict__ x,
                                                            const float* __restrict__ weight, int64_t k, float eps,
                                                            int8_t* __restrict__ x8, float* __restrict__ sx)
{
    __shared__ float part[kBlock];
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * k;
    int8_t* qr = x8 + row * k;
    const int t = threadIdx.x;
    float a = 0.0f;
    for (int64_t j = t; j < k; j += kBlock) a = add_square(a, xr[j]);
    const float r = rms_reciprocal(a, k, eps, part);
    float m = 0.0f;
    for (int64_t j = t; j < k; j += kBlock) m = fmaxf(m, fabsf(rms_value(weight[j], r, xr[j])));
    m = block_max(m, red);
    const float s = scale_from_max(m);
    if (t == 0) sx[row] = s;
    for (int64_t j = t; j < k; j += kBlock) qr[j] = quantize_one(rms_value(weight[j], r, xr[j]), s);
}

constexpr int kGluThreads = 1024;
constexpr int kGluCache = 8;   // values a thread keeps between the two passes (n <= 8192)

// Max over a 1024-thread block; every thread receives the result.
__device__ __forceinline__ float block_max_1024(float v, float* red)
{
    v = wave_max(v);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kGluThreads / kWave; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// One workgroup of 1024 threads per row; up to 8192 columns the gated values
// are computed once and kept in registers for the quantise pass.
__global__ __launch_bounds__(kGluThreads) void k_glu_quantize(const float* __restrict__ gate,
                                                             const float* __restrict__ up, int64_t n, int act,
                                                             int8_t* __restrict__ x8, float* __restrict__ sx)
{
    __shared__ float red[kGluThreads / kWave];
    const int64_t row = blockIdx.x;
    const float* gr = gate + row * n;
    const float* ur = up + row * n;
    int8_t* qr = x8 + row * n;
    const int t = threadIdx.x;
    float m = 0.0f;
    if (n <= (int64_t)kGluThreads * kGluCache) {
        float h[kGluCache];
#pragma unroll
        for (int i = 0; i < kGluCache; ++i) {
            const int64_t j = t + (int64_t)kGluThreads * i;
            h[i] = j < n ? glu_value(gr[j], ur[j], act) : 0.0f;
            m = fmaxf(m, fabsf(h[i]));
        }
        m = block_max_1024(m, red);
        const float s = scale_from_max(m);
        if (t == 0) sx[row] = s;
#pragma unroll
        for (int i = 0; i < kGluCache; ++i) {
            const int64_t j = t + (int64_t)kGluThreads * i;
            if (j < n) qr[j] = quantize_one(h[i], s);
        }
    } else {
        for (int64_t j = t; j < n; j += kGluThreads) m = fmaxf(m, fabsf(glu_value(gr[j], ur[j], act)));
        m = block_max_1024(m, red);
        const float s = scale_from_max(m);
        if (t == 0) sx[row] = s;
        for (int64_t j = t; j < n; j += kGluThreads) qr[j] = quantize_one(glu_value(gr[j], ur[j], act), s);
    }
}

// ---------------------------------------------------------------------------
// Packing.
// ---------------------------------------------------------------------------
__global__ void k_fill_pack_header(float* scale_out, float scale, int32_t* bad)
{
    if (threadIdx.x == 0) {
        *scale_out = scale;
        if (bad) *bad = 0;
    }
}

// One thread per output byte, in device order: o = (c * n + r) * 16 + jj.
__global__ __launch_bounds__(kBlock) void k_pack_ternary(const int8_t* __restrict__ t, int64_t n, int64_t k,
                                                        int64_t total, uint8_t* __restrict__ out,
                                                        int32_t* __restrict__ bad)
{
    int nbad = 0;
    for (int64_t o = (int64_t)blockIdx.x * kBlock + threadIdx.x; o < total; o += (int64_t)gridDim.x * kBlock) {
        const int64_t slot = o >> 4;
        const int64_t c = slot / n;
        const int64_t r = slot - c * n;
        const int64_t j = c * 16 + (o & 15);
        const int8_t* tr = t + r * k;
        int code = 0, place = 1;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int64_t col = 5 * j + i;
            int trit = 0;
            if (col < k) {
                trit = tr[col];
                if (trit < -1 || trit > 1) {
                    ++nbad;
                    trit = 0;
                }
            }
            code += (trit + 1) * place;
            place *= 3;
        }
        out[o] = (uint8_t)code;
    }
    if (bad && nbad) atomicAdd(bad, nbad);
}

__global__ void k_zero_u32(uint32_t* p)
{
    if (threadIdx.x == 0) *p = 0u;
}

// Max |w| over the tensor into *cell (fp32 bits; non-negative, so unsigned
// order is float order).
__global__ __launch_bounds__(kBlock) void k_absmax(const float* __restrict__ w, int64_t count, uint32_t* cell)
{
    __shared__ float red[4];
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count; i += (int64_t)gridDim.x * kBlock)
        m = fmaxf(m, fabsf(w[i]));
    m = block_max(m, red);
    if (threadIdx.x == 0) atomicMax(cell, __float_as_uint(m));
}

__global__ __launch_bounds__(kBlock) void k_pack_int8(const float* __restrict__ w, int64_t n, int64_t k,
                                                     int64_t total, int8_t* __restrict__ out,
                                                     const uint32_t* __restrict__ cell)
{
    const float s = scale_from_max(__uint_as_float(*cell));
    for (int64_t o = (int64_t)blockIdx.x * kBlock + threadIdx.x; o < total; o += (int64_t)gridDim.x * kBlock) {
        const int64_t slot = o >> 4;
        const int64_t c = slot / n;
        const int64_t r = slot - c * n;
        const int64_t j = c * 16 + (o & 15);
        out[o] = (j < k) ? quantize_one(w[r * k + j], s) : (int8_t)0;
    }
}

__global__ void k_finish_int8_scale(float* scale_out)
{
    if (threadIdx.x == 0) *scale_out = scale_from_max(*scale_out);
}

int grid_for(int64_t items)
{
    int64_t g = (items + kBlock - 1) / kBlock;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

hipError_t launch_quantize_rows(const float* x, int64_t m, int64_t k, int8_t* x8, float* sx, hipStream_t s)
{
    hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)m), dim3(kQuantThreads), 0, s, x, k, x8, sx);
    return hipGetLastError();
}

hipError_t launch_quantize_many(const ActSets& sets, int64_t rows, hipStream_t s)
{
    hipLaunchKernelGGL(k_quantize_many, dim3((unsigned)rows), dim3(kQuantThreads), 0, s, sets);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const float* x, const float* weight, int64_t m, int64_t k, float eps, int8_t* x8,
                                   float* sx, hipStream_t s)
{
    hipLaunchKernelGGL(k_rmsnorm_quantize, dim3((unsigned)m), dim3(kBlock), 0, s, x, weight, k, eps, x8, sx);
    return hipGetLastError();
}

hipError_t launch_glu_quantize(const float* gate, const float* up, int64_t m, int64_t n, int act, int8_t* x8,
                               float* sx, hipStream_t s)
{
    hipLaunchKernelGGL(k_glu_quantize, dim3((unsigned)m), dim3(kGluThreads), 0, s, gate, up, n, act, x8, sx);
    return hipGetLastError();
}

hipError_t launch_fill_pack_header(float* scale_out, float scale, int32_t* bad, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_pack_header, dim3(1), dim3(kWave), 0, s, scale_out, scale, bad);
    return hipGetLastError();
}

hipError_t launch_pack_ternary(const int8_t* trits, int64_t n, int64_t k, int64_t chunks, uint8_t* out,
                               int32_t* bad, hipStream_t s)
{
    const int64_t total = n * chunks * 16;
    hipLaunchKernelGGL(k_pack_ternary, dim3(grid_for(total)), dim3(kBlock), 0, s, trits, n, k, total, out, bad);
    return hipGetLastError();
}

hipError_t launch_pack_int8(const float* w, int64_t n, int64_t k, int64_t chunks, int8_t* out, float* scale_out,
                            hipStream_t s)
{
    uint32_t* cell = reinterpret_cast<uint32_t*>(scale_out);
    const int64_t count = n * k;
    const int64_t total = n * chunks * 16;
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(kWave), 0, s, cell);
    hipLaunchKernelGGL(k_absmax, dim3(grid_for(count)), dim3(kBlock), 0, s, w, count, cell);
    hipLaunchKernelGGL(k_pack_int8, dim3(grid_for(total)), dim3(kBlock), 0, s, w, n, k, total, out,
                       (const uint32_t*)cell);
    hipLaunchKernelGGL(k_finish_int8_scale, dim3(1), dim3(kWave), 0, s, scale_out);
    return hipGetLastError();
}

}  // namespace qmv
