// actq.hpp -- per-token activation quantisation and the fused steps around
// the matrix products, shared by the kernels that compute them, so that every
// path that produces a code or a value does it with the same instructions.
//
// Quantisation (cpp20gemma README, "Architecture & implementation"; "Gemma 3
// 1B at 114 tokens per second on a laptop CPU", "Step 2"): scale =
// max(max|v|, 1e-9) / 127, code = clip(round(v / scale), -128, 127), IEEE fp32
// division (the library is built with correctly rounded division and square
// root) and round-half-to-even.  RMSNorm (llama2.c tour, "forward", Steps 1
// and 6): o = weight * (r * x), r = 1 / sqrt(ss / k + eps).  Gated
// feed-forward ("forward", Step 5): h = act(gate) * up.  Nothing here is
// contracted into fused multiply-adds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {
namespace {

// Max over a wave of values >= 0 (every lane receives it): DPP row shifts
// within each row of 16 lanes (a lane shifted in from outside the row brings
// 0, which changes no such maximum), then the four rows' last lanes.  fmaxf,
// so a NaN never wins.
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false)));
    const float a = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15)),
                          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31)));
    const float b = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47)),
                          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63)));
    return fmaxf(a, b);
}

// Max over a block of BS threads of values >= 0 (red: BS / 64 floats of
// LDS); every thread receives it.
template <int BS = 256>
__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < BS / 64; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ float scale_from_max(float m)
{
    return fmaxf(m, 1e-9f) / 127.0f;
}

__device__ __forceinline__ int8_t quantize_one(float v, float s)
{
    float q = __builtin_rintf(v / s);
    q = fminf(fmaxf(q, -128.0f), 127.0f);
    return (int8_t)(int)q;
}

// quantize_one(v, s) for a row whose scale s = scale_from_max(m) has |v| <= m,
// given r = 1 / s (IEEE), with one multiply in place of the division.  Each of
// r, y = v * r and the quotient v / s is within a relative 2^-24 of its exact
// value and |v / s| <= 127 (1 + 2^-23), so y lies within 2^-15 of the rounded
// quotient: both round to the same integer unless y is within 2^-14 of a
// half-integer (or is NaN), and there the division decides.  The same code for
// every such input.
__device__ __forceinline__ int8_t quantize_one_r(float v, float s, float r)
{
#pragma clang fp contract(off)
    const float y = v * r;
    const float n = __builtin_rintf(y);
    float q = fabsf(y - n) < 0.5f - 0x1p-14f ? n : __builtin_rintf(v / s);
    q = fminf(fmaxf(q, -128.0f), 127.0f);
    return (int8_t)(int)q;
}

// a + x * x, rounded twice.
__device__ __forceinline__ float add_square(float a, float x)
{
#pragma clang fp contract(off)
    return a + x * x;
}

// RMSNorm's reciprocal from the 256 per-thread partial sums of squares of a
// row of k values in part[0..255] (LDS): thread t has added x[j]^2 for j = t,
// t + 256, ... in order; the partials meet pairwise, part[t] += part[t + s] for
// s = 128, 64, 32, .., 1 (the last six levels inside wave 0 by lane shuffles and
// DPP moves: the same additions in the same order; lanes t >= s compute values
// nobody reads).  Every thread of the block calls it
// (blocks of 256 threads or more) and receives r.
__device__ __forceinline__ float rms_tree(float* part, int64_t k, float eps)
{
#pragma clang fp contract(off)
    const int t = threadIdx.x;
    __syncthreads();
    if (t < 128) part[t] += part[t + 128];
    __syncthreads();
    if (t < 64) {
        float v = part[t] + part[t + 64];
        for (int st = 32; st >= 16; st >>= 1) {
            const float o = __shfl_down(v, st, 64);
            if (t < st) v += o;
        }
        // s = 8 .. 1 stay inside a row of 16 lanes: DPP row_shl:s hands lane t
        // the value of lane t + s
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x108, 0xf, 0xf, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x104, 0xf, 0xf, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x102, 0xf, 0xf, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x101, 0xf, 0xf, true));
        if (t == 0) part[0] = 1.0f / sqrtf(v / (float)k + eps);
    }
    __syncthreads();
    const float r = part[0];
    __syncthreads();
    return r;
}

// The same from a 256-thread block whose thread t holds partial a.
__device__ __forceinline__ float rms_reciprocal(float a, int64_t k, float eps, float* part)
{
    part[threadIdx.x] = a;
    return rms_tree(part, k, eps);
}

__device__ __forceinline__ float rms_value(float weight, float r, float x)
{
#pragma clang fp contract(off)
    return weight * (r * x);
}

// h = act(gate) * up, act 1 = GeLU (tanh form), 2 = SiLU, in fp32 with the
// device's expf / tanhf.
__device__ __forceinline__ float glu_value(float g, float u, int act)
{
#pragma clang fp contract(off)
    float a;
    if (act == 1) {
        const float c = 0.7978845608028654f;   // sqrt(2 / pi)
        a = 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
    } else {
        a = g / (1.0f + expf(-g));
    }
    return a * u;
}

// The dequantised output of an exact dot: (acc * sx) * sw.
__device__ __forceinline__ float dequant(int acc, float sx, float sw)
{
#pragma clang fp contract(off)
    return (float)acc * sx * sw;
}

}  // namespace
}  // namespace qmv
