// unpack.hpp -- five-trits-per-byte decoding helpers for the GEMV kernels.
//
// A packed dword [b0 b1 b2 b3] (20 trits) becomes the prefix-quotient planes
// P_j = floor(b / 3^(5-j)), j = 1..4, plus b itself entering as b ^ 0x80.
// Digit d_(5-j) = P_j - 3 P_(j-1), so for the activation planes X_i (the x
// values that meet digit i of each byte)
//     sum_i d_i . X_i = sum_(j=1..5) P_j . X_(5-j) - 3 sum_(j=1..4) P_j . X_(4-j).
// floor(v/3) for two bytes at once: the bytes sit in two fp16 lanes as
// 1024 + v, and one packed fp16 FMA (1024+v)*0.332763671875 + 683, rounded to
// nearest even, yields exactly 1024 + floor(v/3) for every v in 0..242
// (checked exhaustively); chaining it gives floor(v/9), floor(v/27), floor(v/81).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Two fp16 lanes holding 1024 + v (v <= 242) -> 1024 + floor(v / 3).
__device__ __forceinline__ uint32_t third2(uint32_t h)
{
    const half2_t mul = __builtin_bit_cast(half2_t, 0x35533553u);  // 0.332763671875
    const half2_t add = __builtin_bit_cast(half2_t, 0x61566156u);  // 683.0
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, h), mul, add));
}

struct Planes {
    uint32_t p1, p2, p3, p4, b5;
};

// One packed dword [b0 b1 b2 b3] -> prefix-quotient planes, byte k of each
// plane belonging to packed byte k.
__device__ __forceinline__ Planes unpack(uint32_t w)
{
    const uint32_t mag = 0x64646464u;                          // fp16 high byte of 1024
    const uint32_t lo = __builtin_amdgcn_perm(mag, w, 0x04020400u);  // [b0 64 b2 64]
    const uint32_t hi = __builtin_amdgcn_perm(mag, w, 0x04030401u);  // [b1 64 b3 64]
    const uint32_t lo4 = third2(lo), hi4 = third2(hi);
    const uint32_t lo3 = third2(lo4), hi3 = third2(hi4);
    const uint32_t lo2 = third2(lo3), hi2 = third2(hi3);
    const uint32_t lo1 = third2(lo2), hi1 = third2(hi2);
    Planes p;
    p.p4 = __builtin_amdgcn_perm(hi4, lo4, 0x06020400u);
    p.p3 = __builtin_amdgcn_perm(hi3, lo3, 0x06020400u);
    p.p2 = __builtin_amdgcn_perm(hi2, lo2, 0x06020400u);
    p.p1 = __builtin_amdgcn_perm(hi1, lo1, 0x06020400u);
    p.b5 = w ^ 0x80808080u;
    return p;
}

__device__ __forceinline__ uint32_t sel(const uint4& v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 16 packed weight bytes as a native vector (loadable through a global pointer).
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t sel(const v4u32& v, int i)
{
    return v[i];
}

constexpr uint32_t bsel(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3)
{
    return s0 | (s1 << 8) | (s2 << 16) | (s3 << 24);
}

// The page's input reorder for one 20-column group: natural bytes B0..B19
// (dwords n0..n4) -> plane i = [B_i, B_(5+i), B_(10+i), B_(15+i)], i = 0..4,
// i.e. the x values that meet digit i of the group's four packed bytes.
__device__ __forceinline__ void reorder20(const uint32_t n0, const uint32_t n1, const uint32_t n2,
                                          const uint32_t n3, const uint32_t n4, uint32_t out[5])
{
    constexpr uint32_t merge = bsel(0, 1, 4, 5);
    out[0] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(n3, n2, bsel(2, 7, 12, 12)),
                                   __builtin_amdgcn_perm(n1, n0, bsel(0, 5, 12, 12)), merge);
    out[1] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(n4, n2, bsel(3, 4, 12, 12)),
                                   __builtin_amdgcn_perm(n1, n0, bsel(1, 6, 12, 12)), merge);
    out[2] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(n4, n3, bsel(0, 5, 12, 12)),
                                   __builtin_amdgcn_perm(n1, n0, bsel(2, 7, 12, 12)), merge);
    out[3] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(n4, n3, bsel(1, 6, 12, 12)),
                                   __builtin_amdgcn_perm(n2, n0, bsel(3, 4, 12, 12)), merge);
    out[4] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(n4, n3, bsel(2, 7, 12, 12)),
                                   __builtin_amdgcn_perm(n2, n1, bsel(0, 5, 12, 12)), merge);
}

}  // namespace
}  // namespace qmv
