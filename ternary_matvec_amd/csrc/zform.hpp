// zform.hpp -- the Z form of a token's activations for five-trits-per-byte
// weights, shared by the kernels that stream ternary rows against one staged
// token ("Gemma 3 1B at 114 tokens per second on a laptop CPU", "Step 1": the
// inputs are reordered once per token so that each unpacked digit plane meets
// its activations).
//
// For a packed byte b with base-3 digits d_1..d_5 (d_1 the most significant,
// digit d = trit + 1) meeting activations X_1..X_5, let P_j = floor(b / 3^(5-j)),
// so d_j = P_j - 3 P_(j-1) and
//     sum_j d_j X_j = sum_j P_j Z_j,   Z_j = X_j - 3 X_(j+1) (j < 5),  Z_5 = X_5.
// The unpacker holds P_j of two bytes as the fp16 pair 1024 + P_j, whose int16
// bit pattern is 25600 + P_j, so one v_dot2_i32_i16 with the int16 pair of Z
// values adds P.Z plus 25600 * (Z sum); that constant and sum x (trit = d - 1)
// are taken off once per row.  Sums are modulo 2^32, exact whenever the true
// dot fits int32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {
namespace {

typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int dot2(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot2(__builtin_bit_cast(s16x2, a), __builtin_bit_cast(s16x2, b), c, false);
}

// Z values of one 20-column group (natural dwords nat[0..4]; packed byte q of
// the group covers columns 5q .. 5q+4, column 5q+e meeting the digit of 3^e,
// so X_j = x[5q + 5 - j]).  out[2i + r] is the int16 pair of Z_(i+1) for bytes
// r (low half) and r + 2 (high half): the same byte pairs the unpacker puts
// into one fp16 register.  Adds the group's Z sum and x sum to sum_z, sum_x.
__device__ __forceinline__ void z_group(const uint32_t nat[5], uint32_t out[10], int& sum_z, int& sum_x)
{
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        int za[5], zb[5];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = r + 2 * h;
            int x[5];
#pragma unroll
            for (int e = 0; e < 5; ++e) {
                const int b = 5 * q + e;
                x[e] = (int)(int8_t)(uint8_t)(nat[b >> 2] >> (8 * (b & 3)));
                sum_x += x[e];
            }
            int* z = h ? zb : za;
            z[0] = x[4] - 3 * x[3];
            z[1] = x[3] - 3 * x[2];
            z[2] = x[2] - 3 * x[1];
            z[3] = x[1] - 3 * x[0];
            z[4] = x[0];
            // Z_1 + .. + Z_5 = x4 - 2 (x3 + x2 + x1 + x0)
            sum_z += x[4] - 2 * (x[3] + x[2] + x[1] + x[0]);
        }
#pragma unroll
        for (int i = 0; i < 5; ++i) out[2 * i + r] = __builtin_amdgcn_perm((uint32_t)zb[i], (uint32_t)za[i], 0x05040100u);
    }
}

// The row correction of a token: 25600 * sum Z + sum x, modulo 2^32.
__device__ __forceinline__ int z_correction(int sum_z, int sum_x)
{
    return (int)(25600u * (uint32_t)sum_z + (uint32_t)sum_x);
}

}  // namespace
}  // namespace qmv
