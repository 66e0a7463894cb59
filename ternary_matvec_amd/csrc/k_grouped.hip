// k_grouped.hip -- int8 weights and activations with group-wise scales.
//
// Weights come in groups of 128 consecutive columns of a row with one fp32
// scale each (gemma.cpp tour, "Weights, Blobs, and the .sbs Format": int8
// groups of 128 sharing a scale); activations get one scale per 32 columns
// ("Gemma 3 1B at 114 tokens per second on a laptop CPU", "A side finding:
// Gemma 4 E4B in 4-bit").  Every group is quantised with the per-token rule
// (cpp20gemma README, "Architecture & implementation": absmax / 127 with a
// 1e-9 floor, IEEE division, half-to-even, clip).
//
// GEMV: activation group h (columns 32h .. 32h+31) lies inside weight group
// h / 4, so its dot product is an exact int32 sum of eight v_dot4_i32_i8, and
// the two scales are applied after it:
//     y[m][n] = sum_h (sw[n][h/4] * sx[m][h]) * D_h
// in fp32: each lane adds its groups with one fused multiply-add each, in
// increasing h, then the lanes of a row meet in a butterfly.
//
// Layout: weights row-major, rows padded with zero bytes to a multiple of 16;
// weight scales [n][ceil(k/128)]; activations [m][k] natural; activation
// scales [m][ceil(k/32)].
#include "qmv_internal.hpp"

namespace qmv {
namespace {

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

// ---------------------------------------------------------------------------
// Group quantisation: LANES = min(GROUP, 64) lanes per group, GROUP / LANES
// values per lane; a block of 256 threads covers 256 / LANES groups.  Output
// rows have stride q_stride >= k; the bytes of [k, q_stride) are written as
// zeros by the lanes of the row's last group (q_stride <= its column span).
// ---------------------------------------------------------------------------
template <int GROUP>
__global__ __launch_bounds__(kBlock) void k_quantize_groups(const float* __restrict__ x, int64_t rows, int64_t k,
                                                           int64_t q_stride, int8_t* __restrict__ q,
                                                           float* __restrict__ s)
{
    constexpr int kLanes = GROUP < kWave ? GROUP : kWave;
    constexpr int kPer = GROUP / kLanes;
    const int64_t ng = (k + GROUP - 1) / GROUP;
    const int64_t gid = (int64_t)blockIdx.x * (kBlock / kLanes) + threadIdx.x / kLanes;
    const int li = threadIdx.x % kLanes;
    const bool live = gid < rows * ng;
    const int64_t row = live ? gid / ng : 0, g = live ? gid % ng : 0;
    float v[kPer];
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t c = g * GROUP + li + (int64_t)kLanes * j;
        v[j] = (live && c < k) ? x[row * k + c] : 0.0f;
        mx = fmaxf(mx, fabsf(v[j]));
    }
#pragma unroll
    for (int off = kLanes / 2; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    if (!live) return;
    const float sc = fmaxf(mx, 1e-9f) / 127.0f;
    if (li == 0) s[row * ng + g] = sc;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t c = g * GROUP + li + (int64_t)kLanes * j;
        if (c < k) {
            float r = __builtin_rintf(v[j] / sc);
            r = fminf(fmaxf(r, -128.0f), 127.0f);
            q[row * q_stride + c] = (int8_t)(int)r;
        } else if (c < q_stride) {
            q[row * q_stride + c] = 0;
        }
    }
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---------------------------------------------------------------------------
// GEMV.  One workgroup per tile entry (problem slot << kTileRowBits | row
// block).  P = lanes_per_row lanes share a row (P in 4 .. 64, a power of two,
// consecutive lanes of one wave), so a tile is 256 / P rows; lane s of a row
// takes activation groups s, s + P, ...  The tokens' activations and scales
// are staged in LDS first: x8 rows zero-padded to a multiple of 32 columns.
// Weight reads are raw buffer loads over the matrix, so the 16 bytes past a
// row's padded end (read for its last group when k % 32 is 1..16) are the next
// row's or zeros; they meet zero activations.
// ---------------------------------------------------------------------------
constexpr int kGBatch = 4;   // groups a lane loads before it computes

template <int MT>
__global__ __launch_bounds__(kBlock) void k_gemv_grouped(const DevProblem* __restrict__ probs,
                                                        const uint32_t* __restrict__ tiles)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const uint32_t te = cload_ptr(tiles)[blockIdx.x];
    const DevProblem* P = probs + (te >> kTileRowBits);
    const int rb = (int)(te & ((1u << kTileRowBits) - 1));
    const int n = P->n, k = P->k, m = P->m;
    const int lshift = 31 - __builtin_clz((uint32_t)P->lanes_per_row);
    const int pl = 1 << lshift;
    const int kp = (k + 31) & ~31;                 // staged columns per token
    const int hn = kp >> 5;                        // activation groups per row
    const int gn = (k + 127) >> 7;                 // weight groups per row
    const uint32_t stride = (uint32_t)P->chunks * 16u;
    const int8_t* x8 = P->x8;
    const float* sx = P->sx;
    uint8_t* xs = smem;
    float* sxs = reinterpret_cast<float*>(smem + (size_t)m * kp);

    const int tid = threadIdx.x;
    const int s = tid & (pl - 1);
    const int row = rb * (kBlock >> lshift) + (tid >> lshift);
    const bool live = row < n;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)P->w, (short)0, (int)((uint32_t)n * stride), (int)kRsrcWord3);
    const float* swr = P->sw + (size_t)(live ? row : 0) * gn;
    const uint32_t roff = (uint32_t)(live ? row : 0) * stride;
    uint4 wlo[kGBatch], whi[kGBatch];
    float wsc[kGBatch];
    // one batch of the lane's groups: its weights and weight scales
    auto load_batch = [&](int h0) {
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            const int h = h0 + b * pl;
            if (b == 0 || h < hn) {
                const uint32_t o = roff + 32u * (uint32_t)h;
                wlo[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, o, 0, 0));
                whi[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, o + 16, 0, 0));
                wsc[b] = gload_ptr(swr)[h < hn ? h >> 2 : 0];
            }
        }
    };
    // the first batch goes out before the activations are staged, so the
    // staging round trip overlaps the weight stream
    if (live && s < hn) load_batch(s);

    // ---- stage: x8 rows (k bytes each, any alignment) as dwords, zero past k
    for (int mi = 0; mi < m; ++mi) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(x8) + (uintptr_t)mi * (uintptr_t)k;
        const uint32_t sh = (uint32_t)(a & 3);
        const uint32_t words = (sh + (uint32_t)k + 3u) >> 2;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a & ~(uintptr_t)3), (short)0, (int)(4 * words), (int)kRsrcWord3);
        uint32_t* dst = reinterpret_cast<uint32_t*>(xs + (size_t)mi * kp);
        for (int d = tid; d < (kp >> 2); d += kBlock) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * d, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * d + 4, 0, 0);
            const uint32_t v = __builtin_amdgcn_alignbyte(hi, lo, sh);
            const int valid = k - 4 * d;
            dst[d] = valid >= 4 ? v : valid <= 0 ? 0u : v & ((1u << (8 * valid)) - 1u);
        }
    }
    for (int i = tid; i < m * hn; i += kBlock) sxs[i] = gload_ptr(sx)[i];
    __syncthreads();
    if (!live) return;   // no barrier follows

    float acc[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) acc[mi] = 0.0f;
    for (int h0 = s; h0 < hn; h0 += kGBatch * pl) {
        if (h0 != s) load_batch(h0);
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            const int h = h0 + b * pl;
            if (b > 0 && h >= hn) break;
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                if (mi < m) {
                    const uint4* xp = reinterpret_cast<const uint4*>(xs + (size_t)mi * kp + 32 * h);
                    const uint4 xa = xp[0], xb = xp[1];
                    int d = dot4(wlo[b].x, xa.x, 0);
                    d = dot4(wlo[b].y, xa.y, d);
                    d = dot4(wlo[b].z, xa.z, d);
                    d = dot4(wlo[b].w, xa.w, d);
                    d = dot4(whi[b].x, xb.x, d);
                    d = dot4(whi[b].y, xb.y, d);
                    d = dot4(whi[b].z, xb.z, d);
                    d = dot4(whi[b].w, xb.w, d);
                    acc[mi] = __builtin_fmaf(wsc[b] * sxs[mi * hn + h], (float)d, acc[mi]);
                }
            }
        }
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
        for (int off = pl >> 1; off >= 1; off >>= 1) acc[mi] += __shfl_xor(acc[mi], off, kWave);
    if (s == 0) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
            if (mi < m) gstore_ptr(P->y)[(size_t)mi * n + row] = acc[mi];
    }
}

template <int MT>
hipError_t launch_grouped_one(const DevProblem* probs, const uint32_t* tiles, int32_t count, size_t lds,
                              hipStream_t s)
{
    hipLaunchKernelGGL((k_gemv_grouped<MT>), dim3((unsigned)count), dim3(kBlock), lds, s, probs, tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_groups(const float* x, int64_t rows, int64_t k, int group, int64_t q_stride, int8_t* q,
                                  float* s, hipStream_t st)
{
    const int64_t ng = (k + group - 1) / group;
    const int lanes = group < kWave ? group : kWave;
    const int64_t per_block = kBlock / lanes;
    const int64_t blocks = (rows * ng + per_block - 1) / per_block;
    if (group == 32)
        hipLaunchKernelGGL(k_quantize_groups<32>, dim3((unsigned)blocks), dim3(kBlock), 0, st, x, rows, k, q_stride,
                           q, s);
    else if (group == 128)
        hipLaunchKernelGGL(k_quantize_groups<128>, dim3((unsigned)blocks), dim3(kBlock), 0, st, x, rows, k,
                           q_stride, q, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

int grouped_lanes_per_row(int64_t k)
{
    const int64_t hn = (k + 31) / 32;
    int p = 4;
    while (p < 64 && p * kGBatch < hn) p *= 2;
    return p;
}

size_t grouped_lds_bytes(int64_t m, int64_t k)
{
    const int64_t kp = (k + 31) / 32 * 32;
    return (size_t)(m * kp + 4 * m * (kp / 32));
}

namespace {
template <int MT>
hipError_t grouped_lds_limit()
{
    return raise_lds_limit(reinterpret_cast<const void*>(&k_gemv_grouped<MT>));
}
}  // namespace

hipError_t setup_grouped_attributes()
{
    hipError_t e = grouped_lds_limit<1>();
    if (e == hipSuccess) e = grouped_lds_limit<2>();
    if (e == hipSuccess) e = grouped_lds_limit<4>();
    if (e == hipSuccess) e = grouped_lds_limit<8>();
    if (e == hipSuccess) e = grouped_lds_limit<16>();
    return e;
}

hipError_t launch_gemv_grouped(const DevProblem* probs, const uint32_t* tiles, int32_t count, int max_m, size_t lds,
                               hipStream_t s)
{
    if (max_m <= 1) return launch_grouped_one<1>(probs, tiles, count, lds, s);
    if (max_m <= 2) return launch_grouped_one<2>(probs, tiles, count, lds, s);
    if (max_m <= 4) return launch_grouped_one<4>(probs, tiles, count, lds, s);
    if (max_m <= 8) return launch_grouped_one<8>(probs, tiles, count, lds, s);
    return launch_grouped_one<16>(probs, tiles, count, lds, s);
}

}  // namespace qmv
