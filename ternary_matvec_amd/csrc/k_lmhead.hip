// k_lmhead.hip -- bf16 output-layer GEMV fused with the greedy choice (gfx950).
//
// logit[r] = sum_c float(w[r][c]) * x[c] with fp32 accumulation, then the
// first index holding the largest logit ("Gemma 3 1B at 114 tokens per second
// on a laptop CPU", "Step 3: the output layer became the bottleneck": every
// vocabulary row is scored against the final hidden state; llama2.c tour,
// "Sampling": greedy argmax keeps the first maximum).
//
// Layout of the work: 16 lanes share one row; lane l reads 16-byte chunks
// l, l+16, ... so each load instruction covers four 256-byte runs of four
// rows.  x lives in LDS.  The 16 partial sums meet through lane shuffles; the
// workgroup's best (value, index) goes to the workspace and a second small
// kernel picks the overall first maximum.  Ties compare indices, so the result
// does not depend on the order in which workgroups finish.
#include "qmv_internal.hpp"

namespace qmv {
namespace {

constexpr int kGroup = 16;                 // lanes per row
constexpr int kRowsPerIter = kBlock / kGroup;  // 16 rows in flight per workgroup
constexpr int kIters = 4;                  // rows per group
constexpr int kRowsPerBlock = kRowsPerIter * kIters;
constexpr int kMaxLdsK = 16384;            // x staged in LDS up to this many columns
constexpr int kUnroll = 8;                 // chunk loads in flight per lane
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));

struct Best {
    float v;
    int32_t i;
};

__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi)
{
    return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__global__ __launch_bounds__(kBlock) void k_lmhead(const uint16_t* __restrict__ w, const float* __restrict__ x,
                                                  int64_t v, int64_t k, float* __restrict__ logits,
                                                  Best* __restrict__ partial, int fast)
{
    extern __shared__ __align__(16) float xs[];
    __shared__ float sb[kRowsPerIter];
    __shared__ int32_t si[kRowsPerIter];

    const int tid = threadIdx.x;
    const int g = tid / kGroup;
    const int l = tid & (kGroup - 1);
    if (fast)
        for (int64_t i = tid; i < k; i += kBlock) xs[i] = x[i];
    __syncthreads();

    float best = -INFINITY;
    int32_t besti = 0x7FFFFFFF;
    const int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock;
    const int nch = (int)(k >> 3);
    for (int it = 0; it < kIters; ++it) {
        const int64_t row = row0 + it * kRowsPerIter + g;
        if (row >= v) break;
        float sum = 0.0f;
        if (fast) {
            const uint4* wr = reinterpret_cast<const uint4*>(w + row * k);
            for (int c0 = l; c0 < nch; c0 += kGroup * kUnroll) {
                uint4 q[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int c = c0 + u * kGroup;
                    // the weights are read once: a non-temporal load
                    q[u] = (c < nch) ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                           reinterpret_cast<const nt_u32x4*>(wr) + c))
                                     : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int c = c0 + u * kGroup;
                    if (c < nch) {
                        const float4 xa = *reinterpret_cast<const float4*>(xs + 8 * c);
                        const float4 xb = *reinterpret_cast<const float4*>(xs + 8 * c + 4);
                        sum = fmaf(bf_lo(q[u].x), xa.x, sum);
                        sum = fmaf(bf_hi(q[u].x), xa.y, sum);
                        sum = fmaf(bf_lo(q[u].y), xa.z, sum);
                        sum = fmaf(bf_hi(q[u].y), xa.w, sum);
                        sum = fmaf(bf_lo(q[u].z), xb.x, sum);
                        sum = fmaf(bf_hi(q[u].z), xb.y, sum);
                        sum = fmaf(bf_lo(q[u].w), xb.z, sum);
                        sum = fmaf(bf_hi(q[u].w), xb.w, sum);
                    }
                }
            }
        } else {
            const uint16_t* wr = w + row * k;
            for (int64_t c = l; c < k; c += kGroup) sum = fmaf(__uint_as_float((uint32_t)wr[c] << 16), x[c], sum);
        }
#pragma unroll
        for (int off = kGroup / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, kGroup);
        if (logits && l == 0) logits[row] = sum;
        if (better(sum, (int32_t)row, best, besti)) {
            best = sum;
            besti = (int32_t)row;
        }
    }
    if (l == 0) {
        sb[g] = best;
        si[g] = besti;
    }
    __syncthreads();
    if (tid == 0) {
        float bv = sb[0];
        int32_t bi = si[0];
        for (int j = 1; j < kRowsPerIter; ++j)
            if (better(sb[j], si[j], bv, bi)) {
                bv = sb[j];
                bi = si[j];
            }
        partial[blockIdx.x].v = bv;
        partial[blockIdx.x].i = bi;
    }
}

constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(kFinalThreads) void k_argmax_final(const Best* __restrict__ partial, int64_t count,
                                                               int32_t* idx, float* max_logit)
{
    __shared__ float sb[kFinalThreads];
    __shared__ int32_t si[kFinalThreads];
    float bv = -INFINITY;
    int32_t bi = 0x7FFFFFFF;
    for (int64_t j = threadIdx.x; j < count; j += kFinalThreads) {
        const Best p = partial[j];
        if (better(p.v, p.i, bv, bi)) {
            bv = p.v;
            bi = p.i;
        }
    }
    sb[threadIdx.x] = bv;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int s = kFinalThreads / 2; s >= 1; s >>= 1) {
        if ((int)threadIdx.x < s) {
            const float ov = sb[threadIdx.x + s];
            const int32_t oi = si[threadIdx.x + s];
            if (better(ov, oi, sb[threadIdx.x], si[threadIdx.x])) {
                sb[threadIdx.x] = ov;
                si[threadIdx.x] = oi;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *idx = si[0];
        if (max_logit) *max_logit = sb[0];
    }
}

}  // namespace

int64_t lmhead_partials(int64_t v) { return (v + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t launch_lmhead(const uint16_t* w, const float* x, int64_t v, int64_t k, int32_t* idx, float* max_logit,
                         float* logits, void* workspace, hipStream_t s)
{
    const int64_t blocks = lmhead_partials(v);
    const int fast = ((k & 7) == 0) && (k <= kMaxLdsK) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0);
    const size_t lds = fast ? (size_t)k * sizeof(float) : 0;
    Best* partial = reinterpret_cast<Best*>(workspace);
    hipLaunchKernelGGL(k_lmhead, dim3((unsigned)blocks), dim3(kBlock), lds, s, w, x, v, k, logits, partial, fast);
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(kFinalThreads), 0, s, (const Best*)partial, blocks, idx,
                       max_logit);
    return hipGetLastError();
}

}  // namespace qmv
