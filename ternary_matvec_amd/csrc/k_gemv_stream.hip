// k_gemv_stream.hip -- persistent grouped GEMV for 1..2 tokens (gfx950).
//
// Same results as k_gemv.hip (exact int32 dot of int8 activations with
// five-trits-per-byte or int8 weights, scales applied once after the sum:
// "Gemma 3 1B at 114 tokens per second on a laptop CPU", "Step 1"; cpp20gemma
// README, "Architecture & implementation"), organised for streaming:
//
//  * Every wave is an independent worker with a static share of the tiles:
//    wave g takes tiles g, g + G, g + 2G, ... of the launch (G waves), and the
//    host lists tiles largest first.  No atomics, no workgroup barriers.
//  * A tile is 64 / L rows of one problem, L = lanes per row (1, 2 or 4,
//    larger for longer rows) so every tile moves a similar number of bytes.
//    Lane s*R + r (R = 64 / L rows) streams chunks s, s + L, ... of row r; for
//    a fixed s the R rows' chunk is one contiguous run of R * 16 bytes.  The L
//    partial sums of a row meet through lane shuffles at the end of the tile.
//  * A wave stages its tile's activations in its own LDS slice, already in
//    trit-plane order (the page's once-per-token input reorder); a wave-local
//    fence orders its LDS writes and reads.
#include "qmv_internal.hpp"
#include "unpack.hpp"

namespace qmv {
namespace {

#ifndef QMV_STREAM_BATCH
#define QMV_STREAM_BATCH 2
#endif
#ifndef QMV_STREAM_WAVES_PER_CU
#define QMV_STREAM_WAVES_PER_CU 16
#endif
#ifndef QMV_STREAM_MIN_WAVES_PER_EU
#define QMV_STREAM_MIN_WAVES_PER_EU 1
#endif
constexpr int kSBatch = QMV_STREAM_BATCH;  // chunks per step batch; the next batch is in flight meanwhile
constexpr int kStreamWavesPerCU = QMV_STREAM_WAVES_PER_CU;

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// One natural-order activation dword (columns 4d .. 4d+3 of a row of k int8
// values, k a multiple of 4, row 4-byte aligned): the load address is clamped
// into the row and bytes past column k are zeroed, so no lane branches.
__device__ __forceinline__ uint32_t x_dword(const QMV_GLOBAL uint32_t* xr4, int d, int k)
{
    const int last = (k >> 2) - 1;
    const uint32_t v = xr4[d < last ? d : last];
    const int valid = k - 4 * d;
    return valid >= 4 ? v : valid <= 0 ? 0u : v & ((1u << (8 * valid)) - 1u);
}

// Byte-wise variant for rows that are not 4-byte aligned or k % 4 != 0.
__device__ __forceinline__ uint32_t x_dword_bytes(const QMV_GLOBAL int8_t* xr, int d, int k)
{
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int col = 4 * d + b;
        v |= (col < k ? (uint32_t)(uint8_t)xr[col] : 0u) << (8 * b);
    }
    return v;
}

template <int MT, int WT>
__global__ __launch_bounds__(kBlock, QMV_STREAM_MIN_WAVES_PER_EU) void k_gemv_stream(const DevProblem* __restrict__ probs,
                                                       const uint32_t* __restrict__ tiles, int32_t tile_base,
                                                       int32_t tile_count, int32_t wave_lds_bytes)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint32_t* xl = reinterpret_cast<uint32_t*>(smem + (size_t)wave * wave_lds_bytes);
    const uint4* xl4 = reinterpret_cast<const uint4*>(xl);
    constexpr int kXdwPerChunk = (WT == 1) ? 20 : 4;

    const int gw = blockIdx.x * (kBlock / kWave) + wave;
    const int G = gridDim.x * (kBlock / kWave);
    for (int t = gw; t < tile_count; t += G) {
        const uint32_t te = tiles[tile_base + t];
        const DevProblem* P = probs + (te >> kTileRowBits);
        const int rb = (int)(te & ((1u << kTileRowBits) - 1));
        const int n = P->n, k = P->k, m = P->m, C = P->chunks;
        const int L = P->lanes_per_row;
        const int R = kWave / L;
        const int s_part = lane / R;            // which of the row's L chunk streams this lane takes
        const int row = rb * R + (lane - s_part * R);
        const bool live = row < n;
        // Loads are never predicated: dead rows read row n-1 and chunk indices
        // past the row read its last chunk; both are discarded (dead rows) or
        // meet the all-zero activation chunk C (see below).
        const QMV_GLOBAL v4u32* wp = gload_ptr(reinterpret_cast<const v4u32*>(P->w)) + (live ? row : n - 1);
        const size_t cstride = (size_t)n;
        const int nmax = (C + L - 1) / L;       // chunk steps of the row group (uniform)
        const int nsteps = (nmax + kSBatch - 1) / kSBatch * kSBatch;
        const int xdw_per_tok = kXdwPerChunk * (C + 1);

        // ---- activation loads for the first staging pass go out first ----------
        const bool fast_x = ((k & 3) == 0) && ((reinterpret_cast<uintptr_t>(P->x8) & 3) == 0);
        const int ngroups = (WT == 1) ? 4 * C : 4 * C;   // 20-column groups (ternary) or dwords (int8)
        uint32_t nat0[MT][5];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            const QMV_GLOBAL int8_t* xr = gload_ptr(P->x8) + (size_t)min(mi, m - 1) * k;
            const QMV_GLOBAL uint32_t* xr4 = reinterpret_cast<const QMV_GLOBAL uint32_t*>(xr);
#pragma unroll
            for (int j = 0; j < (WT == 1 ? 5 : 1); ++j) {
                const int d = (WT == 1) ? 5 * lane + j : lane;
                nat0[mi][j] = fast_x ? x_dword(xr4, d, k) : x_dword_bytes(xr, d, k);
            }
        }

        // ---- first batch of weights --------------------------------------------
        v4u32 buf[kSBatch];
#pragma unroll
        for (int u = 0; u < kSBatch; ++u) buf[u] = wp[(size_t)min(s_part + u * L, C - 1) * cstride];

        // ---- stage this tile's activations in the wave's LDS slice --------------
        // Chunk C of each token is all zeros: a lane whose row has no chunk left
        // at some step reads it, so that step adds nothing.
        int sum_all[MT], sum_d0[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            sum_all[mi] = 0;
            sum_d0[mi] = 0;
            if (mi < m) {
                const QMV_GLOBAL int8_t* xr = gload_ptr(P->x8) + (size_t)mi * k;
                const QMV_GLOBAL uint32_t* xr4 = reinterpret_cast<const QMV_GLOBAL uint32_t*>(xr);
                uint32_t* xo = xl + mi * xdw_per_tok;
                if (lane < kXdwPerChunk) xo[kXdwPerChunk * C + lane] = 0u;
                int s_all = 0, s_0 = 0;
                for (int g = lane; g < ngroups; g += kWave) {
                    if (WT == 1) {
                        uint32_t nat[5];
                        if (g == lane) {
#pragma unroll
                            for (int j = 0; j < 5; ++j) nat[j] = nat0[mi][j];
                        } else {
#pragma unroll
                            for (int j = 0; j < 5; ++j)
                                nat[j] = fast_x ? x_dword(xr4, 5 * g + j, k) : x_dword_bytes(xr, 5 * g + j, k);
                        }
                        uint32_t pl[5];
                        reorder20(nat[0], nat[1], nat[2], nat[3], nat[4], pl);
                        const int c = g >> 2, w = g & 3;
#pragma unroll
                        for (int i = 0; i < 5; ++i) {
                            xo[20 * c + 4 * i + w] = pl[i];
                            s_all = dot4(pl[i], 0x01010101u, s_all);
                        }
                        s_0 = dot4(pl[0], 0x01010101u, s_0);
                    } else {
                        xo[g] = (g == lane) ? nat0[mi][0] : (fast_x ? x_dword(xr4, g, k) : x_dword_bytes(xr, g, k));
                    }
                }
                if (WT == 1) {
                    sum_all[mi] = wave_sum(s_all);
                    sum_d0[mi] = wave_sum(s_0);
                }
            }
        }
        wave_lds_sync();

        // ---- stream the tile ---------------------------------------------------
        // Two register batches in ping-pong: batch b+1's loads are issued before
        // batch b is consumed, so a batch is always in flight.  Loads past the
        // last step re-read the row's last chunk (a cache hit) and are unused.
        int acc_a[MT], acc_b[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            acc_a[mi] = 0;
            acc_b[mi] = 0;
        }
        const int x4_per_tok = xdw_per_tok / 4;
        auto load_batch = [&](v4u32* dst, int i0) {
#pragma unroll
            for (int u = 0; u < kSBatch; ++u) dst[u] = wp[(size_t)min(s_part + (i0 + u) * L, C - 1) * cstride];
        };
        auto run_batch = [&](const v4u32* src, int i0) {
#pragma unroll
            for (int u = 0; u < kSBatch; ++u) {
                const int c = min(s_part + (i0 + u) * L, C);   // C = the zero activation chunk
                if (WT == 1) {
                    Planes pl[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) pl[j] = unpack(src[u][j]);
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi) {
                        if (mi < m) {
                            const uint4* xq = xl4 + mi * x4_per_tok + 5 * c;
                            const uint4 X0 = xq[0], X1 = xq[1], X2 = xq[2], X3 = xq[3], X4 = xq[4];
                            int a = acc_a[mi], b = acc_b[mi];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const uint32_t x0 = sel(X0, j), x1 = sel(X1, j), x2 = sel(X2, j);
                                const uint32_t x3 = sel(X3, j), x4 = sel(X4, j);
                                a = dot4(pl[j].p1, x4, a);
                                a = dot4(pl[j].p2, x3, a);
                                a = dot4(pl[j].p3, x2, a);
                                a = dot4(pl[j].p4, x1, a);
                                a = dot4(pl[j].b5, x0, a);
                                b = dot4(pl[j].p1, x3, b);
                                b = dot4(pl[j].p2, x2, b);
                                b = dot4(pl[j].p3, x1, b);
                                b = dot4(pl[j].p4, x0, b);
                            }
                            acc_a[mi] = a;
                            acc_b[mi] = b;
                        }
                    }
                } else {
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi) {
                        if (mi < m) {
                            const uint4 X = xl4[mi * x4_per_tok + c];
                            int a = acc_a[mi];
                            a = dot4(src[u][0], X.x, a);
                            a = dot4(src[u][1], X.y, a);
                            a = dot4(src[u][2], X.z, a);
                            a = dot4(src[u][3], X.w, a);
                            acc_a[mi] = a;
                        }
                    }
                }
            }
        };
        v4u32 bufb[kSBatch];
        for (int i0 = 0; i0 < nsteps; i0 += 2 * kSBatch) {
            load_batch(bufb, i0 + kSBatch);
            run_batch(buf, i0);
            load_batch(buf, i0 + 2 * kSBatch);
            if (i0 + kSBatch < nsteps) run_batch(bufb, i0 + kSBatch);
        }

        // ---- combine the L lanes of each row and write the tile --------------------
        for (int off = R; off < kWave; off <<= 1) {
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                acc_a[mi] += __shfl_xor(acc_a[mi], off, kWave);
                acc_b[mi] += __shfl_xor(acc_b[mi], off, kWave);
            }
        }
        if (live && s_part == 0) {
            const float sw = *gload_ptr(P->sw);
            const QMV_GLOBAL float* sx = gload_ptr(P->sx);
            QMV_GLOBAL float* y = gstore_ptr(P->y);
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                if (mi < m) {
                    int total;
                    if (WT == 1)
                        total = (int)((uint32_t)acc_a[mi] + 128u * (uint32_t)sum_d0[mi] -
                                      3u * (uint32_t)acc_b[mi] - (uint32_t)sum_all[mi]);
                    else
                        total = acc_a[mi];
                    const size_t o = (size_t)mi * n + row;
                    y[o] = (float)total * sx[mi] * sw;
                    if (P->acc) gstore_ptr(P->acc)[o] = total;
                }
            }
        }
        // the next tile overwrites this wave's LDS slice
        wave_lds_sync();
    }
}

template <int MT, int WT>
hipError_t launch_stream_one(const DevProblem* probs, const uint32_t* tiles, int32_t tile_begin, int32_t tile_count,
                             int max_chunks, int cus, hipStream_t s)
{
    const int wave_lds = (WT == 1 ? 80 : 16) * (max_chunks + 1) * MT;
    int waves_per_cu = kStreamWavesPerCU;
    const int lds_waves = (int)(kMaxLds / (wave_lds > 0 ? wave_lds : 1)) & ~3;
    if (lds_waves < waves_per_cu) waves_per_cu = lds_waves < 4 ? 4 : lds_waves;
    int blocks = cus * waves_per_cu / 4;
    const int max_blocks = (tile_count + 3) / 4;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    const size_t lds = (size_t)wave_lds * 4;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_stream<MT, WT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_gemv_stream<MT, WT>), dim3((unsigned)blocks), dim3(kBlock), lds, s, probs, tiles,
                       tile_begin, tile_count, wave_lds);
    return hipGetLastError();
}

}  // namespace

int gemv_stream_lanes_per_row(int chunks)
{
    return chunks <= 32 ? 1 : chunks <= 64 ? 2 : 4;
}

bool gemv_stream_fits(int wtype, int max_m, int max_chunks)
{
    const int mt = max_m <= 1 ? 1 : 2;
    return max_m <= 2 && (int64_t)(wtype == 1 ? 80 : 16) * (max_chunks + 1) * mt * 4 <= 64 * 1024;
}

hipError_t launch_gemv_stream(const DevProblem* probs, const uint32_t* tiles, int32_t tile_begin, int32_t tile_count,
                              int wtype, int max_m, int max_chunks, hipStream_t s)
{
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (wtype == 1) {
        if (max_m <= 1) return launch_stream_one<1, 1>(probs, tiles, tile_begin, tile_count, max_chunks, cus, s);
        return launch_stream_one<2, 1>(probs, tiles, tile_begin, tile_count, max_chunks, cus, s);
    }
    if (max_m <= 1) return launch_stream_one<1, 2>(probs, tiles, tile_begin, tile_count, max_chunks, cus, s);
    return launch_stream_one<2, 2>(probs, tiles, tile_begin, tile_count, max_chunks, cus, s);
}

}  // namespace qmv
