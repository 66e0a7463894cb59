// k_gemv.hip -- grouped weight-streaming GEMV for 1..16 tokens (gfx950).
//
// What is computed: for each problem, acc[m][r] = sum_c x8[m][c] * w[r][c]
// exactly in int32 and y = acc * sx[m] * sw ("Gemma 3 1B at 114 tokens per
// second on a laptop CPU", "Step 1": the weights are unpacked back to int8
// and multiplied with a 4-way int8 dot product, exact integer arithmetic;
// cpp20gemma README, "Architecture & implementation": the scales are applied
// once, after the dot).
//
// How (MI355X):
//  * Weights sit in the chunk-interleaved layout (chunk c of every row before
//    chunk c+1), so lane l of a wave owns row r0+l and a wave's 16-byte load of
//    one chunk is 1 KiB of contiguous HBM.  Each lane accumulates its own row:
//    no cross-lane reduction is needed; the 4 waves of a workgroup split the
//    row's chunks and meet in LDS at the end.
//  * The activation vector is staged once per workgroup in LDS, reordered into
//    trit-plane order (the page's "trit number i of 4 neighbouring bytes"
//    grouping, "Step 1"): inside each 80-column chunk,
//        xq[80c + 16i + 4w + b] = x8[80c + 20w + 5b + i],
//    so digit plane i of packed dword w meets the 4-byte x group it multiplies.
//    Every lane reads the same LDS address (a broadcast).
//  * Unpacking a packed dword (4 bytes, 20 trits) uses prefix quotients
//    P_j = floor(b / 3^(5-j)), j = 1..5 (P_5 = b).  Digit d_(5-j) = P_j - 3 P_(j-1),
//    so  sum_i d_i X_i = sum_j P_j . X_(5-j) - 3 sum_(j<5) P_j . X_(4-j):
//    two int32 accumulators, no digit subtraction.  floor(v/3) is one packed
//    fp16 FMA on two bytes held as fp16 values 1024 + v: the product-sum
//    (1024+v)*0.332763671875 + 683 rounds (round-to-nearest-even, exact
//    fused FMA) to 1024 + floor(v/3) for every v in 0..242, checked
//    exhaustively.  Four chained FMAs give P_4, P_3, P_2, P_1; v_perm_b32 gathers
//    the bytes into dot4 operands.  P_5 = b may exceed 127, so it enters as
//    b ^ 0x80 = b - 128 and 128 * sum(X_0) is added back.  From 4 tokens on
//    the digit planes themselves are formed once per dword instead (d_i =
//    Q_i - 3 Q_(i+1) bytewise, Q_i = floor(b / 3^i)), so each token needs 5
//    dot products rather than 9.  Trits are t = d - 1, so sum(x) is
//    subtracted.  All sums are modulo 2^32; the final value is exact whenever
//    the true dot fits int32.
#include "qmv_internal.hpp"
#include "unpack.hpp"

namespace qmv {
namespace {

constexpr int kBatch = 4;  // chunks in flight per lane
// From 4 tokens on, the digits of each packed dword are formed once (22 VALU)
// and each token costs 5 dot products instead of 9 (the prefix-quotient form,
// 15 VALU shared), and each lane takes two rows (see rows_per_lane).
// Measured on 24 BitNet-shaped layers: 4 tokens 96 -> 81 us, 16 tokens
// 462 -> 343 us; below 4 tokens the quotient form with one row per lane stays.
constexpr int kDigitMT = 4;

// Rows per lane: from kDigitMT tokens on each lane takes two rows (64 apart),
// so every activation read from LDS serves both; a tile is then 128 rows.
template <int MT, int WT>
constexpr int rows_per_lane()
{
    return (WT == 1 && MT >= kDigitMT) ? 2 : 1;
}

template <int MT, int WT>
__global__ __launch_bounds__(kBlock) void k_gemv(const DevProblem* __restrict__ probs,
                                                const uint32_t* __restrict__ tiles, int32_t tile_base)
{
    constexpr int RPL = rows_per_lane<MT, WT>();
    constexpr int kB = RPL == 1 ? kBatch : kBatch / 2;   // chunks in flight per row
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_sum[MT];
    __shared__ int s_sum0[MT];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    const uint32_t te = tiles[tile_base + blockIdx.x];
    const DevProblem* P = probs + (te >> kTileRowBits);
    const int rb = (int)(te & ((1u << kTileRowBits) - 1));
    const int n = P->n, k = P->k, m = P->m, C = P->chunks;
    const int row = rb * kRowsPerTile * RPL + lane;   // + 64 h for row h of the lane

    const int per = (C + 3) >> 2;
    const int c_lo = min(C, wave * per);
    const int c_hi = min(C, c_lo + per);

    const QMV_GLOBAL v4u32* wp = gload_ptr(reinterpret_cast<const v4u32*>(P->w)) + row;
    const size_t cstride = (size_t)n;
    bool live[RPL];
#pragma unroll
    for (int h = 0; h < RPL; ++h) live[h] = row + kWave * h < n;

    // Issue the first weight loads before staging the activations.
    v4u32 buf[kB][RPL];
#pragma unroll
    for (int u = 0; u < kB; ++u)
#pragma unroll
        for (int h = 0; h < RPL; ++h) {
            const int c = c_lo + u;
            buf[u][h] = (live[h] && c < c_hi) ? wp[(size_t)c * cstride + kWave * h] : v4u32{0u, 0u, 0u, 0u};
        }

    // ---- stage activations in LDS ------------------------------------------
    constexpr int kXBytesPerChunk = (WT == 1) ? 80 : 16;
    const int dw_per_tok = (kXBytesPerChunk / 4) * C;
    uint32_t* xs = reinterpret_cast<uint32_t*>(smem);
    if (WT == 1) {
        if (tid < MT) {
            s_sum[tid] = 0;
            s_sum0[tid] = 0;
        }
        __syncthreads();
    }
    if (WT == 1) {
        // one 20-column unit (packed dword w of chunk c, u = 4c + w) per step: its
        // aligned dwords loaded with a funnel shift (rows may start anywhere),
        // bytes past k cleared, then regrouped into the five planes
        const int units = 4 * C;
        for (int q = tid; q < m * units; q += kBlock) {
            const int mi = q / units;
            const int u = q - mi * units;
            const uintptr_t a = reinterpret_cast<uintptr_t>(P->x8) + (uintptr_t)mi * (uintptr_t)k;
            const uint32_t sh = (uint32_t)(a & 3);
            const uint32_t words = (sh + (uint32_t)k + 3u) >> 2;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(a & ~(uintptr_t)3), (short)0, (int)(4 * words), (int)0x00020000);
            uint32_t raw[6], nat[5], pl[5];
#pragma unroll
            for (int j = 0; j < 6; ++j) raw[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (5 * u + j), 0, 0);
            int sum = 0;
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const uint32_t v = __builtin_amdgcn_alignbyte(raw[j + 1], raw[j], sh);
                const int valid = k - 4 * (5 * u + j);
                nat[j] = valid >= 4 ? v : valid <= 0 ? 0u : v & ((1u << (8 * valid)) - 1u);
                sum = dot4(nat[j], 0x01010101u, sum);
            }
            reorder20(nat[0], nat[1], nat[2], nat[3], nat[4], pl);
            const int c = u >> 2, wd = u & 3;
#pragma unroll
            for (int i = 0; i < 5; ++i) xs[mi * dw_per_tok + 20 * c + 4 * i + wd] = pl[i];
            if (sum) atomicAdd(&s_sum[mi], sum);
            const int s0 = dot4(pl[0], 0x01010101u, 0);
            if (s0) atomicAdd(&s_sum0[mi], s0);
        }
    } else {
        for (int q = tid; q < m * dw_per_tok; q += kBlock) {
            const int mi = q / dw_per_tok;
            const int d = q - mi * dw_per_tok;
            const QMV_GLOBAL int8_t* xr = gload_ptr(P->x8) + (size_t)mi * k;
            uint32_t v = 0;
            const int col0 = 4 * d;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int col = col0 + b;
                const uint32_t byte = (col < k) ? (uint32_t)(uint8_t)xr[col] : 0u;
                v |= byte << (8 * b);
            }
            xs[q] = v;
        }
    }
    __syncthreads();

    // ---- stream the wave's chunks --------------------------------------------
    int acc_a[RPL][MT], acc_b[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int h = 0; h < RPL; ++h) acc_a[h][mi] = 0;
        acc_b[mi] = 0;
    }
    const uint4* xs4 = reinterpret_cast<const uint4*>(smem);
    const int x4_per_tok = dw_per_tok / 4;

    for (int c0 = c_lo; c0 < c_hi; c0 += kB) {
        v4u32 nxt[kB][RPL];
#pragma unroll
        for (int u = 0; u < kB; ++u)
#pragma unroll
            for (int h = 0; h < RPL; ++h) {
                const int c = c0 + kB + u;
                nxt[u][h] = (live[h] && c < c_hi) ? wp[(size_t)c * cstride + kWave * h] : v4u32{0u, 0u, 0u, 0u};
            }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int c = c0 + u;
            if (c < c_hi) {
                if (WT == 1 && MT >= kDigitMT) {
                    // digit planes D_i = Q_i - 3 Q_(i+1), Q_i = floor(b / 3^i) bytewise
                    // (each byte's result is 0..2 and 3 Q_(i+1) <= Q_i, so no byte borrows
                    // or carries), then 5 dot products per token
                    uint32_t D[RPL][4][5];
#pragma unroll
                    for (int h = 0; h < RPL; ++h)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t w = sel(buf[u][h], j);
                            const Planes q = unpack(w);
                            D[h][j][0] = w - (q.p4 + (q.p4 << 1));
                            D[h][j][1] = q.p4 - (q.p3 + (q.p3 << 1));
                            D[h][j][2] = q.p3 - (q.p2 + (q.p2 << 1));
                            D[h][j][3] = q.p2 - (q.p1 + (q.p1 << 1));
                            D[h][j][4] = q.p1;
                        }
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi) {
                        if (mi < m) {
                            const uint4* xq = xs4 + mi * x4_per_tok + 5 * c;
                            const uint4 X0 = xq[0], X1 = xq[1], X2 = xq[2], X3 = xq[3], X4 = xq[4];
#pragma unroll
                            for (int h = 0; h < RPL; ++h) {
                                int a = acc_a[h][mi];
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    a = dot4(D[h][j][0], sel(X0, j), a);
                                    a = dot4(D[h][j][1], sel(X1, j), a);
                                    a = dot4(D[h][j][2], sel(X2, j), a);
                                    a = dot4(D[h][j][3], sel(X3, j), a);
                                    a = dot4(D[h][j][4], sel(X4, j), a);
                                }
                                acc_a[h][mi] = a;
                            }
                        }
                    }
                } else if (WT == 1) {
                    Planes pl[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) pl[j] = unpack(sel(buf[u][0], j));
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi) {
                        if (mi < m) {
                            const uint4* xq = xs4 + mi * x4_per_tok + 5 * c;
                            const uint4 X0 = xq[0], X1 = xq[1], X2 = xq[2], X3 = xq[3], X4 = xq[4];
                            int a = acc_a[0][mi], b = acc_b[mi];
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
                            acc_a[0][mi] = a;
                            acc_b[mi] = b;
                        }
                    }
                } else {
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi) {
                        if (mi < m) {
                            const uint4 X = xs4[mi * x4_per_tok + c];
                            int a = acc_a[0][mi];
                            a = dot4(buf[u][0][0], X.x, a);
                            a = dot4(buf[u][0][1], X.y, a);
                            a = dot4(buf[u][0][2], X.z, a);
                            a = dot4(buf[u][0][3], X.w, a);
                            acc_a[0][mi] = a;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kB; ++u)
#pragma unroll
            for (int h = 0; h < RPL; ++h) buf[u][h] = nxt[u][h];
    }

    // ---- combine the four waves and write ------------------------------------
    // per row of the lane: the a sums of waves 1..3 (and b of the quotient form)
    int* red = reinterpret_cast<int*>(smem + (size_t)MT * dw_per_tok * 4);
    constexpr int kParts = RPL + 1;   // a per row, then b
    if (wave > 0) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
            for (int h = 0; h < RPL; ++h) red[(((wave - 1) * MT + mi) * kParts + h) * kWave + lane] = acc_a[h][mi];
            red[(((wave - 1) * MT + mi) * kParts + RPL) * kWave + lane] = acc_b[mi];
        }
    }
    __syncthreads();
    if (wave == 0) {
        const float sw = *gload_ptr(P->sw);
#pragma unroll
        for (int h = 0; h < RPL; ++h) {
            const int r = row + kWave * h;
            if (!live[h]) continue;
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                if (mi < m) {
                    int a = acc_a[h][mi], b = acc_b[mi];
#pragma unroll
                    for (int w = 0; w < 3; ++w) {
                        a += red[((w * MT + mi) * kParts + h) * kWave + lane];
                        b += red[((w * MT + mi) * kParts + RPL) * kWave + lane];
                    }
                    int total;
                    if (WT == 1 && MT >= kDigitMT) {
                        total = (int)((uint32_t)a - (uint32_t)s_sum[mi]);   // digits are t + 1
                    } else if (WT == 1) {
                        total = (int)((uint32_t)a + 128u * (uint32_t)s_sum0[mi] - 3u * (uint32_t)b -
                                      (uint32_t)s_sum[mi]);
                    } else {
                        total = a;
                    }
                    const size_t o = (size_t)mi * n + r;
                    gstore_ptr(P->y)[o] = (float)total * gload_ptr(P->sx)[mi] * sw;
                    if (P->acc) gstore_ptr(P->acc)[o] = total;
                }
            }
        }
    }
}

int mt_for(int max_m)
{
    return max_m <= 1 ? 1 : max_m <= 2 ? 2 : max_m <= 4 ? 4 : max_m <= 8 ? 8 : 16;
}

size_t lds_bytes(int mt, int wt, int max_chunks)
{
    const int rpl = (wt == 1 && mt >= kDigitMT) ? 2 : 1;
    return (size_t)(wt == 1 ? 80 : 16) * max_chunks * mt + (size_t)3 * mt * (rpl + 1) * kWave * 4;
}

template <int MT, int WT>
hipError_t launch_one(const DevProblem* probs, const uint32_t* tiles, int32_t tile_begin, int32_t tile_count,
                      int max_chunks, hipStream_t s)
{
    const size_t lds = lds_bytes(MT, WT, max_chunks);
    hipLaunchKernelGGL((k_gemv<MT, WT>), dim3((unsigned)tile_count), dim3(kBlock), lds, s, probs, tiles,
                       tile_begin);
    return hipGetLastError();
}

template <int WT>
hipError_t launch_wt(const DevProblem* probs, const uint32_t* tiles, int32_t tile_begin, int32_t tile_count,
                     int max_m, int max_chunks, hipStream_t s)
{
    if (max_m <= 1) return launch_one<1, WT>(probs, tiles, tile_begin, tile_count, max_chunks, s);
    if (max_m <= 2) return launch_one<2, WT>(probs, tiles, tile_begin, tile_count, max_chunks, s);
    if (max_m <= 4) return launch_one<4, WT>(probs, tiles, tile_begin, tile_count, max_chunks, s);
    if (max_m <= 8) return launch_one<8, WT>(probs, tiles, tile_begin, tile_count, max_chunks, s);
    return launch_one<16, WT>(probs, tiles, tile_begin, tile_count, max_chunks, s);
}

}  // namespace

int gemv_rows_per_tile(int wtype, int max_m)
{
    return kRowsPerTile * ((wtype == 1 && mt_for(max_m) >= kDigitMT) ? 2 : 1);
}

int64_t gemv_lds_bytes(int wtype, int max_m, int max_chunks)
{
    return (int64_t)lds_bytes(mt_for(max_m), wtype, max_chunks);
}

namespace {
template <int MT, int WT>
hipError_t lds_limit_one()
{
    return raise_lds_limit(reinterpret_cast<const void*>(&k_gemv<MT, WT>));
}

template <int WT>
hipError_t lds_limit_wt()
{
    hipError_t e = lds_limit_one<1, WT>();
    if (e == hipSuccess) e = lds_limit_one<2, WT>();
    if (e == hipSuccess) e = lds_limit_one<4, WT>();
    if (e == hipSuccess) e = lds_limit_one<8, WT>();
    if (e == hipSuccess) e = lds_limit_one<16, WT>();
    return e;
}
}  // namespace

hipError_t setup_workgroup_gemv_attributes()
{
    hipError_t e = lds_limit_wt<1>();
    return e == hipSuccess ? lds_limit_wt<2>() : e;
}

hipError_t launch_gemv(const DevProblem* probs, const uint32_t* tiles, int32_t tile_begin, int32_t tile_count,
                       int wtype, int max_m, int max_chunks, hipStream_t s)
{
    if (wtype == 1) return launch_wt<1>(probs, tiles, tile_begin, tile_count, max_m, max_chunks, s);
    return launch_wt<2>(probs, tiles, tile_begin, tile_count, max_m, max_chunks, s);
}

}  // namespace qmv
