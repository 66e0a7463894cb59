// k_prefill.hip -- grouped ternary GEMM for many tokens on int8 matrix cores (gfx950).
//
// acc[m][r] = sum_c x8[m][c] * t[r][c] exactly, y = acc * sx[m] * sw, for all
// prompt tokens of a matrix in one pass over its weights ("Gemma 3 1B at 114
// tokens per second on a laptop CPU", "Step 1": prompt processing runs every
// prompt token through each weight matrix in one pass; cpp20gemma README,
// "Architecture & implementation": scales applied once after the dot).
//
// Work: a workgroup (4 waves) owns a 256-token x 256-row tile of one problem;
// wave w owns rows 64w..64w+63 (two 32-row blocks) for all 256 tokens (eight
// 32-token blocks): 16 accumulators of v_mfma_i32_32x32x32_i8.  The K loop
// advances two 16-byte chunks (160 columns) per step.
//  * A (activations, natural column order): the step's 256 x 160 tile is
//    copied HBM -> LDS with global_load_lds_dwordx4 (no registers), double
//    buffered; operand i of lane (m, g) is columns 80g + 16i .. +15 of row m.
//  * B (weights): lane (r = lane % 32, g = lane / 32) loads chunk 2s+g of its
//    row and expands the 16 packed bytes into 80 digits d = t + 1 in natural
//    column order, in registers: floor(b/3^j) by the packed-fp16 chain of
//    unpack.hpp, digit j = P_(5-j) - 3 P_(4-j) by one packed 16-bit
//    multiply-add per two bytes, then byte permutes into column order.
//  * 5 MFMAs per (token block, row block) cover the 160 columns.  Because the
//    digits are t + 1, the epilogue subtracts sum_c x8[m][c], summed from the
//    staged tile.  Columns at or past k meet zeroed B operands.
// Operand layout of v_mfma_i32_32x32x32_i8 (checked on the hardware): A row =
// B column = lane % 32, lanes 32..63 hold the second 16 K-bytes; accumulator
// register i of lane l is row 8*(i/4) + 4*(l/32) + i%4, column l % 32.
#include "qmv_internal.hpp"
#include "unpack.hpp"

namespace qmv {
namespace {

typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef int v16i32 __attribute__((ext_vector_type(16)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr int kPBM = 256;                 // tokens per tile
constexpr int kPBN = 256;                 // rows per tile (64 per wave)
constexpr int kSlots = 11;                // 16-byte slots per staged token row (10 used)
constexpr int kARow = 16 * kSlots;        // 176 bytes: odd number of 16-byte units
constexpr int kABuf = kPBM * kARow;       // one staged A buffer (45056 bytes)
constexpr int kANBuf = 3;                 // staged buffers (two steps in flight)
constexpr int kBBuf = 4 * 2 * 64 * 16;    // one staged B buffer: wave x row block x lane x 16 bytes
constexpr int kBOff = kANBuf * kABuf;     // B ring after the A ring
constexpr int kEpiOff = kBOff + kANBuf * kBBuf;
constexpr int kPrefillLds = kEpiOff + 2 * kPBM * 4;   // 161792 bytes of the 163840 per CU
constexpr int kParkPitch = kPBN + 4;      // parked row pitch (ints): 16-byte rows, token rows 4 banks apart

// (1024 + P_(j-1), 1024 + P_j) per 16-bit lane -> low byte = P_j - 3 P_(j-1).
__device__ __forceinline__ uint32_t digit2(uint32_t prev, uint32_t cur)
{
    const s16x2 m3 = {-3, -3};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, prev) * m3 + __builtin_bit_cast(s16x2, cur));
}

// One packed dword (20 trits, columns 0..19 relative) -> five dwords of
// digits d = t + 1 in natural column order: nat[u] holds columns 4u .. 4u+3.
__device__ __forceinline__ void natural_digits(uint32_t w, uint32_t nat[5])
{
    const uint32_t mag = 0x64646464u;
    const uint32_t lo = __builtin_amdgcn_perm(mag, w, 0x04020400u);  // [b0 64 b2 64]
    const uint32_t hi = __builtin_amdgcn_perm(mag, w, 0x04030401u);  // [b1 64 b3 64]
    const uint32_t L4 = third2(lo), H4 = third2(hi);
    const uint32_t L3 = third2(L4), H3 = third2(H4);
    const uint32_t L2 = third2(L3), H2 = third2(H3);
    const uint32_t L1 = third2(L2), H1 = third2(H2);
    // digit i of bytes (b0, b2) in the low bytes of E_iL, of (b1, b3) in E_iH
    const uint32_t E4L = L1, E4H = H1;
    const uint32_t E3L = digit2(L1, L2), E3H = digit2(H1, H2);
    const uint32_t E2L = digit2(L2, L3), E2H = digit2(H2, H3);
    const uint32_t E1L = digit2(L3, L4), E1H = digit2(H3, H4);
    const uint32_t E0L = digit2(L4, lo), E0H = digit2(H4, hi);
    const uint32_t X01L = __builtin_amdgcn_perm(E1L, E0L, bsel(0, 4, 2, 6));  // d0 b0, d1 b0, d0 b2, d1 b2
    const uint32_t X23L = __builtin_amdgcn_perm(E3L, E2L, bsel(0, 4, 2, 6));  // d2 b0, d3 b0, d2 b2, d3 b2
    const uint32_t X01H = __builtin_amdgcn_perm(E1H, E0H, bsel(0, 4, 2, 6));  // d0 b1, d1 b1, d0 b3, d1 b3
    const uint32_t X23H = __builtin_amdgcn_perm(E3H, E2H, bsel(0, 4, 2, 6));  // d2 b1, d3 b1, d2 b3, d3 b3
    const uint32_t X4 = __builtin_amdgcn_perm(E4H, E4L, bsel(0, 4, 2, 6));    // d4 of b0 b1 b2 b3
    nat[0] = __builtin_amdgcn_perm(X23L, X01L, bsel(0, 1, 4, 5));
    nat[1] = __builtin_amdgcn_perm(X23H, __builtin_amdgcn_perm(X01H, X4, bsel(0, 4, 5, 12)), bsel(0, 1, 2, 4));
    nat[2] = __builtin_amdgcn_perm(X01L, __builtin_amdgcn_perm(X4, X23H, bsel(1, 5, 12, 12)), bsel(0, 1, 6, 7));
    nat[3] = __builtin_amdgcn_perm(X01H, __builtin_amdgcn_perm(X4, X23L, bsel(2, 3, 6, 12)), bsel(0, 1, 2, 6));
    nat[4] = __builtin_amdgcn_perm(X4, __builtin_amdgcn_perm(X23H, X01H, bsel(3, 6, 7, 12)), bsel(0, 1, 2, 7));
}

// Byte-wise activation dword for rows that are not 16-byte aligned.
__device__ __forceinline__ uint32_t x_bytes(const QMV_GLOBAL int8_t* xr, int col, int k)
{
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) v |= (col + b < k ? (uint32_t)(uint8_t)xr[col + b] : 0u) << (8 * b);
    return v;
}

__global__ __launch_bounds__(kBlock, 1) void k_prefill(const DevProblem* __restrict__ probs,
                                                       const uint64_t* __restrict__ tiles)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 5;  // which 16 K-bytes of the MFMA operands this lane holds
    const int l32 = lane & 31;

    const uint64_t te = tiles[blockIdx.x];
    if (te == ~0ull) return;  // padding entry of the XCD-ordered tile list
    const DevProblem* P = probs + (int)(te >> 48);
    const int mt = (int)((te >> 32) & 0xFFFF);
    const int nt = (int)(te & 0xFFFFFFFFu);
    const int n = P->n, k = P->k, mtok = P->m, C = P->chunks;
    const int m0 = mt * kPBM, n0 = nt * kPBN;
    const int steps = (C + 1) >> 1;

    // ---- B addressing: two 32-row blocks per wave ----------------------------------
    const QMV_GLOBAL v4u32* wbase = gload_ptr(reinterpret_cast<const v4u32*>(P->w));
    static_assert(kPrefillLds <= 160 * 1024, "LDS budget of one CU");
    int brow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int r = n0 + 64 * wave + 32 * nb + l32;
        brow[nb] = r < n ? r : n - 1;
    }
    // B goes HBM -> LDS too (lane l of a row block -> 16 bytes at lane * 16), so
    // the two-step prefetch needs no registers; each lane reads its own chunk back.
    auto stage_b = [&](int s, int buf) {
        const int c = min(2 * s + g, C - 1);
        uint8_t* bbuf = smem + kBOff + buf * kBBuf;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            __builtin_amdgcn_global_load_lds((const void QMV_GLOBAL*)(wbase + (size_t)c * n + brow[nb]),
                                             (void __attribute__((address_space(3)))*)(bbuf + 1024 * (2 * wave + nb)),
                                             16, 0, 0);
    };

    // ---- A staging ---------------------------------------------------------------
    // Fast path: slot f of a buffer = row f / 11, 16-byte piece f % 11 (piece 10 is
    // padding); wave w fills slots [64 (11 w + j), +64) for j = 0..10, one per lane.
    const QMV_GLOBAL int8_t* xbase = gload_ptr(P->x8);
    const bool fast = ((k & 15) == 0) && ((reinterpret_cast<uintptr_t>(P->x8) & 15) == 0);
    const int f0 = 64 * kSlots * wave + lane;
    auto stage_a = [&](int s, int buf) {
        uint8_t* abuf = smem + buf * kABuf;
        if (fast) {
            const int colmax = k - 16;
#pragma unroll
            for (int j = 0; j < kSlots; ++j) {
                const int f = f0 + 64 * j;
                const int r = f / kSlots;
                const int p = f - r * kSlots;
                const int tok = min(m0 + r, mtok - 1);
                const int col = min(160 * s + 16 * min(p, 9), colmax);
                __builtin_amdgcn_global_load_lds(
                    (const void QMV_GLOBAL*)(xbase + (size_t)tok * k + col),
                    (void __attribute__((address_space(3)))*)(abuf + 1024 * (kSlots * wave + j)), 16, 0, 0);
            }
        } else {
            // thread t writes row t: 40 dwords, zero past column k or past the last token
            const int tok = m0 + tid;
            uint32_t* row = reinterpret_cast<uint32_t*>(abuf + tid * kARow);
            const QMV_GLOBAL int8_t* xr = xbase + (size_t)min(tok, mtok - 1) * k;
            for (int d = 0; d < 40; ++d) row[d] = tok < mtok ? x_bytes(xr, 160 * s + 4 * d, k) : 0u;
        }
    };
    // sum of row tid's staged columns below k
    int rsum = 0;
    auto sum_a = [&](int s, int buf) {
        const uint4* row = reinterpret_cast<const uint4*>(smem + buf * kABuf + tid * kARow);
#pragma unroll
        for (int p = 0; p < 10; ++p) {
            if (160 * s + 16 * p < k) {
                const uint4 v = row[p];
                rsum = dot4(v.x, 0x01010101u, rsum);
                rsum = dot4(v.y, 0x01010101u, rsum);
                rsum = dot4(v.z, 0x01010101u, rsum);
                rsum = dot4(v.w, 0x01010101u, rsum);
            }
        }
    };
    v16i32 acc[8][2];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = v16i32{};

    // Digits of step s: this lane's 16 packed bytes of each row block (braw, read
    // from the B ring) -> 5 B operands of 16 natural-order digits each.  Work is
    // split in parts so it can ride along the MFMAs: part j (0..3) expands dword j
    // of both row blocks, part 4 assembles the operands (zero past column k).
    uint32_t nat[2][20];
    auto read_b = [&](int buf, v4u32 (&braw)[2]) {
        const uint8_t* bbuf = smem + kBOff + buf * kBBuf;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            braw[nb] = *reinterpret_cast<const v4u32*>(bbuf + 1024 * (2 * wave + nb) + 16 * lane);
    };
    auto digits_part = [&](int s, const v4u32 (&braw)[2], int part, v4i32 (&bop)[2][5]) {
        if (part < 4) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) natural_digits(braw[nb][part], nat[nb] + 5 * part);
        } else {
            const int cbase = 80 * (2 * s + g);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    const bool on = cbase + 16 * i < k;   // columns past k (and chunks past the row) add 0
                    bop[nb][i] = on ? v4i32{(int)nat[nb][4 * i], (int)nat[nb][4 * i + 1], (int)nat[nb][4 * i + 2],
                                            (int)nat[nb][4 * i + 3]}
                                    : v4i32{0, 0, 0, 0};
                }
        }
    };

    // Pipeline: at step s the MFMAs use A(s) (LDS) and the digits of B(s)
    // (registers, expanded during step s-1, assembled into operands at its end),
    // while the digits of B(s+1) are expanded and the loads of step s+2 fly.  Issue order per step is B then A,
    // so "B(s+2) and everything older has landed" is vmcnt(A loads of one step).
    stage_b(0, 0);
    stage_a(0, 0);
    if (steps > 1) {
        stage_b(1, 1);
        stage_a(1, 1);
    }
    wait_vmcnt<0>();
    __syncthreads();
    sum_a(0, 0);
    v4i32 bop[2][5];
    {
        v4u32 braw[2];
        read_b(0, braw);
#pragma unroll
        for (int part = 0; part < 5; ++part) digits_part(0, braw, part, bop);
    }

    for (int s = 0; s < steps; ++s) {
        const int buf = s % kANBuf;
        const bool more = s + 1 < steps;
        const bool more2 = s + 2 < steps;
        if (more2) {
            stage_b(s + 2, (s + 2) % kANBuf);
            stage_a(s + 2, (s + 2) % kANBuf);
        }
        // Plane-outer order: each accumulator is touched once per plane, so 16
        // independent MFMAs separate two that depend on each other.  The A
        // operands of plane i+1 are read from LDS and a fifth of the next step's
        // digit expansion is done while plane i's MFMAs run (one wave per SIMD:
        // nothing else would hide the LDS latency or fill the MFMA pipe).
        // the next step's packed weights (stale data after the last step: expanded
        // and never used, which keeps the MFMA block free of branches)
        v4u32 bnext[2];
        read_b((s + 1) % kANBuf, bnext);
        const uint8_t* arow = smem + buf * kABuf + l32 * kARow + 80 * g;
        // A operands in half planes (4 token blocks): the next half's reads fly
        // while the current half's 8 MFMAs run
        v4i32 aop[2][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) aop[0][mb] = *reinterpret_cast<const v4i32*>(arow + 32 * mb * kARow);
        auto plane = [&](int i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int hs = 2 * i + h;                 // half-plane index 0..9
                if (hs + 1 < 10) {
                    const int ni = (hs + 1) >> 1, nh = (hs + 1) & 1;
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
                        aop[(hs + 1) & 1][mb] =
                            *reinterpret_cast<const v4i32*>(arow + 32 * (4 * nh + mb) * kARow + 16 * ni);
                }
                if (h == 0 && i < 4) {
                    digits_part(s + 1, bnext, i, bop);
                    // keep this part's work here, among the MFMAs (the compiler
                    // would otherwise sink it to the end of the step)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        asm volatile("" ::"v"(nat[nb][5 * i]), "v"(nat[nb][5 * i + 1]), "v"(nat[nb][5 * i + 2]),
                                     "v"(nat[nb][5 * i + 3]), "v"(nat[nb][5 * i + 4]));
                }
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const int tb = 4 * h + mb;
                    acc[tb][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[hs & 1][mb], bop[0][i], acc[tb][0], 0, 0, 0);
                    acc[tb][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[hs & 1][mb], bop[1][i], acc[tb][1], 0, 0, 0);
                }
                // one MFMA (its operands were read a half plane ago), then the next
                // half's LDS reads, then one MFMA per few VALU ops
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
#pragma unroll
                for (int q = 1; q < 8; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
#pragma unroll
        for (int i = 0; i < 5; ++i) plane(i);
        // the next step's operands replace this step's once its MFMAs are issued
        digits_part(s + 1, bnext, 4, bop);
        if (more) {
            // A(s+1) and B(s+2) have landed once only A(s+2) may still fly
            if (more2 && fast) wait_vmcnt<kSlots>();
            else wait_vmcnt<0>();
            __syncthreads();
            sum_a(s + 1, (s + 1) % kANBuf);
        }
    }

    // ---- per-token sums and scales in LDS, then the epilogue -------------------------
    int* tsum = reinterpret_cast<int*>(smem + kEpiOff);
    float* tscale = reinterpret_cast<float*>(smem + kEpiOff + kPBM * 4);
    __syncthreads();
    {
        const float sw = *gload_ptr(P->sw);
        const int tok = m0 + tid;
        tsum[tid] = rsum;
        tscale[tid] = tok < mtok ? gload_ptr(P->sx)[tok] * sw : 0.0f;
    }
    __syncthreads();
    // The tile leaves through LDS, 128 tokens at a time: the exact sums (acc
    // minus the token's digit offset) are parked as [token][row] and written out
    // as whole 1 KB token rows with 16-byte stores, y = sum * sx * sw (long
    // contiguous writes instead of 128-byte pieces per accumulator register).
    QMV_GLOBAL float* y = gstore_ptr(P->y);
    QMV_GLOBAL int32_t* accout = P->acc ? gstore_ptr(P->acc) : nullptr;
    const bool vec = ((reinterpret_cast<uintptr_t>(P->y) & 15) == 0) && ((n & 3) == 0) &&
                     (!P->acc || (reinterpret_cast<uintptr_t>(P->acc) & 15) == 0);
    int* park = reinterpret_cast<int*>(smem);   // [128][kParkPitch]
    static_assert(128 * kParkPitch * 4 <= kEpiOff, "parking fits below the token sums");
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int mh = 0; mh < 4; ++mh) {
            const int mb = 4 * half + mh;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int ml = 32 * mb + 8 * q4 + 4 * g;   // tile token of register 4*q4 (+e)
                const int4 ts = *reinterpret_cast<const int4*>(tsum + ml);
                const int tsv[4] = {ts.x, ts.y, ts.z, ts.w};
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        park[(ml + e - 128 * half) * kParkPitch + 64 * wave + 32 * nb + l32] =
                            acc[mb][nb][4 * q4 + e] - tsv[e];
            }
        }
        __syncthreads();
        for (int it = 0; it < 128 / 4; ++it) {
            const int tl = 4 * it + wave;                  // token within the half
            const int tok = m0 + 128 * half + tl;
            const int r = n0 + 4 * lane;
            if (tok < mtok && r < n) {
                const int4 v = *reinterpret_cast<const int4*>(park + tl * kParkPitch + 4 * lane);
                const float sc = tscale[128 * half + tl];
                const size_t o = (size_t)tok * n + r;
                if (vec && r + 3 < n) {
                    *reinterpret_cast<QMV_GLOBAL v4u32*>(y + o) =
                        v4u32{__float_as_uint((float)v.x * sc), __float_as_uint((float)v.y * sc),
                              __float_as_uint((float)v.z * sc), __float_as_uint((float)v.w * sc)};
                    if (accout)
                        *reinterpret_cast<QMV_GLOBAL v4u32*>(accout + o) =
                            v4u32{(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
                } else {
                    const int vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (r + e < n) {
                            y[o + e] = (float)vv[e] * sc;
                            if (accout) accout[o + e] = vv[e];
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

int64_t prefill_tiles(int64_t m, int64_t n) { return ((m + kPBM - 1) / kPBM) * ((n + kPBN - 1) / kPBN); }

void prefill_tile_entries(int32_t slot, int64_t m, int64_t n, uint64_t* out)
{
    const int64_t mts = (m + kPBM - 1) / kPBM, nts = (n + kPBN - 1) / kPBN;
    int64_t i = 0;
    for (int64_t mt = 0; mt < mts; ++mt)
        for (int64_t nt = 0; nt < nts; ++nt) out[i++] = ((uint64_t)slot << 48) | ((uint64_t)mt << 32) | (uint64_t)nt;
}

hipError_t launch_prefill(const DevProblem* probs, const uint64_t* tiles, int64_t tile_count, hipStream_t s)
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_prefill),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPrefillLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_prefill, dim3((unsigned)tile_count), dim3(kBlock), kPrefillLds, s, probs, tiles);
    return hipGetLastError();
}

}  // namespace qmv
