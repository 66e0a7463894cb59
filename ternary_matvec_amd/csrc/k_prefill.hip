// k_prefill.hip -- grouped ternary GEMM for many tokens on int8 matrix cores (gfx950).
//
// acc[m][r] = sum_c x8[m][c] * t[r][c] exactly, y = acc * sx[m] * sw, for all
// prompt tokens of a matrix in one pass over its weights ("Gemma 3 1B at 114
// tokens per second on a laptop CPU", "Step 1": prompt processing runs every
// prompt token through each weight matrix in one pass; cpp20gemma README,
// "Architecture & implementation": scales applied once after the dot).
//
// Work: a workgroup (4 waves) owns a 128-token x 256-row tile of one problem;
// wave w owns rows 64w..64w+63 (two 32-row blocks) for all 128 tokens (four
// 32-token blocks): 8 accumulators of v_mfma_i32_32x32x32_i8 in 128 registers.
// Two workgroups share a compute unit (registers and LDS are sized for it), so
// the output stores of one drain while the matrix cores run the other.  The K
// loop advances two 16-byte chunks (160 columns) per step.
//  * Weights are the MFMA B operand (rows): lane (r = lane % 32, g = lane / 32)
//    takes chunk 2s+g of its row, HBM -> LDS (two-step ring) -> registers, and
//    expands its 16 packed bytes into 80 digits d = t + 1 in natural column
//    order, one packed dword per plane just ahead of the plane that uses it:
//    floor(b/3^j) by the packed-fp16 chain of unpack.hpp, digit j = P_(5-j) -
//    3 P_(4-j) by one packed 16-bit multiply-add per two bytes, then byte
//    permutes into column order.
//  * Activations are the A operand (tokens): the step's 128 x 160 tile goes
//    HBM -> LDS (three-step ring) with global_load_lds_dwordx4, no registers.
//    Columns at or past k are copied from a block of zeros, so whatever digits
//    meet them (row padding, clamped chunks) add nothing.
//  * 5 MFMAs per (row block, token block) cover the 160 columns.  Because the
//    digits are t + 1, the epilogue subtracts sum_c x8[m][c], summed from the
//    staged tiles.
//  * C = activations x digits^T: a register of the accumulators holds, per
//    half-wave, 32 consecutive outputs of one token; the epilogue stores whole
//    128-byte lines straight from the registers.
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

constexpr int kPBM = (int)kPrefillTileM;  // tokens per tile (128)
constexpr int kPBN = (int)kPrefillTileN;  // rows per tile (256, 64 per wave)
constexpr int kPieces = 10;               // 16-byte pieces per staged token row (160 columns)
constexpr int kARow = 16 * kPieces;       // 160 bytes, rows 8..15 of each 16 rotated by one piece
constexpr int kABuf = kPBM * kARow;       // one staged activation buffer (20480 bytes)
constexpr int kANBuf = 3;                 // activation ring: the step in use + two in flight
constexpr int kADma = kABuf / (16 * kBlock);   // activation copies per wave per step (5)
constexpr int kBBuf = 4 * 2 * 64 * 16;    // one staged weight buffer: wave x row block x lane x 16 bytes
constexpr int kBNBuf = 2;                 // weight ring: read into registers one step ahead
constexpr int kBOff = kANBuf * kABuf;
constexpr int kEpiOff = kBOff + kBNBuf * kBBuf;
constexpr int kPrefillLds = kEpiOff + 3 * kPBM * 4;   // + token sums (two halves) and scales: 79360 bytes
static_assert(kADma * 16 * kBlock == kABuf, "activation tile splits evenly over the copies");
static_assert(2 * kPrefillLds <= 160 * 1024, "two workgroups per compute unit");

// Byte offset of 16-byte piece p (0..9) of staged token row r.  Rows 8..15 of
// every 16 are rotated by one piece, so 16 lanes reading one piece of 16
// consecutive rows cover all 64 banks.
__device__ __forceinline__ int apos(int r, int p)
{
    const int q = p + ((r >> 3) & 1);
    return r * kARow + 16 * (q >= kPieces ? q - kPieces : q);
}

// Workgroup barrier for LDS hand-offs that leaves this wave's copies into LDS
// in flight: it waits only for the wave's own LDS (and scalar) accesses; the
// copies a hand-off depends on are waited for explicitly (wait_vmcnt) before
// it.  The memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// HBM -> LDS copy of 16 bytes per lane: lane i's bytes land at lds + 16 i (lds
// wave-uniform).  Issued as inline assembly so that the compiler's wait-count
// pass does not track it: it would wait for every copy in flight before each
// later LDS read, which allows no copy to overlap a step.  The kernel waits for
// these copies itself (wait_vmcnt) before the barrier that hands them over.
// M0 is written here; this kernel has no other use of it (LDS instructions do
// not read it on gfx9 and later).
__device__ __forceinline__ void copy16_to_lds(const void QMV_GLOBAL* src, const uint8_t* lds)
{
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(a) : "memory");
}

// (1024 + P_(j-1), 1024 + P_j) per 16-bit lane -> low byte = P_j - 3 P_(j-1).
__device__ __forceinline__ uint32_t digit2(uint32_t prev, uint32_t cur)
{
    const s16x2 m3 = {-3, -3};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, prev) * m3 + __builtin_bit_cast(s16x2, cur));
}

// One packed dword (20 trits, columns 0..19 relative) -> five dwords of
// digits d = t + 1 in natural column order: nat[u] holds columns 4u .. 4u+3.
__device__ __forceinline__ void natural_digits(uint32_t w, uint32_t* nat)
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

__global__ __launch_bounds__(kBlock, 2) void k_prefill(const DevProblem* __restrict__ probs,
                                                       const uint64_t* __restrict__ tiles,
                                                       const int8_t* __restrict__ zeros)
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

    // ---- weights: two 32-row blocks per wave, HBM -> LDS ------------------------------
    // lane l of a row block -> 16 bytes at l * 16 of the wave's region; each
    // lane reads its own chunk back.  Rows past n repeat row n - 1 (never stored).
    const QMV_GLOBAL v4u32* wbase = gload_ptr(reinterpret_cast<const v4u32*>(P->w));
    int brow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int r = n0 + 64 * wave + 32 * nb + l32;
        brow[nb] = r < n ? r : n - 1;
    }
    auto copy_b = [&](int s, int buf, int nb) {
        const int c = min(2 * s + g, C - 1);
        copy16_to_lds(wbase + (size_t)c * n + brow[nb], smem + kBOff + buf * kBBuf + 1024 * (2 * wave + nb));
    };
    auto stage_b = [&](int s, int buf) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) copy_b(s, buf, nb);
    };
    auto read_b = [&](int buf, v4u32 (&braw)[2]) {
        const uint8_t* bbuf = smem + kBOff + buf * kBBuf;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            braw[nb] = *reinterpret_cast<const v4u32*>(bbuf + 1024 * (2 * wave + nb) + 16 * lane);
    };

    // ---- activations: 128 token rows x 10 pieces per step --------------------------------
    // Fast path (k % 16 == 0, 16-byte aligned rows): copy j of wave w fills
    // stored slots 64 (5w + j) + lane, slot f = row f / 10 at stored piece
    // f % 10.  Tokens past m repeat token m - 1 (never stored).
    const QMV_GLOBAL int8_t* xbase = gload_ptr(P->x8);
    const QMV_GLOBAL int8_t* zsrc = gload_ptr(zeros);
    const bool fast = ((k & 15) == 0) && ((reinterpret_cast<uintptr_t>(P->x8) & 15) == 0);
    int a_tp[kADma];   // token << 4 | source piece of each copy
#pragma unroll
    for (int j = 0; j < kADma; ++j) {
        const int f = 64 * (kADma * wave + j) + lane;
        const int r = f / kPieces;
        const int q = f - r * kPieces;                     // stored piece
        const int p = q - ((r >> 3) & 1);                  // source piece
        a_tp[j] = (min(m0 + r, mtok - 1) << 4) | (p < 0 ? p + kPieces : p);
    }
    auto copy_a = [&](int s, int buf, int j) {
        const int col = 160 * s + 16 * (a_tp[j] & 15);
        const QMV_GLOBAL int8_t* src = col < k ? xbase + (size_t)(a_tp[j] >> 4) * k + col : zsrc;
        copy16_to_lds(src, smem + buf * kABuf + 1024 * (kADma * wave + j));
    };
    auto stage_a = [&](int s, int buf) {
        uint8_t* abuf = smem + buf * kABuf;
        if (fast) {
#pragma unroll
            for (int j = 0; j < kADma; ++j) copy_a(s, buf, j);
        } else {
            // thread t writes pieces 5h .. 5h+4 of row r (h = t / 128), zero past column k
            const int r = tid & (kPBM - 1), h = tid >> 7;
            const int tok = m0 + r;
            const QMV_GLOBAL int8_t* xr = xbase + (size_t)min(tok, mtok - 1) * k;
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const int p = 5 * h + j;
                uint32_t* dst = reinterpret_cast<uint32_t*>(abuf + apos(r, p));
#pragma unroll
                for (int d = 0; d < 4; ++d) dst[d] = tok < mtok ? x_bytes(xr, 160 * s + 16 * p + 4 * d, k) : 0u;
            }
        }
    };
    // Sum of row (tid % 128)'s staged columns, pieces 5h .. 5h+4 (h = tid / 128),
    // one piece per plane; zero past k.
    int rsum = 0;
    // pieces 5h .. 5h+3 of a row are consecutive; only 5h+4 can wrap to piece 0
    const int sbase = apos(tid & (kPBM - 1), 5 * (tid >> 7));
    const int slast = apos(tid & (kPBM - 1), 5 * (tid >> 7) + 4);
    auto sum_piece = [&](int buf, int j) {
        const uint4 v = *reinterpret_cast<const uint4*>(smem + buf * kABuf + (j < 4 ? sbase + 16 * j : slast));
        rsum = dot4(v.x, 0x01010101u, rsum);
        rsum = dot4(v.y, 0x01010101u, rsum);
        rsum = dot4(v.z, 0x01010101u, rsum);
        rsum = dot4(v.w, 0x01010101u, rsum);
    };
    // This lane's activation operand of plane i is piece 5g + i of token row
    // 32 tb + l32: a per-lane offset (rows of a lane share one rotation).
    const int abase = apos(l32, 5 * g);       // pieces 5g .. 5g+3 are consecutive
    const int alast = apos(l32, 5 * g + 4);   // piece 5g+4 can wrap to piece 0
    auto aoff = [&](int i) { return i < 4 ? abase + 16 * i : alast; };

    v16i32 acc[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[tb][nb] = v16i32{};

    // Pipeline: at step s the MFMAs use the activations of step s (LDS ring slot
    // s % 3) and the weights of step s (registers, read from the LDS ring during
    // step s - 1, digits expanded one dword per plane).  Copies for step s + 2
    // are issued during step s, weights first (plane 0), then the activations
    // spread over planes 1..4 so that no wave stalls long on a burst of copies:
    // "weights of s + 2 and everything older have landed" is vmcnt(activation
    // copies of one step).
    stage_b(0, 0);
    stage_a(0, 0);
    if (steps > 1) {
        stage_b(1, 1);
        stage_a(1, 1);
    }
    wait_vmcnt<0>();
    lds_barrier();
    v4u32 braw[2];
    read_b(0, braw);
    uint32_t nat[2][20];   // the step's digits in natural column order, 4 per dword
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) natural_digits(braw[nb][0], &nat[nb][0]);

    for (int s = 0; s < steps; ++s) {
        const int buf = s % kANBuf;
        const bool more2 = s + 2 < steps;
        const int abuf2 = (s + 2) % kANBuf;
        if (more2 && !fast) stage_a(s + 2, abuf2);
        // the next step's packed weights (after the last step: stale, expanded and
        // never used, which keeps the MFMA block free of branches)
        v4u32 bnext[2];
        read_b((s + 1) & 1, bnext);
        uint32_t nxt[2][5];
        const uint8_t* arow = smem + buf * kABuf;   // + aoff: this lane's token row and piece
        v4i32 aop[2][4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) aop[0][tb] = *reinterpret_cast<const v4i32*>(arow + 32 * tb * kARow + aoff(0));
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            // copies for step s + 2: weights (into the slot of step s's weights,
            // already in registers), then activations
            if (more2) {
                if (i == 0) stage_b(s + 2, s & 1);
                else if (fast) {
                    if (i == 1) copy_a(s + 2, abuf2, 0);
                    copy_a(s + 2, abuf2, i);
                }
            }
            sum_piece(buf, i);
            // plane i covers columns 16i .. 16i+15 of each lane's chunk: digit
            // dwords 4i .. 4i+3, from packed dwords i-1 and i (expanded a plane ahead)
            if (i < 4) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    aop[(i + 1) & 1][tb] = *reinterpret_cast<const v4i32*>(arow + 32 * tb * kARow + aoff(i + 1));
            }
            if (i < 3) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) natural_digits(braw[nb][i + 1], &nat[nb][5 * (i + 1)]);
            } else if (i == 3) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) natural_digits(bnext[nb][0], nxt[nb]);
            }
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const v4i32 wop = {(int)nat[nb][4 * i], (int)nat[nb][4 * i + 1], (int)nat[nb][4 * i + 2],
                                       (int)nat[nb][4 * i + 3]};
                    acc[tb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[i & 1][tb], wop, acc[tb][nb], 0, 0, 0);
                }
            // one MFMA (its operands are ready), the next plane's LDS reads, then
            // one MFMA per few VALU ops of the next dword's expansion
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
            for (int q = 1; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            braw[nb] = bnext[nb];
#pragma unroll
            for (int u = 0; u < 5; ++u) nat[nb][u] = nxt[nb][u];
        }
        if (s + 1 < steps) {
            // activations of s + 1 and weights of s + 2 have landed once only the
            // activation copies of s + 2 may still fly
            if (more2 && fast) wait_vmcnt<kADma>();
            else wait_vmcnt<0>();
            lds_barrier();
        }
    }

    // ---- epilogue ---------------------------------------------------------------------
    // Token sums and scales go to LDS.  Accumulator register 4q+e of lane l is
    // token 8q + 4g + e of its 32-token block and row l % 32 of its 32-row block,
    // so each register's half-wave holds 32 consecutive outputs of one token: a
    // whole 128-byte line, stored straight from the registers.
    int* tsum = reinterpret_cast<int*>(smem + kEpiOff);                 // [2][128]
    float* tscale = reinterpret_cast<float*>(smem + kEpiOff + 2 * kPBM * 4);
    tsum[tid] = rsum;   // half tid / 128 of row tid % 128
    if (tid < kPBM) {
        const int tok = m0 + tid;
        tscale[tid] = tok < mtok ? gload_ptr(P->sx)[tok] * *gload_ptr(P->sw) : 0.0f;
    }
    __syncthreads();
    QMV_GLOBAL float* y = gstore_ptr(P->y);
    QMV_GLOBAL int32_t* accout = P->acc ? gstore_ptr(P->acc) : nullptr;
    const bool full = m0 + kPBM <= mtok && n0 + kPBN <= n;
    const int rl = n0 + 64 * wave + l32;   // this lane's row in row block 0 (+32 in block 1)
    const int loff = 4 * g * n + rl;       // + (token block base + 8q + e) * n
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t0 = 32 * tb + 8 * q + 4 * g;   // tile token of register 4q (+e)
            const int4 ta = *reinterpret_cast<const int4*>(tsum + t0);
            const int4 tc = *reinterpret_cast<const int4*>(tsum + kPBM + t0);
            const float4 sc4 = *reinterpret_cast<const float4*>(tscale + t0);
            const int tsv[4] = {ta.x + tc.x, ta.y + tc.y, ta.z + tc.z, ta.w + tc.w};
            const float scv[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const size_t urow = (size_t)(m0 + 32 * tb + 8 * q + e) * n;   // uniform part of the offset
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int v = acc[tb][nb][4 * q + e] - tsv[e];
                    if (full || (m0 + t0 + e < mtok && rl + 32 * nb < n)) {
                        y[urow + loff + 32 * nb] = (float)v * scv[e];
                        if (accout) accout[urow + loff + 32 * nb] = v;
                    }
                }
            }
        }
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

hipError_t launch_prefill(const DevProblem* probs, const uint64_t* tiles, int64_t tile_count, const int8_t* zeros,
                          hipStream_t s)
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_prefill),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPrefillLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_prefill, dim3((unsigned)tile_count), dim3(kBlock), kPrefillLds, s, probs, tiles, zeros);
    return hipGetLastError();
}

}  // namespace qmv
