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
constexpr int kNextOff = kEpiOff + 3 * kPBM * 4;      // + token sums (two halves) and scales
constexpr int kPrefillLds = kNextOff + 16;             // + the next tile's index: 79376 bytes
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format
constexpr int kBufStoreMaxN = 1 << 22;          // tile rows x n x 4 bytes stays below 2^31
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

// The same for 4 bytes per lane: lane i's dword lands at lds + 4 i.
__device__ __forceinline__ void copy4_to_lds(const void QMV_GLOBAL* src, const uint8_t* lds)
{
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(a) : "memory");
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

// Uniform description of one tile.
struct PTile {
    const DevProblem* P;
    const QMV_GLOBAL v4u32* wbase;
    const QMV_GLOBAL int8_t* xbase;
    float* y;
    int32_t* acc;
    const float* sx;
    float sw;
    int n, k, mtok, C, m0, n0, steps;
    bool fast;               // k % 16 == 0 and 16-byte aligned rows: activation copies
};

__device__ __forceinline__ PTile tile_of(const DevProblem* probs, uint64_t te)
{
    PTile T;
    T.P = probs + (int)(te >> 48);
    const int mt = (int)((te >> 32) & 0xFFFF);
    const int nt = (int)(te & 0xFFFFFFFFu);
    T.n = T.P->n;
    T.k = T.P->k;
    T.mtok = T.P->m;
    T.C = T.P->chunks;
    T.m0 = mt * kPBM;
    T.n0 = nt * kPBN;
    T.steps = (T.C + 1) >> 1;
    T.wbase = gload_ptr(reinterpret_cast<const v4u32*>(T.P->w));
    T.xbase = gload_ptr(T.P->x8);
    T.y = T.P->y;
    T.acc = T.P->acc;
    T.sx = T.P->sx;
    T.sw = *cload_ptr(T.P->sw);
    T.fast = ((T.k & 15) == 0) && ((reinterpret_cast<uintptr_t>(T.P->x8) & 15) == 0);
    return T;
}

// Per-lane values of the copies.  Activation copy j of wave w fills stored
// slots 64 (5w + j) + lane, slot f = row f / 10 at stored piece f % 10.
struct PLane {
    int lane, g, l32;
    int a_rp[kADma];   // tile row << 4 | source piece of each activation copy
};

__device__ __forceinline__ PLane lane_of(int tid, int wave)
{
    PLane L;
    L.lane = tid & (kWave - 1);
    L.g = L.lane >> 5;
    L.l32 = L.lane & 31;
#pragma unroll
    for (int j = 0; j < kADma; ++j) {
        const int f = 64 * (kADma * wave + j) + L.lane;
        const int r = f / kPieces;
        const int q = f - r * kPieces;                     // stored piece
        const int p = q - ((r >> 3) & 1);                  // source piece
        L.a_rp[j] = (r << 4) | (p < 0 ? p + kPieces : p);
    }
    return L;
}

// Weights: two 32-row blocks per wave, HBM -> LDS; lane l of a row block ->
// 16 bytes at l * 16 of the wave's region.  Rows past n repeat row n - 1
// (never stored).
__device__ __forceinline__ void copy_b(const PTile& T, const PLane& L, uint8_t* smem, int wave, int s, int buf, int nb)
{
    const int c = min(2 * s + L.g, T.C - 1);
    const int row = min(T.n0 + 64 * wave + 32 * nb + L.l32, T.n - 1);
    copy16_to_lds(T.wbase + (size_t)c * T.n + row, smem + kBOff + buf * kBBuf + 1024 * (2 * wave + nb));
}

// Activations (fast path: k % 16 == 0, 16-byte aligned rows): 128 token rows
// x 10 pieces per step; tokens past m repeat token m - 1 (never stored),
// columns past k come from the block of zeros.
__device__ __forceinline__ void copy_a(const PTile& T, const PLane& L, uint8_t* smem, const QMV_GLOBAL int8_t* zsrc,
                                       int wave, int s, int buf, int j)
{
    const int col = 160 * s + 16 * (L.a_rp[j] & 15);
    const int tok = min(T.m0 + (L.a_rp[j] >> 4), T.mtok - 1);
    const QMV_GLOBAL int8_t* src = col < T.k ? T.xbase + (size_t)tok * T.k + col : zsrc;
    copy16_to_lds(src, smem + buf * kABuf + 1024 * (kADma * wave + j));
}

// The copies of steps 0 and 1 of a fast-path tile.
__device__ __forceinline__ void first_copies_fast(const PTile& T, const PLane& L, uint8_t* smem,
                                                  const QMV_GLOBAL int8_t* zsrc, int wave)
{
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if (s == 1 && T.steps < 2) break;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) copy_b(T, L, smem, wave, s, s, nb);
#pragma unroll
        for (int j = 0; j < kADma; ++j) copy_a(T, L, smem, zsrc, wave, s, s, j);
    }
}

// Next tile for a workgroup, called by all of wave 0 (lane 0 takes the
// tickets, so x and tries stay wave-uniform): a ticket from list x, or from
// the following lists once x is used up; -1 when every list is.
__device__ __forceinline__ int take_tile(const uint64_t* table, uint32_t* tickets, int lane, int& x, int& tries)
{
    while (tries < kXcds) {
        const int b = (int)table[x], e = (int)table[x + 1];
        if (b < e) {
            uint32_t t = 0;
            if (lane == 0) t = atomicAdd(tickets + x, 1u);
            t = __builtin_amdgcn_readfirstlane(t);
            if (t < (uint32_t)(e - b)) return b + (int)t;
        }
        x = x + 1 == kXcds ? 0 : x + 1;
        ++tries;
    }
    return -1;
}

// A workgroup that found no tile left counts itself out (lane 0 of wave 0);
// the last one resets the tickets for the next launch on the stream.
__device__ __forceinline__ void finish_tiles(uint32_t* tickets)
{
    if (atomicAdd(tickets + kXcds, 1u) == gridDim.x - 1) {
#pragma unroll
        for (int i = 0; i <= kXcds; ++i) __hip_atomic_store(tickets + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Persistent: the table holds 8 tile lists (offsets table[0..8], entries
// after them), one per XCD, and then the tickets.  Workgroup b starts on the
// list of its XCD (b % 8, round-robin dispatch) and takes tiles in list order
// with a ticket each; when that list is used up it helps with the others.
// The next tile is known before a tile's epilogue, so the copies that start
// its K loop are issued before the output stores and their latency and the
// tile set-up hide behind them.
__global__ __launch_bounds__(kBlock, 2) void k_prefill(const DevProblem* __restrict__ probs,
                                                       const uint64_t* __restrict__ table,
                                                       const int8_t* __restrict__ zeros)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);

    const uint64_t* ent = table + kXcds + 1;
    uint32_t* tickets = const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(ent + table[kXcds]));
    int* next_lds = reinterpret_cast<int*>(smem + kNextOff);
    const QMV_GLOBAL int8_t* zsrc = gload_ptr(zeros);
    // ticket state, used by wave 0 only (wave-uniform)
    int tx = (int)(blockIdx.x % kXcds), ttries = 0;
    if (wave == 0) {
        const int first = take_tile(table, tickets, (int)threadIdx.x, tx, ttries);
        if (threadIdx.x == 0) {
            if (first < 0) finish_tiles(tickets);
            next_lds[0] = first;
        }
    }
    __syncthreads();
    int it = __builtin_amdgcn_readfirstlane(next_lds[0]);
    if (it < 0) return;

    PTile T = tile_of(probs, ent[it]);
    bool staged = false;   // the copies of the tile's first two steps are issued
    for (;;) {
        // Per-lane values come from an opaque copy of the thread index, so the
        // compiler derives them inside the tile loop instead of hoisting dozens
        // of them out of it into registers the K loop needs.
        int tid = (int)threadIdx.x;
        asm volatile("" : "+v"(tid));
        const PLane L = lane_of(tid, wave);
        const int lane = L.lane, g = L.g, l32 = L.l32;

        auto stage_b = [&](const PTile& T, int s, int buf) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) copy_b(T, L, smem, wave, s, buf, nb);
        };
        auto read_b = [&](int buf, v4u32 (&braw)[2]) {
            const uint8_t* bbuf = smem + kBOff + buf * kBBuf;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                braw[nb] = *reinterpret_cast<const v4u32*>(bbuf + 1024 * (2 * wave + nb) + 16 * lane);
        };
        auto stage_a = [&](const PTile& T, int s, int buf) {
            uint8_t* abuf = smem + buf * kABuf;
            if (T.fast) {
#pragma unroll
                for (int j = 0; j < kADma; ++j) copy_a(T, L, smem, zsrc, wave, s, buf, j);
            } else {
                // thread t writes pieces 5h .. 5h+4 of row r (h = t / 128), zero past column k
                const int r = tid & (kPBM - 1), h = tid >> 7;
                const int tok = T.m0 + r;
                const QMV_GLOBAL int8_t* xr = T.xbase + (size_t)min(tok, T.mtok - 1) * T.k;
#pragma unroll
                for (int j = 0; j < 5; ++j) {
                    const int p = 5 * h + j;
                    uint32_t* dst = reinterpret_cast<uint32_t*>(abuf + apos(r, p));
#pragma unroll
                    for (int d = 0; d < 4; ++d) dst[d] = tok < T.mtok ? x_bytes(xr, 160 * s + 16 * p + 4 * d, T.k) : 0u;
                }
            }
        };
        // the copies of steps 0 and 1 of a tile
        auto stage_first = [&](const PTile& T) {
            stage_b(T, 0, 0);
            stage_a(T, 0, 0);
            if (T.steps > 1) {
                stage_b(T, 1, 1);
                stage_a(T, 1, 1);
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
        int* tsum = reinterpret_cast<int*>(smem + kEpiOff);                 // [2][128]
        float* tscale = reinterpret_cast<float*>(smem + kEpiOff + 2 * kPBM * 4);
        if (!staged) stage_first(T);
        const int steps = T.steps;
        v16i32 acc[4][2];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) acc[tb][nb] = v16i32{};
        rsum = 0;

        // Pipeline: at step s the MFMAs use the activations of step s (LDS ring
        // slot s % 3) and the weights of step s (registers, read from the LDS ring
        // during step s - 1, digits expanded one dword per plane).  Copies for step
        // s + 2 are issued during step s, weights first (plane 0), then the
        // activations spread over planes 1..4 so that no wave stalls long on a
        // burst of copies: "weights of s + 2 and everything older have landed" is
        // vmcnt(activation copies of one step).  The copies of steps 0 and 1 were
        // issued before the previous tile's stores; waiting for them also waits
        // for those stores.
        wait_vmcnt<0>();
        lds_barrier();
        v4u32 braw[2];
        read_b(0, braw);
        uint32_t nat[2][20];   // the step's digits in natural column order, 4 per dword
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) natural_digits(braw[nb][0], &nat[nb][0]);

        uint32_t tk = 0;   // lane 0 of wave 0: a ticket of list tx, taken during the last step
        for (int s = 0; s < steps; ++s) {
            if (s + 1 == steps) {
                // a step before the epilogue: the next tile's ticket, and the token
                // scales of this tile copied into LDS (tokens past m repeat token m - 1)
                // (the ticket is read only after the step's matrix work; the copy goes
                // first so that no wait placed before it covers the ticket)
                if (wave < kPBM / kWave)
                    copy4_to_lds(gload_ptr(T.sx) + min(T.m0 + tid, T.mtok - 1), smem + kEpiOff + 2 * kPBM * 4 + 4 * kWave * wave);
                if (wave == 0 && lane == 0 && ttries < kXcds) tk = atomicAdd(tickets + tx, 1u);
            }
            const int buf = s % kANBuf;
            const bool more2 = s + 2 < steps;
            const int abuf2 = (s + 2) % kANBuf;
            if (more2 && !T.fast) stage_a(T, s + 2, abuf2);
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
                    if (i == 0) stage_b(T, s + 2, s & 1);
                    else if (T.fast) {
                        if (i == 1) copy_a(T, L, smem, zsrc, wave, s + 2, abuf2, 0);
                        copy_a(T, L, smem, zsrc, wave, s + 2, abuf2, i);
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
                if (more2 && T.fast) wait_vmcnt<kADma>();
                else wait_vmcnt<0>();
                lds_barrier();
            }
        }

        // ---- epilogue ---------------------------------------------------------------------
        // Token sums and scales go to LDS.  Accumulator register 4q+e of lane l is
        // token 8q + 4g + e of its 32-token block and row l % 32 of its 32-row block,
        // so each register's half-wave holds 32 consecutive outputs of one token: a
        // whole 128-byte line, stored straight from the registers.
        // Lane values rederived from a fresh opaque thread index: nothing per-lane
        // has to stay live across the K loop for the epilogue.
        int te = (int)threadIdx.x;
        asm volatile("" : "+v"(te));
        const PLane LE = lane_of(te, wave);
        tsum[te] = rsum;   // half te / 128 of row te % 128
        if (wave == 0) {
            int nxt = -1;
            if (ttries < kXcds) {
                const int b = (int)table[tx], e = (int)table[tx + 1];
                const uint32_t t = __builtin_amdgcn_readfirstlane(tk);
                if (t < (uint32_t)(e - b)) {
                    nxt = b + (int)t;
                } else {
                    tx = tx + 1 == kXcds ? 0 : tx + 1;
                    ++ttries;
                    nxt = take_tile(table, tickets, LE.lane, tx, ttries);
                }
            }
            if (te == 0) {
                if (nxt < 0) finish_tiles(tickets);
                next_lds[0] = nxt;
            }
        }
        // the token scales have landed (waves 0 and 1 copied them); every wave is
        // past its last read of the copy rings
        wait_vmcnt<0>();
        __syncthreads();
        // the next tile's first copies, ahead of this tile's stores (fast path;
        // the byte-wise path stages after the stores)
        const PTile E = T;
        it = __builtin_amdgcn_readfirstlane(next_lds[0]);
        const bool more = it >= 0;
        staged = false;
        if (more) {
            T = tile_of(probs, ent[it]);
            if (T.fast) {
                first_copies_fast(T, LE, smem, zsrc, wave);
                staged = true;
            }
        }
        const bool full = E.m0 + kPBM <= E.mtok && E.n0 + kPBN <= E.n;
        const int rl = E.n0 + 64 * wave + LE.l32;   // this lane's row in row block 0 (+32 in block 1)
        const int loff = 4 * LE.g * E.n + rl;       // + (token block base + 8q + e) * n
        if (full && !E.acc && E.n < kBufStoreMaxN) {
            // The whole tile is in range: buffer stores over the tile's 128 token
            // rows, the lane's offset in a VGPR fixed for the tile and the token's
            // row offset in an SGPR, so a store costs the three VALU of its value.
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(E.y + (size_t)E.m0 * E.n), (short)0, kPBM * 4 * E.n, (int)kRsrcWord3);
            const int voff = 4 * loff;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t0 = 32 * tb + 8 * q + 4 * LE.g;
                    const int4 ta = *reinterpret_cast<const int4*>(tsum + t0);
                    const int4 tc = *reinterpret_cast<const int4*>(tsum + kPBM + t0);
                    const float4 sc4 = *reinterpret_cast<const float4*>(tscale + t0);
                    const int tsv[4] = {ta.x + tc.x, ta.y + tc.y, ta.z + tc.z, ta.w + tc.w};
                    const float scv[4] = {sc4.x * E.sw, sc4.y * E.sw, sc4.z * E.sw, sc4.w * E.sw};   // sx * sw
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int soff = 4 * (32 * tb + 8 * q + e) * E.n;
#pragma unroll
                        for (int nb = 0; nb < 2; ++nb) {
                            const float v = (float)(acc[tb][nb][4 * q + e] - tsv[e]) * scv[e];
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, voff + 128 * nb, soff, 0);
                        }
                    }
                }
            }
        } else {
            QMV_GLOBAL float* y = gstore_ptr(E.y);
            QMV_GLOBAL int32_t* accout = E.acc ? gstore_ptr(E.acc) : nullptr;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t0 = 32 * tb + 8 * q + 4 * LE.g;   // tile token of register 4q (+e)
                    const int4 ta = *reinterpret_cast<const int4*>(tsum + t0);
                    const int4 tc = *reinterpret_cast<const int4*>(tsum + kPBM + t0);
                    const float4 sc4 = *reinterpret_cast<const float4*>(tscale + t0);
                    const int tsv[4] = {ta.x + tc.x, ta.y + tc.y, ta.z + tc.z, ta.w + tc.w};
                    const float scv[4] = {sc4.x * E.sw, sc4.y * E.sw, sc4.z * E.sw, sc4.w * E.sw};   // sx * sw
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const size_t urow = (size_t)(E.m0 + 32 * tb + 8 * q + e) * E.n;   // uniform part of the offset
#pragma unroll
                        for (int nb = 0; nb < 2; ++nb) {
                            const int v = acc[tb][nb][4 * q + e] - tsv[e];
                            if (full || (E.m0 + t0 + e < E.mtok && rl + 32 * nb < E.n)) {
                                y[urow + loff + 32 * nb] = (float)v * scv[e];
                                if (accout) accout[urow + loff + 32 * nb] = v;
                            }
                        }
                    }
                }
            }
        }
        if (!more) break;
        // tsum and tscale are rewritten only after the next tile's K loop, whose
        // barriers every wave passes after its reads above
    }
}

}  // namespace

int64_t prefill_tiles(int64_t m, int64_t n) { return ((m + kPBM - 1) / kPBM) * ((n + kPBN - 1) / kPBN); }

hipError_t setup_prefill_attributes()
{
    return raise_lds_limit(reinterpret_cast<const void*>(&k_prefill));
}

hipError_t launch_prefill(const DevProblem* probs, const uint64_t* table, int64_t grid, const int8_t* zeros,
                          hipStream_t s)
{
    hipLaunchKernelGGL(k_prefill, dim3((unsigned)grid), dim3(kBlock), kPrefillLds, s, probs, table, zeros);
    return hipGetLastError();
}

}  // namespace qmv
