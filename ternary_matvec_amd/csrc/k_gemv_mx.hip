// k_gemv_mx.hip -- persistent grouped ternary GEMV for 1..16 tokens whose
// multiply-adds run on the int8 matrix cores (gfx950).
//
// Same results as the other GEMV kernels: the exact int32 dot product of int8
// activations with five-trits-per-byte weights, the two scales applied once
// after the sum ("Gemma 3 1B at 114 tokens per second on a laptop CPU",
// "Step 1" and "Many users at once"; cpp20gemma README, "Architecture &
// implementation").
//
// Why matrix cores for a product that streams its weights once.  Decoding a
// packed byte and multiplying its five trits costs vector instructions, and
// with dot-product instructions the multiplies grow with the token count.
// Here the vector units only decode (15 instructions per packed dword,
// whatever the token count) and the matrix cores, otherwise idle, do every
// multiply-add.
//
// Arithmetic.  A packed byte b has base-3 digits d_1..d_5 (d_1 the most
// significant, digit = trit + 1); byte q of a chunk covers columns 5q..5q+4 and
// its digit of 3^e meets column 5q+e, so digit d_j meets X_j = x[5q + 5 - j].
// With the prefix quotients P_j = floor(b / 3^(5-j)) (P_5 = b), d_j = P_j - 3
// P_(j-1), hence
//     sum_j d_j X_j = sum_j P_j X_j  -  3 sum_(j<5) P_j X_(j+1).
// Both sums are int8 dot products of the bytes P_j with activation bytes, so
// each token takes two matrix columns: column A holds X_j where the operand
// holds P_j, column B holds X_(j+1) (nothing for P_5).  The integer result is
// A - 3 B + 128 sum X_5 - sum x: P_5 enters as b XOR 0x80 = b - 128, and
// trit = digit - 1.
//   * P_4..P_1 come from the packed-fp16 floor-by-3 chain (unpack.hpp) on the
//     pairs 1024 + P of the even and of the odd bytes; one byte permute per
//     level puts the four quotient bytes of a packed dword back in byte order.
//   * Per packed dword: 1 XOR, 2 byte permutes, 8 packed-fp16 FMAs and 4 byte
//     permutes; per level one operand of 16 quotient bytes.
//
// Matrix instruction: v_mfma_i32_16x16x64_i8 with the activations as the
// first operand (16 columns: token t's A and B are columns 2t and 2t + 1 of
// its column set; tokens 8..15 form a second set) and the weights as the
// second (16 rows).  Lane l supplies column / row l % 16 and K group l / 16.
// A wave step is 16 rows x 4 chunks (lane group g takes chunk 4kr + g of its
// row, one 16-byte load) = 1 KiB of packed weights: five matrix instructions
// per column set (P_5, P_4, .., P_1), each weight operand serving both sets.
// Accumulator register i of lane l holds column 4 (l / 16) + i of row l % 16,
// so lane group g finishes tokens 2g and 2g + 1 of its set and row without
// any cross-lane reduction.
//
// Work and schedule (as the streaming VALU kernel): a workgroup is four
// compute waves and one staging wave; a workgroup tile is 4 x 16 x rgs rows of
// one problem over all of K (each wave rgs row groups of 16, which share every
// activation operand read from LDS; rgs = 2, 4, 4 for up to 4, 8, 16 tokens).
// Tiles are dealt to the 8 XCD lists by the host; each workgroup's first two
// tiles are fixed, later ones come from a per-XCD ticket.  The staging wave
// writes the next tile's activation operands into LDS (two slots) while the
// compute waves stream the current one: per chunk and token 80 bytes, the
// page's input reorder ("Step 1": plane v = the x values that meet digit v of
// each packed byte), plane v holding X_(5-v) of bytes 0..15.  Column A of
// level j reads plane 5 - j, column B plane 4 - j (16 bytes lower; zeros for
// P_5).  The staging wave takes one (token, chunk) per lane over all tokens
// at once, so a tile's staging is a few rounds of loads, not one per token.
#include <type_traits>

#include "qmv_internal.hpp"
#include "unpack.hpp"

namespace qmv {
namespace {

typedef int v4i32 __attribute__((ext_vector_type(4)));

// Shapes per token count (1..4 / 5..8 / 9..16 tokens): register-ring steps,
// row groups of 16 per wave, compute waves, and the waves per SIMD the
// registers are budgeted for.  Build-time knobs; the defaults are the fastest
// measured on the BitNet-large x24 decode (16 tokens: 16-row-group tiles
// 187.6 us, 256-row tiles 56.7 us, once the activations are staged a
// (token, chunk) per lane).
#ifndef QMV_MX_RING
#define QMV_MX_RING 4
#endif
#ifndef QMV_MX_RGS
#define QMV_MX_RGS 2
#endif
#ifndef QMV_MX_WAVES
#define QMV_MX_WAVES 5
#endif
#ifndef QMV_MX8_RING
#define QMV_MX8_RING 4
#endif
#ifndef QMV_MX8_RGS
#define QMV_MX8_RGS 4
#endif
#ifndef QMV_MX8_CWAVES
#define QMV_MX8_CWAVES 4
#endif
#ifndef QMV_MX8_WAVES
#define QMV_MX8_WAVES 3
#endif
#ifndef QMV_MX16_RING
#define QMV_MX16_RING 8
#endif
#ifndef QMV_MX16_RGS
#define QMV_MX16_RGS 4
#endif
#ifndef QMV_MX16_CWAVES
#define QMV_MX16_CWAVES 4
#endif
#ifndef QMV_MX16_WAVES
#define QMV_MX16_WAVES 2
#endif
constexpr int kOps = 5;                        // matrix instructions per step and column set
constexpr int kPlaneBytes = 80;                // staged bytes per chunk and token (5 planes of 16)

// Per token count: weight steps in the register ring (kRing - 1 loads ahead),
// row groups of 16 per wave (a K range's operands serve all of them), compute
// waves per workgroup (plus one staging wave) and the waves per SIMD the
// register budget is made for.
template <int MT>
struct MxShape {
    static constexpr int kRing = MT > 8 ? QMV_MX16_RING : MT > 4 ? QMV_MX8_RING : QMV_MX_RING;
    static constexpr int kRowGroups = MT > 8 ? QMV_MX16_RGS : MT > 4 ? QMV_MX8_RGS : QMV_MX_RGS;
    static constexpr int kComputeWaves = MT > 8 ? QMV_MX16_CWAVES : MT > 4 ? QMV_MX8_CWAVES : 4;
    static constexpr int kThreads = (kComputeWaves + 1) * kWave;
    static constexpr int kWavesPerEu = MT > 8 ? QMV_MX16_WAVES : MT > 4 ? QMV_MX8_WAVES : QMV_MX_WAVES;
    static constexpr int kTileRows = 16 * kRowGroups * kComputeWaves;
    static_assert(kRing % kRowGroups == 0, "a ring group holds whole K ranges");
};
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format
constexpr uint32_t kEnd = 0xffffffffu;         // no tile
constexpr uint32_t kOob = 0xfffffff0u;         // a byte offset past any matrix: the load returns zeros
constexpr int kNonTemporal = 2;                // buffer instruction cache policy: nt
constexpr int kDescSlots = 3;                  // tile descriptors in LDS, used round robin
constexpr int kZeroBytes = 192;                // LDS zeros that idle operand lanes read

// A tile as the staging wave leaves it in LDS for the compute waves.
struct MDesc {
    const uint8_t* w;
    float* y;
    int32_t* acc;
    int32_t n, m, C, wb;
    uint32_t te;            // tile entry, kEnd = no tile
    float sw;
    int32_t pad[4];
};
static_assert(sizeof(MDesc) == 64, "MDesc layout");

// Per token of a staged tile: the integer correction and the scale.
struct TokenData {
    int32_t corr;           // 128 * sum X_5 - sum x
    float sx;
};

// Sum over a wave, exact in int32 arithmetic.
__device__ __forceinline__ int wave_total(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) + __builtin_amdgcn_readlane(v, 47) +
           __builtin_amdgcn_readlane(v, 63);
}

// One ticket from an XCD's counter (one lane); the address is hidden from the
// uniformity analysis so the atomic is waited for where the ticket is used.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* counter)
{
    uintptr_t a = reinterpret_cast<uintptr_t>(counter);
    asm volatile("" : "+v"(a));
    return __hip_atomic_fetch_add(gstore_ptr(reinterpret_cast<uint32_t*>(a)), 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ MDesc desc_of(const DevProblem* P, uint32_t te)
{
    MDesc d;
    d.w = P->w;
    d.y = P->y;
    d.acc = P->acc;
    d.n = P->n;
    d.m = P->m;
    d.C = P->chunks;
    d.wb = (int)(te & ((1u << kTileRowBits) - 1));
    d.te = te;
    d.sw = *cload_ptr(P->sw);
    d.pad[0] = d.pad[1] = d.pad[2] = d.pad[3] = 0;
    return d;
}

__device__ __forceinline__ MDesc desc_load(const MDesc* p)
{
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 q = reinterpret_cast<const uint4*>(p)[i];
        v[4 * i + 0] = __builtin_amdgcn_readfirstlane(q.x);
        v[4 * i + 1] = __builtin_amdgcn_readfirstlane(q.y);
        v[4 * i + 2] = __builtin_amdgcn_readfirstlane(q.z);
        v[4 * i + 3] = __builtin_amdgcn_readfirstlane(q.w);
    }
    return __builtin_bit_cast(MDesc, v);
}

// What a compute wave derives from a tile descriptor.
struct MTile {
    const uint8_t* w;
    uint32_t nrec;          // bytes of the matrix: C * n * 16 (loads at or past it return zeros)
    uint32_t kstride;       // 4 * n * 16: one K range (4 chunks of every row)
    uint32_t lane_base;     // per lane: byte offset of its row's chunk g in K range 0, row group 0
    int n, nkr, S, Spad, cpad, row0;
};

template <int RGS, int RING, int WAVES>
__device__ __forceinline__ MTile mtile_of(const MDesc& d, int wave, int lane)
{
    MTile T;
    T.w = d.w;
    T.n = d.n;
    const uint32_t cstride = (uint32_t)d.n * 16u;
    T.kstride = 4u * cstride;
    T.nrec = (uint32_t)d.C * cstride;
    T.nkr = (d.C + 3) >> 2;
    T.cpad = 4 * T.nkr;
    T.S = T.nkr * RGS;
    T.Spad = (T.S + RING - 1) / RING * RING;
    T.row0 = (d.wb * WAVES + wave) * 16 * RGS;
    T.lane_base = (uint32_t)(lane >> 4) * cstride + (uint32_t)(T.row0 + (lane & 15)) * 16u;
    return T;
}

// 16 weight bytes at byte offset voff of a matrix of nrec bytes (zeros past it).
__device__ __forceinline__ v4u32 load_at(const uint8_t* w, uint32_t nrec, uint32_t voff)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)nrec, (int)kRsrcWord3);
    return __builtin_bit_cast(v4u32, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kNonTemporal));
}

// The 16 weight bytes of this lane for step s of tile `a` (when `first`) or of
// tile `b`: K range s / RGS, row group s % RGS; steps past the tile's
// last are loads that return zeros.  One load instruction whatever the tile,
// with the tile's fields chosen by wave-uniform selects: two load
// instructions on two paths would make the compiler wait for every
// outstanding load before each use.
template <int RGS>
__device__ __forceinline__ v4u32 load_step(const MTile& a, const MTile& b, bool first, int s)
{
    const uint8_t* w = first ? a.w : b.w;
    const uint32_t nrec = first ? a.nrec : b.nrec;
    const uint32_t kstride = first ? a.kstride : b.kstride;
    const uint32_t base = first ? a.lane_base : b.lane_base;
    const int S = first ? a.S : b.S;
    const uint32_t step_off = (uint32_t)(s / RGS) * kstride + (uint32_t)(s % RGS) * 256u;
    return load_at(w, nrec, s < S ? base + step_off : kOob);
}

// ---------------------------------------------------------------------------
// Staging (one wave).  Unit u of a token is the 20-column group d = u % 4 of
// chunk c = u / 4: its aligned dwords are read through a buffer sized to the
// row (zeros past it), shifted into place, bytes past column k cleared.
// ---------------------------------------------------------------------------

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const int8_t* row, int k, uint32_t& sh)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(row);
    sh = (uint32_t)(a & 3);
    const uint32_t words = (sh + (uint32_t)k + 3u) >> 2;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a & ~(uintptr_t)3), (short)0, (int)(4 * words), (int)kRsrcWord3);
}

__device__ __forceinline__ void unit_load(__amdgpu_buffer_rsrc_t rs, int u, uint32_t raw[6])
{
#pragma unroll
    for (int j = 0; j < 6; ++j) raw[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (5 * u + j), 0, 0);
}

__device__ __forceinline__ void unit_of(int k, uint32_t sh, int u, const uint32_t raw[6], uint32_t nat[5])
{
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const uint32_t v = __builtin_amdgcn_alignbyte(raw[j + 1], raw[j], sh);
        const int valid = k - 4 * (5 * u + j);
        nat[j] = valid >= 4 ? v : valid <= 0 ? 0u : v & ((1u << (8 * valid)) - 1u);
    }
}

// The five plane dwords of one 20-column group (natural bytes B0..B19 in
// dwords nat[0..4]; packed byte q covers B(5q)..B(5q+4)) written into dword d
// of the chunk's five 16-byte planes (plane v = [B(v), B(5+v), B(10+v),
// B(15+v)], the x values that meet digit v); adds the group's sum X_5 (plane
// 0) and sum x.
__device__ __forceinline__ void put_group(uint8_t* blk, int d, const uint32_t nat[5], int& s5, int& s)
{
    uint32_t* o = reinterpret_cast<uint32_t*>(blk);
    uint32_t pl[5];
    reorder20(nat[0], nat[1], nat[2], nat[3], nat[4], pl);
#pragma unroll
    for (int v = 0; v < 5; ++v) o[4 * v + d] = pl[v];
    s5 = dot4(pl[0], 0x01010101u, s5);
#pragma unroll
    for (int i = 0; i < 5; ++i) s = dot4(nat[i], 0x01010101u, s);
}

// Stage tile P / te into an LDS slot: the operand blocks of chunks 0 .. cpad-1
// for every token (zeros past k) and the tokens' corrections and scales.
// `after_loads` runs once, right after the first activation loads are issued.
// Chunk c of token t (rows 16-byte aligned, k a multiple of 16): the 80
// columns as five 16-byte loads through one buffer over the staged tokens'
// rows (pieces past the row read as zeros), then the four groups' planes,
// plane v of the chunk written as one 16-byte block.
__device__ __forceinline__ void chunk_load(__amdgpu_buffer_rsrc_t rs, int k, int t, int c, v4u32 raw[5])
{
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int o = 80 * c + 16 * i;
        const uint32_t voff = o < k ? (uint32_t)(t * k + o) : kOob;
        raw[i] = __builtin_bit_cast(v4u32, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
    }
}

__device__ __forceinline__ int put_chunk(const v4u32 raw[5], uint8_t* blk)
{
    uint32_t nat[20];
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) nat[4 * i + j] = raw[i][j];
    uint32_t pl[4][5];
#pragma unroll
    for (int d = 0; d < 4; ++d) reorder20(nat[5 * d], nat[5 * d + 1], nat[5 * d + 2], nat[5 * d + 3], nat[5 * d + 4], pl[d]);
#pragma unroll
    for (int v = 0; v < 5; ++v)
        *reinterpret_cast<v4u32*>(blk + 16 * v) = v4u32{pl[0][v], pl[1][v], pl[2][v], pl[3][v]};
    int s5 = 0, s = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) s5 = dot4(pl[d][0], 0x01010101u, s5);
#pragma unroll
    for (int i = 0; i < 20; ++i) s = dot4(nat[i], 0x01010101u, s);
    return (int)(128u * (uint32_t)s5 - (uint32_t)s);   // the chunk's share of the token's correction
}

// Stage tile P / te into an LDS slot: the operand planes of chunks 0 .. cpad-1
// for every token (zeros past k) and the tokens' corrections and scales.
// Rows that start on 16 bytes with k a multiple of 16 go a (token, chunk) per
// lane, all tokens together; others a 20-column group per lane, token by
// token.  `after_loads` runs once, right after the first activation loads
// are issued (in wave-uniform control flow: it may hold a barrier).
template <int MT, class F>
__device__ __forceinline__ void stage(const DevProblem* P, int lane, uint8_t* slot, TokenData* tok, F after_loads)
{
    constexpr int kBatch = 2;   // units or chunks per lane loaded before any is used
    const int k = P->k, m = P->m;
    const int cpad = 4 * ((P->chunks + 3) >> 2);
    const int units = 4 * cpad;
    const int8_t* x8 = P->x8;
    const bool whole = ((reinterpret_cast<uintptr_t>(x8) | (uintptr_t)k) & 15) == 0;
    bool first = true;
    if (whole) {
        const int mm = m < MT ? m : MT;   // tokens staged
        const int total = mm * cpad;
        // t = i / cpad as (i * inv) >> 22, exact for i * cpad < 2^22 (here
        // i < MT * cpad, which the LDS bounds to about a thousand)
        const uint32_t inv = ((1u << 22) + (uint32_t)cpad - 1) / (uint32_t)cpad;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)x8, (short)0, mm * k, (int)kRsrcWord3);
        if (lane < mm) tok[lane].corr = 0;
        for (int i0 = 0; i0 < total; i0 += kBatch * kWave) {   // uniform: after_loads may hold a barrier
            v4u32 raw[kBatch][5];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int i = i0 + b * kWave + lane;
                if (i < total) {
                    const int t = (int)(((uint32_t)i * inv) >> 22);
                    chunk_load(rs, k, t, i - t * cpad, raw[b]);
                }
            }
            if (first) {
                after_loads();
                first = false;
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int i = i0 + b * kWave + lane;
                if (i < total) {
                    const int t = (int)(((uint32_t)i * inv) >> 22);
                    const int corr = put_chunk(raw[b], slot + (size_t)i * kPlaneBytes);   // token t, chunk i - t cpad
                    atomicAdd(&tok[t].corr, corr);
                }
            }
        }
        if (lane < mm) tok[lane].sx = cload_ptr(P->sx)[lane];
        return;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t > 0 && t >= m) continue;
        uint8_t* base = slot + (size_t)t * cpad * kPlaneBytes;
        int s5 = 0, s = 0;
        uint32_t sh;
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(x8 + (size_t)t * k, k, sh);
        for (int u0 = 0; u0 < units; u0 += kWave * kBatch) {
            uint32_t raw[kBatch][6];
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (b == 0 || u0 + kWave * b < units) unit_load(rs, u0 + kWave * b + lane, raw[b]);
            if (first) {
                after_loads();
                first = false;
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int u = u0 + kWave * b + lane;
                if (u < units) {
                    uint32_t nat[5];
                    unit_of(k, sh, u, raw[b], nat);
                    put_group(base + (size_t)(u >> 2) * kPlaneBytes, u & 3, nat, s5, s);
                }
            }
        }
        const int corr = wave_total((int)(128u * (uint32_t)s5 - (uint32_t)s));
        if (lane == 0) {
            tok[t].corr = corr;
            tok[t].sx = cload_ptr(P->sx)[t];
        }
    }
}

// Schedule words (as the streaming VALU kernel): [counters: 8 tile counters + 8
// done counters, 64 words apart][first two tile entries of each workgroup]
// [8 x (list offset, list size)][tile entries of the 8 XCD lists].
// LDS: [2 slots of slot_bytes][3 descriptors][2 x MT token data][zeros].
template <int MT>
__global__ __launch_bounds__(MxShape<MT>::kThreads) __attribute__((amdgpu_waves_per_eu(MxShape<MT>::kWavesPerEu))) void k_gemv_mx(const DevProblem* __restrict__ probs,
                                                      uint32_t* __restrict__ sched, int32_t slot_bytes)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int kSets = (2 * MT + 15) / 16;   // column sets of 8 tokens
    constexpr int kRing = MxShape<MT>::kRing;
    constexpr int kRowGroups = MxShape<MT>::kRowGroups;
    constexpr int kComputeWaves = MxShape<MT>::kComputeWaves;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // Tile q's descriptor is in descs[q % 3]: the staging wave writes tile q + 2's
    // after barrier q + 1, and the compute waves last read that slot (as tile
    // q - 1's) before barrier q.
    MDesc* const descs = reinterpret_cast<MDesc*>(smem + 2 * (size_t)slot_bytes);
    TokenData* const tokd = reinterpret_cast<TokenData*>(descs + kDescSlots);
    uint8_t* const zeros = reinterpret_cast<uint8_t*>(tokd + 2 * MT);

    const int xcd = blockIdx.x % kStreamXcds;
    const uint32_t wgs = (gridDim.x - xcd + kStreamXcds - 1) / kStreamXcds;   // workgroups of this XCD
    const uint32_t te0 = cload_ptr(sched + kStreamHdr)[2 * blockIdx.x];
    const uint32_t* const hdr = sched + kStreamHdr + 2 * gridDim.x;

    if (wave == kComputeWaves) {
        // ---- staging wave: tile q into slot q & 1, the next tile's descriptor,
        // then barrier q ---------------------------------------------------------
        for (int i = lane; i < kZeroBytes / 4; i += kWave) reinterpret_cast<uint32_t*>(zeros)[i] = 0u;
        const uint32_t te1 = cload_ptr(sched + kStreamHdr)[2 * blockIdx.x + 1];
        uint32_t te = te0;
        uint32_t ticket = 0;
        const DevProblem* P = te != kEnd ? probs + (te >> kTileRowBits) : nullptr;
        const DevProblem* P1 = te1 != kEnd ? probs + (te1 >> kTileRowBits) : nullptr;
        MDesc d1;
        if (P1) d1 = desc_of(P1, te1);
        const uint32_t list_off = cload_ptr(hdr)[2 * xcd];
        const uint32_t list_size = cload_ptr(hdr)[2 * xcd + 1];
        const uint32_t* const list = hdr + 2 * kStreamXcds + list_off;
        bool first = true;
        for (int par = 0, q = 0; te != kEnd; par ^= 1, q = q == kDescSlots - 1 ? 0 : q + 1) {
            const int qn = q == kDescSlots - 1 ? 0 : q + 1;   // the next tile's descriptor slot
            stage<MT>(P, lane, smem + (size_t)par * slot_bytes, tokd + par * MT, [&] {
                if (first) {
                    // Tile 0: release the compute waves' weight prefetch only once
                    // these loads (and the tile's scale) are back.
                    const MDesc d0 = desc_of(P, te);
                    wait_vmcnt<0>();
                    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the scalar loads
                    __builtin_amdgcn_s_barrier();
                    if (lane == 0) {
                        descs[0] = d0;
                        if (te1 != kEnd) ticket = take_ticket(&sched[64 * xcd]);
                    }
                }
            });
            uint32_t nx = kEnd;
            if (first) {
                nx = te1;
                first = false;
            } else {
                if (lane == 0) {
                    const uint32_t i = 2 * wgs + ticket;
                    nx = i < list_size ? list[i] : kEnd;
                    if (nx != kEnd) ticket = take_ticket(&sched[64 * xcd]);
                }
                nx = __builtin_amdgcn_readfirstlane(nx);
            }
            if (nx != kEnd && par == 0 && nx == te1) {
                P = P1;
                if (lane == 0) descs[qn] = d1;
            } else if (nx != kEnd) {
                P = probs + (nx >> kTileRowBits);
                if (lane == 0) descs[qn] = desc_of(P, nx);
            } else if (lane == 0) {
                descs[qn].te = kEnd;
            }
            te = nx;
            // the tile's LDS writes are done; the ticket taken above stays in flight
            lds_barrier();
        }
        // Every workgroup of the XCD counts itself done once; the last one resets
        // both counters for the next launch (relaxed order suffices: every ticket
        // of the launch was taken before the last done count).
        if (lane == 0) {
            uint32_t* done = &sched[64 * (kStreamXcds + xcd)];
            if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == wgs - 1) {
                __hip_atomic_store(&sched[64 * xcd], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        return;
    }
    if (te0 == kEnd) return;

    // ---- compute waves ----------------------------------------------------------
    const int col = lane & 15;        // matrix column of this lane's activation operand
    const int g = lane >> 4;          // K group: chunk 4kr + g
    const int tcol = col >> 1;        // token of that column
    const int colb = col & 1;         // 0: column A, 1: column B
    MTile cur = mtile_of<kRowGroups, kRing, kComputeWaves>(desc_of(probs + (te0 >> kTileRowBits), te0), wave, lane);
    __builtin_amdgcn_s_barrier();     // the staging wave has issued tile 0's activation loads
    v4u32 ring[kRing];
#pragma unroll
    for (int r = 0; r + 1 < kRing; ++r) ring[r] = load_step<kRowGroups>(cur, cur, true, r);

    for (int par = 0, q = 0;; par ^= 1, q = q == kDescSlots - 1 ? 0 : q + 1) {
        // this tile is staged and the next one named; every wave is done with the
        // last; the ring's loads of this tile's first steps stay in flight
        lds_barrier();
        const MDesc cd = desc_load(descs + q);
        const MDesc nd = desc_load(descs + (q == kDescSlots - 1 ? 0 : q + 1));
        const bool has_next = nd.te != kEnd;
        const MTile nxt = mtile_of<kRowGroups, kRing, kComputeWaves>(has_next ? nd : cd, wave, lane);
        const uint8_t* const slot = smem + (size_t)par * slot_bytes;
        const TokenData* const tok = tokd + par * MT;
        const int m = cd.m;
        // This lane's activation planes (chunk 4kr + g of its token, in each
        // column set): column A of level j reads plane 5 - j, column B plane
        // 4 - j, 16 bytes lower, and zeros for P_5.  Columns of tokens past m
        // read token 0's planes: every output column is independent of the
        // others, and those columns are never stored.
        const uint8_t* blk[kSets];
#pragma unroll
        for (int cs = 0; cs < kSets; ++cs) {
            const int tt = 8 * cs + tcol;
            blk[cs] = slot + (size_t)((tt < m ? tt : 0) * cur.cpad + g) * kPlaneBytes;
        }

        v4i32 acc[kRowGroups][kSets] = {};
        v4i32 bop[kSets][kOps];
        // one step: the lane's 16 weight bytes against the K range's operands
        auto run_step = [&](const v4u32& w, v4i32 (&ea)[kSets]) {
            constexpr uint32_t mag = 0x64646464u;
            v4u32 p5, lo, hi, pq;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                p5[d] = w[d] ^ 0x80808080u;
                lo[d] = __builtin_amdgcn_perm(mag, w[d], 0x04020400u);   // [b0 64 b2 64] = fp16 1024 + b
                hi[d] = __builtin_amdgcn_perm(mag, w[d], 0x04030401u);   // [b1 64 b3 64]
            }
#pragma unroll
            for (int cs = 0; cs < kSets; ++cs)
                ea[cs] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop[cs][0], __builtin_bit_cast(v4i32, p5), ea[cs], 0, 0, 0);
#pragma unroll
            for (int lvl = 0; lvl < 4; ++lvl) {   // P_4 .. P_1
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    lo[d] = third2(lo[d]);
                    hi[d] = third2(hi[d]);
                    pq[d] = __builtin_amdgcn_perm(hi[d], lo[d], 0x06020400u);   // the four quotients in byte order
                }
#pragma unroll
                for (int cs = 0; cs < kSets; ++cs)
                    ea[cs] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bop[cs][1 + lvl], __builtin_bit_cast(v4i32, pq),
                                                                   ea[cs], 0, 0, 0);
            }
        };
        // Register ring: while step s is consumed, steps s+1 .. s+kRing-1 are in
        // flight.  Steps run in groups of kRing (a tile pads its steps to a
        // multiple), the row group of step s is s % 2 and its K range s / 2,
        // both static inside a group; only the last group's loads reach past
        // this tile, into the next tile's first steps.
        auto groups = [&](auto rgs_tag) {
            constexpr int RGS = decltype(rgs_tag)::value;
            const int S = cur.S, Spad = cur.Spad;
            auto group = [&](int s0, auto last_tag) {
                constexpr bool LAST = decltype(last_tag)::value;
#pragma unroll
                for (int u = 0; u < kRing; ++u) {
                    const int s = s0 + u;
                    const int b = s + kRing - 1;
                    if (!LAST || u == 0) {
                        const uint32_t off = (uint32_t)(b / RGS) * cur.kstride + (uint32_t)(b % RGS) * 256u;
                        ring[(u + kRing - 1) % kRing] = load_at(cur.w, cur.nrec, b < S ? cur.lane_base + off : kOob);
                    } else {
                        ring[(u + kRing - 1) % kRing] =
                            load_step<kRowGroups>(nxt, nxt, true, has_next ? b - Spad : nxt.Spad);
                    }
                    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the step they overlap
                    if (s < S) {
                        const int rg = u % RGS;   // a constant once the loop is unrolled
                        if (rg == 0) {   // a new K range: its operands from LDS
                            const int off = (s / RGS) * 4 * kPlaneBytes;
#pragma unroll
                            for (int cs = 0; cs < kSets; ++cs) {
#pragma unroll
                                for (int i = 1; i < kOps; ++i)
                                    bop[cs][i] = *reinterpret_cast<const v4i32*>(blk[cs] + off + 16 * (i - colb));
                                bop[cs][0] = *reinterpret_cast<const v4i32*>(colb ? zeros : blk[cs] + off);
                            }
                        }
                        run_step(ring[u], acc[rg]);
                    }
                }
            };
            for (int s0 = 0; s0 < Spad - kRing; s0 += kRing) group(s0, std::false_type{});
            group(Spad - kRing, std::true_type{});
        };
        groups(std::integral_constant<int, kRowGroups>{});

        // ---- epilogue: lane group g holds tokens 2g and 2g + 1 of each column
        // set, for its row ---------------------------------------------------------
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) {
            const int row = cur.row0 + 16 * rg + (lane & 15);
            if (row < cur.n) {
#pragma unroll
                for (int cs = 0; cs < kSets; ++cs) {
                    const v4i32 a = acc[rg][cs];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int t = 8 * cs + 2 * g + h;
                        if (t < MT && t < m) {
                            const int tot =
                                (int)((uint32_t)a[2 * h] - 3u * (uint32_t)a[2 * h + 1] + (uint32_t)tok[t].corr);
                            const size_t o = (size_t)t * cur.n + row;
                            gstore_ptr(cd.y)[o] = (float)tot * tok[t].sx * cd.sw;
                            if (cd.acc) gstore_ptr(cd.acc)[o] = tot;
                        }
                    }
                }
            }
        }
        if (!has_next) break;
        cur = nxt;
    }
}

template <int MT>
hipError_t launch_mx_one(const DevProblem* probs, uint32_t* sched, int nb, int32_t slot_bytes, hipStream_t s)
{
    hipLaunchKernelGGL((k_gemv_mx<MT>), dim3((unsigned)nb), dim3(MxShape<MT>::kThreads), gemv_mx_lds_bytes(MT, slot_bytes), s,
                       probs, sched, slot_bytes);
    return hipGetLastError();
}

template <int MT>
int mx_occupancy_one(int64_t slot_bytes)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&k_gemv_mx<MT>), MxShape<MT>::kThreads,
                                                     gemv_mx_lds_bytes(MT, slot_bytes)) != hipSuccess)
        return 0;
    return n;
}

}  // namespace

int gemv_mx_ring(int mt) { return mt > 8 ? MxShape<16>::kRing : mt > 4 ? MxShape<8>::kRing : MxShape<4>::kRing; }

int gemv_mx_row_groups(int mt)
{
    return mt > 8 ? MxShape<16>::kRowGroups : mt > 4 ? MxShape<8>::kRowGroups : MxShape<4>::kRowGroups;
}

int64_t gemv_mx_tile_rows(int mt)
{
    return mt > 8 ? MxShape<16>::kTileRows : mt > 4 ? MxShape<8>::kTileRows : MxShape<4>::kTileRows;
}

int gemv_mx_tokens(int max_m)
{
    return max_m <= 1 ? 1 : max_m <= 2 ? 2 : max_m <= 4 ? 4 : max_m <= 8 ? 8 : max_m <= 16 ? 16 : 0;
}

int64_t gemv_mx_slot_bytes(int mt, int chunks)
{
    return (int64_t)mt * 4 * ((chunks + 3) / 4) * kPlaneBytes;
}

size_t gemv_mx_lds_bytes(int mt, int64_t slot_bytes)
{
    return (size_t)(2 * slot_bytes + kDescSlots * (int64_t)sizeof(MDesc) + 2 * mt * (int64_t)sizeof(TokenData) +
                    kZeroBytes);
}

int gemv_mx_wg_per_cu(int mt, int64_t slot_bytes)
{
    switch (mt) {
        case 1: return mx_occupancy_one<1>(slot_bytes);
        case 2: return mx_occupancy_one<2>(slot_bytes);
        case 4: return mx_occupancy_one<4>(slot_bytes);
        case 8: return mx_occupancy_one<8>(slot_bytes);
        case 16: return mx_occupancy_one<16>(slot_bytes);
        default: return 0;
    }
}

hipError_t setup_mx_attributes()
{
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&k_gemv_mx<1>));
    if (e == hipSuccess) e = raise_lds_limit(reinterpret_cast<const void*>(&k_gemv_mx<2>));
    if (e == hipSuccess) e = raise_lds_limit(reinterpret_cast<const void*>(&k_gemv_mx<4>));
    if (e == hipSuccess) e = raise_lds_limit(reinterpret_cast<const void*>(&k_gemv_mx<8>));
    if (e == hipSuccess) e = raise_lds_limit(reinterpret_cast<const void*>(&k_gemv_mx<16>));
    return e;
}

hipError_t launch_gemv_mx(const DevProblem* probs, uint32_t* sched, int nb, int mt, int32_t slot_bytes, hipStream_t s)
{
    switch (mt) {
        case 1: return launch_mx_one<1>(probs, sched, nb, slot_bytes, s);
        case 2: return launch_mx_one<2>(probs, sched, nb, slot_bytes, s);
        case 4: return launch_mx_one<4>(probs, sched, nb, slot_bytes, s);
        case 8: return launch_mx_one<8>(probs, sched, nb, slot_bytes, s);
        case 16: return launch_mx_one<16>(probs, sched, nb, slot_bytes, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmv
