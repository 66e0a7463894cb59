// k_gemv_stream.hip -- persistent grouped GEMV for 1..2 tokens (gfx950).
//
// Same results as k_gemv.hip (exact int32 dot of int8 activations with
// five-trits-per-byte or int8 weights, scales applied once after the sum:
// "Gemma 3 1B at 114 tokens per second on a laptop CPU", "Step 1"; cpp20gemma
// README, "Architecture & implementation"), organised for streaming:
//
//  * Work unit = a workgroup tile: 4 * 2R rows of one problem, one 2R-row wave
//    tile per compute wave.  R = 64 / L, L = lanes per row (1, 2, 4 or 8, chosen
//    by the host so tiles are of similar length).  Lane s*R + r of a wave
//    streams chunks s, s + L, s + 2L, ... of rows r and R + r (the two rows
//    share every activation read); for a fixed s the R rows' chunk is one
//    contiguous run of R * 16 bytes.  The L partial sums of a row meet through
//    lane shuffles at the end of the tile.
//  * Tiles are dealt to the 8 XCDs by the host (longest processing time
//    first; workgroup b runs on XCD b mod 8).  Inside an XCD's list a
//    workgroup's first tile is fixed (its rank among the XCD's workgroups) and
//    every later one is taken from a per-XCD atomic counter, one tile ahead, by
//    the staging wave: workgroups that run slower take fewer tiles and all
//    finish within about one tile of each other.  The last workgroup of an XCD
//    to finish resets its counters for the next launch.
//  * A workgroup is four compute waves and one staging wave.  The staging
//    wave prepares the next tile's activations in LDS (two slots) while the
//    compute waves stream the current one, so activation loads never sit in
//    the compute waves' in-order memory counters.  For ternary weights what is
//    staged is not x itself but, per packed byte, the five int16 combinations
//    Z_1..Z_5 of zform.hpp, in the order the weight registers come out of
//    the unpacker: the page's once-per-token input reorder.
//  * Weight loads are raw buffer loads into a register ring (kRing - 1 chunk
//    loads in flight while one is consumed): past the end of the matrix they
//    return zeros instead of faulting, so no lane clamps or branches; loads past
//    a tile's last chunk fetch the next tile's first chunks.
//
// Ternary arithmetic: the Z form of zform.hpp (P_j . Z_j sums on v_dot2_i32_i16,
// one correction per row).
#include "qmv_internal.hpp"
#include "unpack.hpp"
#include "zform.hpp"

namespace qmv {
namespace {

#ifndef QMV_STREAM_RING
#define QMV_STREAM_RING 4
#endif
constexpr int kRPL = kStreamRowsPerLane;       // rows per lane: they share each staged activation read
constexpr int kRing = QMV_STREAM_RING;         // chunk steps in the register ring: kRing - 1 in flight
constexpr int kStepGrain = kRing;              // chunk steps of a tile are a multiple of this
constexpr int kComputeWaves = 4;
constexpr int kStreamThreads = (kComputeWaves + 1) * kWave;   // + the staging wave
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format
constexpr int kZBytes = 192;                   // staged bytes per 16-byte ternary chunk per token (4 x 12 dwords)
constexpr int kXBytes = 16;                    // staged bytes per 16-byte int8 chunk per token
constexpr uint32_t kEnd = 0xffffffffu;         // no tile
constexpr int kNonTemporal = 2;                // buffer instruction cache policy: nt
constexpr int kDescSlots = 3;                  // tile descriptors in LDS, used round robin

// Sum over a wave, exact in int32 arithmetic: prefix sums inside each row of
// 16 lanes by DPP row shifts (lanes shifted in from outside the row add 0),
// then the four row totals through lane reads.
__device__ __forceinline__ int wave_total(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) + __builtin_amdgcn_readlane(v, 47) +
           __builtin_amdgcn_readlane(v, 63);
}

// One ticket from an XCD's counter (one lane).  The address is hidden from the
// compiler's uniformity analysis: otherwise it turns the atomic into a wave-wide
// one whose result is shared out at once, which waits for the atomic (a
// contended counter takes microseconds) right there instead of where the
// ticket is first used, one tile later.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* counter)
{
    uintptr_t a = reinterpret_cast<uintptr_t>(counter);
    asm volatile("" : "+v"(a));
    return __hip_atomic_fetch_add(gstore_ptr(reinterpret_cast<uint32_t*>(a)), 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

// What a wave needs to know about one workgroup tile.
struct Tile {
    const DevProblem* P;
    const int8_t* x8;
    const uint8_t* w;
    int n, k, m, C, lshift, wb, nsteps, cpad, tok_bytes;
    uint32_t chunk_bytes;   // n * 16: one chunk of every row
    int s_part, row;        // per lane (compute waves): its first row (the second is row + R)
    uint32_t voff;          // per lane: byte offset of its first row's chunk s_part
    uint32_t voff_r;        // R rows of one chunk: the second row's offset is voff + voff_r
};

// The part of a tile the compute waves use, as the staging wave leaves it in
// LDS for them (so they never wait on descriptor loads from memory).
struct TileDesc {
    const uint8_t* w;
    float* y;
    int32_t* acc;
    int32_t n, m, C, lshift, wb;
    uint32_t te;            // tile entry, kEnd = no tile
    float sw;
    float sx[2];
    int32_t pad;
};
static_assert(sizeof(TileDesc) == 64, "TileDesc layout");

template <int CB>
__device__ __forceinline__ void tile_derive(Tile& T, int wave, int lane)
{
    const int L = 1 << T.lshift;
    const int rshift = 6 - T.lshift;                          // R = 64 / L rows per wave tile
    T.nsteps = (((T.C + L - 1) >> T.lshift) + kStepGrain - 1) / kStepGrain * kStepGrain;
    T.cpad = T.nsteps << T.lshift;                            // staged chunks: C real, the rest zeros
    T.tok_bytes = T.cpad * CB;
    T.chunk_bytes = (uint32_t)T.n * 16u;
    T.s_part = lane >> rshift;
    T.row = (((T.wb * kComputeWaves + wave) * kRPL) << rshift) + (lane & ((1 << rshift) - 1));
    T.voff = (uint32_t)((T.s_part * T.n + T.row) * 16);
    T.voff_r = 16u << rshift;
}

template <int CB>
__device__ __forceinline__ Tile tile_at(const DevProblem* probs, uint32_t te, int wave, int lane)
{
    Tile T;
    T.P = probs + (te >> kTileRowBits);
    T.wb = (int)(te & ((1u << kTileRowBits) - 1));
    T.x8 = T.P->x8;
    T.w = T.P->w;
    T.n = T.P->n;
    T.k = T.P->k;
    T.m = T.P->m;
    T.C = T.P->chunks;
    T.lshift = 31 - __builtin_clz((uint32_t)T.P->lanes_per_row);   // lanes per row: 1, 2, 4 or 8
    tile_derive<CB>(T, wave, lane);
    return T;
}

__device__ __forceinline__ TileDesc desc_of(const Tile& T, uint32_t te)
{
    TileDesc d;
    d.w = T.w;
    d.y = T.P->y;
    d.acc = T.P->acc;
    d.n = T.n;
    d.m = T.m;
    d.C = T.C;
    d.lshift = T.lshift;
    d.wb = T.wb;
    d.te = te;
    d.sw = *cload_ptr(T.P->sw);
    d.sx[0] = cload_ptr(T.P->sx)[0];
    d.sx[1] = cload_ptr(T.P->sx)[T.m > 1 ? 1 : 0];
    d.pad = 0;
    return d;
}

// A descriptor read back from LDS, made wave-uniform.
__device__ __forceinline__ TileDesc desc_load(const TileDesc* p)
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
    return __builtin_bit_cast(TileDesc, v);
}

template <int CB>
__device__ __forceinline__ Tile tile_of(const TileDesc& d, int wave, int lane)
{
    Tile T;
    T.P = nullptr;
    T.x8 = nullptr;
    T.w = d.w;
    T.n = d.n;
    T.k = 0;
    T.m = d.m;
    T.C = d.C;
    T.lshift = d.lshift;
    T.wb = d.wb;
    tile_derive<CB>(T, wave, lane);
    return T;
}

// Step i of a tile reads chunks iL .. iL+L-1: a buffer based at chunk iL whose
// size is what is left of the matrix, so reads past its end return zeros (the
// host keeps every matrix of this kernel under 2^31 bytes).
__device__ __forceinline__ v4u32 load_step(const Tile& T, int i, uint32_t voff)
{
    const int c0 = min(i << T.lshift, T.C);
    const uint32_t nrec = (uint32_t)(T.C - c0) * T.chunk_bytes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(T.w + (uint32_t)c0 * T.chunk_bytes), (short)0, (int)nrec, (int)kRsrcWord3);
    // weights are read once per launch: non-temporal (aux bit 1), so they do not
    // displace the activations and tables the caches should keep
    return __builtin_bit_cast(v4u32, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kNonTemporal));
}

// ---------------------------------------------------------------------------
// Staging (one wave).  Activation unit u of token mi is a 20-column group (5
// dwords, ternary) or one dword (int8) of the row, at any alignment and for
// any k: the aligned dwords holding it are read through a buffer sized to the
// row's aligned dwords (zeros past them), funnel-shifted into place, and bytes
// past column k are zeroed.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uintptr_t row_addr(const Tile& T, int mi)
{
    return reinterpret_cast<uintptr_t>(T.x8) + (uintptr_t)mi * (uintptr_t)T.k;
}

// The aligned dwords of token mi's row, as a buffer: reads past them return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const Tile& T, int mi, uint32_t& sh)
{
    const uintptr_t a = row_addr(T, mi);
    sh = (uint32_t)(a & 3);
    const uint32_t words = (sh + (uint32_t)T.k + 3u) >> 2;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a & ~(uintptr_t)3), (short)0, (int)(4 * words), (int)kRsrcWord3);
}

// Unit u: its kD + 1 aligned dwords are loaded (unit_load), then shifted into
// place with bytes past column k cleared (unit_of).
template <int WT>
__device__ __forceinline__ void unit_load(__amdgpu_buffer_rsrc_t rs, int u, uint32_t* raw)
{
    constexpr int kD = WT == 1 ? 5 : 1;
#pragma unroll
    for (int j = 0; j <= kD; ++j) raw[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (kD * u + j), 0, 0);
}

template <int WT>
__device__ __forceinline__ void unit_of(const Tile& T, uint32_t sh, int u, const uint32_t* raw, uint32_t* nat)
{
    constexpr int kD = WT == 1 ? 5 : 1;
#pragma unroll
    for (int j = 0; j < kD; ++j) {
        const uint32_t v = __builtin_amdgcn_alignbyte(raw[j + 1], raw[j], sh);
        const int valid = T.k - 4 * (kD * u + j);
        nat[j] = valid >= 4 ? v : valid <= 0 ? 0u : v & ((1u << (8 * valid)) - 1u);
    }
}

// The ten Z words of group g (chunk g / 4, dword g % 4) into their 48-byte
// slot of the staged chunk.
__device__ __forceinline__ void put_z(uint32_t* zo, int g, const uint32_t zz[10])
{
    uint32_t* d = zo + (g >> 2) * 48 + (g & 3) * 12;
    reinterpret_cast<uint4*>(d)[0] = make_uint4(zz[0], zz[1], zz[2], zz[3]);
    reinterpret_cast<uint4*>(d)[1] = make_uint4(zz[4], zz[5], zz[6], zz[7]);
    reinterpret_cast<uint2*>(d)[4] = make_uint2(zz[8], zz[9]);
}

// Stage tile T into an LDS slot (the staging wave): Z values (ternary) or x
// (int8) for chunks 0..C-1, zeros up to cpad, and the ternary correction
// 25600 * sum Z + sum x of each token.  `after_loads` runs once, in uniform
// control flow, right after the first activation loads of every lane are
// issued: work placed there overlaps their latency instead of delaying them.
template <int MT, int WT, bool SKIP, class F>
__device__ __forceinline__ void stage(const Tile& T, int lane, uint8_t* slot, int* corr, F after_loads)
{
    constexpr int kD = WT == 1 ? 5 : 1;
    // Zero-unit mask (SKIP): bit j of word i is set while unit j of the chunks
    // of step i (chunks iL .. iL+L-1) is zero for every token so far; the
    // lanes clear the bits of units they find non-zero.  Units past k count
    // as zero.  The words follow the tokens' staged values.
    uint32_t* const mask = reinterpret_cast<uint32_t*>(slot + (size_t)MT * T.tok_bytes);
    if (SKIP)
        for (int i = lane; i < T.nsteps; i += kWave) mask[i] = 0xfu;
    // units per lane loaded before any is used: a ternary row of up to
    // 64 * 2 * 20 = 2560 columns costs one memory round trip.  Larger batches
    // would cover longer rows in one trip but raise the kernel's register
    // count past what four resident workgroups per compute unit allow.
    constexpr int kBatch = 2;
    bool first = true;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
        if (mi > 0 && mi >= T.m) continue;
        uint32_t* zo = reinterpret_cast<uint32_t*>(slot + (size_t)mi * T.tok_bytes);
        const int units = 4 * T.C;
        uint32_t sh;
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(T, mi, sh);
        int s_z = 0, s_x = 0;
        for (int g0 = 0; g0 < units; g0 += kWave * kBatch) {
            uint32_t raw[kBatch][kD + 1];
            // the batch's loads, wave-uniform conditions (reads past the row
            // return zeros)
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (b == 0 || g0 + kWave * b < units) unit_load<WT>(rs, g0 + kWave * b + lane, raw[b]);
            if (first) {
                after_loads();
                first = false;
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int g = g0 + kWave * b + lane;
                if (g < units) {
                    if (WT == 1) {
                        uint32_t nat[5], zz[10];
                        unit_of<1>(T, sh, g, raw[b], nat);
                        z_group(nat, zz, s_z, s_x);
                        put_z(zo, g, zz);
                        if (SKIP && (nat[0] | nat[1] | nat[2] | nat[3] | nat[4]) != 0u)
                            __hip_atomic_fetch_and(&mask[(g >> 2) >> T.lshift], ~(1u << (g & 3)), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                    } else {
                        unit_of<2>(T, sh, g, raw[b], &zo[g]);
                    }
                }
            }
        }
        if (WT == 1) {
            for (int d = 48 * T.C + lane; d < 48 * T.cpad; d += kWave) zo[d] = 0u;
            const int cw = wave_total(z_correction(s_z, s_x));
            if (lane == 0) corr[mi] = cw;
        } else {
            for (int d = units + lane; d < 4 * T.cpad; d += kWave) zo[d] = 0u;
        }
    }
}

// Schedule words: [counters: 8 tile counters + 8 done counters, 64 words
// apart][first tile entry of each workgroup][8 x (list offset, list size)]
// [tile entries of the 8 XCD lists].
// LDS: [2 tile slots of slot_bytes][3 tile descriptors][corr: 2 x MT]
template <int MT, int WT, bool SKIP>
__global__ __launch_bounds__(kStreamThreads) void k_gemv_stream(const DevProblem* __restrict__ probs,
                                                               uint32_t* __restrict__ sched, int32_t slot_bytes)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int kCB = (WT == 1) ? kZBytes : kXBytes;   // staged bytes per chunk per token
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // Tile q's descriptor is in descs[q % 3]: the staging wave writes tile q + 2's
    // after barrier q + 1, and the compute waves last read that slot (as tile
    // q - 1's) before barrier q.
    TileDesc* const descs = reinterpret_cast<TileDesc*>(smem + 2 * (size_t)slot_bytes);
    int* const corr_base = reinterpret_cast<int*>(descs + kDescSlots);

    const int xcd = blockIdx.x % kStreamXcds;
    const uint32_t wgs = (gridDim.x - xcd + kStreamXcds - 1) / kStreamXcds;   // workgroups of this XCD
    // A workgroup's first two tiles are one load away; the rest of its XCD's
    // list is dealt by the ticket counter, from entry 2 * wgs on.
    const uint32_t te0 = cload_ptr(sched + kStreamHdr)[2 * blockIdx.x];
    const uint32_t* const hdr = sched + kStreamHdr + 2 * gridDim.x;

    if (wave == kComputeWaves) {
        // ---- staging wave: tile q into slot q & 1, the entry of tile q + 1, then
        // barrier q ------------------------------------------------------------------
        // The counter is read one tile ahead of its use (an atomic under
        // contention takes microseconds): the ticket for tile q + 2 is taken
        // while tile q + 1 is streamed.  Tile 1 is the static second entry, so
        // nothing on the way to the first barrier waits for an atomic.
        const uint32_t te1 = cload_ptr(sched + kStreamHdr)[2 * blockIdx.x + 1];
        uint32_t te = te0;
        uint32_t ticket = 0;
        Tile T, T1;
        TileDesc d1;
        if (te != kEnd) T = tile_at<kCB>(probs, te, 0, lane);
        if (te1 != kEnd) {   // tile 1's descriptor, fetched with tile 0's (scalar loads)
            T1 = tile_at<kCB>(probs, te1, 0, lane);
            d1 = desc_of(T1, te1);
        }
        // the XCD's list, read now: these loads return with tile 0's, not behind
        // the chip's first weight loads
        const uint32_t list_off = cload_ptr(hdr)[2 * xcd];
        const uint32_t list_size = cload_ptr(hdr)[2 * xcd + 1];
        const uint32_t* const list = hdr + 2 * kStreamXcds + list_off;
        bool first = true;
        for (int par = 0, q = 0; te != kEnd; par ^= 1, q = q == kDescSlots - 1 ? 0 : q + 1) {
            const int qn = q == kDescSlots - 1 ? 0 : q + 1;   // the next tile's descriptor slot
            stage<MT, WT, SKIP>(T, lane, smem + (size_t)par * slot_bytes, corr_base + par * MT, [&] {
                if (first) {
                    // Tile 0: release the compute waves' weight prefetch only once
                    // these loads (and the tile's scales) are back: they gate every
                    // wave of the workgroup, and behind the prefetch of the whole
                    // chip (tens of MB) they would wait microseconds.  Then the
                    // tile's descriptor and the first ticket.
                    const TileDesc d0 = desc_of(T, te);   // wave-uniform: scalar loads
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
                T = T1;
                if (lane == 0) descs[qn] = d1;
            } else if (nx != kEnd) {
                T = tile_at<kCB>(probs, nx, 0, lane);
                if (lane == 0) descs[qn] = desc_of(T, nx);
            } else if (lane == 0) {
                descs[qn].te = kEnd;
            }
            te = nx;
            // the tile's LDS writes are done; the ticket taken above stays in flight
            lds_barrier();
        }
        // Every workgroup of the XCD counts itself done once; the last one resets
        // both counters.  Relaxed order suffices: a workgroup reaches this point
        // only after the value of its last ticket came back (its loop exit
        // depends on it), so every ticket of the launch has been taken before
        // the last done count, and the resets reach the next launch through the
        // end of this kernel.  (Acquire/release here would write back and
        // invalidate the XCD's L2 per workgroup.)
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

    // ---- compute waves ----------------------------------------------------------------
    Tile cur = tile_at<kCB>(probs, te0, wave, lane);
    __builtin_amdgcn_s_barrier();   // the staging wave has issued tile 0's activation loads
    v4u32 ring[kRing][kRPL];
#pragma unroll
    for (int r = 0; r + 1 < kRing; ++r)
#pragma unroll
        for (int h = 0; h < kRPL; ++h) ring[r][h] = load_step(cur, r, cur.voff + h * cur.voff_r);

    for (int par = 0, q = 0;; par ^= 1, q = q == kDescSlots - 1 ? 0 : q + 1) {
        // this tile is staged and the next one named; every wave is done with the
        // last; the ring's loads of this tile's first steps stay in flight
        lds_barrier();
        // The next tile (after the last one: the tile itself, with its batch loads
        // past the matrix end, so every path is the same).
        const TileDesc cd = desc_load(descs + q);
        const TileDesc nd = desc_load(descs + (q == kDescSlots - 1 ? 0 : q + 1));
        const bool has_next = nd.te != kEnd;
        const Tile nxt = tile_of<kCB>(has_next ? nd : cd, wave, lane);
        const uint8_t* zs = smem + (size_t)par * slot_bytes;
        const int* corr = corr_base + par * MT;

        int acc_lo[kRPL][MT], acc_hi[kRPL][MT];
#pragma unroll
        for (int h = 0; h < kRPL; ++h)
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                acc_lo[h][mi] = 0;
                acc_hi[h][mi] = 0;
            }
        const uint8_t* zlane = zs + cur.s_part * kCB;
        const int zstep = kCB << cur.lshift;
        const int tok_bytes = cur.tok_bytes;
        // one chunk step: the weight chunk of each of the lane's rows against the
        // staged activations of that chunk
        const uint32_t* const zmask = reinterpret_cast<const uint32_t*>(zs + (size_t)MT * tok_bytes);
        auto run_step = [&](const v4u32* src, int i) {
            const uint8_t* zc = zlane + i * zstep;
            if (WT == 1) {
                // SKIP: the step's units whose activations are zero for every
                // token and every lane part add nothing; a wave-uniform skip
                const uint32_t zm = SKIP ? __builtin_amdgcn_readfirstlane(zmask[i]) : 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (SKIP && ((zm >> j) & 1u)) continue;
                    uint4 Z[MT][3];   // the 10 Z pairs of dword j (and two pad words)
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
                        for (int q = 0; q < 3; ++q)
                            Z[mi][q] = reinterpret_cast<const uint4*>(zc + (size_t)mi * tok_bytes + 48 * j)[q];
#pragma unroll
                    for (int h = 0; h < kRPL; ++h) {
                        constexpr uint32_t mag = 0x64646464u;
                        uint32_t lo = __builtin_amdgcn_perm(mag, src[h][j], 0x04020400u);   // 1024 + b0 | b2
                        uint32_t hi = __builtin_amdgcn_perm(mag, src[h][j], 0x04030401u);   // 1024 + b1 | b3
#pragma unroll
                        for (int i5 = 4; i5 >= 0; --i5) {   // P_5 = b, then P_4 .. P_1
#pragma unroll
                            for (int mi = 0; mi < MT; ++mi) {
                                acc_lo[h][mi] = dot2(lo, sel(Z[mi][i5 >> 1], (2 * i5) & 3), acc_lo[h][mi]);
                                acc_hi[h][mi] = dot2(hi, sel(Z[mi][i5 >> 1], (2 * i5 + 1) & 3), acc_hi[h][mi]);
                            }
                            if (i5 > 0) {
                                lo = third2(lo);
                                hi = third2(hi);
                            }
                        }
                    }
                    // one dword at a time: other waves hide the latency, and short
                    // live ranges leave room for the ring
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int mi = 0; mi < MT; ++mi) {
                    const uint4 X = *reinterpret_cast<const uint4*>(zc + (size_t)mi * tok_bytes);
#pragma unroll
                    for (int h = 0; h < kRPL; ++h) {
                        int a = acc_lo[h][mi];
                        a = dot4(src[h][0], X.x, a);
                        a = dot4(src[h][1], X.y, a);
                        a = dot4(src[h][2], X.z, a);
                        a = dot4(src[h][3], X.w, a);
                        acc_lo[h][mi] = a;
                    }
                }
            }
        };
        // Register ring: while step i is consumed, steps i+1 .. i+kRing-1 are in
        // flight; loads past this tile's last step fetch the next tile's first
        // steps (after the last tile: nothing, they lie past the matrix end).
        const int nsteps = cur.nsteps;   // a multiple of kRing, at least kRing
        for (int i0 = 0; i0 < nsteps; i0 += kRing) {
#pragma unroll
            for (int s = 0; s < kRing; ++s) {
                const int b = i0 + s + kRing - 1;
                const bool mine = b < nsteps;
                const Tile& src_t = mine ? cur : nxt;
                const uint32_t vo = mine ? cur.voff : nxt.voff;
                const uint32_t vr = mine ? cur.voff_r : nxt.voff_r;
                const int bb = mine ? b : (has_next ? b - nsteps : nsteps + kRing);
#pragma unroll
                for (int h = 0; h < kRPL; ++h) ring[(s + kRing - 1) % kRing][h] = load_step(src_t, bb, vo + h * vr);
                __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the step they overlap
                run_step(ring[s], i0 + s);
            }
        }

        // ---- combine the L lanes of each row and write the tile --------------------
        int cr[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) cr[mi] = WT == 1 ? corr[mi] : 0;
#pragma unroll
        for (int h = 0; h < kRPL; ++h) {
            int total[MT];
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) total[mi] = acc_lo[h][mi] + acc_hi[h][mi];
            for (int off = kWave >> cur.lshift; off < kWave; off <<= 1) {
#pragma unroll
                for (int mi = 0; mi < MT; ++mi) total[mi] += __shfl_xor(total[mi], off, kWave);
            }
            const int row = cur.row + (h << (6 - cur.lshift));
            if (row < cur.n && cur.s_part == 0) {
                QMV_GLOBAL float* y = gstore_ptr(cd.y);
                int32_t* accp = cd.acc;
#pragma unroll
                for (int mi = 0; mi < MT; ++mi) {
                    if (mi < cur.m) {
                        const int tot = (int)((uint32_t)total[mi] - (uint32_t)cr[mi]);
                        const size_t o = (size_t)mi * cur.n + row;
                        y[o] = (float)tot * cd.sx[mi] * cd.sw;
                        if (accp) gstore_ptr(accp)[o] = tot;
                    }
                }
            }
        }
        if (!has_next) break;
        cur = nxt;
    }
}

template <int MT, int WT, bool SKIP>
hipError_t launch_stream_one(const DevProblem* probs, uint32_t* sched, int nb, int32_t slot_bytes, hipStream_t s)
{
    const size_t lds = gemv_stream_lds_bytes(MT, slot_bytes);
    hipLaunchKernelGGL((k_gemv_stream<MT, WT, SKIP>), dim3((unsigned)nb), dim3(kStreamThreads), lds, s, probs, sched,
                       slot_bytes);
    return hipGetLastError();
}

}  // namespace

int64_t gemv_stream_steps(int chunks, int lanes)
{
    return ((chunks + lanes - 1) / lanes + kStepGrain - 1) / kStepGrain * kStepGrain;
}

int64_t gemv_stream_slot_bytes(int wtype, int mt, int chunks, int lanes)
{
    // ternary slots end with the zero-unit mask of the skipping variant (one
    // word per step)
    const int64_t steps = gemv_stream_steps(chunks, lanes);
    return (int64_t)mt * steps * lanes * (wtype == 1 ? kZBytes : kXBytes) + (wtype == 1 ? 4 * steps : 0);
}

size_t gemv_stream_lds_bytes(int mt, int64_t slot_bytes)
{
    return (size_t)(2 * slot_bytes + kDescSlots * (int64_t)sizeof(TileDesc) + 2 * mt * (int64_t)sizeof(int));
}

template <int MT, int WT, bool SKIP>
int occupancy_one(int64_t slot_bytes)
{
    const size_t lds = gemv_stream_lds_bytes(MT, slot_bytes);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&k_gemv_stream<MT, WT, SKIP>),
                                                     kStreamThreads, lds) != hipSuccess)
        return 0;
    return n;
}

int gemv_stream_wg_per_cu(int wtype, int max_m, int64_t slot_bytes, bool skip)
{
    if (wtype == 1) {
        if (skip) return max_m <= 1 ? occupancy_one<1, 1, true>(slot_bytes) : occupancy_one<2, 1, true>(slot_bytes);
        return max_m <= 1 ? occupancy_one<1, 1, false>(slot_bytes) : occupancy_one<2, 1, false>(slot_bytes);
    }
    return max_m <= 1 ? occupancy_one<1, 2, false>(slot_bytes) : occupancy_one<2, 2, false>(slot_bytes);
}

namespace {
template <int MT, int WT, bool SKIP>
hipError_t stream_lds_limit()
{
    return raise_lds_limit(reinterpret_cast<const void*>(&k_gemv_stream<MT, WT, SKIP>));
}
}  // namespace

hipError_t setup_stream_attributes()
{
    hipError_t e = stream_lds_limit<1, 1, false>();
    if (e == hipSuccess) e = stream_lds_limit<2, 1, false>();
    if (e == hipSuccess) e = stream_lds_limit<1, 1, true>();
    if (e == hipSuccess) e = stream_lds_limit<2, 1, true>();
    if (e == hipSuccess) e = stream_lds_limit<1, 2, false>();
    if (e == hipSuccess) e = stream_lds_limit<2, 2, false>();
    return e;
}

hipError_t launch_gemv_stream(const DevProblem* probs, uint32_t* sched, int nb, int wtype, int max_m,
                              int32_t slot_bytes, bool skip, hipStream_t s)
{
    if (wtype == 1) {
        if (skip) {
            if (max_m <= 1) return launch_stream_one<1, 1, true>(probs, sched, nb, slot_bytes, s);
            return launch_stream_one<2, 1, true>(probs, sched, nb, slot_bytes, s);
        }
        if (max_m <= 1) return launch_stream_one<1, 1, false>(probs, sched, nb, slot_bytes, s);
        return launch_stream_one<2, 1, false>(probs, sched, nb, slot_bytes, s);
    }
    if (max_m <= 1) return launch_stream_one<1, 2, false>(probs, sched, nb, slot_bytes, s);
    return launch_stream_one<2, 2, false>(probs, sched, nb, slot_bytes, s);
}

}  // namespace qmv
