// k_ffn.hip -- the feed-forward half of a stack of decoder layers for one
// token, in one persistent launch (llama2.c tour, "forward": Step 5, the gated
// feed-forward, and the residual connection after it; gemma.cpp tour, "The
// Forward Pass, Layer by Layer").  Per layer, on ternary weights:
//     x8, sx  = quantise(RMSNorm(h, norm))                    per-token int8
//     g, u    = (W_gate . x8) sx s_gate, (W_up . x8) sx s_up    exact int32 dots
//     q8, sq  = quantise(act(g) * u)
//     h       = h + (W_down . q8) sq s_down
// with the instructions of the chain qmv_rmsnorm_quantize -> qmv_gemv (gate
// and up) -> qmv_glu_quantize -> qmv_gemv (down) -> fp32 add, so the two agree
// bit for bit (actq.hpp, zform.hpp).
//
// Design (every workgroup resident for the whole launch):
//  * Every workgroup takes both kinds of task, so each step of a layer has the
//    whole chip.  Gate/up: workgroup b keeps its own copy of h in LDS; per layer
//    it applies the previous layer's residual update, RMSNorm and the int8
//    codes, then computes 32 rows of gate and up (eight waves = gate/up x four
//    quarters of the chunks, lanes 32..63 taking the odd chunks of a quarter)
//    and the GLU value of each row.  Down: workgroup b's task is 64 rows x a
//    run of chunks, split over the eight waves; it quantises the GLU values of
//    its own columns and adds int32 partial sums into one of two accumulators
//    with atomic adds.
//  * No device-wide barrier.  What crosses workgroups travels as 64-bit
//    records (value, tag), tag = launch generation << 8 | layer + 1, written
//    with device-coherent stores: the GLU values, the per-task max |GLU|, and
//    one tag per down task once its atomic adds have completed.  A consumer
//    polls exactly the records it needs until every tag is the one it waits
//    for.  Records of other layers or launches carry other tags, so nothing is
//    cleared between layers.
//  * A ninth wave per workgroup (the io wave) does all polling and gathers the
//    values into LDS, so the compute waves' weight loads, which are issued a
//    layer ahead as soon as their registers are free, never hold up a poll.
//  * Waits are bounded: a poll also reads the error word and the caller's
//    cancel word, and gives up after spin_limit rounds with a status.  The last
//    workgroup to finish (counted per XCD, then over the XCDs) writes the
//    status, clears the accumulators and advances the generation, so the
//    workspace is ready for the next launch whatever happened in this one.
//  * Cross-workgroup reads and writes use the sc1 (device-coherent) cache
//    policy: the XCDs' L2 caches are not coherent with each other for plain
//    accesses.  A record is only read after its producer's earlier writes
//    completed (the producer waits for their acknowledgement before it writes
//    the record).
#include <qmv.h>

#include "actq.hpp"
#include "qmv_internal.hpp"
#include "unpack.hpp"
#include "zform.hpp"

namespace qmv {
namespace {

constexpr int kCompute = kFfnComputeWaves;        // compute waves (two per SIMD)
constexpr int kThreads = (kCompute + 1) * kWave;  // + the io wave
constexpr int kCT = kCompute * kWave;             // compute threads
constexpr int kRmsThreads = 256;                  // RMSNorm's partial sums (the order of qmv_rmsnorm_quantize)
constexpr int kGuRegs = 4;      // gate/up chunks a lane holds in registers
constexpr int kDnRegs = kFfnDownChunks;   // down chunks per wave (the largest run)
constexpr int kNormRegs = 4;    // RMSNorm weights per thread kept in registers (h of up to 2048)
constexpr int64_t kDefaultSpin = 1 << 20;
constexpr int kFfnStamps = QMV_FFN_TRACE_STAMPS;   // trace stamps per layer
constexpr int kSc1 = 16;        // buffer instruction cache policy: sc1 (device-coherent)
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Control words (uint32 index).
constexpr int kGen = 0;                  // launch generation (24 bits)
constexpr int kErr = 64;                 // gen << 8 | QMV_FFN_* code of the launch's first error
constexpr int kExitX = 128;              // [8] workgroups out per XCD, 64 words apart
constexpr int kExitAll = 128 + 64 * 8;   // XCDs out

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_record(uint64_t* p, uint32_t v, uint32_t tag)
{
    __hip_atomic_store(p, (uint64_t)v | ((uint64_t)tag << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ v4u32 load_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, kSc1);
}

// One ternary chunk (16 packed bytes = 80 columns) of a lane's row against
// the chunk's 48 staged Z words (zform.hpp).
__device__ __forceinline__ void dot_chunk(const v4u32 w, const uint32_t* z, int& lo_acc, int& hi_acc)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 z0 = reinterpret_cast<const uint4*>(z + 12 * j)[0];
        const uint4 z1 = reinterpret_cast<const uint4*>(z + 12 * j)[1];
        const uint2 z2 = reinterpret_cast<const uint2*>(z + 12 * j)[4];
        const uint32_t zz[10] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w, z2.x, z2.y};
        constexpr uint32_t mag = 0x64646464u;
        uint32_t lo = __builtin_amdgcn_perm(mag, w[j], 0x04020400u);   // 1024 + b0 | b2
        uint32_t hi = __builtin_amdgcn_perm(mag, w[j], 0x04030401u);   // 1024 + b1 | b3
#pragma unroll
        for (int i5 = 4; i5 >= 0; --i5) {   // P_5 = b, then P_4 .. P_1
            lo_acc = dot2(lo, zz[2 * i5], lo_acc);
            hi_acc = dot2(hi, zz[2 * i5 + 1], hi_acc);
            if (i5 > 0) {
                lo = third2(lo);
                hi = third2(hi);
            }
        }
    }
}

// Z words of the 20-column group g of int8 codes x (LDS, 4-byte aligned) into
// z + 12 g; returns the group's share of the row correction.
__device__ __forceinline__ uint32_t z_of_group(const int8_t* x, int g, uint32_t* z)
{
    uint32_t nat[5], zz[10];
    const uint32_t* xw = reinterpret_cast<const uint32_t*>(x) + 5 * g;
#pragma unroll
    for (int q = 0; q < 5; ++q) nat[q] = xw[q];
    int s_z = 0, s_x = 0;
    z_group(nat, zz, s_z, s_x);
    uint32_t* d = z + 12 * g;
    reinterpret_cast<uint4*>(d)[0] = make_uint4(zz[0], zz[1], zz[2], zz[3]);
    reinterpret_cast<uint4*>(d)[1] = make_uint4(zz[4], zz[5], zz[6], zz[7]);
    reinterpret_cast<uint2*>(d)[4] = make_uint2(zz[8], zz[9]);
    return (uint32_t)z_correction(s_z, s_x);
}

// Wave reductions by DPP row shifts (lanes shifted in from outside a row of 16
// bring 0) and reads of the four row totals; every lane receives the result.
// Call with every lane of the wave active.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 15) + (uint32_t)__builtin_amdgcn_readlane((int)v, 31) +
           (uint32_t)__builtin_amdgcn_readlane((int)v, 47) + (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Max over a wave of non-negative values (float bit patterns order as uint).
__device__ __forceinline__ uint32_t wave_umax(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 15), (uint32_t)__builtin_amdgcn_readlane((int)v, 31)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 47), (uint32_t)__builtin_amdgcn_readlane((int)v, 63)));
}
__device__ __forceinline__ float wave_fmax(float v)   // v >= 0
{
    return __uint_as_float(wave_umax(__float_as_uint(v)));
}

__device__ __forceinline__ v4u32 load_chunk(const uint8_t* base, int64_t n, int c, int64_t row)
{
    const v4u32* p = reinterpret_cast<const v4u32*>(base + ((size_t)c * n + row) * 16);
    return __builtin_nontemporal_load(gload_ptr(p));
}

struct FfnLayerDev {
    const uint8_t* gate;
    const uint8_t* up;
    const uint8_t* down;
    const float* gate_scale;
    const float* up_scale;
    const float* down_scale;
    const float* norm;
};

struct FfnArgs {
    FfnLayerDev layer[QMV_FFN_LAUNCH_LAYERS];
    float* h;               // [hidden] in/out
    uint32_t* ctrl;         // control words
    uint32_t* done;         // [kFfnReplicas][done_rep] tag of each down task's finished layer
    uint64_t* pmax;         // [kFfnReplicas][pmax_rep] x [2][even(gu_tasks)] records: max |GLU| of a
                            // gate/up task (by layer parity)
    int32_t done_rep;       // words between tag replicas
    int32_t pmax_rep;       // records between max replicas
    uint64_t* glu;          // [inter] records: GLU values
    int32_t* acc;           // [2][hp] int32 down sums (by layer parity)
    const int32_t* cancel;  // nonzero: stop (device or host-mapped memory), or null
    int32_t* status;        // the call's status word
    uint64_t* trace;        // [grid][1 + kFfnStamps * nlayers] realtime stamps, or null
    int64_t spin_limit;     // poll rounds per wait
    int32_t nlayers, hidden, inter, hp;
    int32_t cg, cd;         // chunks per gate/up row, per down row
    int32_t dcs, dparts;    // down chunks per wave, chunk runs per 64-row group
    int32_t gu_tasks, dn_tasks;
    int32_t first_launch;   // this launch writes the status even when it is 0
    int32_t act;
    float eps;
};

}  // namespace

size_t ffn_lds_bytes(int64_t hidden, int64_t cg)
{
    const size_t h4 = (size_t)((hidden + 3) & ~3);
    return 8 * h4 + (size_t)272 * cg + (size_t)4 * kCompute * kDnRegs * 80 + (size_t)kCompute * kDnRegs * (192 + 80);
}

namespace {

__global__ __launch_bounds__(kThreads) void k_ffn(FfnArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float part[kRmsThreads];
    __shared__ float red[kCompute];
    __shared__ int tot[kCompute - 1][kWave];
    __shared__ uint32_t ired[kCompute];
    __shared__ float sxb_s;
    __shared__ int stop_s;
    __shared__ uint64_t stamps[1 + kFfnStamps * QMV_FFN_LAUNCH_LAYERS];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(t / kWave);
    const bool io = w == kCompute;
    const int b = blockIdx.x;
    const int G = gridDim.x;
    const int H = a.hidden, I = a.inter;
    uint32_t* const ctrl = a.ctrl;
    // trace stamps go to LDS and are written out once, at the end
    auto stamp = [&](int l, int k) {
        if (a.trace && t == 0) stamps[1 + kFfnStamps * l + k] = __builtin_amdgcn_s_memrealtime();
    };
    if (a.trace && t == 0) {
        stamps[0] = __builtin_amdgcn_s_memrealtime();
        for (int i = 1; i < 1 + kFfnStamps * a.nlayers; ++i) stamps[i] = 0;
    }

    const uint32_t gen = load_agent(&ctrl[kGen]) & 0xffffffu;
    auto tag = [&](int l) -> uint32_t { return (gen << 8) | (uint32_t)(l + 1); };
    // A launch that follows a failed one in the same call does nothing.
    const bool run = a.first_launch || __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;

    // io wave: record the first error of the launch (tagged with its generation)
    auto set_error = [&](uint32_t code) {
        if (lane == 0) {
            uint32_t cur = load_agent(&ctrl[kErr]);
            while ((cur >> 8) != gen || (cur & 0xffu) == 0u) {
                if (__hip_atomic_compare_exchange_strong(&ctrl[kErr], &cur, (gen << 8) | code, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                    break;
            }
        }
    };
    // io wave: poll until ready() holds on every lane (true), or stop (false).
    // ready() issues the round's loads; the error and cancel words ride along.
    uint32_t polls = 0;   // io wave: poll rounds of this layer (trace slot 11)
    auto io_wait = [&](auto ready) -> bool {
        for (int64_t i = 0;; ++i) {
            ++polls;
            uint32_t e = 0, c = 0;
            if (lane == 0) e = load_agent(&ctrl[kErr]);
            if (lane == 1 && a.cancel)
                c = __hip_atomic_load(reinterpret_cast<const uint32_t*>(a.cancel), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
            const bool ok = ready();
            e = __builtin_amdgcn_readlane(e, 0);
            c = __builtin_amdgcn_readlane(c, 1);
            if ((e >> 8) == gen && (e & 0xffu) != 0u) return false;
            if (c != 0u) {
                set_error(QMV_FFN_CANCELLED);
                return false;
            }
            if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
            if (i >= a.spin_limit) {
                set_error(QMV_FFN_TIMEOUT);
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    };
    // io wave: the max |GLU| of layer l over every gate/up task, if all are in
    // (m: the bits of the max, on every lane)
    const int gp = (a.gu_tasks + 1) & ~1;   // records per parity (even: 16-byte aligned halves)
    // polled words are read from this workgroup's XCD's replica (workgroups are
    // dealt round robin over the XCDs)
    const int rep = b % kFfnReplicas;
    const __amdgpu_buffer_rsrc_t rpmax = rsrc(a.pmax + (size_t)rep * a.pmax_rep, (int64_t)16 * gp);
    auto pmax_ready = [&](int l, uint32_t& m) -> bool {
        bool ok = true;
        uint32_t mx = 0;
        const uint32_t base = (uint32_t)(8 * gp * (l & 1));
        for (int i0 = 0; i0 < a.gu_tasks; i0 += 8 * 2 * kWave) {
            v4u32 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + 2 * lane + 2 * kWave * k;
                if (i < a.gu_tasks) v[k] = load_coherent(rpmax, base + 8 * i);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + 2 * lane + 2 * kWave * k;
                if (i < a.gu_tasks) {
                    ok = ok && v[k][1] == tag(l);
                    mx = max(mx, v[k][0]);
                    if (i + 1 < a.gu_tasks) {
                        ok = ok && v[k][3] == tag(l);
                        mx = max(mx, v[k][2]);
                    }
                }
            }
        }
        mx = wave_umax(mx);
        m = mx;
        return ok;
    };
    // Max over the compute threads (io wave: 0); every thread receives it.
    auto cmax = [&](float v) -> float {
        v = wave_fmax(v);
        if (lane == 0 && !io) red[w] = v;
        __syncthreads();
        float r = red[0];
#pragma unroll
        for (int i = 1; i < kCompute; ++i) r = fmaxf(r, red[i]);
        __syncthreads();
        return r;
    };

    // ---- LDS of the two roles ------------------------------------------------------------
    const size_t h4 = (size_t)((H + 3) & ~3);
    float* const hs = reinterpret_cast<float*>(smem);                               // [h4] the residual h
    int32_t* const accs = reinterpret_cast<int32_t*>(smem + 4 * h4);                // [h4] down sums
    uint32_t* const zg = reinterpret_cast<uint32_t*>(smem + 8 * h4);                // [48 cg] Z words
    int8_t* const x8 = reinterpret_cast<int8_t*>(smem + 8 * h4 + (size_t)192 * a.cg);   // [80 cg] codes
    uint8_t* const dsm = smem + 8 * h4 + (size_t)272 * a.cg;
    float* const vals = reinterpret_cast<float*>(dsm);                              // [4 * kDnRegs * 80]
    uint32_t* const zd = reinterpret_cast<uint32_t*>(dsm + 4 * kCompute * kDnRegs * 80) + w * kDnRegs * 48;
    int8_t* const xd = reinterpret_cast<int8_t*>(dsm + 4 * kCompute * kDnRegs * 80 + 4 * kCompute * kDnRegs * 48) +
                       w * kDnRegs * 80;

    // ---- gate/up tasks: 32 rows of both matrices; wave w takes matrix w / 4 and
    // quarter w % 4 of the chunks, lanes 32..63 the odd chunks of that quarter ----------
    const bool has_gu = b < a.gu_tasks;
    const int cgq = (a.cg + 3) >> 2;
    const int gmat = w >> 2;
    const int gpar = lane >> 5;
    const int gq0 = (w & 3) * cgq;
    const int gc0 = gq0 + gpar;                                                     // first chunk of the lane
    const int gn = io ? 0 : (max(0, min(a.cg, gq0 + cgq) - gq0) - gpar + 1) / 2;
    // ---- down tasks: 64 rows x 4 * dcs chunks; wave w takes dcs of them ----------------
    const bool has_dn = b < a.dn_tasks;
    auto task_chunks = [&](int task, int& c0, int& nch, int64_t& row) {
        const int rd = task / a.dparts, p = task - rd * a.dparts;
        c0 = p * kCompute * a.dcs + w * a.dcs;
        nch = io ? 0 : max(0, min(a.cd, c0 + a.dcs) - c0);
        row = (int64_t)64 * rd + lane;
    };

    // Registers of the next layer, loaded as soon as the current one is done with
    // them: gate/up chunks, RMSNorm weights, the three scales; down chunks.
    v4u32 gw[kGuRegs];
    v4u32 dw[kDnRegs];
    float nr[kNormRegs];
    float sg = 0.0f, su = 0.0f, sd = 0.0f, sd_prev = 0.0f;
    auto prefetch_gu = [&](int l) {
        const FfnLayerDev& ly = a.layer[l];
        const uint8_t* base = gmat ? ly.up : ly.gate;
        const int64_t row = min((int64_t)32 * b + (lane & 31), (int64_t)I - 1);
#pragma unroll
        for (int i = 0; i < kGuRegs; ++i)
            if (i < gn) gw[i] = load_chunk(base, I, gc0 + 2 * i, row);
#pragma unroll
        for (int i = 0; i < kNormRegs; ++i)
            if (t + kCT * i < H) nr[i] = ly.norm[t + kCT * i];
        sd_prev = sd;
        sg = *ly.gate_scale;
        su = *ly.up_scale;
        sd = *ly.down_scale;
    };
    auto load_dn = [&](int l, int task) {
        int c0, nch;
        int64_t row;
        task_chunks(task, c0, nch, row);
        const int64_t rr = min(row, (int64_t)H - 1);
#pragma unroll
        for (int i = 0; i < kDnRegs; ++i)
            if (i < nch) dw[i] = load_chunk(a.layer[l].down, H, c0 + i, rr);
    };

    // io wave: wait for layer l's down sums, then gather them and the layer's GLU
    // scale into LDS
    const __amdgpu_buffer_rsrc_t rdone = rsrc(a.done + (size_t)rep * a.done_rep, (int64_t)4 * a.dn_tasks);
    const __amdgpu_buffer_rsrc_t racc = rsrc(a.acc, (int64_t)8 * a.hp);
    const __amdgpu_buffer_rsrc_t rglu = rsrc(a.glu, (int64_t)8 * I);
    auto gather_sums = [&](int l) -> bool {
        uint32_t m = 0;
        const bool ok = io_wait([&]() -> bool {
            bool r = true;
            for (int i0 = 0; i0 < a.dn_tasks; i0 += 8 * 4 * kWave) {
                v4u32 v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = i0 + 4 * lane + 4 * kWave * k;
                    if (i < a.dn_tasks) v[k] = load_coherent(rdone, 4 * i);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int i = i0 + 4 * lane + 4 * kWave * k;
#pragma unroll
                    for (int q = 0; q < 4; ++q) r = r && (i + q >= a.dn_tasks || v[k][q] == tag(l));
                }
            }
            return pmax_ready(l, m) && r;
        });
        if (!ok) return false;
        const uint32_t base = (uint32_t)(4 * a.hp * (l & 1));
        for (int j0 = 0; j0 < H; j0 += 8 * 4 * kWave) {
            v4u32 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = j0 + 4 * lane + 4 * kWave * k;
                if (j < H) v[k] = load_coherent(racc, base + 4 * j);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = j0 + 4 * lane + 4 * kWave * k;
                if (j < H) *reinterpret_cast<v4u32*>(accs + j) = v[k];
            }
        }
        if (lane == 0) sxb_s = scale_from_max(__uint_as_float(m));
        return true;
    };

    if (run && !io) {
        if (has_gu) {
            for (int j = t; j < H; j += kCT) hs[j] = a.h[j];
            prefetch_gu(0);
        }
        if (has_dn) load_dn(0, b);
    }
    int l = 0;
    for (; run && l < a.nlayers; ++l) {
        const FfnLayerDev& ly = a.layer[l];
        stamp(l, 0);
        if (has_gu) {
            // ======== the residual update, RMSNorm and codes, then gate/up and GLU ==========
            float ss = 0.0f;
            if (l > 0) {
                if (io && lane == 0) stop_s = 0;
                if (io && !gather_sums(l - 1) && lane == 0) stop_s = 1;
                __syncthreads();
                if (stop_s) break;
                const float sxb = sxb_s;
                if (t < kRmsThreads)
                    for (int j = t; j < H; j += kRmsThreads) {
                        const float v = hs[j] + dequant(accs[j], sxb, sd_prev);
                        hs[j] = v;
                        ss = add_square(ss, v);
                    }
            } else if (t < kRmsThreads) {
                for (int j = t; j < H; j += kRmsThreads) ss = add_square(ss, hs[j]);
            }
            stamp(l, 1);
            if (t < kRmsThreads) part[t] = ss;
            const float r = rms_tree(part, H, a.eps);
            stamp(l, 2);
            float o[kNormRegs];
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < kNormRegs; ++i) {
                const int j = t + kCT * i;
                o[i] = (!io && j < H) ? rms_value(nr[i], r, hs[j]) : 0.0f;
                m = fmaxf(m, fabsf(o[i]));
            }
            if (!io)
                for (int j = t + kCT * kNormRegs; j < H; j += kCT) m = fmaxf(m, fabsf(rms_value(ly.norm[j], r, hs[j])));
            m = cmax(m);
            const float sxa = scale_from_max(m);
            if (!io) {
#pragma unroll
                for (int i = 0; i < kNormRegs; ++i) {
                    const int j = t + kCT * i;
                    if (j < H) x8[j] = quantize_one(o[i], sxa);
                }
                for (int j = t + kCT * kNormRegs; j < H; j += kCT)
                    x8[j] = quantize_one(rms_value(ly.norm[j], r, hs[j]), sxa);
                for (int j = H + t; j < 80 * a.cg; j += kCT) x8[j] = 0;
            }
            __syncthreads();
            stamp(l, 3);
            uint32_t cpart = 0;
            if (!io)
                for (int g = t; g < 4 * a.cg; g += kCT) cpart += z_of_group(x8, g, zg);
            cpart = wave_sum(cpart);
            if (lane == 0 && !io) ired[w] = cpart;
            __syncthreads();
            uint32_t corr = 0;
#pragma unroll
            for (int i = 0; i < kCompute; ++i) corr += ired[i];
            stamp(l, 4);
            for (int task = b, first = 1; task < a.gu_tasks; task += G, first = 0) {
                const int64_t row = (int64_t)32 * task + (lane & 31);
                int lo = 0, hi = 0;
                for (int i0 = 0; i0 < gn; i0 += kGuRegs) {
                    if (!(first && i0 == 0)) {
                        const uint8_t* base = gmat ? ly.up : ly.gate;
                        const int64_t rr = min(row, (int64_t)I - 1);
#pragma unroll
                        for (int i = 0; i < kGuRegs; ++i)
                            if (i0 + i < gn) gw[i] = load_chunk(base, I, gc0 + 2 * (i0 + i), rr);
                    }
#pragma unroll
                    for (int i = 0; i < kGuRegs; ++i)
                        if (i0 + i < gn) dot_chunk(gw[i], zg + 48 * (gc0 + 2 * (i0 + i)), lo, hi);
                }
                int total = (int)((uint32_t)lo + (uint32_t)hi);
                total = (int)((uint32_t)total + (uint32_t)__shfl_xor(total, 32, kWave));   // odd chunks
                if (w > 0 && !io && lane < 32) tot[w - 1][lane] = total;
                __syncthreads();
                if (w == 0) {
                    float mv = 0.0f;
                    if (lane < 32) {
                        uint32_t g = (uint32_t)total - corr, u = 0u - corr;
#pragma unroll
                        for (int i = 0; i < kCompute / 2 - 1; ++i) g += (uint32_t)tot[i][lane];
#pragma unroll
                        for (int i = kCompute / 2 - 1; i < kCompute - 1; ++i) u += (uint32_t)tot[i][lane];
                        const int tg = (int)g, tu = (int)u;
                        const float v = glu_value(dequant(tg, sxa, sg), dequant(tu, sxa, su), a.act);
                        if (row < I) {
                            store_record(a.glu + row, __float_as_uint(v), tag(l));
                            mv = fabsf(v);
                        }
                    }
                    mv = wave_fmax(mv);
                    if (lane < kFfnReplicas)
                        store_record(a.pmax + (size_t)lane * a.pmax_rep + (size_t)gp * (l & 1) + task, __float_as_uint(mv),
                                     tag(l));
                }
                __syncthreads();
            }
            stamp(l, 5);
            if (l + 1 < a.nlayers && !io) prefetch_gu(l + 1);
        }
        if (has_dn) {
            // ======== down: int32 partial sums into acc[l & 1] ================================
            int32_t* const accl = a.acc + (size_t)a.hp * (l & 1);
            bool stop = false;
            for (int task = b, first = 1; task < a.dn_tasks; task += G, first = 0) {
                const int rd = task / a.dparts, p = task - rd * a.dparts;
                const int cb = p * kCompute * a.dcs;
                const int col0 = 80 * cb;
                const int col1 = min(I, 80 * min(a.cd, cb + kCompute * a.dcs));
                // io wave: this task's GLU values and the layer's scale
                if (io) {
                    uint32_t m = 0;
                    const bool ok = io_wait([&]() -> bool {
                        // every column of the task in one batch of loads (at most 4 * kDnRegs * 80)
                        constexpr int kB = (kCompute * kDnRegs * 80 + 2 * kWave - 1) / (2 * kWave);
                        v4u32 v[kB];
#pragma unroll
                        for (int k = 0; k < kB; ++k) {
                            const int c = col0 + 2 * lane + 2 * kWave * k;
                            if (c < col1) v[k] = load_coherent(rglu, 8 * c);
                        }
                        bool r = true;
#pragma unroll
                        for (int k = 0; k < kB; ++k) {
                            const int c = col0 + 2 * lane + 2 * kWave * k;
                            if (c < col1) {
                                r = r && v[k][1] == tag(l) && (c + 1 >= col1 || v[k][3] == tag(l));
                                vals[c - col0] = __uint_as_float(v[k][0]);
                                if (c + 1 < col1) vals[c - col0 + 1] = __uint_as_float(v[k][2]);
                            }
                        }
                        return pmax_ready(l, m) && r;
                    });
                    if (lane == 0) {
                        stop_s = ok ? 0 : 1;
                        sxb_s = scale_from_max(__uint_as_float(m));
                    }
                }
                __syncthreads();
                if (stop_s) {
                    stop = true;
                    break;
                }
                stamp(l, 6);
                const float sxb = sxb_s;
                int c0, nch;
                int64_t row;
                task_chunks(task, c0, nch, row);
                if (!first) load_dn(l, task);
#pragma unroll
                for (int i = 0; i < (kDnRegs * 80 + kWave - 1) / kWave; ++i) {
                    const int jj = lane + kWave * i;
                    const int col = 80 * c0 + jj;
                    if (jj < 80 * nch) xd[jj] = col < I ? quantize_one(vals[col - col0], sxb) : (int8_t)0;
                }
                __syncthreads();
                uint32_t cp = 0;
                if (lane < 4 * nch) cp = z_of_group(xd, lane, zd);
                cp = wave_sum(cp);
                __syncthreads();
                stamp(l, 7);
                int lo = 0, hi = 0;
#pragma unroll
                for (int i = 0; i < kDnRegs; ++i)
                    if (i < nch) dot_chunk(dw[i], zd + 48 * i, lo, hi);
                const int total = (int)((uint32_t)lo + (uint32_t)hi - cp);
                if (w > 0 && !io) tot[w - 1][lane] = total;
                __syncthreads();
                stamp(l, 8);
                if (w == 0 && row < H) {
                    uint32_t sum = (uint32_t)total;
#pragma unroll
                    for (int i = 0; i < kCompute - 1; ++i) sum += (uint32_t)tot[i][lane];
                    __hip_atomic_fetch_add(&accl[row], (int)sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    // The first task of a row group clears the group's rows of the
                    // accumulator of layer l - 1: every gate/up task read them before
                    // it wrote its max record of this layer, all of which this task
                    // has seen; they are next added to in layer l + 1, which no task
                    // reaches before seeing this task's tag.
                    if (p == 0 && l > 0)
                        store_agent(reinterpret_cast<uint32_t*>(a.acc + (size_t)a.hp * ((l - 1) & 1)) + row, 0u);
                }
                __builtin_amdgcn_s_waitcnt(0);   // the adds (and clears) are done
                stamp(l, 9);
                __syncthreads();
                if (io && lane < kFfnReplicas) store_agent(&a.done[(size_t)lane * a.done_rep + task], tag(l));
            }
            if (stop) break;
            if (l + 1 < a.nlayers && !io) load_dn(l + 1, b);
        }
        stamp(l, 10);
        if (a.trace && io && lane == 0) stamps[1 + kFfnStamps * l + 11] = polls;
        polls = 0;
    }
    // ---- the last residual update, written out by workgroup 0 ----------------------------
    if (run && l == a.nlayers && b == 0) {
        if (io && lane == 0) stop_s = 0;
        if (io && !gather_sums(a.nlayers - 1) && lane == 0) stop_s = 1;
        __syncthreads();
        if (!stop_s && !io) {
            const float sxb = sxb_s;
            for (int j = t; j < H; j += kCT) a.h[j] = hs[j] + dequant(accs[j], sxb, sd);
        }
    }
    if (a.trace && t == 0) {
        uint64_t* tr = a.trace + (size_t)b * (1 + kFfnStamps * a.nlayers);
        for (int i = 0; i < 1 + kFfnStamps * a.nlayers; ++i) tr[i] = stamps[i];
    }

    // ---- exit: the last workgroup out writes the status and readies the workspace ---------
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) {
        const int x = b % kXcds;
        const uint32_t nx = (uint32_t)((G - x + kXcds - 1) / kXcds);
        const uint32_t nxcd = (uint32_t)min(G, kXcds);
        int last = 0;
        if (__hip_atomic_fetch_add(&ctrl[kExitX + 64 * x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nx - 1)
            last = __hip_atomic_fetch_add(&ctrl[kExitAll], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   nxcd - 1;
        stop_s = last;
    }
    __syncthreads();
    if (stop_s) {
        for (int j = t; j < 2 * a.hp; j += kThreads) store_agent(reinterpret_cast<uint32_t*>(a.acc) + j, 0u);
        if (t == 0) {
            const uint32_t e = load_agent(&ctrl[kErr]);
            const uint32_t code = (e >> 8) == gen ? (e & 0xffu) : 0u;
            if (a.first_launch || code != 0u)
                __hip_atomic_store(a.status, (int32_t)code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int x = 0; x < kXcds; ++x) store_agent(&ctrl[kExitX + 64 * x], 0u);
            store_agent(&ctrl[kExitAll], 0u);
            store_agent(&ctrl[kGen], (gen + 1) & 0xffffffu);
        }
    }
}

}  // namespace

int ffn_max_wg_per_cu(size_t lds)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k_ffn), kThreads, lds) !=
        hipSuccess)
        return 0;
    return n;
}

hipError_t setup_ffn_attributes()
{
    return raise_lds_limit(reinterpret_cast<const void*>(k_ffn));
}

hipError_t launch_ffn(const FfnLaunch& f, hipStream_t s)
{
    FfnArgs a = {};
    for (int l = 0; l < f.nlayers; ++l) {
        const qmv_ffn_layer& y = f.layers[l];
        a.layer[l].gate = static_cast<const uint8_t*>(y.gate.data);
        a.layer[l].up = static_cast<const uint8_t*>(y.up.data);
        a.layer[l].down = static_cast<const uint8_t*>(y.down.data);
        a.layer[l].gate_scale = y.gate.scale;
        a.layer[l].up_scale = y.up.scale;
        a.layer[l].down_scale = y.down.scale;
        a.layer[l].norm = y.norm;
    }
    const FfnLayout& o = f.layout;
    uint8_t* ws = static_cast<uint8_t*>(f.workspace);
    a.h = f.h;
    a.ctrl = reinterpret_cast<uint32_t*>(ws);
    a.done = reinterpret_cast<uint32_t*>(ws + o.done);
    a.pmax = reinterpret_cast<uint64_t*>(ws + o.pmax);
    a.done_rep = (int32_t)(o.done_rep / 4);
    a.pmax_rep = (int32_t)(o.pmax_rep / 8);
    a.glu = reinterpret_cast<uint64_t*>(ws + o.glu);
    a.acc = reinterpret_cast<int32_t*>(ws + o.acc);
    a.cancel = f.cancel;
    a.status = f.status;
    a.trace = f.trace;
    a.spin_limit = f.spin_limit > 0 ? f.spin_limit : kDefaultSpin;
    a.nlayers = f.nlayers;
    a.hidden = (int32_t)f.hidden;
    a.inter = (int32_t)f.inter;
    a.hp = (int32_t)o.hp;
    a.cg = (int32_t)f.cg;
    a.cd = (int32_t)f.cd;
    a.dcs = f.dcs;
    a.dparts = f.dparts;
    a.gu_tasks = f.gu_tasks;
    a.dn_tasks = f.dn_tasks;
    a.first_launch = f.first_launch;
    a.act = f.act;
    a.eps = f.eps;
    hipLaunchKernelGGL(k_ffn, dim3(f.grid), dim3(kThreads), f.lds, s, a);
    return hipGetLastError();
}

}  // namespace qmv
