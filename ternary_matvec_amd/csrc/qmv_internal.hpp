// qmv_internal.hpp -- device-side descriptors and helpers shared by the HIP
// kernels of libqmv (gfx950 only).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <qmv.h>

namespace qmv {

constexpr int kWave = 64;         // CDNA wavefront width
constexpr int kBlock = 256;       // threads per workgroup for the streaming kernels
constexpr int kRowsPerTile = 64;  // one output row per lane of a wave
constexpr int kTileProbBits = 14; // tile entry = problem << 18 | row block
constexpr int kTileRowBits = 18;

// One problem as the kernels see it (uploaded into the caller's workspace).
struct DevProblem {
    const uint8_t* w;    // packed weights in the chunk-interleaved layout
    const float* sw;     // 1 fp32 weight scale ([n][ceil(k/128)] for group-scaled int8)
    const int8_t* x8;    // [m][k] int8 activations, natural column order
    const float* sx;     // [m] fp32 activation scales ([m][ceil(k/32)] for group-scaled int8)
    float* y;            // [m][n] fp32 outputs
    int32_t* acc;        // [m][n] int32 exact dots, or null
    int32_t n;           // output rows
    int32_t k;           // input columns
    int32_t m;           // tokens
    int32_t chunks;      // 16-byte chunks per row (row stride / 16)
    int32_t tile_begin;  // first tile of this problem in the launch
    int32_t wtype;       // 1 = five trits per byte, 2 = int8, 3 = int8 with group scales
    int32_t lanes_per_row;  // lanes sharing one row (streaming kernel: 1 .. 8; group-scaled: 4 .. 64)
    int32_t reserved;
};
static_assert(sizeof(DevProblem) == 80, "DevProblem layout");

// Pointers read from a descriptor in memory are generic (FLAT) to the
// compiler; FLAT loads also count against the LDS wait counter, which
// serialises weight streaming with LDS traffic.  These casts make them global.
#define QMV_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const QMV_GLOBAL T* gload_ptr(const T* p)
{
    return (const QMV_GLOBAL T*)p;
}
// Read-only for the whole kernel and wave-uniform: the constant address space
// makes such reads scalar loads (they then never wait behind vector loads).
#define QMV_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const QMV_CONST T* cload_ptr(const T* p)
{
    return (const QMV_CONST T*)p;
}
template <typename T>
__device__ __forceinline__ QMV_GLOBAL T* gstore_ptr(T* p)
{
    return (QMV_GLOBAL T*)p;
}

// Wait until at most N vector memory operations of this wave are outstanding
// (they complete in order); the other counters are left alone.  gfx9
// encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt in 6:4,
// lgkmcnt in 11:8.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-offs that leaves the wave's global memory
// operations in flight (loads into registers or LDS, atomics): it waits only
// for the wave's own LDS (and scalar) accesses, so what was written to LDS
// before it is visible to every wave after it.  Anything else a hand-off
// depends on is waited for explicitly before it.  The memory clobber keeps the
// compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Once-per-device set-up of the kernel translation units: each raises its
// kernels' dynamic-LDS limit to the whole kMaxLds, so launches never set
// attributes.
hipError_t setup_workgroup_gemv_attributes();
hipError_t setup_stream_attributes();
hipError_t setup_grouped_attributes();
hipError_t setup_prefill_attributes();
hipError_t setup_sketch_attributes();
// Launchers implemented in the kernel translation units.
hipError_t launch_rmsnorm_quantize(const float* x, const float* weight, int64_t m, int64_t k, float eps, int8_t* x8,
                                   float* sx, hipStream_t s);
hipError_t launch_glu_quantize(const float* gate, const float* up, int64_t m, int64_t n, int act, int8_t* x8,
                               float* sx, hipStream_t s);
hipError_t launch_fill_pack_header(float* scale_out, float scale, int32_t* bad, hipStream_t s);
hipError_t launch_pack_ternary(const int8_t* trits, int64_t n, int64_t k, int64_t chunks, uint8_t* out,
                               int32_t* bad, hipStream_t s);
hipError_t launch_pack_int8(const float* w, int64_t n, int64_t k, int64_t chunks, int8_t* out,
                            float* scale_out, hipStream_t s);
hipError_t launch_quantize_rows(const float* x, int64_t m, int64_t k, int8_t* x8, float* sx, hipStream_t s);
// Activation sets of one multi-set quantisation launch (a kernel argument).
constexpr int kMaxActSets = 8;
struct ActSet {
    const float* x;
    int8_t* x8;
    float* sx;
    int64_t k;
};
struct ActSets {
    ActSet set[kMaxActSets];
    int64_t first[kMaxActSets + 1];   // first workgroup (row) of each set; first[count] = rows
    int32_t count;
};
hipError_t launch_quantize_many(const ActSets& sets, int64_t rows, hipStream_t s);
int64_t gemv_lds_bytes(int wtype, int max_m, int max_chunks);
// Rows per tile of the workgroup GEMV (64, or 128 from 4 tokens: two rows per lane).
int gemv_rows_per_tile(int wtype, int max_m);
constexpr int64_t kMaxLds = 160 * 1024;  // LDS of one gfx950 compute unit

// Raise a kernel's dynamic-LDS limit to what its static LDS leaves of kMaxLds.
inline hipError_t raise_lds_limit(const void* kernel)
{
    hipFuncAttributes a;
    hipError_t e = hipFuncGetAttributes(&a, kernel);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)(kMaxLds - (int64_t)a.sharedSizeBytes));
}
hipError_t launch_gemv(const DevProblem* probs, const uint32_t* tiles, int32_t tile_begin, int32_t tile_count,
                       int wtype, int max_m, int max_chunks, hipStream_t s);
// Streaming (persistent) GEMV for 1..2 tokens.  Workgroups are 4 compute
// waves + 1 staging wave; a workgroup tile is 4 * 64 / lanes_per_row *
// kStreamRowsPerLane rows of one problem, entry = problem slot << kTileRowBits | row block.  Schedule
// words (in the workspace, writable): [kStreamHdr words of counters, zero
// between launches][the first two tile entries of each workgroup][kStreamXcds x
// (offset, size)][the XCD tile lists].  LDS =
// two staged tiles of slot_bytes + a few words.
constexpr int kStreamXcds = 8;
#ifndef QMV_STREAM_RPL
#define QMV_STREAM_RPL 2
#endif
constexpr int kStreamRowsPerLane = QMV_STREAM_RPL;   // a workgroup tile is 4 * 64 / lanes_per_row * this rows
constexpr int kStreamHdr = 64 * 2 * kStreamXcds;
// At most 8 lanes per row: the smallest workgroup tile, 4 * 64 / 8 * 2 rows,
// is no smaller than a 64-row tile, so entries and table bounds stay as sized.
constexpr int kStreamMaxLanes = 8;
static_assert(4 * 64 / kStreamMaxLanes * kStreamRowsPerLane >= kRowsPerTile, "stream tile rows");
int64_t gemv_stream_steps(int chunks, int lanes);
int64_t gemv_stream_slot_bytes(int wtype, int mt, int chunks, int lanes);
size_t gemv_stream_lds_bytes(int mt, int64_t slot_bytes);
// Workgroups of the streaming kernel resident per compute unit (registers and
// LDS), 0 if it cannot run or no device is usable.
int gemv_stream_wg_per_cu(int wtype, int max_m, int64_t slot_bytes, bool skip);
// skip (ternary only): the variant that skips 20-column units whose
// activations are zero for every token.
hipError_t launch_gemv_stream(const DevProblem* probs, uint32_t* sched, int nb, int wtype, int max_m,
                              int32_t slot_bytes, bool skip, hipStream_t s);
// Persistent ternary GEMV on int8 matrix cores for 1..16 tokens: the same
// schedule words as the streaming kernel; a workgroup tile is
// gemv_mx_tile_rows rows (compute waves x row groups x 16).  Tokens per launch
// are 1, 2, 4, 8 or 16 (gemv_mx_tokens); LDS = two slots of slot_bytes and a
// few words.
int gemv_mx_tokens(int max_m);                  // 0: more than 16 tokens
int gemv_mx_ring(int mt);                       // steps of the kernel's weight ring (tiles pad to it)
int gemv_mx_row_groups(int mt);                 // row groups of 16 per wave
int64_t gemv_mx_tile_rows(int mt);              // rows of a workgroup tile
int64_t gemv_mx_slot_bytes(int mt, int chunks);
size_t gemv_mx_lds_bytes(int mt, int64_t slot_bytes);
int gemv_mx_wg_per_cu(int mt, int64_t slot_bytes);
hipError_t setup_mx_attributes();
hipError_t launch_gemv_mx(const DevProblem* probs, uint32_t* sched, int nb, int mt, int32_t slot_bytes,
                          hipStream_t s);
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin over them
// Prefill (int8 matrix cores): tiles of 128 tokens x 256 rows.
constexpr int64_t kPrefillTileM = 128;
constexpr int64_t kPrefillTileN = 256;
constexpr int64_t kPrefillZeroBytes = 256;   // block of zeros at the end of the prefill workspace
constexpr int64_t kPrefillMaxGrid = 1024;     // persistent workgroups per launch, at most
constexpr int64_t kPrefillTicketWords = 8;    // 64-bit words after the entries: 8 list tickets + 1 count (uint32)
int64_t prefill_tiles(int64_t m, int64_t n);
// table: 9 offsets (list x = entries [table[x], table[x + 1])), the entries
// (slot << 48 | token tile << 32 | row tile), then the zeroed tickets.
hipError_t launch_prefill(const DevProblem* probs, const uint64_t* table, int64_t grid, const int8_t* zeros,
                          hipStream_t s);
// Sketch head of the output layer: build tables, per-token argmax.
constexpr int64_t kSketchMaxK = 8192;
int64_t sketch_bytes(int64_t v, int64_t k);
int64_t sketch_workspace_bytes(int64_t v);
hipError_t launch_sketch_build(const uint16_t* w, int64_t v, int64_t k, void* sketch, hipStream_t s);
hipError_t launch_sketch_argmax(const uint16_t* w, const void* sketch, const float* x, int64_t v, int64_t k,
                                int32_t* idx, float* max_logit, int32_t* ncand, float* scores, void* workspace,
                                hipStream_t s);
hipError_t launch_read_probe(const void* data, int64_t bytes, uint32_t* out, int cus, hipStream_t s);
hipError_t launch_mfma_probe(int kind, int iters, uint32_t* out, int cus, int64_t* ops, hipStream_t s);
hipError_t launch_lmhead(const uint16_t* w, const float* x, int64_t v, int64_t k, int32_t* idx,
                         float* max_logit, float* logits, void* workspace, hipStream_t s);
int64_t lmhead_partials(int64_t v);
// Group-scaled int8 (weights per 128 columns, activations per 32).
hipError_t launch_quantize_groups(const float* x, int64_t rows, int64_t k, int group, int64_t q_stride, int8_t* q,
                                  float* s, hipStream_t st);
int grouped_lanes_per_row(int64_t k);          // lanes sharing one row: 4 .. 64
size_t grouped_lds_bytes(int64_t m, int64_t k);
hipError_t launch_gemv_grouped(const DevProblem* probs, const uint32_t* tiles, int32_t count, int max_m, size_t lds,
                               hipStream_t s);

// Feed-forward half of a layer stack, one token, one persistent launch
// (k_ffn.hip).  Workspace: control words, then kFfnReplicas copies of the down
// tasks' tags and of the per-task GLU maxima (two layer parities), the GLU
// value records and two int32 accumulators; byte offsets in FfnLayout.
constexpr int64_t kFfnCtrlBytes = 4096;
constexpr int kFfnWgPerCu = 1;          // workgroups per compute unit, if occupancy allows
constexpr int kFfnComputeWaves = 8;     // compute waves of a workgroup (plus one io wave)
constexpr int kFfnDownChunks = 2;       // down chunks per wave, at most
constexpr int kFfnReplicas = 8;         // copies of the polled tags and maxima (one per XCD)
struct FfnLayout {
    int64_t hp;                         // accumulator words per parity (hidden rounded up to 64)
    int64_t done, pmax, glu, acc, bytes;
    int64_t done_rep, pmax_rep;         // bytes between the replicas of the tags, of the maxima
};
struct FfnLaunch {
    const qmv_ffn_layer* layers;        // host, nlayers entries (this launch's)
    int32_t nlayers;
    float* h;
    int64_t hidden, inter;
    int64_t cg, cd;                     // 16-byte chunks per gate/up row, per down row
    int32_t dcs, dparts;                // down chunks per wave, chunk runs per 64-row group
    int32_t gu_tasks, dn_tasks;
    int32_t act;
    float eps;
    void* workspace;
    FfnLayout layout;
    const int32_t* cancel;
    int32_t* status;
    uint64_t* trace;
    int64_t spin_limit;
    int32_t first_launch;
    int32_t grid;
    size_t lds;
};
size_t ffn_lds_bytes(int64_t hidden, int64_t cg);
int ffn_max_wg_per_cu(size_t lds);
hipError_t setup_ffn_attributes();
hipError_t launch_ffn(const FfnLaunch& f, hipStream_t s);

}  // namespace qmv
