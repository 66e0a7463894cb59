// k_sketch.hip -- the sketch head: the output layer's greedy choice from
// candidates ("Gemma 3 1B at 114 tokens per second on a laptop CPU", "Step 3:
// the output layer became the bottleneck", the sketch head's three steps).
//
// Per token, two launches:
//  1. k_sketch_score, a workgroup per 1024 rows (two per lane).  Each
//     workgroup reads x, asks for its rows' sign words (they do not depend on
//     the token's plan; issued in batches between the plan's steps) and makes
//     the plan itself in LDS while they are in flight: the T = min(32, k) dimensions with the largest |x| (ties to the
//     lower index) are scored exactly, the other k - T form 4 consecutive rank
//     groups, each weighted by c * mean |x| of the group (c = mean |w| of the
//     table, computed when the sketch is built).  Ranks are never sorted out:
//     the order key at each of the 4 group boundaries is selected by a shared
//     histogram of the top 11 bits of |x|, then (for a bin of more than 64
//     dimensions) further 10-bit digits, and the at most 64 dimensions left in
//     the boundary's bin are ranked against each other (by |x|, then index);
//     a dimension's class is then four compares.  The approximate score of a
//     row is the exact products over the T dimensions (from the
//     dimension-major copy of the table) plus, per group, weight * (n_g - 2 *
//     popcount((signs of w ^ signs of x) & mask_g)) from the 1-bit table.
//     Each row's fp32 score order key goes to the workspace and into a
//     histogram of its top 13 bits; the 256 bins below the workgroup's highest
//     non-empty one are added into one of 8 device copies.
//  2. k_sketch_pick, a workgroup per 1024 rows (one per lane).  Every
//     workgroup finds the cut b*, the highest bin at which the bins from the
//     top down hold min(1024, v) words, among the 256 bins below the highest
//     non-empty one (every workgroup of launch 1 added all of those); if they
//     hold fewer, every word is a candidate.  It scores its own candidates
//     exactly (a wave per word, fp32 like k_lmhead) and leaves its best (logit
//     key, lowest row) and count in its slot; the last workgroup out (counted
//     in 8 groups, then over the groups) takes the first maximum over the
//     slots and writes the choice.
// Every workgroup makes the same plan from the same x in the same order, so
// the scores of one token are consistent over workgroups and calls.
//
// The workspace carries the state between launches and tokens: zero-filled
// before its first use, each token leaves it ready for the next (the score
// launch clears the pick's counters, the pick launch clears the histogram set
// the next token will use; the two sets alternate on a parity word).  Values
// shared between workgroups of one launch go through device-scope atomics:
// the compute dies' L2 caches are not coherent with each other for plain
// accesses.  Atomics on one address are few (at most a group's workgroups),
// since the memory side serialises them.
#include "qmv_internal.hpp"

namespace qmv {
namespace {

constexpr int kSkTop = 32;            // exactly scored dimensions
constexpr int kSkGroups = 4;          // sign-bit groups
constexpr int kSkMinCand = 1024;      // candidates: at least this many words (or all of them)
constexpr int kSkBinBits = 13;        // histogram over the top 13 bits of the score's order key
constexpr int kSkBins = 1 << kSkBinBits;
constexpr int kSkWindow = 256;        // bins searched below the highest non-empty one
constexpr int kSkCopies = 8;          // device histograms: score workgroup b adds into copy b % 8
constexpr int kSkSets = 8;            // max-bin words and exit counters: workgroup b in set b % 8
constexpr int kSkRowBlock = 512;      // build: rows per fp64 partial of the table scale
constexpr int kSkRows = 1024;         // rows per workgroup in both per-token launches (the table pitch)
constexpr int kSkScoreThreads = 512;  // score: two rows per lane
constexpr int kSkScoreWaves = kSkScoreThreads / kWave;
constexpr int kSkPickThreads = 1024;  // pick: one row per lane
constexpr int kSkWords = kSketchMaxK / 32;
constexpr int kSkList = 64;           // dimensions of a boundary's bin ranked against each other
constexpr int kSkPre = 36;            // sign words per lane asked for before the plan (all of them for k <= 1152)
constexpr int kSkBatch = 12;          // sign words per batch after those
constexpr int kSkXLoads = kSketchMaxK / (4 * kSkScoreThreads);   // 16-byte loads of x per lane
constexpr uint32_t kSkMagic = 0x32484b53u;   // "SKH2"

typedef uint32_t sk_u32x2 __attribute__((ext_vector_type(2)));

// Sketch buffer: header, sign words [kw][vp], dimension-major bf16 copy [k][vp],
// vp = v rounded up to a multiple of kSkRows (rows v..vp-1 hold zeros).
struct SketchHeader {
    uint32_t magic;
    int32_t k;
    int64_t v;
    float c;        // mean |w| of the table
    int32_t pad[11];
};
static_assert(sizeof(SketchHeader) == 64, "sketch header");

// Workspace: control words, two histogram sets, a slot per pick workgroup, the
// row keys [vp].  Each control word has a 64-byte line of its own.
constexpr int kCtlParity = 0;                    // histogram set of the next token
constexpr int kCtlMaxBin = 16;                   // [kSkSets]: highest non-empty bin (score; reset by pick)
constexpr int kCtlOut = 16 * (1 + kSkSets);      // [kSkSets]: pick workgroups out; then [kSkSets]: sets out
constexpr int kCtlOutAll = kCtlOut + 16 * kSkSets;
constexpr int64_t kSkCtlBytes = 2048;
static_assert(4 * (kCtlOutAll + 16) <= kSkCtlBytes, "sketch control words");
constexpr int64_t kSkHistOff = kSkCtlBytes;
constexpr int64_t kSkHistSet = (int64_t)kSkCopies * kSkBins;   // words per set
constexpr int64_t kSkSlotOff = kSkHistOff + 2 * 4 * kSkHistSet;   // 16 bytes per pick workgroup

constexpr int64_t sk_round(int64_t n, int64_t a) { return (n + a - 1) / a * a; }
constexpr int64_t sk_pitch(int64_t v) { return sk_round(v, kSkRows); }
constexpr int64_t sk_keys_off(int64_t vp) { return kSkSlotOff + sk_round(16 * (vp / kSkRows), 256); }

__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// ---- build --------------------------------------------------------------------------------

// A thread per row of the padded table: the sign words (word w of row r at
// w * vp + r) and the row's sum of |w| in fp32, column order (into `rowsum`);
// padding rows get zero words.
__global__ __launch_bounds__(kBlock) void k_sketch_rows(const uint16_t* __restrict__ w, int64_t v, int64_t vp, int k,
                                                        uint32_t* __restrict__ signs, float* __restrict__ rowsum)
{
    const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (r >= vp) return;
    if (r >= v) {
        for (int wd = 0; wd < (k + 31) / 32; ++wd) signs[(int64_t)wd * vp + r] = 0u;
        return;
    }
    const uint4* row = reinterpret_cast<const uint4*>(w + r * k);
    float sum = 0.0f;
    uint32_t word = 0;
    for (int c8 = 0; c8 < k / 8; ++c8) {
        const uint4 q = row[c8];
        const uint32_t h[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float f = half ? __uint_as_float(h[j] & 0xFFFF0000u) : __uint_as_float(h[j] << 16);
                const int col = 8 * c8 + 2 * j + half;
                sum += fabsf(f);
                if (f < 0.0f) word |= 1u << (col & 31);
            }
        }
        if ((c8 & 3) == 3 || c8 == k / 8 - 1) {
            signs[(int64_t)(c8 >> 2) * vp + r] = word;
            word = 0;
        }
    }
    rowsum[r] = sum;
}

// One workgroup: c = mean |w|.  Blocks of 512 rows are summed in fp64 in row
// order (thread t takes blocks t, t + 256, ...), then thread 0 adds the block
// sums in order.
__global__ __launch_bounds__(kBlock) void k_sketch_scale(const float* __restrict__ rowsum, int64_t v, int k,
                                                         double* __restrict__ part, SketchHeader* __restrict__ hdr)
{
    const int64_t nb = (v + kSkRowBlock - 1) / kSkRowBlock;
    for (int64_t b = threadIdx.x; b < nb; b += kBlock) {
        double s = 0.0;
        const int64_t end = min(v, (b + 1) * kSkRowBlock);
        for (int64_t r = b * kSkRowBlock; r < end; ++r) s += (double)rowsum[r];
        part[b] = s;
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        double total = 0.0;
        for (int64_t b = 0; b < nb; ++b) total += part[b];
        hdr->magic = kSkMagic;
        hdr->k = k;
        hdr->v = v;
        hdr->c = (float)(total / ((double)v * (double)k));
    }
}

// 64 x 64 tiles through LDS: wt[c][r] = w[r][c], zero for the padding rows.
__global__ __launch_bounds__(kBlock) void k_sketch_transpose(const uint16_t* __restrict__ w, int64_t v, int64_t vp,
                                                             int k, uint16_t* __restrict__ wt)
{
    __shared__ uint16_t tile[64][66];
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int c0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int rr = ty + 4 * i;
        const int64_t r = r0 + rr;
        const int c = c0 + tx;
        tile[rr][tx] = (r < v && c < k) ? w[r * k + c] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int cc = ty + 4 * i;
        const int c = c0 + cc;
        const int64_t r = r0 + tx;
        if (c < k && r < vp) wt[(int64_t)c * vp + r] = tile[tx][cc];
    }
}

// ---- per token: plan and approximate scores ------------------------------------------------

struct ScoreLds {
    uint32_t xb[kSketchMaxK];                    // x's bit patterns
    alignas(16) uint32_t rh0[2048];              // top 11 bits of |x|, shared by the boundaries
    alignas(16) uint32_t rh[2][kSkGroups][1024]; // the next 10-bit digits, then the last (per boundary)
    uint64_t lst[kSkGroups][kSkList];            // order keys of the dimensions in a boundary's bin
    alignas(16) uint32_t word[6][kSkWords + kSkBatch];   // masks: [0] exact, [1..4] groups, [5] signs of x
    float gpart[kSkScoreWaves][kSkGroups];       // the groups' sums of |x| per wave
    uint64_t kb[kSkGroups];                      // order key at each boundary rank (0: none)
    uint32_t lcnt[kSkGroups];
    int32_t top_idx[kSkScoreWaves][kSkTop];      // each wave's copy of the exact dimensions (index order)
    float top_x[kSkScoreWaves][kSkTop];
    uint32_t wmax[kSkScoreWaves];
    alignas(16) uint32_t hist[kSkBins];
};

// Lane l + the lanes up to l - 1, 2, 4, 8 back within its row of 16 (DPP row shifts; a lane
// past the row's start adds 0): an inclusive prefix within each row.
__device__ __forceinline__ uint32_t row_scan_u32(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
    return v;
}

__device__ __forceinline__ float row_scan_f(float a)
{
    a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x111, 0xf, 0xf, false));
    a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x112, 0xf, 0xf, false));
    a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x114, 0xf, 0xf, false));
    a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x118, 0xf, 0xf, false));
    return a;
}

// Sum over the wave in a fixed order (each row's prefix tree, then the four rows in order),
// the same in every lane.
__device__ __forceinline__ float wave_sum_f(float a)
{
    a = row_scan_f(a);
    return ((__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 15)) +
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 31))) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 47))) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 63));
}

// Maximum over the wave (every lane gets it): DPP row shifts (a lane past the row's
// start takes 0), then the four rows' last lanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 15), (uint32_t)__builtin_amdgcn_readlane((int)v, 31)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 47), (uint32_t)__builtin_amdgcn_readlane((int)v, 63)));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int step = 0; step < 4; ++step) {
        uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32), slo, shi;
        switch (step) {   // row_shr:1, 2, 4, 8
        case 0:
            slo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, 0x111, 0xf, 0xf, false);
            shi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, 0x111, 0xf, 0xf, false);
            break;
        case 1:
            slo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, 0x112, 0xf, 0xf, false);
            shi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, 0x112, 0xf, 0xf, false);
            break;
        case 2:
            slo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, 0x114, 0xf, 0xf, false);
            shi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, 0x114, 0xf, 0xf, false);
            break;
        default:
            slo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, 0x118, 0xf, 0xf, false);
            shi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, 0x118, 0xf, 0xf, false);
            break;
        }
        const uint64_t o = ((uint64_t)shi << 32) | slo;
        v = o > v ? o : v;
    }
    uint64_t m = 0ull;
#pragma unroll
    for (int r = 15; r < kWave; r += 16) {
        const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, r);
        m = o > m ? o : m;
    }
    return m;
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v, int lane)
{
    v = row_scan_u32(v);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const int row = lane >> 4;
    return v + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// |x| order key of dimension d: |x| bits above the inverted index, so keys are
// distinct, larger |x| ranks first and equal |x| go to the lower index.
__device__ __forceinline__ uint64_t dim_key(uint32_t ubits, int d)
{
    return ((uint64_t)ubits << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)d);
}

// Rank of the first dimension of group b (b = 0: of the first non-exact one).
__device__ __forceinline__ int boundary_rank(int b, int t, int base)
{
    return b == 0 || base == 0 ? t : t + b * base;
}

// One wave: in the histogram h of 64 * PER bins, the bin D holding rank r
// counted from the top bin down, r's rank within D and D's count (in every
// lane).  Lane l sums bins 64 PER - 1 - PER l down to 64 PER - PER (l + 1).
template <int PER>
__device__ __forceinline__ void find_digit(const uint32_t* h, uint32_t r, int lane, uint32_t& digit, uint32_t& rin,
                                           uint32_t& cnt)
{
    constexpr int kNb = kWave * PER;
    const int lo = kNb - PER * (lane + 1);
    uint32_t q[PER];
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
        const uint4 v4 = *reinterpret_cast<const uint4*>(h + lo + j);
        q[j] = v4.x;
        q[j + 1] = v4.y;
        q[j + 2] = v4.z;
        q[j + 3] = v4.w;
    }
    uint32_t sum = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) sum += q[j];
    const uint32_t incl = wave_scan_incl(sum, lane);
    const uint32_t excl = incl - sum;
    const bool mine = excl <= r && r < incl;
    uint32_t dg = 0u, ri = 0u, c = 0u, run = excl;
    bool done = false;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {   // highest bin first, without branches
        const bool hit = !done && r < run + q[j];
        dg = hit ? (uint32_t)(lo + j) : dg;
        ri = hit ? r - run : ri;
        c = hit ? q[j] : c;
        done = done || hit;
        run += q[j];
    }
    const int src = (int)__builtin_ctzll(__ballot(mine) | (1ull << 63));
    digit = (uint32_t)__builtin_amdgcn_readlane((int)dg, src);
    rin = (uint32_t)__builtin_amdgcn_readlane((int)ri, src);
    cnt = (uint32_t)__builtin_amdgcn_readlane((int)c, src);
}

// One wave, the shared histogram of the top 11 bits (2048 bins): for each active
// boundary b, the bin holding rank B[b] from the top, the rank within it and the
// bin's count (the same in every lane).  Lane l first sums bins 2047 - 32 l down to
// 2016 - 32 l; the lane whose range holds the rank then has its 32 bins spread
// over lanes 0..31 and scanned again.
__device__ __forceinline__ void find_digits4(const uint32_t* h, const int* B, const bool* act, int lane,
                                             uint32_t* pre, uint32_t* res, uint32_t* cnt)
{
    constexpr int kPer = 32;
    const int lo = 2048 - kPer * (lane + 1);
    uint32_t sum = 0u;
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
        const uint4 v4 = *reinterpret_cast<const uint4*>(h + lo + j);
        sum += (v4.x + v4.y) + (v4.z + v4.w);
    }
    const uint32_t incl = wave_scan_incl(sum, lane);
    const uint32_t excl = incl - sum;
#pragma unroll
    for (int b = 0; b < kSkGroups; ++b) {
        pre[b] = res[b] = cnt[b] = 0u;
        if (!act[b]) continue;
        const uint32_t r = (uint32_t)B[b];
        const int src = (int)__builtin_ctzll(__ballot(excl <= r && r < incl) | (1ull << 63));
        const uint32_t e_src = (uint32_t)__builtin_amdgcn_readlane((int)excl, src);
        const int lo_src = 2048 - kPer * (src + 1);
        const uint32_t hv = lane < kPer ? h[lo_src + kPer - 1 - lane] : 0u;   // its bins, highest first
        const uint32_t ci = wave_scan_incl(hv, lane);
        const int j = (int)__builtin_ctzll(__ballot(lane < kPer && e_src + ci > r) | (1ull << 63));
        pre[b] = (uint32_t)(lo_src + kPer - 1 - j);
        cnt[b] = (uint32_t)__builtin_amdgcn_readlane((int)hv, j);
        res[b] = r - e_src - ((uint32_t)__builtin_amdgcn_readlane((int)ci, j) - cnt[b]);
    }
}

__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The cut b*: the highest bin at which the bins from the top down hold `need`
// words, among the kSkWindow bins below the highest non-empty one (0 when they
// hold fewer, or when every word is needed).  The same in every thread.  The
// histogram and the maxima come from the previous launch: plain loads see them.
template <int THREADS>
__device__ __forceinline__ uint32_t find_cut(const uint32_t* ctlw, const uint32_t* hist, uint32_t need, int64_t v,
                                             uint32_t (*part)[kSkWindow], uint32_t& s_bstar, int32_t& s_found,
                                             int tid, int lane, int wave)
{
    if ((int64_t)need >= v) return 0u;
    uint32_t mb = 0u;
#pragma unroll
    for (int g = 0; g < kSkSets; ++g) mb = max(mb, ctlw[kCtlMaxBin + 16 * g]);
    const int max_bin = (int)min(mb, (uint32_t)(kSkBins - 1));
    if (tid == 0) s_found = 0;
    for (int i = tid; i < kSkCopies * kSkWindow; i += THREADS) {
        const int c = i / kSkWindow, j = i % kSkWindow, bin = max_bin - j;
        part[c][j] = bin >= 0 ? hist[c * kSkBins + bin] : 0u;
    }
    __syncthreads();
    if (wave == 0) {   // lane l: bins max_bin - 4 l .. max_bin - 4 l - 3
        uint32_t h4[4], sum = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h4[e] = 0u;
#pragma unroll
            for (int c = 0; c < kSkCopies; ++c) h4[e] += part[c][4 * lane + e];
            sum += h4[e];
        }
        const uint32_t incl = wave_scan_incl(sum, lane);
        const uint32_t excl = incl - sum;
        if (excl < need && incl >= need) {
            uint32_t run = excl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                run += h4[e];
                if (run >= need) {
                    s_bstar = (uint32_t)(max_bin - (4 * lane + e));
                    s_found = 1;
                    break;
                }
            }
        }
    }
    __syncthreads();
    return s_found ? s_bstar : 0u;   // fewer than need words in the window: every word
}

// Exact logits of the workgroup's candidates, a wave per word (x in LDS); the
// wave's best (logit order key << 32 | ~row).
template <int WAVES>
__device__ __forceinline__ unsigned long long rescore(const uint16_t* __restrict__ w, const float* xs, int k,
                                                      const int32_t* list, int n, int lane, int wave)
{
    const int nch = k / 8;
    unsigned long long mine = 0ull;
    for (int c = wave; c < n; c += WAVES) {
        const int64_t row_i = list[c];
        const uint4* row = reinterpret_cast<const uint4*>(w + row_i * k);
        float sum = 0.0f;
        for (int ch0 = lane; ch0 < nch; ch0 += 4 * kWave) {
            uint4 q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = ch0 + u * kWave < nch ? row[ch0 + u * kWave] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ch = ch0 + u * kWave;
                if (ch >= nch) break;
                const float* xc = xs + 8 * ch;
                sum = fmaf(__uint_as_float(q[u].x << 16), xc[0], sum);
                sum = fmaf(__uint_as_float(q[u].x & 0xFFFF0000u), xc[1], sum);
                sum = fmaf(__uint_as_float(q[u].y << 16), xc[2], sum);
                sum = fmaf(__uint_as_float(q[u].y & 0xFFFF0000u), xc[3], sum);
                sum = fmaf(__uint_as_float(q[u].z << 16), xc[4], sum);
                sum = fmaf(__uint_as_float(q[u].z & 0xFFFF0000u), xc[5], sum);
                sum = fmaf(__uint_as_float(q[u].w << 16), xc[6], sum);
                sum = fmaf(__uint_as_float(q[u].w & 0xFFFF0000u), xc[7], sum);
            }
        }
        sum = wave_sum_f(sum);
        const unsigned long long kv =
            ((unsigned long long)order_key(sum) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)row_i);
        mine = kv > mine ? kv : mine;
    }
    return mine;
}

// The workgroup's best and count go to its slot; it counts itself out (per set
// of workgroups, then over the sets), and the last one out takes the first
// maximum over the slots, writes the choice and readies the control words for
// the next token.
template <int THREADS>
__device__ __forceinline__ void finish(uint8_t* ws, uint32_t* ctlw, unsigned long long mine, uint32_t n,
                                       uint32_t parity, int32_t* idx, float* max_logit, int32_t* ncand,
                                       unsigned long long* s_best, uint32_t* s_cnt, int32_t& s_last, int tid,
                                       int lane, int wave)
{
    constexpr int kWaves = THREADS / kWave;
    uint64_t* slots = reinterpret_cast<uint64_t*>(ws + kSkSlotOff);
    if (lane == 0) s_best[wave] = mine;
    __syncthreads();
    if (tid == 0) {
        unsigned long long b = 0ull;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) b = s_best[i] > b ? s_best[i] : b;
        __hip_atomic_store(&slots[2 * blockIdx.x], (uint64_t)b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&slots[2 * blockIdx.x + 1], (uint64_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);   // the slot is written before this workgroup counts itself out
        const uint32_t set = blockIdx.x % kSkSets;
        const uint32_t in_set = (gridDim.x - set + kSkSets - 1) / kSkSets;
        int last = 0;
        if (__hip_atomic_fetch_add(&ctlw[kCtlOut + 16 * set], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            in_set - 1)
            last = __hip_atomic_fetch_add(&ctlw[kCtlOutAll], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   min(gridDim.x, (uint32_t)kSkSets) - 1;
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    unsigned long long b = 0ull;
    uint32_t cnt = 0u;
    for (uint32_t i = tid; i < gridDim.x; i += THREADS) {
        const unsigned long long bi = __hip_atomic_load(&slots[2 * i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        b = bi > b ? bi : b;
        cnt += (uint32_t)__hip_atomic_load(&slots[2 * i + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    b = wave_max_u64(b);
    cnt = wave_scan_incl(cnt, lane);
    if (lane == kWave - 1) {
        s_best[wave] = b;
        s_cnt[wave] = cnt;
    }
    __syncthreads();
    if (tid == 0) {
        unsigned long long fb = 0ull;
        uint32_t fc = 0u;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            fb = s_best[i] > fb ? s_best[i] : fb;
            fc += s_cnt[i];
        }
        *idx = (int32_t)(0xFFFFFFFFu - (uint32_t)(fb & 0xFFFFFFFFu));
        if (max_logit) *max_logit = key_value((uint32_t)(fb >> 32));
        if (ncand) *ncand = (int32_t)fc;
        store_agent(&ctlw[kCtlParity], 1u - parity);
    }
    if (tid < kSkSets) store_agent(&ctlw[kCtlMaxBin + 16 * tid], 0u);
    if (tid < 2 * kSkSets) store_agent(&ctlw[kCtlOut + 16 * tid], 0u);
}

__global__ __launch_bounds__(kSkScoreThreads) void k_sketch_score(const uint32_t* __restrict__ signs,
                                                                  const uint16_t* __restrict__ wt,
                                                                  const float* __restrict__ x,
                                                                  const SketchHeader* __restrict__ hdr, int64_t v,
                                                                  int64_t vp, int k, uint8_t* __restrict__ ws,
                                                                  float* __restrict__ scores)
{
    extern __shared__ __align__(16) uint8_t smem[];
    ScoreLds& s = *reinterpret_cast<ScoreLds*>(smem);
    uint32_t* ctlw = reinterpret_cast<uint32_t*>(ws);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const float ctab = hdr->c;
    const uint32_t parity = ctlw[kCtlParity] & 1u;
    const int kw = (k + 31) >> 5, k4 = k >> 2;
    const int64_t col = ((int64_t)blockIdx.x * kSkRows >> 1) + tid;   // this lane's row pair: rows 2 col, 2 col + 1
    const int64_t vp2 = vp >> 1;

    // x first (its few loads would otherwise wait behind the sign words) ...
    float4 xv[kSkXLoads];
    const float4* x4 = reinterpret_cast<const float4*>(x);
#pragma unroll
    for (int i = 0; i < kSkXLoads; ++i) xv[i] = x4[min(tid + kSkScoreThreads * i, k4 - 1)];
    uint32_t ux[kSkXLoads][4];   // |x| bits of dimensions 4 q .. 4 q + 3, q = tid + 512 i (all ones: none)
#pragma unroll
    for (int i = 0; i < kSkXLoads; ++i) {
        const int q = tid + kSkScoreThreads * i;
        const uint32_t b4[4] = {__float_as_uint(xv[i].x), __float_as_uint(xv[i].y), __float_as_uint(xv[i].z),
                                __float_as_uint(xv[i].w)};
#pragma unroll
        for (int j = 0; j < 4; ++j) ux[i][j] = q < k4 ? (b4[j] & 0x7FFFFFFFu) : 0xFFFFFFFFu;
        if (q < k4) reinterpret_cast<float4*>(s.xb)[q] = xv[i];
    }
    asm volatile("" ::: "memory");
    // ... then the sign words, which stay in flight while the plan is made.  They go out in six
    // batches, one before the plan and one after each of its first five LDS steps: asked for at
    // once, the whole chip's requests fill the memory queues and issuing them holds the wave for
    // microseconds before the plan can start; spread out, the plan runs while the queues drain.
    const sk_u32x2* sg = reinterpret_cast<const sk_u32x2*>(signs);
    sk_u32x2 sw[kSkPre];
    constexpr int kSkPreBatch = kSkPre / 6;
    static_assert(kSkPre % 6 == 0, "six batches of sign words");
    auto issue = [&](int b) {
#pragma unroll
        for (int u = b * kSkPreBatch; u < (b + 1) * kSkPreBatch; ++u)
            sw[u] = __builtin_nontemporal_load(&sg[(int64_t)min(u, kw - 1) * vp2 + col]);
        asm volatile("" ::: "memory");
    };
    issue(0);

    // ---- the plan ----
    for (int i = tid; i < 6 * (kSkWords + kSkBatch) / 4; i += kSkScoreThreads)
        reinterpret_cast<uint4*>(&s.word[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < kSkBins / 4; i += kSkScoreThreads)
        reinterpret_cast<uint4*>(s.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < 2048 / 4; i += kSkScoreThreads)
        reinterpret_cast<uint4*>(s.rh0)[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < 2 * kSkGroups * 1024 / 4; i += kSkScoreThreads)
        reinterpret_cast<uint4*>(&s.rh[0][0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    const int t = min(k, kSkTop), rest = k - t, base = rest / kSkGroups;
    int B[kSkGroups];
    bool act[kSkGroups];
#pragma unroll
    for (int b = 0; b < kSkGroups; ++b) {
        B[b] = boundary_rank(b, t, base);
        act[b] = B[b] < k;
    }
    if (tid < kSkGroups) s.lcnt[tid] = 0u;
    const int nq = (k4 + kSkScoreThreads - 1) / kSkScoreThreads;
    lds_barrier();
    issue(1);
    // the boundaries' bins of the top 11 bits of |x| (every wave finds them; the state stays in registers)
#pragma unroll
    for (int i = 0; i < kSkXLoads; ++i) {
        if (i >= nq) break;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (ux[i][j] != 0xFFFFFFFFu) atomicAdd(&s.rh0[ux[i][j] >> 20], 1u);
    }
    lds_barrier();
    issue(2);
    uint32_t pre[kSkGroups], res[kSkGroups], cnt[kSkGroups], shv[kSkGroups];
    find_digits4(s.rh0, B, act, lane, pre, res, cnt);
#pragma unroll
    for (int b = 0; b < kSkGroups; ++b) shv[b] = 20u;
    // a bin of more than kSkList dimensions: the next 10 bits (then the last 10)
#pragma unroll
    for (int p = 1; p <= 2; ++p) {
        const int sh = 20 - 10 * p;
        bool more[kSkGroups];
        bool any_more = false;
#pragma unroll
        for (int b = 0; b < kSkGroups; ++b) {
            more[b] = act[b] && cnt[b] > (uint32_t)kSkList;
            any_more = any_more || more[b];
        }
        if (!any_more) break;
#pragma unroll 1
        for (int i = 0; i < nq; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t u = ux[i][j];
#pragma unroll
                for (int b = 0; b < kSkGroups; ++b)
                    if (more[b] && (u >> (sh + 10)) == pre[b]) atomicAdd(&s.rh[p - 1][b][(u >> sh) & 1023u], 1u);
            }
        }
        lds_barrier();
#pragma unroll
        for (int b = 0; b < kSkGroups; ++b) {
            if (!more[b]) continue;
            uint32_t dg, rin, c;
            find_digit<16>(s.rh[p - 1][b], res[b], lane, dg, rin, c);
            pre[b] = (pre[b] << 10) | dg;
            res[b] = rin;
            cnt[b] = c;
            shv[b] = (uint32_t)sh;
        }
    }
    // the dimensions left in each boundary's bin
#pragma unroll 1
    for (int i = 0; i < nq; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t u = ux[i][j];
            const int d = 4 * (tid + kSkScoreThreads * i) + j;
#pragma unroll
            for (int b = 0; b < kSkGroups; ++b) {
                if (act[b] && cnt[b] <= (uint32_t)kSkList && (u >> shv[b]) == pre[b]) {
                    const uint32_t slot = atomicAdd(&s.lcnt[b], 1u);
                    if (slot < (uint32_t)kSkList) s.lst[b][slot] = dim_key(u, d);
                }
            }
        }
    }
    lds_barrier();
    issue(3);
    const int nch = (k + 63) >> 6;
    if (wave < kSkGroups) {
        const int b = wave;
        if (!act[b]) {
            if (lane == 0) s.kb[b] = 0ull;   // no such rank: every key is above
        } else if (cnt[b] <= (uint32_t)kSkList) {
            // rank the bin's dimensions against each other
            const uint32_t c = cnt[b], r = res[b];
            const uint64_t my = lane < (int)c ? s.lst[b][lane] : 0ull;
            uint32_t above = 0u;
            for (uint32_t j = 0; j < c; j += 8) {   // entries past c are ignored below
                uint64_t e[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) e[u] = s.lst[b][(j + u) & (kSkList - 1)];
#pragma unroll
                for (int u = 0; u < 8; ++u) above += (j + u < c && e[u] > my) ? 1u : 0u;
            }
            if (lane < (int)c && above == r) s.kb[b] = my;
        } else {
            // more than kSkList dimensions with exactly the boundary's |x|: by index
            const uint32_t ub = pre[b];
            uint32_t r = res[b];
            for (int c = 0; c < nch; ++c) {
                const int d = 64 * c + lane;
                const bool m = d < k && (s.xb[min(d, k - 1)] & 0x7FFFFFFFu) == ub;
                const uint64_t mask = __ballot(m);
                const uint32_t n = (uint32_t)__popcll(mask);
                if (r < n) {
                    if (m && lanes_below(mask) == r) s.kb[b] = dim_key(ub, d);
                    break;
                }
                r -= n;
            }
        }
    }
    lds_barrier();
    issue(4);
    // classes, 64 dimensions per wave step: mask words, the exact dimensions, group sums of |x|
    const uint64_t k0 = s.kb[0], k1 = s.kb[1], k2 = s.kb[2], k3 = s.kb[3];
    {
        float gp[kSkGroups] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int c = wave; c < nch; c += kSkScoreWaves) {
            const int d = 64 * c + lane;
            const bool valid = d < k;
            const uint32_t xbits = valid ? s.xb[d] : 0u;
            const uint64_t key = dim_key(xbits & 0x7FFFFFFFu, d);
            const bool top = valid && key > k0;
            const bool rst = valid && !top;
            const int g = (key <= k1 ? 1 : 0) + (key <= k2 ? 1 : 0) + (key <= k3 ? 1 : 0);
            const float ax = __uint_as_float(xbits & 0x7FFFFFFFu);
            uint64_t m[6];
            m[0] = __ballot(top);
#pragma unroll
            for (int gi = 0; gi < kSkGroups; ++gi) {
                m[1 + gi] = __ballot(rst && g == gi);
                gp[gi] += rst && g == gi ? ax : 0.0f;
            }
            m[5] = __ballot(valid && __uint_as_float(xbits) < 0.0f);
            if (lane == 0) {
#pragma unroll
                for (int q = 0; q < 6; ++q) {
                    s.word[q][2 * c] = (uint32_t)m[q];
                    s.word[q][2 * c + 1] = (uint32_t)(m[q] >> 32);
                }
            }
        }
#pragma unroll
        for (int gi = 0; gi < kSkGroups; ++gi) {
            const float a = wave_sum_f(gp[gi]);
            if (lane == 0) s.gpart[wave][gi] = a;
        }
    }
    lds_barrier();
    issue(5);
    // every wave on its own from here: the group weights (the partial sums in wave order) and the
    // exact dimensions in index order (a scan of the exact-mask words over the 64-dimension steps)
    float wgt[kSkGroups];
    int ng[kSkGroups];
#pragma unroll
    for (int g = 0; g < kSkGroups; ++g) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kSkScoreWaves; ++w) sum += s.gpart[w][g];
        ng[g] = g < kSkGroups - 1 ? base : rest - (kSkGroups - 1) * base;
        wgt[g] = ng[g] > 0 ? ctab * (sum / (float)ng[g]) : 0.0f;
    }
    {
        uint32_t before = 0u;
        for (int c0 = 0; c0 < nch; c0 += kWave) {
            const int c = c0 + lane;
            uint64_t m = 0ull;
            if (c < nch) m = ((uint64_t)s.word[0][2 * c + 1] << 32) | s.word[0][2 * c];
            const uint32_t n = (uint32_t)__popcll(m);
            const uint32_t incl = wave_scan_incl(n, lane);
            uint32_t pos = before + incl - n;
            while (m && pos < (uint32_t)kSkTop) {
                const int d = 64 * c + (int)__builtin_ctzll(m);
                m &= m - 1;
                s.top_idx[wave][pos] = d;
                s.top_x[wave][pos] = __uint_as_float(s.xb[d]);
                ++pos;
            }
            before += (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's list is written before it is read

    // ---- scores of rows 2 col and 2 col + 1 ----
    const uint32_t* wt2 = reinterpret_cast<const uint32_t*>(wt);
    uint32_t hx[kSkTop];
#pragma unroll
    for (int j = 0; j < kSkTop; ++j) {
        const uint32_t d = min((uint32_t)s.top_idx[wave][min(j, t - 1)], (uint32_t)(k - 1));
        hx[j] = __builtin_nontemporal_load(&wt2[(int64_t)d * vp2 + col]);
    }
    int c0[kSkGroups] = {0, 0, 0, 0}, c1[kSkGroups] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kSkPre; ++u) {
        const uint32_t xs = s.word[5][u];
        const uint32_t d0 = sw[u].x ^ xs, d1 = sw[u].y ^ xs;
#pragma unroll
        for (int g = 0; g < kSkGroups; ++g) {
            const uint32_t m = s.word[1 + g][u];
            c0[g] += __popc(d0 & m);
            c1[g] += __popc(d1 & m);
        }
    }
    for (int w0 = kSkPre; w0 < kw; w0 += kSkBatch) {
        sk_u32x2 bw[kSkBatch];
#pragma unroll
        for (int u = 0; u < kSkBatch; ++u)
            bw[u] = __builtin_nontemporal_load(&sg[(int64_t)min(w0 + u, kw - 1) * vp2 + col]);
#pragma unroll
        for (int u = 0; u < kSkBatch; ++u) {
            const uint32_t xs = s.word[5][w0 + u];
            const uint32_t d0 = bw[u].x ^ xs, d1 = bw[u].y ^ xs;
#pragma unroll
            for (int g = 0; g < kSkGroups; ++g) {
                const uint32_t m = s.word[1 + g][w0 + u];
                c0[g] += __popc(d0 & m);
                c1[g] += __popc(d1 & m);
            }
        }
    }
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int j = 0; j < kSkTop; ++j) {
        if (j < t) {
            const float xj = s.top_x[wave][j];
            a0 = fmaf(__uint_as_float(hx[j] << 16), xj, a0);
            a1 = fmaf(__uint_as_float(hx[j] & 0xFFFF0000u), xj, a1);
        }
    }
#pragma unroll
    for (int g = 0; g < kSkGroups; ++g) {
        a0 = fmaf(wgt[g], (float)(ng[g] - 2 * c0[g]), a0);
        a1 = fmaf(wgt[g], (float)(ng[g] - 2 * c1[g]), a1);
    }
    const uint32_t key0 = order_key(a0), key1 = order_key(a1);
    reinterpret_cast<sk_u32x2*>(ws + sk_keys_off(vp))[col] = sk_u32x2{key0, key1};
    const int64_t r0 = 2 * col;
    const bool live0 = r0 < v, live1 = r0 + 1 < v;
    if (scores) {
        if (live0) scores[r0] = a0;
        if (live1) scores[r0 + 1] = a1;
    }
    if (live0) atomicAdd(&s.hist[key0 >> (32 - kSkBinBits)], 1u);
    if (live1) atomicAdd(&s.hist[key1 >> (32 - kSkBinBits)], 1u);
    lds_barrier();
    {
        uint32_t top1 = 0u;   // highest non-empty bin of this thread's, plus one
#pragma unroll
        for (int i = 0; i < kSkBins / kSkScoreThreads; ++i) {
            const int bin = tid + kSkScoreThreads * i;
            top1 = s.hist[bin] ? (uint32_t)bin + 1u : top1;
        }
        top1 = wave_max_u32(top1);
        if (lane == 0) s.wmax[wave] = top1;
    }
    lds_barrier();
    // the kSkWindow bins below the highest non-empty one, two bins per 64-bit add (each
    // 32-bit half holds a bin's count, which never carries over)
    uint32_t top1 = 0u;
#pragma unroll
    for (int w = 0; w < kSkScoreWaves; ++w) top1 = max(top1, s.wmax[w]);
    const int lmax = (int)top1 - 1;   // every workgroup has a live row
    uint64_t* hist64 = reinterpret_cast<uint64_t*>(ws + kSkHistOff) +
                       (parity * kSkHistSet + (int64_t)(blockIdx.x % kSkCopies) * kSkBins) / 2;
    for (int pr = max(lmax - (kSkWindow - 1), 0) / 2 + tid; pr <= lmax / 2; pr += kSkScoreThreads) {
        const uint32_t h0 = s.hist[2 * pr], h1 = s.hist[2 * pr + 1];
        if (h0 | h1)
            __hip_atomic_fetch_add(&hist64[pr], (uint64_t)h0 | ((uint64_t)h1 << 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0)
        __hip_atomic_fetch_max(&ctlw[kCtlMaxBin + 16 * (blockIdx.x % kSkSets)], (uint32_t)lmax, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    if (blockIdx.x == 0 && tid < 2 * kSkSets)   // the pick launch's exit counters, used only after this launch
        ctlw[kCtlOut + 16 * tid] = 0u;
}

// ---- per token, second launch: the cut, exact scores of the candidates, the choice ----------

__global__ __launch_bounds__(kSkPickThreads) void k_sketch_pick(const uint16_t* __restrict__ w,
                                                                const float* __restrict__ x, int64_t v, int64_t vp,
                                                                int k, uint8_t* __restrict__ ws,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ max_logit,
                                                                int32_t* __restrict__ ncand)
{
    __shared__ __align__(16) float xs[kSketchMaxK];
    __shared__ int32_t s_list[kSkRows];
    __shared__ uint32_t s_part[kSkCopies][kSkWindow];
    __shared__ unsigned long long s_best[kSkPickThreads / kWave];
    __shared__ uint32_t s_cnt[kSkPickThreads / kWave];
    __shared__ uint32_t s_n, s_bstar;
    __shared__ int32_t s_found, s_last;
    uint32_t* ctlw = reinterpret_cast<uint32_t*>(ws);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t parity = ctlw[kCtlParity] & 1u;
    const int64_t r = (int64_t)blockIdx.x * kSkRows + tid;
    const uint32_t key = reinterpret_cast<const uint32_t*>(ws + sk_keys_off(vp))[r];
    for (int q = tid; q < (k >> 2); q += kSkPickThreads)
        reinterpret_cast<float4*>(xs)[q] = reinterpret_cast<const float4*>(x)[q];
    if (tid == 0) s_n = 0u;
    // this workgroup's share of clearing the other histogram set (the next token's)
    uint4* other = reinterpret_cast<uint4*>(ws + kSkHistOff) + (int64_t)(1u - parity) * (kSkHistSet / 4);
    for (int64_t i = (int64_t)blockIdx.x * kSkPickThreads + tid; i < kSkHistSet / 4;
         i += (int64_t)gridDim.x * kSkPickThreads)
        other[i] = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t need = (uint32_t)min<int64_t>(v, kSkMinCand);
    const uint32_t bstar = find_cut<kSkPickThreads>(
        ctlw, reinterpret_cast<const uint32_t*>(ws + kSkHistOff) + parity * kSkHistSet, need, v, s_part, s_bstar,
        s_found, tid, lane, wave);
    if (r < v && (key >> (32 - kSkBinBits)) >= bstar) s_list[atomicAdd(&s_n, 1u)] = (int32_t)r;
    __syncthreads();
    const uint32_t n = s_n;
    const unsigned long long mine = rescore<kSkPickThreads / kWave>(w, xs, k, s_list, (int)n, lane, wave);
    finish<kSkPickThreads>(ws, ctlw, mine, n, parity, idx, max_logit, ncand, s_best, s_cnt, s_last, tid, lane, wave);
}

}  // namespace

// The copy's space also holds the build's row sums and block partials until
// the transpose overwrites them.
int64_t sketch_copy_bytes(int64_t v, int64_t k)
{
    const int64_t temp = sk_round(4 * v, 256) + sk_round(8 * ((v + kSkRowBlock - 1) / kSkRowBlock), 256);
    return max(sk_round(2 * k * sk_pitch(v), 256), temp);
}

int64_t sketch_bytes(int64_t v, int64_t k)
{
    const int64_t kw = (k + 31) / 32;
    return 256 + sk_round(4 * kw * sk_pitch(v), 256) + sketch_copy_bytes(v, k);
}

// [control][2 histogram sets][a slot per pick workgroup][row keys: 4 vp]
int64_t sketch_workspace_bytes(int64_t v) { return sk_keys_off(sk_pitch(v)) + 4 * sk_pitch(v); }

hipError_t launch_sketch_build(const uint16_t* w, int64_t v, int64_t k, void* sketch, hipStream_t s)
{
    uint8_t* base = static_cast<uint8_t*>(sketch);
    const int64_t kw = (k + 31) / 32, vp = sk_pitch(v);
    uint32_t* signs = reinterpret_cast<uint32_t*>(base + 256);
    uint16_t* wt = reinterpret_cast<uint16_t*>(base + 256 + sk_round(4 * kw * vp, 256));
    // the row sums and block partials live in the copy's space until the transpose
    float* rowsum = reinterpret_cast<float*>(wt);
    double* part = reinterpret_cast<double*>(reinterpret_cast<uint8_t*>(wt) + sk_round(4 * v, 256));
    hipLaunchKernelGGL(k_sketch_rows, dim3((unsigned)((vp + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, w, v, vp,
                       (int)k, signs, rowsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_scale, dim3(1), dim3(kBlock), 0, s, rowsum, v, (int)k, part,
                       reinterpret_cast<SketchHeader*>(base));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_transpose, dim3((unsigned)(vp / 64), (unsigned)((k + 63) / 64)), dim3(kBlock), 0, s,
                       w, v, vp, (int)k, wt);
    return hipGetLastError();
}

hipError_t setup_sketch_attributes() { return raise_lds_limit(reinterpret_cast<const void*>(&k_sketch_score)); }

hipError_t launch_sketch_argmax(const uint16_t* w, const void* sketch, const float* x, int64_t v, int64_t k,
                                int32_t* idx, float* max_logit, int32_t* ncand, float* scores, void* workspace,
                                hipStream_t s)
{
    const uint8_t* base = static_cast<const uint8_t*>(sketch);
    const int64_t kw = (k + 31) / 32, vp = sk_pitch(v);
    const uint32_t* signs = reinterpret_cast<const uint32_t*>(base + 256);
    const uint16_t* wt = reinterpret_cast<const uint16_t*>(base + 256 + sk_round(4 * kw * vp, 256));
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const unsigned nwg = (unsigned)(vp / kSkRows);
    hipLaunchKernelGGL(k_sketch_score, dim3(nwg), dim3(kSkScoreThreads), sizeof(ScoreLds), s, signs, wt, x,
                       reinterpret_cast<const SketchHeader*>(base), v, vp, (int)k, ws, scores);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_pick, dim3(nwg), dim3(kSkPickThreads), 0, s, w, x, v, vp, (int)k, ws, idx, max_logit,
                       ncand);
    return hipGetLastError();
}

}  // namespace qmv
