// k_sketch.hip -- the sketch head: the output layer's greedy choice from
// candidates ("Gemma 3 1B at 114 tokens per second on a laptop CPU", "Step 3:
// the output layer became the bottleneck", the sketch head's three steps).
//
// Per token:
//  1. k_sketch_rank (many workgroups) ranks the hidden dimensions by |x|
//     (descending, ties to the lower index) by counting larger keys; then
//     k_sketch_plan (one workgroup) takes the first T = min(32, k) as the
//     exactly scored ones and cuts the rest into 4 consecutive rank groups,
//     each weighted by c * mean |x| (c = mean |w| of the table, computed when
//     the sketch is built).  Group bit masks and the sign bits of x go to the
//     workspace; the candidate histograms are cleared.
//  2. k_sketch_score (a thread per row): a = 0; a = fma(w[r][d_j], x[d_j], a)
//     over the exact dimensions in rank order, read from a dimension-major
//     copy of the table; then per group a = fma(weight_g, agreement_g, a),
//     the agreement = n_g - 2 * popcount((signs of w ^ signs of x) & mask_g)
//     from the 1-bit table (one XOR, then AND + bit count per group, 32
//     dimensions per word).  The fp32 score's order key goes to the
//     workspace and into a histogram of its top 12 bits.
//  3. k_sketch_select finds the lowest bin b* such that the bins from b* up
//     hold at least min(1024, v) words; the words in those bins are the
//     candidates.  k_sketch_rescore scores each candidate exactly (a wave per
//     candidate, fp32 like k_lmhead) and keeps each workgroup's best (logit,
//     lowest index); k_sketch_final takes the first maximum over them.
// The score arithmetic is fixed (fp32 FMAs in the order above), so the
// candidate set is exactly the one the oracle computes.
#include "qmv_internal.hpp"

namespace qmv {
namespace {

constexpr int kSkTop = 32;         // exactly scored dimensions
constexpr int kSkGroups = 4;       // sign-bit groups
constexpr int kSkMinCand = 1024;   // candidates: at least this many words (or all of them)
constexpr int kSkBins = 4096;      // histogram over the top 12 bits of the order key
constexpr int kSkRowBlock = 512;   // rows per fp64 partial of the table scale
constexpr int kSkPlanThreads = 1024;
constexpr int kSkRowsPerBlock = 1024;   // score / rescore: rows per workgroup (4 per thread)
constexpr uint32_t kSkMagic = 0x31484b53u;   // "SKH1"

// Sketch buffer: header, sign words [kw][v], dimension-major bf16 copy [k][v].
struct SketchHeader {
    uint32_t magic;
    int32_t k;
    int64_t v;
    float c;        // mean |w| of the table
    int32_t pad[11];
};
static_assert(sizeof(SketchHeader) == 64, "sketch header");

// Workspace: the plan, the histogram, the pick, then the order keys [v].
struct SketchPlan {
    int32_t t;               // exact dimensions
    int32_t kw;              // 32-dimension words
    int32_t n[kSkGroups];    // group sizes
    float wgt[kSkGroups];    // group weights
    int32_t pad[6];
    int32_t top_idx[kSkTop];
    float top_x[kSkTop];
    // then masks [kSkGroups][kw] and the sign words of x [kw]
};
static_assert(sizeof(SketchPlan) == 320, "sketch plan");
constexpr int kSkHistCopies = 8;        // private histograms (workgroup b adds into copy b % 8)
constexpr int kSkScoreThreads = 1024;   // score: a thread per row
constexpr int64_t kSkPlanBytes = 8192;
constexpr int64_t kSkHistOff = kSkPlanBytes;
constexpr int64_t kSkPickOff = kSkHistOff + kSkHistCopies * kSkBins * 4;   // u32 b*
constexpr int64_t kSkWgOff = kSkPickOff + 256;   // per rescore workgroup: u64 best, then u32 counts
constexpr int64_t kSkMaxWg = (((int64_t)1 << 24) + kSkRowsPerBlock - 1) / kSkRowsPerBlock;
constexpr int64_t kSkKeysOff = kSkWgOff + 12 * kSkMaxWg;

constexpr int64_t sk_round(int64_t n, int64_t a) { return (n + a - 1) / a * a; }

__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ---- build --------------------------------------------------------------------------------

// A thread per row: the sign words (word w of row r at w * v + r) and the
// row's sum of |w| in fp32, column order (into `rowsum`).
__global__ __launch_bounds__(kBlock) void k_sketch_rows(const uint16_t* __restrict__ w, int64_t v, int k,
                                                        uint32_t* __restrict__ signs, float* __restrict__ rowsum)
{
    const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (r >= v) return;
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
            signs[(int64_t)(c8 >> 2) * v + r] = word;
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

// 64 x 64 tiles through LDS: wt[c][r] = w[r][c].
__global__ __launch_bounds__(kBlock) void k_sketch_transpose(const uint16_t* __restrict__ w, int64_t v, int k,
                                                             uint16_t* __restrict__ wt)
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
        if (c < k && r < v) wt[(int64_t)c * v + r] = tile[tx][cc];
    }
}

// ---- per token ----------------------------------------------------------------------------

// |x| order key of dimension i: |x| bits above the inverted index, so keys are
// distinct, larger |x| ranks first and equal |x| go to the lower index.
__device__ __forceinline__ uint64_t order_key_of(const float* x, int i)
{
    return ((uint64_t)__float_as_uint(fabsf(x[i])) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// Ranks by counting, spread over many compute units: workgroup b places keys
// 16b .. 16b+15, each compared with every key by 16 threads (a sixteenth of the
// keys each); the rank is the number of larger keys, and the key is written at
// its rank, so `sorted` ends up in descending order.
constexpr int kSkRankPer = 16;
__global__ __launch_bounds__(kBlock) void k_sketch_rank(const float* __restrict__ x, int k,
                                                        uint64_t* __restrict__ sorted)
{
    __shared__ uint64_t key[kSketchMaxK];
    __shared__ uint32_t cnt[kSkRankPer];
    const int tid = threadIdx.x;
    for (int i = tid; i < k; i += kBlock) key[i] = order_key_of(x, i);
    if (tid < kSkRankPer) cnt[tid] = 0u;
    __syncthreads();
    const int e = blockIdx.x * kSkRankPer + (tid % kSkRankPer);
    const int part = tid / kSkRankPer;
    if (e < k) {
        const uint64_t me = key[e];
        uint32_t c = 0;
        for (int j = part; j < k; j += kBlock / kSkRankPer) c += key[j] > me ? 1u : 0u;
        atomicAdd(&cnt[tid % kSkRankPer], c);
    }
    __syncthreads();
    if (tid < kSkRankPer && e < k) sorted[cnt[tid]] = key[e];
}

// One workgroup of 1024 threads; dynamic LDS: the k order keys in descending
// order (from k_sketch_rank) then the masks and x sign words (5 * kw words).
__global__ __launch_bounds__(kSkPlanThreads) void k_sketch_plan(const float* __restrict__ x, int k,
                                                                const uint64_t* __restrict__ sorted,
                                                                const SketchHeader* __restrict__ hdr,
                                                                uint8_t* __restrict__ ws)
{
    extern __shared__ __align__(16) uint8_t sm[];
    uint64_t* key = reinterpret_cast<uint64_t*>(sm);
    const int kw = (k + 31) >> 5;
    uint32_t* mbits = reinterpret_cast<uint32_t*>(sm + 8 * (size_t)k);   // [5][kw]: masks, then x signs
    const int tid = threadIdx.x;
    for (int i = tid; i < k; i += kSkPlanThreads) key[i] = sorted[i];
    for (int i = tid; i < 5 * kw; i += kSkPlanThreads) mbits[i] = 0u;
    __syncthreads();
    SketchPlan* plan = reinterpret_cast<SketchPlan*>(ws);
    const int t = min(k, kSkTop);
    const int rest = k - t, base = rest / kSkGroups;
    auto dim_of = [&](int rank) { return (int)(0xFFFFFFFFu - (uint32_t)(key[rank] & 0xFFFFFFFFu)); };
    auto group_of_rank = [&](int rank) { return base > 0 ? min((rank - t) / base, kSkGroups - 1) : kSkGroups - 1; };
    if (tid < t) {
        const int d = dim_of(tid);
        plan->top_idx[tid] = d;
        plan->top_x[tid] = x[d];
    }
    for (int rank = t + tid; rank < k; rank += kSkPlanThreads) {
        const int d = dim_of(rank);
        atomicOr(&mbits[group_of_rank(rank) * kw + (d >> 5)], 1u << (d & 31));
    }
    for (int i = tid; i < k; i += kSkPlanThreads)
        if (x[i] < 0.0f) atomicOr(&mbits[kSkGroups * kw + (i >> 5)], 1u << (i & 31));
    if (tid < kSkGroups) {
        // group sums of |x| in rank order, fp32; |x| is the high word of the sorted key
        const int lo = t + tid * base;
        const int hi = tid == kSkGroups - 1 ? k : lo + base;
        float sum = 0.0f;
        int rank = lo;
        for (; rank + 8 <= hi; rank += 8) {
            float v8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v8[j] = __uint_as_float((uint32_t)(key[rank + j] >> 32));
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += v8[j];
        }
        for (; rank < hi; ++rank) sum += __uint_as_float((uint32_t)(key[rank] >> 32));
        const float mean = hi > lo ? sum / (float)(hi - lo) : 0.0f;
        plan->n[tid] = hi - lo;
        plan->wgt[tid] = hdr->c * mean;
    }
    if (tid == 0) {
        plan->t = t;
        plan->kw = kw;
    }
    // clear the histograms for this token
    uint4* hist4 = reinterpret_cast<uint4*>(ws + kSkHistOff);
    for (int i = tid; i < kSkHistCopies * kSkBins / 4; i += kSkPlanThreads) hist4[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    uint32_t* mout = reinterpret_cast<uint32_t*>(ws + sizeof(SketchPlan));
    for (int i = tid; i < 5 * kw; i += kSkPlanThreads) mout[i] = mbits[i];
}

// A thread per row, 1024 rows per workgroup; the workgroup's histogram is
// added into private copy blockIdx % 8 (a hot bin then takes few atomics).
__global__ __launch_bounds__(kSkScoreThreads) void k_sketch_score(const uint32_t* __restrict__ signs,
                                                                  const uint16_t* __restrict__ wt, int64_t v,
                                                                  uint8_t* __restrict__ ws, float* __restrict__ scores)
{
    __shared__ uint32_t sbits[5 * 256];
    __shared__ uint32_t shist[kSkBins];
    __shared__ int32_t s_idx[kSkTop];
    __shared__ float s_x[kSkTop];
    const SketchPlan* plan = reinterpret_cast<const SketchPlan*>(ws);
    const int tid = threadIdx.x;
    const int t = plan->t, kw = plan->kw;
    const uint32_t* mbits = reinterpret_cast<const uint32_t*>(ws + sizeof(SketchPlan));
    for (int i = tid; i < 5 * kw; i += kSkScoreThreads) sbits[i] = mbits[i];
    for (int i = tid; i < kSkBins; i += kSkScoreThreads) shist[i] = 0u;
    if (tid < kSkTop) {
        s_idx[tid] = plan->top_idx[tid];
        s_x[tid] = plan->top_x[tid];
    }
    float wgt[kSkGroups];
    int32_t ng[kSkGroups];
#pragma unroll
    for (int g = 0; g < kSkGroups; ++g) {
        wgt[g] = plan->wgt[g];
        ng[g] = plan->n[g];
    }
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * kSkScoreThreads + tid;
    const bool live = r < v;
    const int64_t rr = live ? r : v - 1;   // a valid address for every lane; only live rows count
    // step 1: the exact dimensions, in rank order (loads batched, FMAs in order)
    float a = 0.0f;
    int j = 0;
    for (; j + 8 <= t; j += 8) {
        uint16_t h[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) h[u] = __builtin_nontemporal_load(&wt[(int64_t)s_idx[j + u] * v + rr]);   // read once per token
#pragma unroll
        for (int u = 0; u < 8; ++u) a = fmaf(bf16f(h[u]), s_x[j + u], a);
    }
    for (; j < t; ++j) a = fmaf(bf16f(wt[(int64_t)s_idx[j] * v + rr]), s_x[j], a);
    // step 2: sign agreement per group
    int cnt[kSkGroups] = {0, 0, 0, 0};
    int w = 0;
    for (; w + 6 <= kw; w += 6) {
        uint32_t sw6[6];
#pragma unroll
        for (int u = 0; u < 6; ++u) sw6[u] = __builtin_nontemporal_load(&signs[(int64_t)(w + u) * v + rr]);
#pragma unroll
        for (int u = 0; u < 6; ++u) {
            const uint32_t d = sw6[u] ^ sbits[kSkGroups * kw + w + u];
#pragma unroll
            for (int g = 0; g < kSkGroups; ++g) cnt[g] += __popc(d & sbits[g * kw + w + u]);
        }
    }
    for (; w < kw; ++w) {
        const uint32_t d = signs[(int64_t)w * v + rr] ^ sbits[kSkGroups * kw + w];
#pragma unroll
        for (int g = 0; g < kSkGroups; ++g) cnt[g] += __popc(d & sbits[g * kw + w]);
    }
#pragma unroll
    for (int g = 0; g < kSkGroups; ++g) a = fmaf(wgt[g], (float)(ng[g] - 2 * cnt[g]), a);
    const uint32_t key = order_key(a);
    if (live) {
        reinterpret_cast<uint32_t*>(ws + kSkKeysOff)[r] = key;
        if (scores) scores[r] = a;
        atomicAdd(&shist[key >> 20], 1u);
    }
    __syncthreads();
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + kSkHistOff) + (blockIdx.x % kSkHistCopies) * kSkBins;
    for (int i = tid; i < kSkBins; i += kSkScoreThreads)
        if (shist[i]) atomicAdd(&hist[i], shist[i]);
}

// One workgroup of 1024 threads: b*, the highest bin at which the bins from
// the top down first hold min(1024, v) words.  Thread t owns bins
// 4095 - 4t - 3 .. 4095 - 4t.
__global__ __launch_bounds__(kSkPlanThreads) void k_sketch_select(int64_t v, uint8_t* __restrict__ ws)
{
    __shared__ uint32_t ssum[kSkPlanThreads];
    const int tid = threadIdx.x;
    const uint32_t* hist = reinterpret_cast<const uint32_t*>(ws + kSkHistOff);
    const int hi_bin = kSkBins - 1 - 4 * tid;
    uint32_t hv[4] = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < kSkHistCopies; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) hv[u] += hist[c * kSkBins + hi_bin - u];
    // inclusive scan over the threads: inside each wave by shuffles, then the
    // wave totals (16 of them) in order
    __shared__ uint32_t wtot[kSkPlanThreads / kWave];
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    uint32_t x = hv[0] + hv[1] + hv[2] + hv[3];
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) wtot[wave] = x;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wtot[w];
    ssum[tid] = x + base;
    __syncthreads();
    const uint32_t need = (uint32_t)min<int64_t>(v, kSkMinCand);
    const uint32_t before = tid ? ssum[tid - 1] : 0u;
    if (before < need && ssum[tid] >= need) {
        uint32_t run = before;
        for (int u = 0; u < 4; ++u) {
            run += hv[u];
            if (run >= need) {
                reinterpret_cast<uint32_t*>(ws + kSkPickOff)[0] = (uint32_t)(hi_bin - u);
                break;
            }
        }
    }
}

// 256 threads, 1024 rows per workgroup.  Dynamic LDS: x (k floats).  Each
// workgroup writes its best (logit key << 32 | ~row) and its candidate count.
__global__ __launch_bounds__(kBlock) void k_sketch_rescore(const uint16_t* __restrict__ w, const float* __restrict__ x,
                                                           int64_t v, int k, uint8_t* __restrict__ ws)
{
    extern __shared__ __align__(16) float xs[];
    __shared__ int32_t s_n;
    __shared__ int32_t s_list[kSkRowsPerBlock];
    __shared__ unsigned long long s_best[kBlock / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t bstar = reinterpret_cast<const uint32_t*>(ws + kSkPickOff)[0];
    if (tid == 0) s_n = 0;
    if (lane == 0) s_best[wave] = 0ull;
    __syncthreads();
    // this workgroup's candidates
    const uint32_t* keys = reinterpret_cast<const uint32_t*>(ws + kSkKeysOff);
    const int64_t base = (int64_t)blockIdx.x * kSkRowsPerBlock;
    uint32_t kv4[kSkRowsPerBlock / kBlock];
#pragma unroll
    for (int i = 0; i < kSkRowsPerBlock / kBlock; ++i) {
        const int64_t r = base + tid + kBlock * i;
        kv4[i] = r < v ? keys[r] : 0u;
    }
#pragma unroll
    for (int i = 0; i < kSkRowsPerBlock / kBlock; ++i) {
        const int64_t r = base + tid + kBlock * i;
        if (r < v && (kv4[i] >> 20) >= bstar) s_list[atomicAdd(&s_n, 1)] = (int32_t)r;
    }
    __syncthreads();
    const int n = s_n;
    if (n) {
        for (int i = tid; i < k; i += kBlock) xs[i] = x[i];
        __syncthreads();
        // exact logits: one wave per candidate, 16-byte chunks over the lanes, a
        // row's loads issued together
        const int nch = k / 8;
        unsigned long long mine = 0ull;
        for (int c = wave; c < n; c += kBlock / kWave) {
            const int64_t r = s_list[c];
            const uint4* row = reinterpret_cast<const uint4*>(w + r * k);
            float s = 0.0f;
            for (int ch0 = lane; ch0 < nch; ch0 += 4 * kWave) {
                uint4 q[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) q[u] = ch0 + u * kWave < nch ? row[ch0 + u * kWave] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int ch = ch0 + u * kWave;
                    if (ch >= nch) break;
                    const float* xc = xs + 8 * ch;
                    s = fmaf(__uint_as_float(q[u].x << 16), xc[0], s);
                    s = fmaf(__uint_as_float(q[u].x & 0xFFFF0000u), xc[1], s);
                    s = fmaf(__uint_as_float(q[u].y << 16), xc[2], s);
                    s = fmaf(__uint_as_float(q[u].y & 0xFFFF0000u), xc[3], s);
                    s = fmaf(__uint_as_float(q[u].z << 16), xc[4], s);
                    s = fmaf(__uint_as_float(q[u].z & 0xFFFF0000u), xc[5], s);
                    s = fmaf(__uint_as_float(q[u].w << 16), xc[6], s);
                    s = fmaf(__uint_as_float(q[u].w & 0xFFFF0000u), xc[7], s);
                }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
            const unsigned long long kv =
                ((unsigned long long)order_key(s) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)r);
            mine = kv > mine ? kv : mine;
        }
        if (lane == 0) s_best[wave] = mine;
    }
    __syncthreads();
    if (tid == 0) {
        unsigned long long b = 0ull;
#pragma unroll
        for (int i = 0; i < kBlock / kWave; ++i) b = s_best[i] > b ? s_best[i] : b;
        reinterpret_cast<unsigned long long*>(ws + kSkWgOff)[blockIdx.x] = b;
        reinterpret_cast<uint32_t*>(ws + kSkWgOff + 8 * kSkMaxWg)[blockIdx.x] = (uint32_t)n;
    }
}

// One workgroup: the overall first maximum and the candidate count.
__global__ __launch_bounds__(kBlock) void k_sketch_final(int nwg, const uint8_t* __restrict__ ws,
                                                         int32_t* __restrict__ idx, float* __restrict__ max_logit,
                                                         int32_t* __restrict__ ncand)
{
    __shared__ unsigned long long sb[kBlock];
    __shared__ uint32_t sn[kBlock];
    const int tid = threadIdx.x;
    const unsigned long long* wb = reinterpret_cast<const unsigned long long*>(ws + kSkWgOff);
    const uint32_t* wn = reinterpret_cast<const uint32_t*>(ws + kSkWgOff + 8 * kSkMaxWg);
    unsigned long long b = 0ull;
    uint32_t n = 0;
    for (int i = tid; i < nwg; i += kBlock) {
        b = wb[i] > b ? wb[i] : b;
        n += wn[i];
    }
    sb[tid] = b;
    sn[tid] = n;
    __syncthreads();
    for (int off = kBlock / 2; off > 0; off >>= 1) {
        if (tid < off) {
            sb[tid] = sb[tid + off] > sb[tid] ? sb[tid + off] : sb[tid];
            sn[tid] += sn[tid + off];
        }
        __syncthreads();
    }
    if (tid == 0) {
        *idx = (int32_t)(0xFFFFFFFFu - (uint32_t)(sb[0] & 0xFFFFFFFFu));
        if (max_logit) *max_logit = key_value((uint32_t)(sb[0] >> 32));
        if (ncand) *ncand = (int32_t)sn[0];
    }
}

}  // namespace

// The copy's space also holds the build's row sums and block partials until
// the transpose overwrites them.
int64_t sketch_copy_bytes(int64_t v, int64_t k)
{
    const int64_t temp = sk_round(4 * v, 256) + sk_round(8 * ((v + kSkRowBlock - 1) / kSkRowBlock), 256);
    return max(sk_round(2 * k * v, 256), temp);
}

int64_t sketch_bytes(int64_t v, int64_t k)
{
    const int64_t kw = (k + 31) / 32;
    return 256 + sk_round(4 * kw * v, 256) + sketch_copy_bytes(v, k);
}

// [plan][histograms][pick][per-workgroup bests][row keys: 4 v][sorted |x| keys: 8 * kSketchMaxK]
int64_t sketch_sorted_off(int64_t v) { return kSkKeysOff + sk_round(4 * v, 256); }
int64_t sketch_workspace_bytes(int64_t v) { return sketch_sorted_off(v) + 8 * kSketchMaxK; }

hipError_t launch_sketch_build(const uint16_t* w, int64_t v, int64_t k, void* sketch, hipStream_t s)
{
    uint8_t* base = static_cast<uint8_t*>(sketch);
    const int64_t kw = (k + 31) / 32;
    uint32_t* signs = reinterpret_cast<uint32_t*>(base + 256);
    uint16_t* wt = reinterpret_cast<uint16_t*>(base + 256 + sk_round(4 * kw * v, 256));
    // the row sums and block partials live in the copy's space until the transpose
    float* rowsum = reinterpret_cast<float*>(wt);
    double* part = reinterpret_cast<double*>(reinterpret_cast<uint8_t*>(wt) + sk_round(4 * v, 256));
    hipLaunchKernelGGL(k_sketch_rows, dim3((unsigned)((v + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, w, v, (int)k,
                       signs, rowsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_scale, dim3(1), dim3(kBlock), 0, s, rowsum, v, (int)k, part,
                       reinterpret_cast<SketchHeader*>(base));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_transpose, dim3((unsigned)((v + 63) / 64), (unsigned)((k + 63) / 64)), dim3(kBlock), 0,
                       s, w, v, (int)k, wt);
    return hipGetLastError();
}

hipError_t setup_sketch_attributes()
{
    hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(&k_sketch_plan));
    if (e == hipSuccess)
        e = raise_lds_limit(reinterpret_cast<const void*>(&k_sketch_rescore));
    return e;
}

hipError_t launch_sketch_argmax(const uint16_t* w, const void* sketch, const float* x, int64_t v, int64_t k,
                                int32_t* idx, float* max_logit, int32_t* ncand, float* scores, void* workspace,
                                hipStream_t s)
{
    const uint8_t* base = static_cast<const uint8_t*>(sketch);
    const int64_t kw = (k + 31) / 32;
    const uint32_t* signs = reinterpret_cast<const uint32_t*>(base + 256);
    const uint16_t* wt = reinterpret_cast<const uint16_t*>(base + 256 + sk_round(4 * kw * v, 256));
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint64_t* sorted = reinterpret_cast<uint64_t*>(ws + sketch_sorted_off(v));
    hipLaunchKernelGGL(k_sketch_rank, dim3((unsigned)((k + kSkRankPer - 1) / kSkRankPer)), dim3(kBlock), 0, s, x,
                       (int)k, sorted);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t plan_lds = 8 * (size_t)k + 20 * (size_t)kw;
    hipLaunchKernelGGL(k_sketch_plan, dim3(1), dim3(kSkPlanThreads), plan_lds, s, x, (int)k,
                       (const uint64_t*)sorted, reinterpret_cast<const SketchHeader*>(base), ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_score, dim3((unsigned)((v + kSkScoreThreads - 1) / kSkScoreThreads)),
                       dim3(kSkScoreThreads), 0, s, signs, wt, v, ws, scores);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_select, dim3(1), dim3(kSkPlanThreads), 0, s, v, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nwg = (int)((v + kSkRowsPerBlock - 1) / kSkRowsPerBlock);
    hipLaunchKernelGGL(k_sketch_rescore, dim3((unsigned)nwg), dim3(kBlock), (size_t)(4 * k), s, w, x, v, (int)k, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sketch_final, dim3(1), dim3(kBlock), 0, s, nwg, ws, idx, max_logit, ncand);
    return hipGetLastError();
}

}  // namespace qmv
