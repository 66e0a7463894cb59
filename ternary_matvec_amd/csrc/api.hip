// api.hip -- the C ABI of libqmv: host-side validation, problem tables and
// kernel launches.  Declarations and the contract of every call are in
// include/qmv.h.
#include <qmv.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <queue>
#include <vector>

#include "qmv_internal.hpp"

using namespace qmv;

namespace {

constexpr int64_t kMaxProblems = (int64_t)1 << kTileProbBits;
constexpr int64_t kMaxInt8K = 65536;  // keeps every int8 x int8 dot inside int32
// group-scaled int8: row blocks of as few as 4 rows must fit a tile entry
constexpr int64_t kMaxGroupedN = (int64_t)4 << kTileRowBits;

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int64_t row_stride(int32_t wtype, int64_t k)
{
    if (wtype == QMV_W_TERNARY5) return round_up((k + 4) / 5, 16);
    if (wtype == QMV_W_INT8 || wtype == QMV_W_INT8_G128) return round_up(k, 16);
    return -1;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? QMV_OK : QMV_EHIP; }

int32_t check_weight(const qmv_weight& w)
{
    if (w.wtype != QMV_W_TERNARY5 && w.wtype != QMV_W_INT8 && w.wtype != QMV_W_INT8_G128) return QMV_EUNSUPPORTED;
    if (w.reserved != 0) return QMV_EINVAL;
    if (!w.data || !w.scale) return QMV_EINVAL;
    if (!aligned(w.data, 16)) return QMV_EINVAL;
    if (w.n < 1 || w.k < 1 || w.n > QMV_MAX_N || w.k > QMV_MAX_K) return QMV_ESHAPE;
    if (w.wtype == QMV_W_INT8 && w.k > kMaxInt8K) return QMV_ESHAPE;
    if (w.wtype == QMV_W_INT8_G128 &&
        (w.k > kMaxInt8K || w.n > kMaxGroupedN || w.n * row_stride(w.wtype, w.k) > INT32_MAX))
        return QMV_ESHAPE;
    return QMV_OK;
}

int32_t check_problems(const qmv_problem* probs, int32_t count, int64_t max_m)
{
    if (!probs) return QMV_EINVAL;
    if (count < 1 || count > kMaxProblems) return QMV_ESHAPE;
    for (int32_t i = 0; i < count; ++i) {
        const qmv_problem& p = probs[i];
        int32_t st = check_weight(p.w);
        if (st != QMV_OK) return st;
        if (!p.x8 || !p.sx || !p.y) return QMV_EINVAL;
        if (p.m < 1 || p.m > max_m) return QMV_ESHAPE;
        if (p.w.wtype == QMV_W_INT8_G128) {   // no single exact dot per output; activations staged in LDS
            if (p.acc) return QMV_EINVAL;
            if ((int64_t)grouped_lds_bytes(p.m, p.w.k) > kMaxLds) return QMV_ESHAPE;
        }
    }
    return QMV_OK;
}

// ---------------------------------------------------------------------------
// GEMV problem tables.
//
// Workspace image: [DevProblem x count] then, per weight type present, either
// a tile list for the workgroup kernel (64-row tiles) or a schedule for the
// streaming kernel ([nb + 1 offsets][workgroup tile entries]).  Problems are
// grouped by weight type in the table.
//
// Streaming schedule: every problem gets L lanes per row (1, 2, 4 or 8), so a
// workgroup tile is 4 * 64 / L rows.  Several L assignments are tried (each the
// smallest L that brings a problem under a target number of chunk steps); each
// is scheduled longest-processing-time-first onto the nb workgroups and the
// one with the shortest modelled makespan is kept.
// ---------------------------------------------------------------------------

#ifndef QMV_STREAM_WG_PER_CU
#define QMV_STREAM_WG_PER_CU 4
#endif
constexpr int kStreamWgPerCu = QMV_STREAM_WG_PER_CU;   // at most 16 compute waves per compute unit
constexpr int kStreamMaxM = 2;
// Token counts whose ternary problems go to the matrix-core kernel.  At one
// token the streaming dot-product kernel is faster (measured on the Gemma-3-1B
// x26 step); from two tokens the matrix cores' cost does not grow with the
// tokens while the dot products' does.
constexpr int kMxMinM = 2;
constexpr int kMxMaxM = 16;

// The kernel that serves one weight type of a launch.
enum GemvKernel { kWorkgroupDot = 0, kStreamDot = 1, kMatrixCore = 2 };

struct Table {
    std::vector<uint8_t> bytes;
    int kernel[4] = {kWorkgroupDot, kWorkgroupDot, kWorkgroupDot, kWorkgroupDot};
    int mx_tokens = 0;                     // kMatrixCore: tokens per launch (1, 2, 4 or 8)
    bool skip_zero = false;                // kStreamDot, ternary: skip zero activation units
    int64_t region[4] = {0, 0, 0, 0};      // byte offset of the type's tile list or schedule
    int32_t count[4] = {0, 0, 0, 0};       // tiles (workgroup kernels) or workgroup tiles (streaming)
    int32_t max_m[4] = {0, 0, 0, 0}, max_chunks[4] = {0, 0, 0, 0};
    int32_t nb[4] = {0, 0, 0, 0}, slot_bytes[4] = {0, 0, 0, 0};   // slot_bytes[3]: LDS of the grouped kernel
};

int32_t chunks_of(const qmv_problem& p) { return (int32_t)(row_stride(p.w.wtype, p.w.k) / 16); }

int64_t rows_tiles(int64_t n, int64_t rows) { return (n + rows - 1) / rows; }

// Upper bound of the table bytes for any device with at most `cus` compute units.
int64_t table_bound(const qmv_problem* probs, int32_t count, int cus)
{
    int64_t tiles64 = 0;
    for (int32_t i = 0; i < count; ++i) tiles64 += rows_tiles(probs[i].w.n, kRowsPerTile);
    int64_t b = round_up((int64_t)sizeof(DevProblem) * count, 256);
    (void)cus;
    // per weight type: counters, list offsets, tile entries (at most one per 64
    // rows) and the first two entries of each workgroup (no more workgroups
    // than tiles)
    for (int wt = 1; wt <= 2; ++wt) b += round_up((3 * tiles64 + kStreamHdr + 2 * kStreamXcds) * 4, 256);
    // group-scaled int8: one entry per tile of 256 / lanes_per_row rows
    int64_t gtiles = 0;
    for (int32_t i = 0; i < count; ++i)
        if (probs[i].w.wtype == QMV_W_INT8_G128)
            gtiles += rows_tiles(probs[i].w.n, kBlock / grouped_lanes_per_row(probs[i].w.k));
    b += round_up(gtiles * 4, 256);
    return b;
}

// A persistent kernel's tile model: per problem a choice (lanes per row of the
// streaming kernel, row groups per wave of the matrix-core kernel) made for a
// target number of steps per tile, the rows and modelled cost of a workgroup
// tile under that choice, and the LDS slot it needs.
struct TileModel {
    std::vector<int> targets;
    std::function<int(const qmv_problem&, int target)> choose;
    std::function<int64_t(int choice)> rows;
    std::function<double(const qmv_problem&, int choice)> cost;
    std::function<int64_t(const qmv_problem&, int choice)> slot_bytes;
    std::function<size_t(int64_t slot)> lds;
    std::function<int(int64_t slot)> wg_per_cu;   // resident workgroups per CU, 0 if unknown
    int max_wg_per_cu;
    int min_wg_per_cu;
};

struct StreamChoice {
    std::vector<int32_t> lanes;        // per table slot: the model's choice
    std::vector<uint32_t> words;       // offsets + entries
    int nb = 0;
    int64_t slot_bytes = 0;
    double makespan = 0;
};

// Schedule the problems `sp` (table slots `slots`) for a persistent kernel.
// For each distinct choice vector the tiles are dealt longest first to the 8
// XCD lists and the makespan of the kernel's dealing is modelled; the shortest
// is kept.
bool schedule_persistent(const std::vector<const qmv_problem*>& sp, const std::vector<int32_t>& slots,
                         const TileModel& model, int cus, StreamChoice& best)
{
    for (const qmv_problem* p : sp)   // the kernels size their weight buffers in 32 bits
        if ((int64_t)chunks_of(*p) * 16 * p->w.n >= ((int64_t)1 << 31)) return false;
    std::vector<std::vector<int32_t>> tried;
    bool found = false;
    for (int target : model.targets) {
        std::vector<int32_t> lanes(sp.size());
        for (size_t i = 0; i < sp.size(); ++i) lanes[i] = model.choose(*sp[i], target);
        if (std::find(tried.begin(), tried.end(), lanes) != tried.end()) continue;
        tried.push_back(lanes);
        int64_t slot = 0;
        for (size_t i = 0; i < sp.size(); ++i) slot = std::max(slot, model.slot_bytes(*sp[i], lanes[i]));
        slot = round_up(slot, 16);
        const size_t lds = model.lds(slot);
        if ((int64_t)lds > kMaxLds) continue;
        // resident workgroups per compute unit: the runtime's answer for this
        // kernel and LDS size, else (no usable device) the LDS bound
        int wg_per_cu = model.wg_per_cu(slot);
        if (wg_per_cu <= 0) wg_per_cu = (int)std::min<int64_t>(model.max_wg_per_cu, kMaxLds / (int64_t)lds);
        wg_per_cu = std::min(wg_per_cu, model.max_wg_per_cu);
        if (wg_per_cu < model.min_wg_per_cu) continue;
        // workgroup tiles, longest first
        struct Item { double cost; uint32_t entry; };
        std::vector<Item> items;
        for (size_t i = 0; i < sp.size(); ++i) {
            const qmv_problem& p = *sp[i];
            const double cost = model.cost(p, lanes[i]);
            const int64_t nt = rows_tiles(p.w.n, model.rows(lanes[i]));
            for (int64_t r = 0; r < nt; ++r)
                items.push_back({cost, ((uint32_t)slots[i] << kTileRowBits) | (uint32_t)r});
        }
        std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.cost > b.cost; });
        const int nb = (int)std::max<int64_t>(1, std::min<int64_t>((int64_t)cus * wg_per_cu, (int64_t)items.size()));
        // The kernel deals tiles per XCD: the same items, longest first, onto
        // the 8 XCD lists (each list stays longest first).
        std::vector<std::vector<uint32_t>> xl(kStreamXcds);
        std::vector<std::vector<double>> xc(kStreamXcds);
        std::vector<double> load(kStreamXcds, 0.0);
        std::vector<int> wgs(kStreamXcds);
        for (int x = 0; x < kStreamXcds; ++x) wgs[x] = (nb - x + kStreamXcds - 1) / kStreamXcds;
        for (const Item& it : items) {
            int bx = -1;
            for (int x = 0; x < kStreamXcds; ++x)   // least loaded per workgroup
                if (wgs[x] > 0 && (bx < 0 || load[x] / wgs[x] < load[bx] / wgs[bx])) bx = x;
            xl[bx].push_back(it.entry);
            xc[bx].push_back(it.cost);
            load[bx] += it.cost;
        }
        // Workgroup r of an XCD's w starts with list entries r and 2w - 1 - r
        // (the longest tiles pair with the shortest of the second w), then takes
        // the entries from 2w on by ticket, whenever it is free.  The modelled
        // makespan replays that on each list.
        double makespan = 0;
        for (int x = 0; x < kStreamXcds; ++x) {
            const size_t w = (size_t)wgs[x], sz = xc[x].size();
            std::priority_queue<double, std::vector<double>, std::greater<double>> busy;
            for (size_t r = 0; r < w; ++r)
                busy.push((r < sz ? xc[x][r] : 0.0) + (2 * w - 1 - r < sz ? xc[x][2 * w - 1 - r] : 0.0));
            for (size_t i = 2 * w; i < sz; ++i) {
                const double t = busy.top();
                busy.pop();
                busy.push(t + xc[x][i]);
            }
            while (busy.size() > 1) busy.pop();
            if (!busy.empty()) makespan = std::max(makespan, busy.top());
        }
        if (found && makespan >= best.makespan) continue;
        found = true;
        best.lanes = lanes;
        best.nb = nb;
        best.slot_bytes = slot;
        best.makespan = makespan;
        // [counters][first two entries of each workgroup][list offsets and
        // sizes][lists]; workgroup b runs on XCD b % 8, as the XCD's workgroup
        // r = b / 8 of w: its tiles are entries 2w - 1 - r and r (the shorter
        // first: the lists are longest first, and the longer one is then staged
        // while the shorter one streams), then the entries from 2w on as its
        // tickets name them
        best.words.assign(kStreamHdr + 2 * nb + 2 * kStreamXcds, 0u);
        for (int b = 0; b < nb; ++b) {
            const int x = b % kStreamXcds;
            const auto& l = xl[x];
            const size_t r = (size_t)(b / kStreamXcds), w = (size_t)wgs[x];
            const uint32_t e0 = r < l.size() ? l[r] : 0xffffffffu;
            const uint32_t e1 = 2 * w - 1 - r < l.size() ? l[2 * w - 1 - r] : 0xffffffffu;
            best.words[kStreamHdr + 2 * b] = e1 != 0xffffffffu ? e1 : e0;
            best.words[kStreamHdr + 2 * b + 1] = e1 != 0xffffffffu ? e0 : e1;
        }
        uint32_t off = 0;
        for (int x = 0; x < kStreamXcds; ++x) {
            best.words[kStreamHdr + 2 * nb + 2 * x] = off;
            best.words[kStreamHdr + 2 * nb + 2 * x + 1] = (uint32_t)xl[x].size();
            off += (uint32_t)xl[x].size();
        }
        for (int x = 0; x < kStreamXcds; ++x) best.words.insert(best.words.end(), xl[x].begin(), xl[x].end());
    }
    return found;
}

// The streaming dot-product kernel (1..2 tokens): L lanes per row, a
// workgroup tile of 4 * 64 / L * kStreamRowsPerLane rows.
TileModel stream_model(int wtype, int mt, bool skip)
{
    TileModel m;
    m.targets = {4, 6, 8, 12, 16, 24, 32, 48, 64, 1 << 30};
    m.choose = [](const qmv_problem& p, int target) {
        const int c = chunks_of(p);
        int L = 1;
        while (L < kStreamMaxLanes && gemv_stream_steps(c, L) > target) L *= 2;
        return L;
    };
    m.rows = [](int L) { return (int64_t)4 * (kRowsPerTile / L) * kStreamRowsPerLane; };
    // chunk steps (an int8 step is a quarter of a ternary one) plus the tile
    // boundary (barrier, epilogue, ring refill), which measures at about six
    // ternary steps
    m.cost = [wtype](const qmv_problem& p, int L) {
        return ((double)gemv_stream_steps(chunks_of(p), L) * (wtype == 1 ? p.m : 0.3 * p.m) + 6.0) *
               kStreamRowsPerLane;
    };
    m.slot_bytes = [wtype, mt](const qmv_problem& p, int L) {
        return gemv_stream_slot_bytes(wtype, mt, chunks_of(p), L);
    };
    m.lds = [mt](int64_t slot) { return gemv_stream_lds_bytes(mt, slot); };
    m.wg_per_cu = [wtype, mt, skip](int64_t slot) { return gemv_stream_wg_per_cu(wtype, mt, slot, skip); };
    m.max_wg_per_cu = kStreamWgPerCu;
    m.min_wg_per_cu = 1;
    return m;
}

// The matrix-core kernel (ternary, 2..16 tokens): a workgroup tile of compute
// waves x rgs row groups of 16 rows over all of K; a step is one K range (4
// chunks) of one row group, 1 KiB of weights per wave.
TileModel mx_model(int mt)
{
    TileModel m;
    const int rgs = gemv_mx_row_groups(mt);
    m.targets = {0};
    m.choose = [rgs](const qmv_problem&, int) { return rgs; };
    m.rows = [mt](int) { return gemv_mx_tile_rows(mt); };
    // steps (padded to a multiple of the register ring) plus about two steps
    // of tile boundary
    m.cost = [mt, rgs](const qmv_problem& p, int) {
        const int steps = (chunks_of(p) + 3) / 4 * rgs;
        const int ring = gemv_mx_ring(mt);
        return (double)((steps + ring - 1) / ring * ring) + 2.0;
    };
    m.slot_bytes = [mt](const qmv_problem& p, int) { return gemv_mx_slot_bytes(mt, chunks_of(p)); };
    m.lds = [mt](int64_t slot) { return gemv_mx_lds_bytes(mt, slot); };
    m.wg_per_cu = [mt](int64_t slot) { return gemv_mx_wg_per_cu(mt, slot); };
    m.max_wg_per_cu = kStreamWgPerCu;
    m.min_wg_per_cu = 1;
    return m;
}

// Builds the table; returns QMV_OK or a status.  With allow_mx, ternary
// problems of 2..16 tokens go to the matrix-core kernel (when its LDS slots fit); with skip_zero,
// ternary problems of one or two tokens go to the streaming kernel that skips
// zero activation units.
int32_t build_table(const qmv_problem* probs, int32_t count, int cus, bool allow_mx, bool skip_zero, Table& t)
{
    std::vector<int32_t> order(count);
    for (int32_t i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return probs[a].w.wtype < probs[b].w.wtype; });
    for (int32_t i = 0; i < count; ++i) {
        const int32_t wt = probs[i].w.wtype;
        t.max_m[wt] = std::max<int32_t>(t.max_m[wt], (int32_t)probs[i].m);
        t.max_chunks[wt] = std::max<int32_t>(t.max_chunks[wt], chunks_of(probs[i]));
    }
    const int64_t pbytes = round_up((int64_t)sizeof(DevProblem) * count, 256);
    std::vector<int32_t> lanes(count, 1);             // per table slot
    std::vector<uint32_t> words[4];
    for (int wt = 1; wt <= 2; ++wt) {
        if (t.max_m[wt] == 0) continue;
        std::vector<const qmv_problem*> sp;
        std::vector<int32_t> slots;
        for (int32_t slot = 0; slot < count; ++slot)
            if (probs[order[slot]].w.wtype == wt) {
                sp.push_back(&probs[order[slot]]);
                slots.push_back(slot);
            }
        StreamChoice ch;
        const int mxt = gemv_mx_tokens(t.max_m[wt]);
        bool ok = false;
        if (wt == QMV_W_TERNARY5 && allow_mx && t.max_m[wt] >= kMxMinM && t.max_m[wt] <= kMxMaxM && mxt > 0 &&
            schedule_persistent(sp, slots, mx_model(mxt), cus, ch)) {
            t.kernel[wt] = kMatrixCore;
            t.mx_tokens = mxt;
            ok = true;
        } else if (t.max_m[wt] <= kStreamMaxM &&
                   schedule_persistent(sp, slots,
                                       stream_model(wt, t.max_m[wt] <= 1 ? 1 : 2, skip_zero && wt == QMV_W_TERNARY5),
                                       cus, ch)) {
            t.kernel[wt] = kStreamDot;
            t.skip_zero = skip_zero && wt == QMV_W_TERNARY5;
            ok = true;
        }
        if (ok) {
            t.nb[wt] = ch.nb;
            t.slot_bytes[wt] = (int32_t)ch.slot_bytes;
            t.count[wt] = (int32_t)(ch.words.size() - kStreamHdr - 2 * ch.nb - 2 * kStreamXcds);
            for (size_t i = 0; i < slots.size(); ++i) lanes[slots[i]] = ch.lanes[i];
            words[wt] = std::move(ch.words);
        } else {
            if (gemv_lds_bytes(wt, t.max_m[wt], t.max_chunks[wt]) > kMaxLds) return QMV_ESHAPE;
            for (size_t i = 0; i < sp.size(); ++i) {
                const int64_t nt = rows_tiles(sp[i]->w.n, gemv_rows_per_tile(wt, t.max_m[wt]));
                for (int64_t r = 0; r < nt; ++r) words[wt].push_back(((uint32_t)slots[i] << kTileRowBits) | (uint32_t)r);
            }
            t.count[wt] = (int32_t)words[wt].size();
        }
    }
    if (t.max_m[QMV_W_INT8_G128] > 0) {   // group-scaled int8: one workgroup per tile
        size_t lds = 0;
        for (int32_t slot = 0; slot < count; ++slot) {
            const qmv_problem& p = probs[order[slot]];
            if (p.w.wtype != QMV_W_INT8_G128) continue;
            lanes[slot] = grouped_lanes_per_row(p.w.k);
            const int64_t nt = rows_tiles(p.w.n, kBlock / lanes[slot]);
            for (int64_t r = 0; r < nt; ++r)
                words[QMV_W_INT8_G128].push_back(((uint32_t)slot << kTileRowBits) | (uint32_t)r);
            lds = std::max(lds, grouped_lds_bytes(p.m, p.w.k));
        }
        t.count[QMV_W_INT8_G128] = (int32_t)words[QMV_W_INT8_G128].size();
        t.slot_bytes[QMV_W_INT8_G128] = (int32_t)lds;
    }
    int64_t total = pbytes;
    for (int wt = 1; wt <= 3; ++wt) {
        t.region[wt] = total;
        total += round_up((int64_t)words[wt].size() * 4, 256);
    }
    t.bytes.assign(total, 0);
    DevProblem* dp = reinterpret_cast<DevProblem*>(t.bytes.data());
    for (int32_t slot = 0; slot < count; ++slot) {
        const qmv_problem& p = probs[order[slot]];
        DevProblem& d = dp[slot];
        d.w = static_cast<const uint8_t*>(p.w.data);
        d.sw = p.w.scale;
        d.x8 = p.x8;
        d.sx = p.sx;
        d.y = p.y;
        d.acc = p.acc;
        d.n = (int32_t)p.w.n;
        d.k = (int32_t)p.w.k;
        d.m = (int32_t)p.m;
        d.chunks = chunks_of(p);
        d.tile_begin = 0;
        d.wtype = p.w.wtype;
        d.lanes_per_row = lanes[slot];
        d.reserved = 0;
    }
    for (int wt = 1; wt <= 3; ++wt)
        if (!words[wt].empty())
            std::memcpy(t.bytes.data() + t.region[wt], words[wt].data(), words[wt].size() * 4);
    return QMV_OK;
}

// ---------------------------------------------------------------------------
// Per-device set-up, done once per device on first use: the compute-unit
// count, the kernels' dynamic-LDS limit raised to the whole 160 KB (launches
// then never set attributes), and the device address of `scratch`.
// ---------------------------------------------------------------------------

constexpr int kMaxDevices = 64;

constexpr int64_t kStaticScratchBytes = 256 * 1024;

}  // namespace

// The scratch of qmv_lmhead_argmax_static (the output layer's per-workgroup
// maxima): one copy per device.  Host code never uses this name as an
// address: device_setup takes each device's address once, and the entry point
// passes that.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

struct DeviceSetup {
    std::once_flag once;
    int32_t status = QMV_EHIP;
    int cus = 0;
    void* scratch = nullptr;   // device address of `scratch` on this device (null: not found)
    int ffn_grid = 0;          // workgroups of a qmv_ffn_decode launch (0: cannot run)
};

DeviceSetup g_devices[kMaxDevices];

// The current device's record (set up on first use), or null with no usable
// device.
const DeviceSetup* device_setup(int* dev_out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceSetup& d = g_devices[dev];
    std::call_once(d.once, [&d, dev] {
        int cus = 0;
        hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess && cus < 1) e = hipErrorInvalidDevice;
        if (e == hipSuccess) e = setup_workgroup_gemv_attributes();
        if (e == hipSuccess) e = setup_stream_attributes();
        if (e == hipSuccess) e = setup_mx_attributes();
        if (e == hipSuccess) e = setup_grouped_attributes();
        if (e == hipSuccess) e = setup_prefill_attributes();
        if (e == hipSuccess) e = setup_sketch_attributes();
        if (e == hipSuccess) e = setup_ffn_attributes();
        if (e == hipSuccess) {
            // residency of the largest feed-forward launch decides the grid of all
            const int64_t cg = row_stride(QMV_W_TERNARY5, QMV_FFN_MAX_HIDDEN) / 16;
            const int occ = ffn_max_wg_per_cu(ffn_lds_bytes(QMV_FFN_MAX_HIDDEN, cg));
            d.ffn_grid = cus * std::min(occ, kFfnWgPerCu);
        }
        // the scratch address only serves qmv_lmhead_argmax_static, which
        // refuses to run without it
        void* p = nullptr;
        if (e == hipSuccess && hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
        d.cus = cus;
        d.scratch = p;
        d.status = e == hipSuccess ? QMV_OK : QMV_EHIP;
    });
    if (d.status != QMV_OK) return nullptr;
    if (dev_out) *dev_out = dev;
    return &d;
}

// Workspace layout of qmv_ffn_decode: sized for any grid (down tasks number
// at most one per kFfnComputeWaves chunks of a 64-row group).
FfnLayout ffn_layout(int64_t hidden, int64_t inter)
{
    FfnLayout o;
    const int64_t cd = row_stride(QMV_W_TERNARY5, inter) / 16;
    const int64_t dn_cap = ((hidden + 63) / 64) * ((cd + kFfnComputeWaves - 1) / kFfnComputeWaves);
    const int64_t gu = (inter + 31) / 32;
    o.hp = round_up(hidden, 64);
    o.done_rep = round_up(4 * dn_cap, 4096);
    o.pmax_rep = round_up(2 * 8 * round_up(gu, 2), 4096);
    o.done = kFfnCtrlBytes;
    o.pmax = o.done + kFfnReplicas * o.done_rep;
    o.glu = o.pmax + kFfnReplicas * o.pmax_rep;
    o.acc = o.glu + round_up(8 * inter, 256);
    o.bytes = o.acc + 2 * 4 * o.hp;
    return o;
}

int64_t ffn_workspace(int64_t hidden, int64_t inter) { return ffn_layout(hidden, inter).bytes; }

int32_t check_ffn_layer(const qmv_ffn_layer& y, int64_t hidden, int64_t inter)
{
    const qmv_weight* ws[3] = {&y.gate, &y.up, &y.down};
    for (const qmv_weight* w : ws) {
        const int32_t st = check_weight(*w);
        if (st != QMV_OK) return st;
        if (w->wtype != QMV_W_TERNARY5) return QMV_EUNSUPPORTED;
    }
    if (y.gate.n != inter || y.gate.k != hidden || y.up.n != inter || y.up.k != hidden || y.down.n != hidden ||
        y.down.k != inter)
        return QMV_ESHAPE;
    if (!y.norm) return QMV_EINVAL;
    return QMV_OK;
}

constexpr int64_t kMaxPrefillM = 65536;

int32_t check_prefill(const qmv_problem* probs, int32_t count)
{
    int32_t st = check_problems(probs, count, kMaxPrefillM);
    if (st != QMV_OK) return st;
    for (int32_t i = 0; i < count; ++i)
        if (probs[i].w.wtype != QMV_W_TERNARY5) return QMV_EUNSUPPORTED;
    return QMV_OK;
}


// Workspace of a prefill problem list: the problem table, the tile table (9
// list offsets, every tile once, then the tickets) and a block of zeros the
// kernel copies for activation columns past k.
int64_t prefill_table_bytes(const qmv_problem* probs, int32_t count)
{
    int64_t tiles = 0;
    for (int32_t i = 0; i < count; ++i) tiles += prefill_tiles(probs[i].m, probs[i].w.n);
    return round_up((int64_t)sizeof(DevProblem) * count, 256) +
           round_up((kXcds + 1 + tiles + kPrefillTicketWords) * 8, 256) + kPrefillZeroBytes;
}

// The prefill workspace image: the problem table (longest rows first), the
// tile table and its zeroed tickets, and the block of zeros; `grid` is the
// persistent workgroup count.
int32_t build_prefill_image(const qmv_problem* probs, int32_t count, int cus, std::vector<uint8_t>& img,
                            int64_t& pbytes, int64_t& grid)
{
    const int64_t need = prefill_table_bytes(probs, count);
    std::vector<int32_t> order(count);
    for (int32_t i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return probs[a].w.k > probs[b].w.k; });
    pbytes = round_up((int64_t)sizeof(DevProblem) * count, 256);
    img.assign(need, 0);
    DevProblem* dp = reinterpret_cast<DevProblem*>(img.data());
    // Tile list, XCD-aware: workgroup b runs on XCD b % 8 (round-robin dispatch).
    // All tiles of a problem go to one XCD's list, row block major (its token
    // blocks side by side), so the tiles in flight on an XCD share both their
    // weight row blocks and their activation blocks in that XCD's L2: a weight
    // row block is fetched once per pass instead of once per token block.  The
    // problems are spread over the XCDs longest first, to the least loaded one.
    struct Prob {
        int32_t slot;
        int64_t mts, nts, work;
    };
    std::vector<Prob> pr;
    for (int32_t slot = 0; slot < count; ++slot) {
        const qmv_problem& p = probs[order[slot]];
        DevProblem& d = dp[slot];
        d.w = static_cast<const uint8_t*>(p.w.data);
        d.sw = p.w.scale;
        d.x8 = p.x8;
        d.sx = p.sx;
        d.y = p.y;
        d.acc = p.acc;
        d.n = (int32_t)p.w.n;
        d.k = (int32_t)p.w.k;
        d.m = (int32_t)p.m;
        d.chunks = (int32_t)(row_stride(p.w.wtype, p.w.k) / 16);
        d.tile_begin = 0;
        d.wtype = p.w.wtype;
        d.lanes_per_row = 1;
        d.reserved = 0;
        const int64_t mts = (p.m + kPrefillTileM - 1) / kPrefillTileM;
        const int64_t nts = (p.w.n + kPrefillTileN - 1) / kPrefillTileN;
        pr.push_back({slot, mts, nts, mts * nts * ((d.chunks + 1) / 2)});
    }
    std::stable_sort(pr.begin(), pr.end(), [](const Prob& a, const Prob& b) { return a.work > b.work; });
    std::vector<std::vector<uint64_t>> lists(kXcds);
    std::vector<int64_t> load(kXcds, 0);
    for (const Prob& q : pr) {
        int x = 0;
        for (int i = 1; i < kXcds; ++i)
            if (load[i] < load[x]) x = i;
        load[x] += q.work;
        for (int64_t nt = 0; nt < q.nts; ++nt)
            for (int64_t mt = 0; mt < q.mts; ++mt)
                lists[x].push_back(((uint64_t)q.slot << 48) | ((uint64_t)mt << 32) | (uint64_t)nt);
    }
    // Persistent workgroups, two per compute unit: each starts on its XCD's
    // list and takes tiles by ticket (the tickets follow the entries and start
    // at zero; the kernel leaves them at zero).
    size_t longest = 0, total = 0;
    for (const auto& l : lists) {
        longest = std::max(longest, l.size());
        total += l.size();
    }
    const int64_t per_xcd =
        std::max<int64_t>(1, std::min<int64_t>({2 * std::max(1, cus / kXcds), kPrefillMaxGrid / kXcds, (int64_t)longest}));
    grid = per_xcd * kXcds;
    if (pbytes + (kXcds + 1 + (int64_t)total + kPrefillTicketWords) * 8 > need - kPrefillZeroBytes)
        return QMV_EWORKSPACE;  // cannot happen: need covers every tile
    uint64_t* tt = reinterpret_cast<uint64_t*>(img.data() + pbytes);
    uint64_t pos = 0;
    for (int x = 0; x < kXcds; ++x) {
        tt[x] = pos;
        for (uint64_t e : lists[x]) tt[kXcds + 1 + pos++] = e;
    }
    tt[kXcds] = pos;
    return QMV_OK;
}

constexpr int kNoDevice = -1;

}  // namespace

// A launch plan: the workspace image of one problem list and the launch
// parameters, made for one device.
struct qmv_plan {
    int32_t kind = 0;
    int dev = kNoDevice;            // device the plan was made for (kNoDevice: none usable)
    std::vector<uint8_t> image;     // uploaded into the workspace
    Table table;                    // QMV_PLAN_GEMV: launch parameters per weight type
    int64_t pbytes = 0, grid = 0;   // QMV_PLAN_PREFILL: tile table offset, persistent grid
};

namespace {

// A plan for the current device; with no usable device it is made for a
// 256-CU part and cannot be uploaded or launched.
int32_t make_plan(int32_t kind, const qmv_problem* probs, int32_t count, qmv_plan& plan)
{
    int dev = kNoDevice;
    const DeviceSetup* d = device_setup(&dev);
    const int cus = d ? d->cus : 256;
    plan.kind = kind;
    plan.dev = d ? dev : kNoDevice;
    if (kind == QMV_PLAN_GEMV || kind == QMV_PLAN_GEMV_DOT || kind == QMV_PLAN_GEMV_SKIP_ZERO) {
        const int32_t st =
            build_table(probs, count, cus, kind == QMV_PLAN_GEMV, kind == QMV_PLAN_GEMV_SKIP_ZERO, plan.table);
        if (st != QMV_OK) return st;
        plan.image.swap(plan.table.bytes);
        return QMV_OK;
    }
    return build_prefill_image(probs, count, cus, plan.image, plan.pbytes, plan.grid);
}

int32_t check_plan_use(const qmv_plan* plan, const void* workspace, int64_t ws_bytes)
{
    if (!plan) return QMV_EINVAL;
    if (!workspace || !aligned(workspace, 256) || ws_bytes < (int64_t)plan->image.size()) return QMV_EWORKSPACE;
    if (plan->dev == kNoDevice) return QMV_EHIP;
    return QMV_OK;
}

int32_t upload_plan(const qmv_plan& plan, void* workspace, hipStream_t s)
{
    return hip_status(hipMemcpyAsync(workspace, plan.image.data(), plan.image.size(), hipMemcpyHostToDevice, s));
}

int32_t launch_plan(const qmv_plan& plan, void* workspace, hipStream_t s)
{
    uint8_t* base = static_cast<uint8_t*>(workspace);
    if (plan.kind == QMV_PLAN_PREFILL)
        return hip_status(launch_prefill(reinterpret_cast<const DevProblem*>(base),
                                         reinterpret_cast<const uint64_t*>(base + plan.pbytes), plan.grid,
                                         reinterpret_cast<const int8_t*>(base + plan.image.size() - kPrefillZeroBytes),
                                         s));
    const Table& t = plan.table;
    const DevProblem* dp = reinterpret_cast<const DevProblem*>(base);
    for (int wt = 1; wt <= 3; ++wt) {
        if (t.count[wt] == 0) continue;
        uint32_t* words = reinterpret_cast<uint32_t*>(base + t.region[wt]);
        hipError_t e;
        if (wt == QMV_W_INT8_G128)
            e = launch_gemv_grouped(dp, words, t.count[wt], t.max_m[wt], (size_t)t.slot_bytes[wt], s);
        else if (t.kernel[wt] == kMatrixCore)
            e = launch_gemv_mx(dp, words, t.nb[wt], t.mx_tokens, t.slot_bytes[wt], s);
        else if (t.kernel[wt] == kStreamDot)
            e = launch_gemv_stream(dp, words, t.nb[wt], wt, t.max_m[wt], t.slot_bytes[wt],
                                   wt == QMV_W_TERNARY5 && t.skip_zero, s);
        else
            e = launch_gemv(dp, words, 0, t.count[wt], wt, t.max_m[wt], t.max_chunks[wt], s);
        if (e != hipSuccess) return QMV_EHIP;
    }
    return QMV_OK;
}

// A plan made, uploaded and launched in one call (qmv_gemv, qmv_gemm_prefill).
// The upload copies from pageable host memory that is freed on return, which
// a stream capture would keep a pointer to: such calls are refused while the
// stream is capturing.
int32_t one_shot(int32_t kind, const qmv_problem* probs, int32_t count, void* workspace, int64_t ws_bytes,
                 int64_t bound, void* stream)
{
    if (!workspace || !aligned(workspace, 256) || ws_bytes < bound) return QMV_EWORKSPACE;
    const hipStream_t s = as_stream(stream);
    qmv_plan plan;
    int32_t st = make_plan(kind, probs, count, plan);
    if (st != QMV_OK) return st;
    st = check_plan_use(&plan, workspace, ws_bytes);
    if (st != QMV_OK) return st;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return QMV_EHIP;
    if (cap != hipStreamCaptureStatusNone) return QMV_EUNSUPPORTED;
    st = upload_plan(plan, workspace, s);
    return st != QMV_OK ? st : launch_plan(plan, workspace, s);
}

}  // namespace

extern "C" {

const char* qmv_version(void) { return "qmv 0.1 (gfx950)"; }

const char* qmv_status_str(int32_t status)
{
    switch (status) {
        case QMV_OK: return "ok";
        case QMV_EINVAL: return "invalid argument";
        case QMV_ESHAPE: return "bad or unsupported shape";
        case QMV_EVALUE: return "value out of range";
        case QMV_EHIP: return "HIP runtime error";
        case QMV_EUNSUPPORTED: return "unsupported weight type";
        case QMV_EWORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

int64_t qmv_packed_bytes(int32_t wtype, int64_t n, int64_t k)
{
    if (n < 1 || k < 1 || n > QMV_MAX_N || k > QMV_MAX_K) return -1;
    const int64_t s = row_stride(wtype, k);
    return s < 0 ? -1 : n * s;
}

int32_t qmv_pack_ternary(const int8_t* trits, int64_t n, int64_t k, float scale, void* packed, float* scale_out,
                         int32_t* bad_count, qmv_weight* desc_out, void* stream)
{
    if (!trits || !packed || !scale_out) return QMV_EINVAL;
    if (n < 1 || k < 1 || n > QMV_MAX_N || k > QMV_MAX_K) return QMV_ESHAPE;
    if (!aligned(packed, 16)) return QMV_EINVAL;
    if (!std::isfinite(scale)) return QMV_EVALUE;
    const hipStream_t s = as_stream(stream);
    const int64_t chunks = row_stride(QMV_W_TERNARY5, k) / 16;
    hipError_t e = launch_fill_pack_header(scale_out, scale, bad_count, s);
    if (e == hipSuccess) e = launch_pack_ternary(trits, n, k, chunks, static_cast<uint8_t*>(packed), bad_count, s);
    if (e != hipSuccess) return QMV_EHIP;
    if (desc_out) {
        desc_out->wtype = QMV_W_TERNARY5;
        desc_out->reserved = 0;
        desc_out->n = n;
        desc_out->k = k;
        desc_out->data = packed;
        desc_out->scale = scale_out;
    }
    return QMV_OK;
}

int32_t qmv_pack_int8(const float* w, int64_t n, int64_t k, void* packed, float* scale_out, qmv_weight* desc_out,
                      void* stream)
{
    if (!w || !packed || !scale_out) return QMV_EINVAL;
    if (n < 1 || k < 1 || n > QMV_MAX_N || k > kMaxInt8K) return QMV_ESHAPE;
    if (!aligned(packed, 16)) return QMV_EINVAL;
    const int64_t chunks = row_stride(QMV_W_INT8, k) / 16;
    hipError_t e = launch_pack_int8(w, n, k, chunks, static_cast<int8_t*>(packed), scale_out, as_stream(stream));
    if (e != hipSuccess) return QMV_EHIP;
    if (desc_out) {
        desc_out->wtype = QMV_W_INT8;
        desc_out->reserved = 0;
        desc_out->n = n;
        desc_out->k = k;
        desc_out->data = packed;
        desc_out->scale = scale_out;
    }
    return QMV_OK;
}

int32_t qmv_pack_int8_grouped(const float* w, int64_t n, int64_t k, void* packed, float* scales,
                              qmv_weight* desc_out, void* stream)
{
    if (!w || !packed || !scales) return QMV_EINVAL;
    if (n < 1 || k < 1 || n > kMaxGroupedN || k > kMaxInt8K) return QMV_ESHAPE;
    if (n * row_stride(QMV_W_INT8_G128, k) > INT32_MAX) return QMV_ESHAPE;
    if (!aligned(packed, 16)) return QMV_EINVAL;
    hipError_t e = launch_quantize_groups(w, n, k, QMV_WEIGHT_GROUP, row_stride(QMV_W_INT8_G128, k),
                                          static_cast<int8_t*>(packed), scales, as_stream(stream));
    if (e != hipSuccess) return QMV_EHIP;
    if (desc_out) {
        desc_out->wtype = QMV_W_INT8_G128;
        desc_out->reserved = 0;
        desc_out->n = n;
        desc_out->k = k;
        desc_out->data = packed;
        desc_out->scale = scales;
    }
    return QMV_OK;
}

int32_t qmv_quantize_act_grouped(const float* x, int64_t m, int64_t k, int8_t* x8, float* sx, void* stream)
{
    if (!x || !x8 || !sx) return QMV_EINVAL;
    if (m < 1 || k < 1 || k > QMV_MAX_K || m > ((int64_t)1 << 31) - 1 || m * ((k + 31) / 32) > INT32_MAX)
        return QMV_ESHAPE;
    return hip_status(launch_quantize_groups(x, m, k, QMV_ACT_GROUP, k, x8, sx, as_stream(stream)));
}

int32_t qmv_quantize_act_many(const qmv_act* acts, int32_t count, void* stream)
{
    if (!acts) return QMV_EINVAL;
    if (count < 1 || count > QMV_MAX_ACT_SETS) return QMV_ESHAPE;
    static_assert(QMV_MAX_ACT_SETS == kMaxActSets, "activation set count");
    ActSets sets{};
    int64_t rows = 0;
    for (int32_t i = 0; i < count; ++i) {
        const qmv_act& a = acts[i];
        if (!a.x || !a.x8 || !a.sx) return QMV_EINVAL;
        if (a.m < 1 || a.k < 1 || a.k > QMV_MAX_K) return QMV_ESHAPE;
        sets.set[i] = ActSet{a.x, a.x8, a.sx, a.k};
        sets.first[i] = rows;
        rows += a.m;
        if (rows > ((int64_t)1 << 31) - 1) return QMV_ESHAPE;
    }
    sets.first[count] = rows;
    sets.count = count;
    return hip_status(launch_quantize_many(sets, rows, as_stream(stream)));
}

int32_t qmv_quantize_act(const float* x, int64_t m, int64_t k, int8_t* x8, float* sx, void* stream)
{
    if (!x || !x8 || !sx) return QMV_EINVAL;
    if (m < 1 || k < 1 || k > QMV_MAX_K || m > ((int64_t)1 << 31) - 1) return QMV_ESHAPE;
    return hip_status(launch_quantize_rows(x, m, k, x8, sx, as_stream(stream)));
}

int32_t qmv_rmsnorm_quantize(const float* x, const float* weight, int64_t m, int64_t k, float eps, int8_t* x8,
                             float* sx, void* stream)
{
    if (!x || !weight || !x8 || !sx) return QMV_EINVAL;
    if (m < 1 || k < 1 || k > QMV_MAX_K || m > ((int64_t)1 << 31) - 1) return QMV_ESHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return QMV_EVALUE;
    return hip_status(launch_rmsnorm_quantize(x, weight, m, k, eps, x8, sx, as_stream(stream)));
}

int32_t qmv_glu_quantize(const float* gate, const float* up, int64_t m, int64_t n, int32_t act, int8_t* x8, float* sx,
                         void* stream)
{
    if (!gate || !up || !x8 || !sx) return QMV_EINVAL;
    if (m < 1 || n < 1 || n > QMV_MAX_K || m > ((int64_t)1 << 31) - 1) return QMV_ESHAPE;
    if (act != QMV_ACT_GELU_TANH && act != QMV_ACT_SILU) return QMV_EINVAL;
    return hip_status(launch_glu_quantize(gate, up, m, n, act, x8, sx, as_stream(stream)));
}

int64_t qmv_ffn_workspace_bytes(int64_t hidden, int64_t inter)
{
    if (hidden < 1 || hidden > QMV_FFN_MAX_HIDDEN || inter < 1 || inter > QMV_FFN_MAX_INTER) return -1;
    return ffn_workspace(hidden, inter);
}

int32_t qmv_ffn_grid(int32_t* grid)
{
    if (!grid) return QMV_EINVAL;
    const DeviceSetup* d = device_setup(nullptr);
    if (!d) return QMV_EHIP;
    if (d->ffn_grid < 1) return QMV_EUNSUPPORTED;
    *grid = d->ffn_grid;
    return QMV_OK;
}

int32_t qmv_ffn_decode(const qmv_ffn_layer* layers, int32_t nlayers, float* h, float eps, int32_t act,
                       void* workspace, int64_t ws_bytes, const int32_t* cancel, int64_t spin_limit,
                       int32_t* status, uint64_t* trace, void* stream)
{
    if (!layers || !h || !status) return QMV_EINVAL;
    if (nlayers < 1) return QMV_ESHAPE;
    const int64_t hidden = layers[0].gate.k, inter = layers[0].gate.n;
    if (hidden < 1 || hidden > QMV_FFN_MAX_HIDDEN || inter < 1 || inter > QMV_FFN_MAX_INTER) return QMV_ESHAPE;
    for (int32_t l = 0; l < nlayers; ++l) {
        const int32_t st = check_ffn_layer(layers[l], hidden, inter);
        if (st != QMV_OK) return st;
    }
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return QMV_EVALUE;
    if (act != QMV_ACT_GELU_TANH && act != QMV_ACT_SILU) return QMV_EINVAL;
    if (spin_limit < 0) return QMV_EVALUE;
    if (trace && nlayers > QMV_FFN_LAUNCH_LAYERS) return QMV_EINVAL;
    if (!workspace || !aligned(workspace, 256) || ws_bytes < ffn_workspace(hidden, inter)) return QMV_EWORKSPACE;
    const DeviceSetup* d = device_setup(nullptr);
    if (!d) return QMV_EHIP;
    if (d->ffn_grid < 1) return QMV_EUNSUPPORTED;
    FfnLaunch f{};
    f.h = h;
    f.hidden = hidden;
    f.inter = inter;
    f.cg = row_stride(QMV_W_TERNARY5, hidden) / 16;
    f.cd = row_stride(QMV_W_TERNARY5, inter) / 16;
    // every workgroup takes gate/up tasks (32 rows of both) and down tasks (64
    // rows x runs of W * dcs chunks, W compute waves, dcs <= kFfnDownChunks), one
    // of each where the grid allows
    const int64_t grid = d->ffn_grid;
    const int64_t W = kFfnComputeWaves;
    f.gu_tasks = (int32_t)((inter + 31) / 32);
    const int64_t groups = (hidden + 63) / 64;
    const int64_t dcs = std::min<int64_t>(kFfnDownChunks, std::max<int64_t>(1, (groups * f.cd + W * grid - 1) / (W * grid)));
    f.dcs = (int32_t)dcs;
    f.dparts = (int32_t)((f.cd + W * dcs - 1) / (W * dcs));
    f.dn_tasks = (int32_t)(groups * f.dparts);
    f.layout = ffn_layout(hidden, inter);
    f.act = act;
    f.eps = eps;
    f.workspace = workspace;
    f.cancel = cancel;
    f.status = status;
    f.trace = trace;
    f.spin_limit = spin_limit;
    f.grid = (int32_t)grid;
    f.lds = ffn_lds_bytes(hidden, f.cg);
    const hipStream_t s = as_stream(stream);
    for (int32_t l0 = 0; l0 < nlayers; l0 += QMV_FFN_LAUNCH_LAYERS) {
        f.layers = layers + l0;
        f.nlayers = std::min<int32_t>(QMV_FFN_LAUNCH_LAYERS, nlayers - l0);
        f.first_launch = l0 == 0;
        const hipError_t e = launch_ffn(f, s);
        if (e != hipSuccess) return QMV_EHIP;
    }
    return QMV_OK;
}

int64_t qmv_gemv_workspace_bytes(const qmv_problem* probs, int32_t count)
{
    if (check_problems(probs, count, QMV_MAX_GEMV_M) != QMV_OK) return -1;
    return table_bound(probs, count, 0);
}

int64_t qmv_prefill_workspace_bytes(const qmv_problem* probs, int32_t count)
{
    if (check_prefill(probs, count) != QMV_OK) return -1;
    return prefill_table_bytes(probs, count);
}

int64_t qmv_workspace_bytes(const qmv_problem* probs, int32_t count)
{
    const int64_t g = qmv_gemv_workspace_bytes(probs, count);
    const int64_t p = qmv_prefill_workspace_bytes(probs, count);
    return std::max(g, p);
}

int32_t qmv_gemv(const qmv_problem* probs, int32_t count, void* workspace, int64_t ws_bytes, void* stream)
{
    const int32_t st = check_problems(probs, count, QMV_MAX_GEMV_M);
    if (st != QMV_OK) return st;
    return one_shot(QMV_PLAN_GEMV, probs, count, workspace, ws_bytes, table_bound(probs, count, 0), stream);
}

int32_t qmv_gemm_prefill(const qmv_problem* probs, int32_t count, void* workspace, int64_t ws_bytes, void* stream)
{
    const int32_t st = check_prefill(probs, count);
    if (st != QMV_OK) return st;
    return one_shot(QMV_PLAN_PREFILL, probs, count, workspace, ws_bytes, prefill_table_bytes(probs, count), stream);
}

int32_t qmv_plan_create(int32_t kind, const qmv_problem* probs, int32_t count, qmv_plan** plan)
{
    if (!plan) return QMV_EINVAL;
    *plan = nullptr;
    int32_t st;
    if (kind == QMV_PLAN_GEMV || kind == QMV_PLAN_GEMV_DOT || kind == QMV_PLAN_GEMV_SKIP_ZERO)
        st = check_problems(probs, count, QMV_MAX_GEMV_M);
    else if (kind == QMV_PLAN_PREFILL)
        st = check_prefill(probs, count);
    else
        return QMV_EINVAL;
    if (st != QMV_OK) return st;
    qmv_plan* p = new (std::nothrow) qmv_plan;
    if (!p) return QMV_EINVAL;
    st = make_plan(kind, probs, count, *p);
    if (st != QMV_OK) {
        delete p;
        return st;
    }
    *plan = p;
    return QMV_OK;
}

int64_t qmv_plan_workspace_bytes(const qmv_plan* plan)
{
    return plan ? (int64_t)plan->image.size() : -1;
}

int32_t qmv_plan_upload(const qmv_plan* plan, void* workspace, int64_t ws_bytes, void* stream)
{
    const int32_t st = check_plan_use(plan, workspace, ws_bytes);
    return st != QMV_OK ? st : upload_plan(*plan, workspace, as_stream(stream));
}

int32_t qmv_plan_launch(const qmv_plan* plan, void* workspace, int64_t ws_bytes, void* stream)
{
    const int32_t st = check_plan_use(plan, workspace, ws_bytes);
    return st != QMV_OK ? st : launch_plan(*plan, workspace, as_stream(stream));
}

void qmv_plan_destroy(qmv_plan* plan) { delete plan; }

int64_t qmv_lmhead_workspace_bytes(int64_t v, int64_t k)
{
    if (v < 1 || k < 1 || v > QMV_MAX_N || k > QMV_MAX_K) return -1;
    return round_up(lmhead_partials(v) * 8, 256);
}

int32_t qmv_mfma_probe(int32_t kind, int32_t iters, uint32_t* out, int64_t* ops, void* stream)
{
    if (!out || !ops || (kind != 0 && kind != 1) || iters < 1 || iters > (1 << 20)) return QMV_EINVAL;
    const DeviceSetup* d = device_setup(nullptr);
    if (!d) return QMV_EHIP;
    return hip_status(launch_mfma_probe(kind, iters, out, d->cus, ops, as_stream(stream)));
}

int32_t qmv_read_probe(const void* data, int64_t bytes, uint32_t* out, void* stream)
{
    if (!data || !out || bytes < 0 || !aligned(data, 16) || (bytes & 15)) return QMV_EINVAL;
    if (bytes == 0) return QMV_OK;
    const DeviceSetup* d = device_setup(nullptr);
    if (!d) return QMV_EHIP;
    return hip_status(launch_read_probe(data, bytes, out, d->cus, as_stream(stream)));
}

int32_t qmv_lmhead_argmax(const uint16_t* w_bf16, const float* x, int64_t v, int64_t k, int32_t* idx,
                          float* max_logit, float* logits, void* workspace, int64_t ws_bytes, void* stream)
{
    if (!w_bf16 || !x || !idx) return QMV_EINVAL;
    if (v < 1 || k < 1 || v > QMV_MAX_N || k > QMV_MAX_K) return QMV_ESHAPE;
    const int64_t need = qmv_lmhead_workspace_bytes(v, k);
    if (!workspace || !aligned(workspace, 256) || ws_bytes < need) return QMV_EWORKSPACE;
    return hip_status(launch_lmhead(w_bf16, x, v, k, idx, max_logit, logits, workspace, as_stream(stream)));
}

int32_t qmv_lmhead_argmax_static(const uint16_t* w_bf16, const float* x, int64_t v, int64_t k, int32_t* idx,
                                 float* max_logit, float* logits, void* stream)
{
    if (!w_bf16 || !x || !idx) return QMV_EINVAL;
    if (v < 1 || k < 1 || v > QMV_MAX_N || k > QMV_MAX_K) return QMV_ESHAPE;
    if (lmhead_partials(v) * 8 > kStaticScratchBytes) return QMV_ESHAPE;
    const DeviceSetup* d = device_setup(nullptr);
    if (!d || !d->scratch) return QMV_EHIP;
    return hip_status(launch_lmhead(w_bf16, x, v, k, idx, max_logit, logits, d->scratch, as_stream(stream)));
}

int64_t qmv_sketch_bytes(int64_t v, int64_t k)
{
    if (v < 1 || v > QMV_MAX_N || k < 8 || k > kSketchMaxK || k % 8) return -1;
    return sketch_bytes(v, k);
}

int64_t qmv_sketch_workspace_bytes(int64_t v, int64_t k)
{
    if (v < 1 || v > QMV_MAX_N || k < 8 || k > kSketchMaxK || k % 8) return -1;
    return sketch_workspace_bytes(v);
}

int32_t qmv_sketch_build(const uint16_t* w_bf16, int64_t v, int64_t k, void* sketch, int64_t sketch_bytes_,
                         void* stream)
{
    if (!w_bf16 || !sketch || !aligned(w_bf16, 16) || !aligned(sketch, 256)) return QMV_EINVAL;
    if (v < 1 || v > QMV_MAX_N || k < 8 || k > kSketchMaxK || k % 8) return QMV_ESHAPE;
    if (sketch_bytes_ < sketch_bytes(v, k)) return QMV_EWORKSPACE;
    return hip_status(launch_sketch_build(w_bf16, v, k, sketch, as_stream(stream)));
}

int32_t qmv_lmhead_sketch_argmax(const uint16_t* w_bf16, const void* sketch, const float* x, int64_t v, int64_t k,
                                 int32_t* idx, float* max_logit, int32_t* candidates, float* scores,
                                 void* workspace, int64_t ws_bytes, void* stream)
{
    if (!w_bf16 || !sketch || !x || !idx || !aligned(w_bf16, 16) || !aligned(sketch, 256) || !aligned(x, 16))
        return QMV_EINVAL;
    if (v < 1 || v > QMV_MAX_N || k < 8 || k > kSketchMaxK || k % 8) return QMV_ESHAPE;
    if (!workspace || !aligned(workspace, 256) || ws_bytes < sketch_workspace_bytes(v)) return QMV_EWORKSPACE;
    if (!device_setup(nullptr)) return QMV_EHIP;
    return hip_status(launch_sketch_argmax(w_bf16, sketch, x, v, k, idx, max_logit, candidates, scores, workspace,
                                           as_stream(stream)));
}

}  // extern "C"
