// api.hip -- the C ABI of libqmv: host-side validation, problem tables and
// kernel launches.  Declarations and the contract of every call are in
// include/qmv.h.
#include <qmv.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "qmv_internal.hpp"

using namespace qmv;

namespace {

constexpr int64_t kMaxProblems = (int64_t)1 << kTileProbBits;
constexpr int64_t kMaxInt8K = 65536;  // keeps every int8 x int8 dot inside int32

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int64_t row_stride(int32_t wtype, int64_t k)
{
    if (wtype == QMV_W_TERNARY5) return round_up((k + 4) / 5, 16);
    if (wtype == QMV_W_INT8) return round_up(k, 16);
    return -1;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? QMV_OK : QMV_EHIP; }

int32_t check_weight(const qmv_weight& w)
{
    if (w.wtype != QMV_W_TERNARY5 && w.wtype != QMV_W_INT8) return QMV_EUNSUPPORTED;
    if (w.reserved != 0) return QMV_EINVAL;
    if (!w.data || !w.scale) return QMV_EINVAL;
    if (!aligned(w.data, 16)) return QMV_EINVAL;
    if (w.n < 1 || w.k < 1 || w.n > QMV_MAX_N || w.k > QMV_MAX_K) return QMV_ESHAPE;
    if (w.wtype == QMV_W_INT8 && w.k > kMaxInt8K) return QMV_ESHAPE;
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
    }
    return QMV_OK;
}

// Workspace image of a problem list: [DevProblem x count][tile entries].
// Problems are grouped by weight type; inside a group the largest tiles come
// first so they start first.  A tile is a block of rows of one problem:
// 64 rows for the workgroup kernel, 64 / lanes_per_row rows for the streaming
// kernel.
struct Table {
    std::vector<uint8_t> bytes;
    int64_t tiles_offset = 0;
    int32_t total_tiles = 0;
    // per weight type: streaming kernel?, first tile, tile count, max m, max chunks
    bool stream[3] = {false, false, false};
    int32_t first[3] = {0, 0, 0}, count[3] = {0, 0, 0}, max_m[3] = {0, 0, 0}, max_chunks[3] = {0, 0, 0};
};

struct Plan {
    std::vector<int32_t> order;    // problem index per table slot
    std::vector<int32_t> rows;     // rows per tile, per problem
    std::vector<int32_t> lanes;    // lanes per row, per problem
    int64_t tiles = 0;
    bool stream[3] = {false, false, false};
    int32_t max_m[3] = {0, 0, 0}, max_chunks[3] = {0, 0, 0};
};

void make_plan(const qmv_problem* probs, int32_t count, Plan& pl)
{
    for (int32_t i = 0; i < count; ++i) {
        const int32_t wt = probs[i].w.wtype;
        pl.max_m[wt] = std::max<int32_t>(pl.max_m[wt], (int32_t)probs[i].m);
        pl.max_chunks[wt] = std::max<int32_t>(pl.max_chunks[wt], (int32_t)(row_stride(wt, probs[i].w.k) / 16));
    }
    for (int wt = 1; wt <= 2; ++wt)
        pl.stream[wt] = pl.max_m[wt] > 0 && gemv_stream_fits(wt, pl.max_m[wt], pl.max_chunks[wt]);
    pl.rows.resize(count);
    pl.lanes.resize(count);
    pl.order.resize(count);
    for (int32_t i = 0; i < count; ++i) {
        const int32_t wt = probs[i].w.wtype;
        const int32_t chunks = (int32_t)(row_stride(wt, probs[i].w.k) / 16);
        pl.lanes[i] = pl.stream[wt] ? gemv_stream_lanes_per_row(chunks) : 1;
        pl.rows[i] = kRowsPerTile / pl.lanes[i];
        pl.tiles += (probs[i].w.n + pl.rows[i] - 1) / pl.rows[i];
        pl.order[i] = i;
    }
    std::stable_sort(pl.order.begin(), pl.order.end(), [&](int32_t a, int32_t b) {
        if (probs[a].w.wtype != probs[b].w.wtype) return probs[a].w.wtype < probs[b].w.wtype;
        const int64_t ta = (int64_t)pl.rows[a] * row_stride(probs[a].w.wtype, probs[a].w.k);
        const int64_t tb = (int64_t)pl.rows[b] * row_stride(probs[b].w.wtype, probs[b].w.k);
        return ta > tb;
    });
}

int64_t plan_bytes(const Plan& pl, int32_t count)
{
    return round_up((int64_t)sizeof(DevProblem) * count, 256) + round_up(pl.tiles * 4, 256);
}

bool plan_tiles_fit(const qmv_problem* probs, int32_t count, const Plan& pl)
{
    for (int32_t i = 0; i < count; ++i)
        if ((probs[i].w.n + pl.rows[i] - 1) / pl.rows[i] > ((int64_t)1 << kTileRowBits)) return false;
    return true;
}

int64_t table_bytes(const qmv_problem* probs, int32_t count)
{
    Plan pl;
    make_plan(probs, count, pl);
    return plan_bytes(pl, count);
}

void build_table(const qmv_problem* probs, int32_t count, const Plan& pl, Table& t)
{
    const int64_t pbytes = round_up((int64_t)sizeof(DevProblem) * count, 256);
    t.bytes.assign(plan_bytes(pl, count), 0);
    t.tiles_offset = pbytes;
    t.total_tiles = (int32_t)pl.tiles;
    DevProblem* dp = reinterpret_cast<DevProblem*>(t.bytes.data());
    uint32_t* te = reinterpret_cast<uint32_t*>(t.bytes.data() + pbytes);
    int32_t tile = 0;
    for (int wt = 1; wt <= 2; ++wt) {
        t.stream[wt] = pl.stream[wt];
        t.max_m[wt] = pl.max_m[wt];
        t.max_chunks[wt] = pl.max_chunks[wt];
    }
    for (int32_t slot = 0; slot < count; ++slot) {
        const int32_t pi = pl.order[slot];
        const qmv_problem& p = probs[pi];
        const int32_t wt = p.w.wtype;
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
        d.chunks = (int32_t)(row_stride(wt, p.w.k) / 16);
        d.tile_begin = tile;
        d.wtype = wt;
        d.lanes_per_row = pl.lanes[pi];
        d.reserved = 0;
        if (t.count[wt] == 0) t.first[wt] = tile;
        const int32_t ntiles = (int32_t)((p.w.n + pl.rows[pi] - 1) / pl.rows[pi]);
        for (int32_t r = 0; r < ntiles; ++r) te[tile + r] = ((uint32_t)slot << kTileRowBits) | (uint32_t)r;
        tile += ntiles;
        t.count[wt] += ntiles;
    }
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

constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

// Workspace of a prefill problem list: the problem table and the XCD-ordered
// tile list (8 lists padded to the longest, bounded by 8 x all tiles).
int64_t prefill_table_bytes(const qmv_problem* probs, int32_t count)
{
    int64_t tiles = 0;
    for (int32_t i = 0; i < count; ++i) tiles += prefill_tiles(probs[i].m, probs[i].w.n);
    // no XCD list can be longer than all tiles together
    const int64_t bound = kXcds * tiles;
    return round_up((int64_t)sizeof(DevProblem) * count, 256) + round_up(bound * 8, 256);
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

int32_t qmv_quantize_act(const float* x, int64_t m, int64_t k, int8_t* x8, float* sx, void* stream)
{
    if (!x || !x8 || !sx) return QMV_EINVAL;
    if (m < 1 || k < 1 || k > QMV_MAX_K || m > ((int64_t)1 << 31) - 1) return QMV_ESHAPE;
    return hip_status(launch_quantize_rows(x, m, k, x8, sx, as_stream(stream)));
}

int64_t qmv_gemv_workspace_bytes(const qmv_problem* probs, int32_t count)
{
    if (check_problems(probs, count, QMV_MAX_GEMV_M) != QMV_OK) return -1;
    return table_bytes(probs, count);
}

int32_t qmv_gemv(const qmv_problem* probs, int32_t count, void* workspace, int64_t ws_bytes, uint32_t flags,
                 void* stream)
{
    int32_t st = check_problems(probs, count, QMV_MAX_GEMV_M);
    if (st != QMV_OK) return st;
    if (flags & ~(uint32_t)QMV_F_TABLE_READY) return QMV_EINVAL;
    Plan pl;
    make_plan(probs, count, pl);
    if (!plan_tiles_fit(probs, count, pl)) return QMV_ESHAPE;
    for (int wt = 1; wt <= 2; ++wt)
        if (pl.max_m[wt] && !pl.stream[wt] && gemv_lds_bytes(wt, pl.max_m[wt], pl.max_chunks[wt]) > kMaxLds)
            return QMV_ESHAPE;
    if (!workspace || !aligned(workspace, 256) || ws_bytes < plan_bytes(pl, count)) return QMV_EWORKSPACE;
    Table t;
    build_table(probs, count, pl, t);
    const hipStream_t s = as_stream(stream);
    if (!(flags & QMV_F_TABLE_READY)) {
        hipError_t e = hipMemcpyAsync(workspace, t.bytes.data(), t.bytes.size(), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return QMV_EHIP;
    }
    const uint8_t* base = static_cast<const uint8_t*>(workspace);
    const DevProblem* dp = reinterpret_cast<const DevProblem*>(base);
    const uint32_t* tiles = reinterpret_cast<const uint32_t*>(base + t.tiles_offset);
    for (int wt = 1; wt <= 2; ++wt) {
        if (t.count[wt] == 0) continue;
        hipError_t e;
        if (t.stream[wt])
            e = launch_gemv_stream(dp, tiles, t.first[wt], t.count[wt], wt, t.max_m[wt], t.max_chunks[wt], s);
        else
            e = launch_gemv(dp, tiles, t.first[wt], t.count[wt], wt, t.max_m[wt], t.max_chunks[wt], s);
        if (e != hipSuccess) return QMV_EHIP;
    }
    return QMV_OK;
}

int64_t qmv_prefill_workspace_bytes(const qmv_problem* probs, int32_t count)
{
    if (check_prefill(probs, count) != QMV_OK) return -1;
    return prefill_table_bytes(probs, count);
}

int32_t qmv_gemm_prefill(const qmv_problem* probs, int32_t count, void* workspace, int64_t ws_bytes, uint32_t flags,
                         void* stream)
{
    int32_t st = check_prefill(probs, count);
    if (st != QMV_OK) return st;
    if (flags & ~(uint32_t)QMV_F_TABLE_READY) return QMV_EINVAL;
    const int64_t need = prefill_table_bytes(probs, count);
    if (!workspace || !aligned(workspace, 256) || ws_bytes < need) return QMV_EWORKSPACE;
    // Problem table: longest rows first.
    std::vector<int32_t> order(count);
    for (int32_t i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return probs[a].w.k > probs[b].w.k; });
    const int64_t pbytes = round_up((int64_t)sizeof(DevProblem) * count, 256);
    std::vector<uint8_t> img(need, 0);
    DevProblem* dp = reinterpret_cast<DevProblem*>(img.data());
    // Tile list, XCD-aware: workgroup b runs on XCD b % 8 (round-robin dispatch),
    // so tiles that share an activation block (same problem and token block) go
    // to one XCD's list and run back to back there, reusing that XCD's L2.  The
    // token-block groups are spread over the XCDs longest first, to the least
    // loaded one.
    struct Group {
        int32_t slot;
        int64_t mt, ntiles, work;
    };
    std::vector<Group> groups;
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
        for (int64_t mt = 0; mt < mts; ++mt) groups.push_back({slot, mt, nts, nts * ((d.chunks + 1) / 2)});
    }
    std::stable_sort(groups.begin(), groups.end(), [](const Group& a, const Group& b) { return a.work > b.work; });
    std::vector<std::vector<uint64_t>> lists(kXcds);
    std::vector<int64_t> load(kXcds, 0);
    for (const Group& gr : groups) {
        int x = 0;
        for (int i = 1; i < kXcds; ++i)
            if (load[i] < load[x]) x = i;
        load[x] += gr.work;
        for (int64_t nt = 0; nt < gr.ntiles; ++nt)
            lists[x].push_back(((uint64_t)gr.slot << 48) | ((uint64_t)gr.mt << 32) | (uint64_t)nt);
    }
    size_t longest = 0;
    for (const auto& l : lists) longest = std::max(longest, l.size());
    const int64_t grid = (int64_t)longest * kXcds;
    if (pbytes + grid * 8 > need) return QMV_EWORKSPACE;  // cannot happen: need covers 8 x all tiles
    uint64_t* te = reinterpret_cast<uint64_t*>(img.data() + pbytes);
    for (int64_t b = 0; b < grid; ++b) {
        const auto& l = lists[b % kXcds];
        const size_t j = (size_t)(b / kXcds);
        te[b] = j < l.size() ? l[j] : ~0ull;
    }
    const hipStream_t s = as_stream(stream);
    if (!(flags & QMV_F_TABLE_READY)) {
        hipError_t e = hipMemcpyAsync(workspace, img.data(), img.size(), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return QMV_EHIP;
    }
    const uint8_t* base = static_cast<const uint8_t*>(workspace);
    return hip_status(launch_prefill(reinterpret_cast<const DevProblem*>(base),
                                     reinterpret_cast<const uint64_t*>(base + pbytes), grid, s));
}

int64_t qmv_lmhead_workspace_bytes(int64_t v, int64_t k)
{
    if (v < 1 || k < 1 || v > QMV_MAX_N || k > QMV_MAX_K) return -1;
    return round_up(lmhead_partials(v) * 8, 256);
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

}  // extern "C"
