// C ABI of libmla: host-side validation, the split-KV planner and launch
// dispatch.  Argument checks and the planner make no HIP call, so they run
// (and are tested) on machines without a GPU.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <queue>
#include <vector>

#include "common.hpp"

using namespace mla;

namespace {

thread_local char g_err[512] = "";

// measurement events for the next kernel launches of this thread
constexpr int kMaxTimedLaunches = 16;
thread_local LaunchTiming g_timing[kMaxTimedLaunches];
thread_local int g_timing_n = 0, g_timing_next = 0;

mla_status_t fail(mla_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

mla_status_t ok() {
    g_err[0] = '\0';
    return MLA_OK;
}

mla_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int elem_bytes(mla_dtype_t dt) {
    switch (dt) {
    case MLA_DT_F32: return 4;
    case MLA_DT_BF16: return 2;
    case MLA_DT_FP8_E4M3: return 1;
    case MLA_DT_F16: return 2;
    case MLA_DT_FP8_E5M2: return 1;
    case MLA_DT_FP8_E4M3_ROW: return 1;
    }
    return 0;
}

int64_t block_bytes_of(mla_dtype_t kv, int32_t d_c, int32_t d_r) {
    switch (kv) {
    case MLA_DT_F32: return (int64_t)kBlock * (d_c + d_r) * 4;
    case MLA_DT_BF16: return (int64_t)kBlock * (d_c + d_r) * 2;
    case MLA_DT_FP8_E4M3:
    case MLA_DT_FP8_E5M2: return (int64_t)kBlock * d_c + (int64_t)kBlock * d_r * 2;
    case MLA_DT_F16: return (int64_t)kBlock * (d_c + d_r) * 2;
    case MLA_DT_FP8_E4M3_ROW: return (int64_t)kBlock * (d_c + d_r);
    }
    return -1;
}

bool is_kv_dtype(mla_dtype_t kv) { return kv >= MLA_DT_F32 && kv <= MLA_DT_FP8_E4M3_ROW; }

bool is_fp8_kv(mla_dtype_t kv) {
    return kv == MLA_DT_FP8_E4M3 || kv == MLA_DT_FP8_E5M2 || kv == MLA_DT_FP8_E4M3_ROW;
}

bool is_fast_shape(mla_dtype_t kv, int32_t d_c, int32_t d_r) {
    return kv != MLA_DT_F32 && is_kv_dtype(kv) && d_c == 512 && d_r == 64;
}

mla_status_t check_cache(const mla_cache_desc_t *c) {
    if (!c) return fail(MLA_ERR_INVALID_ARG, "cache descriptor is NULL");
    if (!c->base) return fail(MLA_ERR_INVALID_ARG, "cache base is NULL");
    if (c->num_blocks < 1) return fail(MLA_ERR_INVALID_ARG, "cache is empty (num_blocks=%lld)", (long long)c->num_blocks);
    if (c->block_size != kBlock)
        return fail(MLA_ERR_UNSUPPORTED, "block_size %d unsupported (only %d)", c->block_size, kBlock);
    if (!is_kv_dtype(c->kv_dtype)) return fail(MLA_ERR_UNSUPPORTED, "kv dtype %d unsupported", (int)c->kv_dtype);
    if (c->d_c < 4 || c->d_c > 1024 || c->d_c % 4 || c->d_r < 0 || c->d_r > 256 || c->d_r % 4)
        return fail(MLA_ERR_UNSUPPORTED, "cache dims d_c=%d d_r=%d unsupported (d_c in [4,1024], d_r in [0,256], multiples of 4)",
                    c->d_c, c->d_r);
    if (is_fp8_kv(c->kv_dtype) && !c->block_scales)
        return fail(MLA_ERR_INVALID_ARG, "fp8 cache needs block_scales");
    if (c->flags & ~MLA_CACHE_FP8_EXACT) return fail(MLA_ERR_INVALID_ARG, "unknown cache flags %d", c->flags);
    if (!aligned(c->base, 16)) return fail(MLA_ERR_ALIGN, "cache base not 16-byte aligned");
    return MLA_OK;
}

}  // namespace

namespace mla {
LaunchTiming next_launch_timing() {
    if (g_timing_next >= g_timing_n) return LaunchTiming{nullptr, nullptr};
    return g_timing[g_timing_next++];
}
}  // namespace mla

extern "C" {

const char *mla_last_error(void) { return g_err; }

mla_status_t mla_set_launch_events(void *const *events, int32_t pairs) {
    if (pairs < 0 || pairs > kMaxTimedLaunches)
        return fail(MLA_ERR_INVALID_ARG, "pairs=%d outside [0, %d]", pairs, kMaxTimedLaunches);
    if (pairs > 0 && !events) return fail(MLA_ERR_INVALID_ARG, "events is NULL");
    for (int k = 0; k < pairs; ++k) {
        if (!events[2 * k] || !events[2 * k + 1]) return fail(MLA_ERR_INVALID_ARG, "event %d is NULL", k);
        g_timing[k] = LaunchTiming{(hipEvent_t)events[2 * k], (hipEvent_t)events[2 * k + 1]};
    }
    g_timing_n = pairs;
    g_timing_next = 0;
    return ok();
}

int32_t mla_launch_events_used(void) { return g_timing_next; }

const char *mla_version(void) { return "mla-mi355x 0.1.0 (gfx950)"; }

int64_t mla_cache_bytes(const mla_cache_desc_t *cache) {
    if (!cache || cache->block_size != kBlock || cache->num_blocks < 0) return 0;
    int64_t bb = block_bytes_of(cache->kv_dtype, cache->d_c, cache->d_r);
    return bb < 0 ? 0 : bb * cache->num_blocks;
}

mla_status_t mla_decode_plan(const int32_t *seq_lens_host, int32_t B, int32_t q_len,
                             int32_t n_h, int32_t d_c, int32_t d_r, mla_dtype_t kv_dtype,
                             int32_t num_cus, int32_t *plan_host, int64_t plan_capacity,
                             mla_plan_t *info) {
    if (!info) return fail(MLA_ERR_INVALID_ARG, "info is NULL");
    if (!seq_lens_host) return fail(MLA_ERR_INVALID_ARG, "seq_lens_host is NULL");
    if (B < 1 || q_len < 1 || n_h < 1 || d_c < 1 || d_r < 0)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes B=%d q_len=%d n_h=%d d_c=%d d_r=%d", B, q_len, n_h, d_c, d_r);
    if (num_cus < 1) return fail(MLA_ERR_INVALID_ARG, "num_cus=%d", num_cus);
    if (!is_kv_dtype(kv_dtype)) return fail(MLA_ERR_UNSUPPORTED, "kv dtype %d unsupported", (int)kv_dtype);
    int64_t rows = (int64_t)q_len * n_h;
    if (rows > (1 << 20)) return fail(MLA_ERR_INVALID_ARG, "q_len*n_h too large");
    int32_t row_chunks = (int32_t)((rows + kRowsPerChunk - 1) / kRowsPerChunk);

    int64_t max_seq_blocks = 0;
    for (int b = 0; b < B; ++b) {
        if (seq_lens_host[b] < 0) return fail(MLA_ERR_INVALID_ARG, "seq_lens[%d] = %d < 0", b, seq_lens_host[b]);
        max_seq_blocks = std::max<int64_t>(max_seq_blocks, (seq_lens_host[b] + (int64_t)kBlock - 1) / kBlock);
    }

    // Work list: every (sequence, row chunk) segment with at least one block,
    // in order.  A work item is a block range of one segment, run by one
    // workgroup.  Item sizes: pack the list into at most num_cus bins
    // minimising the largest bin cost, each item costing its 32-token stages
    // plus kItemCost for its query prologue and output epilogue (binary
    // search on the budget M, greedy fill: a bin takes whole segments while
    // they fit, then as many whole blocks of the next as fit); the pieces cut
    // this way are the items.  Uniform batches get the even split (the
    // measured 32 x 4096 batch: 8 items of 8 blocks per sequence); ragged
    // ones get pieces sized so that short sequences fill the gaps left by
    // long ones, instead of every compute unit waiting for the longest split.
    // (segments of an empty sequence get one item of no blocks each, which
    // writes their rows' o_lat = 0 and lse = -inf)
    struct Seg { int32_t sc; int64_t nb, st; };
    std::vector<Seg> segs;
    for (int b = 0; b < B; ++b) {
        const int64_t nb = (seq_lens_host[b] + kBlock - 1) / kBlock;
        const int64_t st = (seq_lens_host[b] + 31) / 32;
        for (int c = 0; c < row_chunks; ++c) segs.push_back({b * row_chunks + c, nb, st});
    }
    constexpr int64_t kItemCost = 6;
    auto piece_stages = [](const Seg &g, int64_t k0, int64_t k1) {
        return std::min<int64_t>(2 * (k1 - k0), g.st - 2 * k0);
    };
    struct Piece { int32_t seg; int64_t k0, k1; };
    // bins used at budget M (stops counting past `limit` unless pieces are wanted)
    auto fill = [&](int64_t M, int64_t limit, std::vector<Piece> *out) {
        int64_t bins = 0, load = 0;
        bool open = false;
        for (size_t i = 0; i < segs.size(); ++i) {
            const Seg &g = segs[i];
            int64_t k = 0;
            while (k < g.nb) {
                if (!open) {
                    if (++bins > limit && !out) return bins;
                    load = 0;
                    open = true;
                }
                const int64_t rest = piece_stages(g, k, g.nb);
                int64_t kk;
                if (load + rest + kItemCost <= M) {
                    kk = g.nb;
                } else {
                    kk = std::min<int64_t>(g.nb, k + std::max<int64_t>(0, (M - load - kItemCost) / 2));
                    open = false;   // full after this piece
                }
                if (kk > k) {
                    if (out) out->push_back({(int32_t)i, k, kk});
                    load += piece_stages(g, k, kk) + kItemCost;
                    k = kk;
                }
            }
        }
        return bins;
    };
    std::vector<Piece> pieces;
    if (!segs.empty()) {
        int64_t total = 0;
        for (const Seg &g : segs) total += g.st + kItemCost;
        int64_t lo = kItemCost + 1, hi = std::max<int64_t>(total, kItemCost + 2);   // fill(hi) uses one bin
        while (hi - lo > 1) {
            const int64_t mid = lo + (hi - lo) / 2;
            (fill(mid, num_cus, nullptr) <= num_cus ? hi : lo) = mid;
        }
        fill(hi, num_cus, &pieces);
        for (size_t i = 0; i < segs.size(); ++i)
            if (segs[i].nb == 0) pieces.push_back({(int32_t)i, 0, 0});
    }
    const int64_t num_items = (int64_t)pieces.size();
    const int64_t nseg = (int64_t)B * row_chunks;
    if (num_items > (1 << 24)) return fail(MLA_ERR_INVALID_ARG, "too many work items");

    // Dispatch order of the MFMA decode.  Workgroup k runs on XCD k % 8, and
    // each XCD starts its workgroups in order on whichever of its compute
    // units frees first.  Simulate longest-first list scheduling of the
    // items over the num_cus compute units (numbered XCD-major, ties to the
    // lowest number, so that equal pieces of one sequence share an XCD and
    // its L2) and give each XCD its items in simulated start order.
    constexpr int kXcds = 8;
    const int64_t per_x = (num_cus + kXcds - 1) / kXcds;
    std::vector<std::vector<int32_t>> queue(kXcds);
    {
        std::vector<int64_t> cost(num_items);
        for (int64_t i = 0; i < num_items; ++i)
            cost[i] = piece_stages(segs[pieces[i].seg], pieces[i].k0, pieces[i].k1) + kItemCost;
        std::vector<int32_t> order(num_items);
        for (int64_t i = 0; i < num_items; ++i) order[i] = (int32_t)i;
        std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
        typedef std::pair<int64_t, int32_t> Slot;   // (free at, compute unit)
        std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> free_at;
        for (int32_t c = 0; c < num_cus; ++c) free_at.push({0, c});
        for (int32_t i : order) {
            const Slot u = free_at.top();
            free_at.pop();
            queue[u.second / per_x].push_back(i);
            free_at.push({u.first + cost[i], u.second});
        }
    }
    size_t longest = 0;
    for (const auto &q : queue) longest = std::max(longest, q.size());
    const int64_t grid_wgs = kXcds * (int64_t)longest;

    // pieces per segment -> partial slots (segments split more than once)
    std::vector<int32_t> count(segs.size(), 0);
    for (const Piece &q : pieces) ++count[q.seg];
    int64_t num_partials = 0, max_blocks = 0;
    int32_t max_splits = 0;
    for (size_t i = 0; i < segs.size(); ++i) {
        if (count[i] > 1) num_partials += count[i];
        max_splits = std::max(max_splits, count[i]);
    }
    for (const Piece &q : pieces) max_blocks = std::max<int64_t>(max_blocks, q.k1 - q.k0);

    info->B = B; info->q_len = q_len; info->n_h = n_h; info->d_c = d_c;
    info->num_items = (int32_t)num_items;
    info->row_chunks = row_chunks;
    info->num_partials = (int32_t)num_partials;
    info->needs_combine = num_partials > 0 ? 1 : 0;
    info->max_splits = max_splits;
    info->blocks_per_item = (int32_t)max_blocks;
    info->partial_dtype = is_fast_shape(kv_dtype, d_c, d_r) ? MLA_DT_BF16 : MLA_DT_F32;
    info->grid_wgs = (int32_t)grid_wgs;
    info->kv_dtype = (int32_t)kv_dtype;
    info->d_r = d_r;
    info->max_seq_blocks = (int32_t)max_seq_blocks;
    info->plan_ints = plan_flags_off((int32_t)num_items, (int32_t)grid_wgs, (int32_t)nseg) + nseg;
    int64_t o_bytes = num_partials * rows * d_c * elem_bytes((mla_dtype_t)info->partial_dtype);
    int64_t o_bytes_al = (o_bytes + 255) / 256 * 256;
    info->workspace_bytes = num_partials ? o_bytes_al + num_partials * rows * 4 : 0;

    if (!plan_host) return ok();
    if (plan_capacity < info->plan_ints)
        return fail(MLA_ERR_INVALID_ARG, "plan capacity %lld < %lld", (long long)plan_capacity, (long long)info->plan_ints);

    int32_t *items = plan_host + plan_items_off();
    int32_t *wg_item = plan_host + plan_wg_off((int32_t)num_items);
    int32_t *split_off = plan_host + plan_split_off((int32_t)num_items, (int32_t)grid_wgs);
    int32_t *flags = plan_host + plan_flags_off((int32_t)num_items, (int32_t)grid_wgs, (int32_t)nseg);
    for (int k = 0; k < kPlanHeader; ++k) plan_host[k] = 0;
    plan_host[0] = (int32_t)num_items;
    plan_host[1] = B;
    plan_host[2] = row_chunks;
    plan_host[3] = (int32_t)num_partials;
    plan_host[4] = (int32_t)grid_wgs;
    // slots: the pieces of a split segment, in order
    std::vector<int32_t> first_slot(segs.size(), -1);
    {
        int64_t slot = 0;
        size_t i = 0;
        for (int64_t sc = 0; sc < nseg; ++sc) {
            split_off[sc] = (int32_t)slot;
            flags[sc] = 0;
            if (i < segs.size() && segs[i].sc == sc) {
                if (count[i] == 1) flags[sc] = 1;
                else { first_slot[i] = (int32_t)slot; slot += count[i]; }
                ++i;
            }
        }
        split_off[nseg] = (int32_t)slot;
    }
    std::vector<int32_t> seen(segs.size(), 0);
    for (int64_t it = 0; it < num_items; ++it) {
        const Piece &q = pieces[it];
        items[4 * it + 0] = segs[q.seg].sc;
        items[4 * it + 1] = (int32_t)q.k0;
        items[4 * it + 2] = (int32_t)q.k1;
        items[4 * it + 3] = count[q.seg] == 1 ? -1 : first_slot[q.seg] + seen[q.seg];
        ++seen[q.seg];
    }
    for (int64_t k = 0; k < grid_wgs; ++k) {
        const auto &q = queue[k % kXcds];
        const size_t j = (size_t)(k / kXcds);
        wg_item[k] = j < q.size() ? q[j] : -1;
    }
    return ok();
}

namespace {

// Validate mla_decode's arguments and resolve them into kernel arguments.
mla_status_t prepare_decode(const void *q_lat, const void *q_rope, mla_dtype_t q_dtype,
                            const mla_cache_desc_t *cache, const int32_t *block_table,
                            int32_t bt_stride, const int32_t *seq_lens, int32_t B, int32_t q_len,
                            int32_t n_h, float scale, const mla_plan_t *plan,
                            const int32_t *plan_dev, void *workspace, int64_t workspace_bytes,
                            void *o_lat, float *lse, DecodeArgs *out) {
    mla_status_t st = check_cache(cache);
    if (st != MLA_OK) return st;
    if (!q_lat || !o_lat || !lse || !block_table || !seq_lens)
        return fail(MLA_ERR_INVALID_ARG, "NULL q_lat/o_lat/lse/block_table/seq_lens");
    if (cache->d_r > 0 && !q_rope) return fail(MLA_ERR_INVALID_ARG, "q_rope is NULL");
    if (!plan || !plan_dev) return fail(MLA_ERR_INVALID_ARG, "missing decode plan");
    if (B < 1 || q_len < 1 || n_h < 1 || bt_stride < 1)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes B=%d q_len=%d n_h=%d bt_stride=%d", B, q_len, n_h, bt_stride);
    if (plan->B != B || plan->q_len != q_len || plan->n_h != n_h || plan->d_c != cache->d_c ||
        plan->d_r != cache->d_r)
        return fail(MLA_ERR_INVALID_ARG, "plan was built for other sizes");
    if (plan->kv_dtype != (int32_t)cache->kv_dtype)
        return fail(MLA_ERR_INVALID_ARG, "plan was built for kv dtype %d, cache is %d", plan->kv_dtype,
                    (int)cache->kv_dtype);
    if (bt_stride < plan->max_seq_blocks)
        return fail(MLA_ERR_INVALID_ARG, "bt_stride %d < %d blocks of the longest planned sequence", bt_stride,
                    plan->max_seq_blocks);
    if (plan->partial_dtype != (is_fast_shape(cache->kv_dtype, cache->d_c, cache->d_r) ? MLA_DT_BF16 : MLA_DT_F32))
        return fail(MLA_ERR_INVALID_ARG, "plan partial dtype does not match the cache format");
    if (q_dtype != MLA_DT_F32 && q_dtype != MLA_DT_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "q dtype %d unsupported", (int)q_dtype);
    if (!aligned(q_lat, 16) || !aligned(o_lat, 16) || (q_rope && !aligned(q_rope, 16)) || !aligned(lse, 4))
        return fail(MLA_ERR_ALIGN, "q_lat/q_rope/o_lat must be 16-byte aligned");
    if (workspace_bytes < plan->workspace_bytes)
        return fail(MLA_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)workspace_bytes,
                    (long long)plan->workspace_bytes);
    if (plan->workspace_bytes > 0 && (!workspace || !aligned(workspace, 256)))
        return fail(MLA_ERR_ALIGN, "workspace NULL or not 256-byte aligned");
    if (!(scale > 0.0f) || scale != scale) return fail(MLA_ERR_INVALID_ARG, "scale must be positive");

    DecodeArgs a{};
    a.q_lat = q_lat; a.q_rope = q_rope; a.pool = cache->base; a.block_scales = cache->block_scales;
    a.block_table = block_table; a.seq_lens = seq_lens; a.plan = plan_dev;
    const int64_t rows = (int64_t)q_len * n_h;
    if (plan->partial_dtype != MLA_DT_F32 && plan->partial_dtype != MLA_DT_BF16)
        return fail(MLA_ERR_INVALID_ARG, "plan has a bad partial dtype");
    if (plan->num_partials > 0) {
        const int64_t o_bytes = (int64_t)plan->num_partials * rows * cache->d_c *
                                elem_bytes((mla_dtype_t)plan->partial_dtype);
        a.o_part = workspace;
        a.lse_part = (float *)((char *)workspace + (o_bytes + 255) / 256 * 256);
    }
    a.o_lat = o_lat; a.lse = lse;
    a.block_bytes = block_bytes_of(cache->kv_dtype, cache->d_c, cache->d_r);
    a.num_pool_blocks = cache->num_blocks;
    a.bt_stride = bt_stride; a.B = B; a.q_len = q_len; a.n_h = n_h;
    a.d_c = cache->d_c; a.d_r = cache->d_r; a.rows = (int32_t)rows;
    a.num_items = plan->num_items; a.row_chunks = plan->row_chunks; a.grid_wgs = plan->grid_wgs;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q_dtype = q_dtype; a.kv_dtype = cache->kv_dtype;
    a.partial_dtype = (mla_dtype_t)plan->partial_dtype;
    a.cache_flags = cache->flags;
    *out = a;
    return MLA_OK;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    if (a.num_items == 0) return hipSuccess;
    if (is_fast_shape(a.kv_dtype, a.d_c, a.d_r) && a.q_dtype == MLA_DT_BF16) {
        if (a.kv_dtype == MLA_DT_FP8_E4M3 && !(a.cache_flags & MLA_CACHE_FP8_EXACT)) return launch_decode_f8w8(a, s);
        return launch_decode_mfma(a, s);
    }
    return launch_decode_generic(a, s);
}

mla_status_t finish_decode(const mla_plan_t *plan, const int32_t *plan_dev, void *workspace,
                           mla_dtype_t out_dtype, void *o_lat, float *lse, hipStream_t s) {
    if (!plan->needs_combine) return ok();
    const int64_t rows = (int64_t)plan->q_len * plan->n_h;
    const mla_dtype_t pdt = (mla_dtype_t)plan->partial_dtype;
    void *o_part = nullptr;
    float *lse_part = nullptr;
    if (plan->num_partials > 0) {
        const int64_t o_bytes = (int64_t)plan->num_partials * rows * plan->d_c * elem_bytes(pdt);
        o_part = workspace;
        lse_part = (float *)((char *)workspace + (o_bytes + 255) / 256 * 256);
    }
    const int32_t nseg = plan->B * plan->row_chunks;
    const int32_t *split_off = plan_dev + plan_split_off(plan->num_items, plan->grid_wgs);
    const int32_t *flags = plan_dev + plan_flags_off(plan->num_items, plan->grid_wgs, nseg);
    return hip_status(launch_combine(o_part, pdt, lse_part, split_off, flags, plan->B,
                                     (int32_t)rows, kRowsPerChunk, plan->d_c, o_lat, out_dtype, lse,
                                     plan->max_splits, s),
                      "combine launch");
}

}  // namespace

}  // extern "C"

namespace {
bool debug_on();
mla_status_t device_check(const int32_t *bt, int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                          int64_t num_blocks, hipStream_t s);
}  // namespace

extern "C" {

mla_status_t mla_decode(const void *q_lat, const void *q_rope, mla_dtype_t q_dtype,
                        const mla_cache_desc_t *cache, const int32_t *block_table,
                        int32_t bt_stride, const int32_t *seq_lens, int32_t B, int32_t q_len,
                        int32_t n_h, float scale, const mla_plan_t *plan,
                        const int32_t *plan_dev, void *workspace, int64_t workspace_bytes,
                        void *o_lat, float *lse, mla_stream_t stream) {
    DecodeArgs a;
    mla_status_t st = prepare_decode(q_lat, q_rope, q_dtype, cache, block_table, bt_stride, seq_lens,
                                     B, q_len, n_h, scale, plan, plan_dev, workspace,
                                     workspace_bytes, o_lat, lse, &a);
    if (st != MLA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (debug_on()) {
        st = device_check(block_table, bt_stride, seq_lens, B, cache->num_blocks, s);
        if (st != MLA_OK) return st;
    }
    hipError_t e = launch_decode(a, s);
    if (e != hipSuccess) return hip_status(e, "decode launch");
    return finish_decode(plan, plan_dev, workspace, q_dtype, o_lat, lse, s);
}

}  // extern "C"

namespace {

// Scratch of the entry point that allocates nothing (mla_decode_noalloc):
// each GPU the library runs on holds one copy until the process ends.  In
// host code `scratch` is only a stand-in for the symbol; its device address
// comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

mla_status_t scratch_address(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MLA_OK;
}

}  // namespace

namespace {

// Device checks (mla_set_debug): the offence counter and the first offence,
// one copy per GPU, zero between checks (a failing check clears it).
static __device__ __align__(16) int32_t check_flag[4];

std::atomic<int> g_debug{-1};   // -1: MLA_DEBUG not read yet
void *g_check_ptr[kMaxDevices] = {};

bool debug_on() {
    int d = g_debug.load();
    if (d < 0) {
        const char *e = std::getenv("MLA_DEBUG");
        d = (e && std::atoi(e) != 0) ? 1 : 0;
        int expect = -1;
        if (!g_debug.compare_exchange_strong(expect, d)) d = g_debug.load();
    }
    return d > 0;
}

mla_status_t device_check(const int32_t *bt, int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                          int64_t num_blocks, hipStream_t s) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    int32_t *flag = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_check_ptr[dev]) {
            void *p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_flag));
            if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(check_flag)");
            if (!p) return fail(MLA_ERR_HIP, "hipGetSymbolAddress(check_flag) returned NULL");
            g_check_ptr[dev] = p;
        }
        flag = (int32_t *)g_check_ptr[dev];
    }
    e = launch_table_check(bt, bt_stride, seq_lens, B, num_blocks, flag, s);
    if (e != hipSuccess) return hip_status(e, "device check launch");
    int32_t h[4] = {0, 0, 0, 0};
    e = hipMemcpyAsync(h, flag, sizeof(h), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "device check read-back");
    if (h[0] == 0) return MLA_OK;
    static const int32_t zeros[4] = {0, 0, 0, 0};
    e = hipMemcpyAsync(flag, zeros, sizeof(zeros), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "device check reset");
    if (h[2] < 0)
        return fail(MLA_ERR_DEVICE_CHECK, "device check: %d offences; first: sequence %d has length %d, outside "
                    "[0, 64 * bt_stride = %lld]", h[0], h[1], h[3], (long long)kBlock * bt_stride);
    return fail(MLA_ERR_DEVICE_CHECK, "device check: %d offences; first: sequence %d, table entry %d holds block id "
                "%d, outside [0, %lld)", h[0], h[1], h[2], h[3], (long long)num_blocks);
}

}  // namespace

extern "C" {

mla_status_t mla_set_debug(int32_t on) {
    if (on != 0 && on != 1) return fail(MLA_ERR_INVALID_ARG, "mla_set_debug takes 0 or 1, not %d", on);
    g_debug.store(on);
    return ok();
}

int32_t mla_debug(void) { return debug_on() ? 1 : 0; }

mla_status_t mla_decode_noalloc(const void *q_lat, const void *q_rope, mla_dtype_t q_dtype,
                                const mla_cache_desc_t *cache, const int32_t *block_table,
                                int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                                int32_t q_len, int32_t n_h, float scale, const mla_plan_t *plan,
                                const int32_t *plan_dev, void *o_lat, float *lse,
                                mla_stream_t stream) {
    if (!plan) return fail(MLA_ERR_INVALID_ARG, "missing decode plan");
    if (plan->workspace_bytes < 0 || plan->workspace_bytes > (int64_t)MLA_NOALLOC_SCRATCH_BYTES)
        return fail(MLA_ERR_WORKSPACE, "plan needs %lld workspace bytes, beyond the %lld-byte scratch of "
                    "mla_decode_noalloc", (long long)plan->workspace_bytes, (long long)MLA_NOALLOC_SCRATCH_BYTES);
    // every argument check first (the scratch address is only a stand-in
    // here: a non-NULL, 256-byte aligned placeholder), then the one HIP call
    // that resolves it
    DecodeArgs a;
    mla_status_t st = prepare_decode(q_lat, q_rope, q_dtype, cache, block_table, bt_stride, seq_lens, B, q_len,
                                     n_h, scale, plan, plan_dev, (void *)(uintptr_t)256,
                                     MLA_NOALLOC_SCRATCH_BYTES, o_lat, lse, &a);
    if (st != MLA_OK) return st;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != MLA_OK) return st;
    st = prepare_decode(q_lat, q_rope, q_dtype, cache, block_table, bt_stride, seq_lens, B, q_len, n_h, scale,
                        plan, plan_dev, ws, MLA_NOALLOC_SCRATCH_BYTES, o_lat, lse, &a);
    if (st != MLA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (debug_on()) {
        st = device_check(block_table, bt_stride, seq_lens, B, cache->num_blocks, s);
        if (st != MLA_OK) return st;
    }
    hipError_t e = launch_decode(a, s);
    if (e != hipSuccess) return hip_status(e, "decode launch");
    return finish_decode(plan, plan_dev, ws, q_dtype, o_lat, lse, s);
}

mla_status_t mla_decode_partial(const void *q_lat, const void *q_rope, mla_dtype_t q_dtype,
                                const mla_cache_desc_t *cache, const int32_t *block_table,
                                int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                                int32_t q_len, int32_t n_h, float scale, const mla_plan_t *plan,
                                const int32_t *plan_dev, void *workspace,
                                int64_t workspace_bytes, void *o_lat, float *lse,
                                mla_stream_t stream) {
    DecodeArgs a;
    mla_status_t st = prepare_decode(q_lat, q_rope, q_dtype, cache, block_table, bt_stride, seq_lens,
                                     B, q_len, n_h, scale, plan, plan_dev, workspace,
                                     workspace_bytes, o_lat, lse, &a);
    if (st != MLA_OK) return st;
    if (debug_on()) {
        st = device_check(block_table, bt_stride, seq_lens, B, cache->num_blocks, (hipStream_t)stream);
        if (st != MLA_OK) return st;
    }
    return hip_status(launch_decode(a, (hipStream_t)stream), "decode launch");
}

mla_status_t mla_decode_finish(const mla_plan_t *plan, const int32_t *plan_dev, void *workspace,
                               int64_t workspace_bytes, mla_dtype_t out_dtype, void *o_lat,
                               float *lse, mla_stream_t stream) {
    if (!plan || !plan_dev || !o_lat || !lse)
        return fail(MLA_ERR_INVALID_ARG, "NULL plan/plan_dev/o_lat/lse");
    if (out_dtype != MLA_DT_F32 && out_dtype != MLA_DT_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "out dtype %d unsupported", (int)out_dtype);
    if (workspace_bytes < plan->workspace_bytes)
        return fail(MLA_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)workspace_bytes,
                    (long long)plan->workspace_bytes);
    if (plan->workspace_bytes > 0 && (!workspace || !aligned(workspace, 256)))
        return fail(MLA_ERR_ALIGN, "workspace NULL or not 256-byte aligned");
    return finish_decode(plan, plan_dev, workspace, out_dtype, o_lat, lse, (hipStream_t)stream);
}

mla_status_t mla_combine_lse(const float *o_part, const float *lse_part,
                             const int32_t *split_off, const int32_t *seq_flags, int32_t B,
                             int32_t rows, int32_t d_c, void *o_lat, mla_dtype_t out_dtype,
                             float *lse, mla_stream_t stream) {
    if (!split_off || !o_lat || !lse) return fail(MLA_ERR_INVALID_ARG, "NULL split_off/o_lat/lse");
    if (B < 1 || rows < 1 || d_c < 4 || d_c > 1024 || d_c % 4)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes B=%d rows=%d d_c=%d (d_c in [4,1024], multiple of 4)", B, rows, d_c);
    if (!o_part || !lse_part) return fail(MLA_ERR_INVALID_ARG, "NULL o_part/lse_part");
    if (!aligned(o_part, 16)) return fail(MLA_ERR_ALIGN, "o_part not 16-byte aligned");
    if (out_dtype != MLA_DT_F32 && out_dtype != MLA_DT_BF16)
        return fail(MLA_ERR_UNSUPPORTED, "out dtype %d unsupported", (int)out_dtype);
    return hip_status(launch_combine(o_part, MLA_DT_F32, lse_part, split_off, seq_flags, B, rows,
                                     rows, d_c, o_lat, out_dtype, lse, 0, (hipStream_t)stream),
                      "combine launch");
}

mla_status_t mla_absorb_q(const void *q_nope, int64_t ld_q, const void *w_uk, void *q_lat,
                          int32_t T, int32_t n_h, int32_t d_nope, int32_t d_c,
                          mla_dtype_t dt, mla_stream_t stream) {
    if (!q_nope || !w_uk || !q_lat) return fail(MLA_ERR_INVALID_ARG, "NULL q_nope/w_uk/q_lat");
    if (T < 1 || n_h < 1 || d_nope < 1 || d_c < 1 || ld_q < (int64_t)n_h * d_nope)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes T=%d n_h=%d d_nope=%d d_c=%d ld_q=%lld", T, n_h,
                    d_nope, d_c, (long long)ld_q);
    if (dt != MLA_DT_F32 && dt != MLA_DT_BF16) return fail(MLA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
    if (!aligned(q_nope, 16) || !aligned(w_uk, 16) || !aligned(q_lat, 16) || (ld_q * elem_bytes(dt)) % 16 ||
        (d_nope * elem_bytes(dt)) % 16 || (d_c * elem_bytes(dt)) % 16)
        return fail(MLA_ERR_ALIGN, "absorb_q operands and rows must be 16-byte aligned");
    return hip_status(launch_absorb_q(q_nope, ld_q, w_uk, q_lat, T, n_h, d_nope, d_c, dt,
                                      (hipStream_t)stream),
                      "absorb_q launch");
}

int64_t mla_absorb_out_workspace(int32_t T, int32_t n_h, int32_t d_v, int32_t d_model,
                                 mla_dtype_t dt) {
    if (T < 1 || n_h < 1 || d_v < 1 || d_model < 1) return 0;
    return absorb_out_workspace(T, n_h, d_v, d_model, dt);
}

mla_status_t mla_absorb_out(const void *o_lat, const void *w_uv, const void *w_o, void *u_ws,
                            void *out, void *f32_ws, int64_t f32_ws_bytes, int32_t T,
                            int32_t n_h, int32_t d_c, int32_t d_v, int32_t d_model,
                            mla_dtype_t dt, mla_stream_t stream) {
    if (!o_lat || !w_uv || !w_o || !u_ws || !out)
        return fail(MLA_ERR_INVALID_ARG, "NULL o_lat/w_uv/w_o/u_ws/out");
    if (T < 1 || n_h < 1 || d_c < 1 || d_v < 1 || d_model < 1)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes T=%d n_h=%d d_c=%d d_v=%d d_model=%d", T, n_h, d_c, d_v, d_model);
    if (dt != MLA_DT_F32 && dt != MLA_DT_BF16) return fail(MLA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
    int64_t need = absorb_out_workspace(T, n_h, d_v, d_model, dt);
    if (f32_ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "absorb_out workspace %lld < %lld", (long long)f32_ws_bytes, (long long)need);
    if (need > 0 && (!f32_ws || !aligned(f32_ws, 256))) return fail(MLA_ERR_ALIGN, "absorb_out workspace NULL or unaligned");
    int eb = elem_bytes(dt);
    if (!aligned(o_lat, 16) || !aligned(w_uv, 16) || !aligned(w_o, 16) || !aligned(u_ws, 16) || !aligned(out, 16) ||
        (d_c * eb) % 16 || (d_v * eb) % 16 || (d_model * eb) % 16)
        return fail(MLA_ERR_ALIGN, "absorb_out operands and rows must be 16-byte aligned");
    return hip_status(launch_absorb_out(o_lat, w_uv, w_o, u_ws, out, (float *)f32_ws, T, n_h, d_c,
                                        d_v, d_model, dt, (hipStream_t)stream),
                      "absorb_out launch");
}

mla_status_t mla_rope_freqs(const mla_rope_t *rope, int32_t d_r, double *theta_host) {
    if (!rope || !theta_host) return fail(MLA_ERR_INVALID_ARG, "NULL rope/theta_host");
    RopeTab t;
    if (!rope_table(rope, d_r, &t))
        return fail(MLA_ERR_INVALID_ARG, "bad rope (d_r=%d base=%g factor=%g orig_ctx=%g mscale=%g)", d_r,
                    rope->base, rope->factor, rope->orig_ctx, rope->mscale);
    for (int j = 0; j < t.half; ++j) theta_host[j] = t.theta[j];
    return ok();
}

int64_t mla_cache_append_workspace(int32_t T, int32_t d_model, int32_t d_c, int32_t d_r,
                                   mla_dtype_t dt) {
    if (T < 1 || d_model < 1 || d_c < 1 || d_r < 0) return 0;
    return cache_append_workspace(T, d_model, d_c, d_r, dt);
}

mla_status_t mla_cache_append(const void *h, const void *w_kv, mla_dtype_t dt,
                              const mla_cache_desc_t *cache, const int32_t *block_table,
                              int32_t bt_stride, const int32_t *pos0, int32_t B, int32_t q_len,
                              int32_t d_model, const mla_rope_t *rope, void *workspace,
                              int64_t workspace_bytes, mla_stream_t stream) {
    mla_status_t st = check_cache(cache);
    if (st != MLA_OK) return st;
    if (!h || !w_kv || !block_table || !pos0) return fail(MLA_ERR_INVALID_ARG, "NULL h/w_kv/block_table/pos0");
    if (B < 1 || q_len < 1 || d_model < 1 || bt_stride < 1)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes B=%d q_len=%d d_model=%d bt_stride=%d", B, q_len, d_model, bt_stride);
    if (dt != MLA_DT_F32 && dt != MLA_DT_BF16) return fail(MLA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
    RopeTab t{};
    if (cache->d_r > 0) {
        if (!rope) return fail(MLA_ERR_INVALID_ARG, "rope is NULL with d_r=%d", cache->d_r);
        if (!rope_table(rope, cache->d_r, &t))
            return fail(MLA_ERR_INVALID_ARG, "bad rope (base=%g factor=%g orig_ctx=%g mscale=%g)", rope->base,
                        rope->factor, rope->orig_ctx, rope->mscale);
    }
    const int32_t T = B * q_len;
    const int64_t need = cache_append_workspace(T, d_model, cache->d_c, cache->d_r, dt);
    if (workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE, "cache_append workspace %lld < %lld", (long long)workspace_bytes, (long long)need);
    if (!workspace || !aligned(workspace, 256)) return fail(MLA_ERR_ALIGN, "workspace NULL or not 256-byte aligned");
    // (row alignment is part of the MFMA path's shape test; other shapes run a generic kernel)
    if (!aligned(h, 16) || !aligned(w_kv, 16)) return fail(MLA_ERR_ALIGN, "h / w_kv must be 16-byte aligned");
    return hip_status(launch_cache_append(h, w_kv, dt, (uint8_t *)cache->base, (float *)cache->block_scales,
                                          block_bytes_of(cache->kv_dtype, cache->d_c, cache->d_r),
                                          cache->num_blocks, cache->kv_dtype, block_table, bt_stride, pos0, B,
                                          q_len, d_model, cache->d_c, cache->d_r, t, (float *)workspace,
                                          (hipStream_t)stream),
                      "cache_append launch");
}

int64_t mla_project_q_workspace(int32_t T, int32_t d_model, int32_t q_lora, int32_t n_h,
                                int32_t d_nope, int32_t d_c, int32_t d_r, mla_dtype_t dt) {
    if (T < 1 || d_model < 1 || q_lora < 1 || n_h < 1 || d_nope < 1 || d_c < 1 || d_r < 0) return 0;
    return project_q_workspace(T, d_model, q_lora, n_h, d_nope, d_c, d_r, dt);
}

mla_status_t mla_project_q(const void *h, const void *w_dq, const void *w_uq, const void *w_qr,
                           const void *w_uk, mla_dtype_t dt, const int32_t *pos, int32_t T,
                           int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope,
                           int32_t d_c, int32_t d_r, const mla_rope_t *rope, void *q_lat,
                           void *q_rope, void *workspace, int64_t workspace_bytes,
                           mla_stream_t stream) {
    if (!h || !w_dq || !w_uq || !w_uk || !pos || !q_lat)
        return fail(MLA_ERR_INVALID_ARG, "NULL h/w_dq/w_uq/w_uk/pos/q_lat");
    if (T < 1 || d_model < 1 || q_lora < 1 || n_h < 1 || d_nope < 1 || d_c < 1 || d_r < 0)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes T=%d d_model=%d q_lora=%d n_h=%d d_nope=%d d_c=%d d_r=%d", T,
                    d_model, q_lora, n_h, d_nope, d_c, d_r);
    if (dt != MLA_DT_F32 && dt != MLA_DT_BF16) return fail(MLA_ERR_UNSUPPORTED, "dtype %d", (int)dt);
    RopeTab t{};
    if (d_r > 0) {
        if (!w_qr || !q_rope || !rope) return fail(MLA_ERR_INVALID_ARG, "NULL w_qr/q_rope/rope with d_r=%d", d_r);
        if (!rope_table(rope, d_r, &t))
            return fail(MLA_ERR_INVALID_ARG, "bad rope (d_r=%d base=%g factor=%g orig_ctx=%g mscale=%g)", d_r,
                        rope->base, rope->factor, rope->orig_ctx, rope->mscale);
    }
    const int64_t need = project_q_workspace(T, d_model, q_lora, n_h, d_nope, d_c, d_r, dt);
    if (workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE, "project_q workspace %lld < %lld", (long long)workspace_bytes, (long long)need);
    if (!workspace || !aligned(workspace, 256)) return fail(MLA_ERR_ALIGN, "workspace NULL or not 256-byte aligned");
    if (!aligned(h, 16) || !aligned(w_dq, 16) || !aligned(w_uq, 16) || !aligned(w_uk, 16) || !aligned(q_lat, 16) ||
        (d_r > 0 && (!aligned(w_qr, 16) || !aligned(q_rope, 16))))
        return fail(MLA_ERR_ALIGN, "project_q operands must be 16-byte aligned");
    if (d_r == 0) return fail(MLA_ERR_UNSUPPORTED, "project_q needs d_r > 0");
    return hip_status(launch_project_q(h, w_dq, w_uq, w_qr, w_uk, dt, pos, T, d_model, q_lora, n_h, d_nope, d_c,
                                       d_r, t, q_lat, q_rope, workspace, (hipStream_t)stream),
                      "project_q launch");
}

int64_t mla_project_step_workspace(int32_t B, int32_t q_len, int32_t d_model, int32_t q_lora, int32_t n_h,
                                   int32_t d_nope, int32_t d_c, int32_t d_r, mla_dtype_t dt) {
    if (B < 1 || q_len < 1 || (int64_t)B * q_len > INT32_MAX || d_model < 1 || q_lora < 1 || n_h < 1 ||
        d_nope < 1 || d_c < 1 || d_r < 1)
        return 0;
    if (!project_step_ok(dt, B * q_len, d_model, q_lora, n_h, d_nope, d_c, d_r)) return 0;
    return project_step_workspace(B * q_len, d_model, q_lora, n_h, d_c, d_r);
}

mla_status_t mla_project_step(const void *h, const void *w_dkvq, const void *w_uq, const void *w_qr,
                              const void *w_uk, mla_dtype_t dt, const mla_cache_desc_t *cache,
                              const int32_t *block_table, int32_t bt_stride, const int32_t *pos0, int32_t B,
                              int32_t q_len, int32_t d_model, int32_t q_lora, int32_t n_h, int32_t d_nope,
                              const mla_rope_t *rope, void *q_lat, void *q_rope, void *workspace,
                              int64_t workspace_bytes, mla_stream_t stream) {
    mla_status_t st = check_cache(cache);
    if (st != MLA_OK) return st;
    if (!h || !w_dkvq || !w_uq || !w_qr || !w_uk || !block_table || !pos0 || !rope || !q_lat || !q_rope)
        return fail(MLA_ERR_INVALID_ARG, "NULL h/w_dkvq/w_uq/w_qr/w_uk/block_table/pos0/rope/q_lat/q_rope");
    if (B < 1 || q_len < 1 || (int64_t)B * q_len > INT32_MAX || d_model < 1 || q_lora < 1 || n_h < 1 ||
        d_nope < 1 || bt_stride < 1)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes B=%d q_len=%d d_model=%d q_lora=%d n_h=%d d_nope=%d bt_stride=%d",
                    B, q_len, d_model, q_lora, n_h, d_nope, bt_stride);
    const int32_t d_c = cache->d_c, d_r = cache->d_r, T = B * q_len;
    if (d_r < 1) return fail(MLA_ERR_UNSUPPORTED, "project_step needs d_r > 0");
    if (!project_step_ok(dt, T, d_model, q_lora, n_h, d_nope, d_c, d_r))
        return fail(MLA_ERR_UNSUPPORTED,
                    "project_step shape (dt=%d T=%d d_model=%d q_lora=%d n_h=%d d_nope=%d d_c=%d d_r=%d): use "
                    "mla_project_q and mla_cache_append", (int)dt, T, d_model, q_lora, n_h, d_nope, d_c, d_r);
    RopeTab t{};
    if (!rope_table(rope, d_r, &t))
        return fail(MLA_ERR_INVALID_ARG, "bad rope (d_r=%d base=%g factor=%g orig_ctx=%g mscale=%g)", d_r,
                    rope->base, rope->factor, rope->orig_ctx, rope->mscale);
    const int64_t need = project_step_workspace(T, d_model, q_lora, n_h, d_c, d_r);
    if (workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE, "project_step workspace %lld < %lld", (long long)workspace_bytes,
                    (long long)need);
    if (!workspace || !aligned(workspace, 256)) return fail(MLA_ERR_ALIGN, "workspace NULL or not 256-byte aligned");
    if (!aligned(h, 16) || !aligned(w_dkvq, 16) || !aligned(w_uq, 16) || !aligned(w_qr, 16) || !aligned(w_uk, 16) ||
        !aligned(q_lat, 16) || !aligned(q_rope, 16))
        return fail(MLA_ERR_ALIGN, "project_step operands must be 16-byte aligned");
    return hip_status(launch_project_step(h, w_dkvq, w_uq, w_qr, w_uk, (uint8_t *)cache->base,
                                          (float *)cache->block_scales,
                                          block_bytes_of(cache->kv_dtype, d_c, d_r), cache->num_blocks,
                                          cache->kv_dtype, block_table, bt_stride, pos0, B, q_len, d_model, q_lora,
                                          n_h, d_c, d_r, t, q_lat, q_rope, workspace, (hipStream_t)stream),
                      "project_step launch");
}

mla_status_t mla_gather_paged(const mla_cache_desc_t *cache, const int32_t *block_table,
                              int32_t bt_stride, const int32_t *seq_lens, int32_t B,
                              int32_t max_tokens, void *out, mla_stream_t stream) {
    mla_status_t st = check_cache(cache);
    if (st != MLA_OK) return st;
    if (!block_table || !seq_lens || !out) return fail(MLA_ERR_INVALID_ARG, "NULL block_table/seq_lens/out");
    if (B < 1 || max_tokens < 1 || bt_stride < 1)
        return fail(MLA_ERR_INVALID_ARG, "bad sizes B=%d max_tokens=%d bt_stride=%d", B, max_tokens, bt_stride);
    if ((int64_t)max_tokens > (int64_t)kBlock * bt_stride)
        return fail(MLA_ERR_INVALID_ARG, "max_tokens %d > %d positions of a block-table row", max_tokens,
                    kBlock * bt_stride);
    if (!aligned(out, 16)) return fail(MLA_ERR_ALIGN, "out not 16-byte aligned");
    if (debug_on()) {
        st = device_check(block_table, bt_stride, seq_lens, B, cache->num_blocks, (hipStream_t)stream);
        if (st != MLA_OK) return st;
    }
    int eb = elem_bytes(cache->kv_dtype);
    bool split = cache->kv_dtype == MLA_DT_FP8_E4M3 || cache->kv_dtype == MLA_DT_FP8_E5M2;
    int32_t c_bytes = split ? cache->d_c : (cache->d_c + cache->d_r) * eb;
    int32_t r_bytes = split ? cache->d_r * 2 : 0;
    return hip_status(launch_gather((const uint8_t *)cache->base,
                                    block_bytes_of(cache->kv_dtype, cache->d_c, cache->d_r),
                                    cache->num_blocks, c_bytes, r_bytes, split, block_table, bt_stride,
                                    seq_lens, B,
                                    max_tokens, (uint8_t *)out, (hipStream_t)stream),
                      "gather launch");
}

mla_status_t mla_clock_probe(int64_t *out, int32_t wgs, int32_t iters, mla_stream_t stream) {
    if (!out) return fail(MLA_ERR_INVALID_ARG, "out is NULL");
    if (wgs < 1 || wgs > (1 << 16) || iters < 1 || iters > (1 << 24))
        return fail(MLA_ERR_INVALID_ARG, "bad probe size wgs=%d iters=%d", wgs, iters);
    if (!aligned(out, 8)) return fail(MLA_ERR_ALIGN, "out not 8-byte aligned");
    return hip_status(launch_clock_probe(out, wgs, iters, (hipStream_t)stream), "clock probe launch");
}

}  // extern "C"
