// plan.cpp -- host-side split-KV partitioner of libpa.
//
// The plan is computed once per decode step and reused by every layer
// (Agent-Infer page, "Agent-Infer: 纯 Rust 编写的高性能 LLM 推理引擎", section
// "分页 KV 缓存", and stage 3 of the table in "优化历程").  How the work is cut
// is not on the pages; this file's policy is:
//
// Decode.  The work of request b is Hkv independent streams (one per KV head)
// of L_b tokens.  A work unit is one workgroup: one (request, KV head) and a
// contiguous part of the list.  Parts have a fixed length S for the whole
// step, so part j of every request covers list positions [j*S, (j+1)*S) --
// requests that share a prompt prefix (radix prefix cache, Agent-Infer page,
// section "前缀缓存") read the same slots in their part-0 units.  S is chosen
// so the launch holds about kTargetUnitsPerCu workgroups per compute unit,
// never below kMinUnitBytes of K+V per unit, rounded to kUnitGranule tokens.
// A request cut into n > 1 parts writes n partial results that a merge unit
// combines by log-sum-exp weights.
//
// Prefill.  A unit is one (request, KV head, tile of chunk rows); the tile
// stacks the group's query heads so it holds kPrefillTileRows rows.  The KV
// range of a tile ends at the causal window of its last row.  When there are
// too few tiles to fill the GPU, the KV range is also cut into parts and
// merged the same way.
//
// XCD order.  Workgroup i runs on XCD i % 8 and each XCD has its own L2.  Units
// are grouped into clusters (same part, same KV head, 16 consecutive
// requests), clusters are spread over the XCDs to balance tokens (largest
// first onto the least loaded XCD), and each XCD's queue is turned into
// workgroup ids x, x+8, x+16, ...  Units of one cluster therefore run close in
// time on one XCD, where reads of shared slots can hit its L2.  Queues are
// padded to equal length with empty units.
#include <algorithm>
#include <cstring>
#include <numeric>
#include <vector>

#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kClusterRequests = 16;

struct Unit {
    pa_work_unit u;
    int32_t part;      // index of the part within its (request, head) range
    int64_t tokens;    // list entries the unit reads (for balance)
};

int32_t forced_splits(uint32_t flags) {
    return (int32_t)((flags & PA_PLAN_FORCE_SPLITS_MASK) >> PA_PLAN_FORCE_SPLITS_SHIFT);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Place units on XCD queues and return them in workgroup-id order (with
// padding units).  `units` are in the natural (request, head, part) order.
std::vector<pa_work_unit> xcd_order(const std::vector<Unit> &units, int num_xcd) {
    if (units.empty())
        return {};
    struct Cluster {
        int64_t tokens = 0;
        std::vector<int32_t> members;
        int32_t part, head, block;
    };
    // cluster key: (part, head, request block)
    std::vector<int32_t> order(units.size());
    std::iota(order.begin(), order.end(), 0);
    auto key = [&](int32_t i) {
        const Unit &x = units[i];
        return std::make_tuple(x.part, x.u.kv_head, x.u.request / kClusterRequests, x.u.request,
                               x.u.q_begin);
    };
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return key(a) < key(b); });
    std::vector<Cluster> clusters;
    for (int32_t i : order) {
        const Unit &x = units[i];
        int32_t blk = x.u.request / kClusterRequests;
        if (clusters.empty() || clusters.back().part != x.part ||
            clusters.back().head != x.u.kv_head || clusters.back().block != blk) {
            clusters.push_back(Cluster{});
            clusters.back().part = x.part;
            clusters.back().head = x.u.kv_head;
            clusters.back().block = blk;
        }
        clusters.back().tokens += std::max<int64_t>(x.tokens, 1);
        clusters.back().members.push_back(i);
    }
    // largest cluster first onto the least loaded XCD (ties: lower XCD)
    std::vector<int32_t> corder(clusters.size());
    std::iota(corder.begin(), corder.end(), 0);
    std::stable_sort(corder.begin(), corder.end(), [&](int32_t a, int32_t b) {
        return clusters[a].tokens > clusters[b].tokens;
    });
    std::vector<int64_t> load(num_xcd, 0);
    std::vector<std::vector<int32_t>> queue(num_xcd);
    for (int32_t c : corder) {
        int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
        load[x] += clusters[c].tokens;
        for (int32_t m : clusters[c].members)
            queue[x].push_back(m);
    }
    size_t depth = 0;
    for (auto &q : queue)
        depth = std::max(depth, q.size());
    pa_work_unit pad;
    std::memset(&pad, 0, sizeof pad);
    pad.request = -1;
    pad.partial = -1;
    std::vector<pa_work_unit> out(depth * num_xcd, pad);
    for (int x = 0; x < num_xcd; x++)
        for (size_t p = 0; p < queue[x].size(); p++)
            out[p * num_xcd + x] = units[queue[x][p]].u;
    return out;
}

pa_status fail(const char **detail, const char *msg, pa_status s) {
    if (detail)
        *detail = msg;
    return s;
}

}  // namespace

bool supported_shape(int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim) {
    if (num_kv_heads <= 0 || num_qo_heads <= 0 || num_qo_heads % num_kv_heads != 0)
        return false;
    int32_t g = num_qo_heads / num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return false;
    return head_dim == 128 || head_dim == 256;
}

static int64_t min_unit_tokens(int32_t head_dim) {
    // K and V rows of one head: 2 * head_dim bf16 values per token
    return std::max<int64_t>(kUnitGranule, kMinUnitBytes / (4 * (int64_t)head_dim));
}

static int32_t prefill_tile_tokens(int32_t group) { return kPrefillTileRows / group; }

void partition_capacity(int32_t max_batch, int64_t max_kv_total, int32_t max_q_total,
                        int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t num_xcd, int64_t *max_units, int64_t *max_merges,
                        int64_t *max_partial_rows) {
    int32_t g = num_qo_heads / num_kv_heads;
    // decode, automatic split: ceil(L/S) <= L/S + 1 with S >= the minimum
    int64_t dec = (int64_t)num_kv_heads * (max_batch + ceil_div(max_kv_total, min_unit_tokens(head_dim)));
    // prefill: tiles, then at most ~4 units per CU after KV splitting
    int64_t tiles = 0, pre = 0;
    if (max_q_total > 0) {
        int32_t qt = prefill_tile_tokens(g);
        tiles = (int64_t)num_kv_heads * (ceil_div(max_q_total, qt) + max_batch);
        pre = std::max<int64_t>(tiles, 4LL * kNumCu + tiles);
    }
    int64_t units = std::max(dec, pre);
    // padding to equal XCD queues can at worst multiply by the XCD count
    *max_units = units * num_xcd;
    *max_merges = std::max(dec, tiles);
    // partial storage is counted in rows of head_dim floats: a decode partial
    // slot holds the group's g rows, a prefill slot a whole tile
    int64_t dec_rows = dec * g;
    int64_t pre_rows = (max_q_total > 0) ? pre * kPrefillTileRows : 0;
    *max_partial_rows = std::max(dec_rows, pre_rows);
}

pa_status partition(const PartitionArgs &a, pa_work_unit *units_out, int32_t unit_capacity,
                    pa_merge_unit *merges_out, int32_t merge_capacity, PartitionResult *res,
                    const char **detail) {
    *res = PartitionResult{};
    if (a.batch < 0)
        return fail(detail, "batch < 0", PA_ERR_INVALID_ARG);
    if (a.batch > 0 && !a.kv_indptr)
        return fail(detail, "kv_indptr is null", PA_ERR_INVALID_ARG);
    if (!supported_shape(a.num_qo_heads, a.num_kv_heads, a.head_dim))
        return fail(detail, "unsupported head shape (need Hq/Hkv in {1,2,4,8}, D in {128,256})",
                    PA_ERR_UNSUPPORTED);
    const int32_t Hkv = a.num_kv_heads;
    const int32_t g = a.num_qo_heads / a.num_kv_heads;
    const int32_t forced = forced_splits(a.flags);
    if (forced > PA_MAX_FORCED_SPLITS)
        return fail(detail, "forced split count above PA_MAX_FORCED_SPLITS", PA_ERR_INVALID_ARG);
    if ((a.flags & ~(PA_PLAN_FORCE_SPLITS_MASK | PA_PLAN_NO_XCD_ORDER)) != 0)
        return fail(detail, "unknown flag bits", PA_ERR_INVALID_ARG);
    if (a.batch > 0) {
        if (a.kv_indptr[0] != 0)
            return fail(detail, "kv_indptr[0] != 0", PA_ERR_INVALID_ARG);
        for (int32_t b = 0; b < a.batch; b++)
            if (a.kv_indptr[b + 1] < a.kv_indptr[b])
                return fail(detail, "kv_indptr decreases", PA_ERR_INVALID_ARG);
    }
    const bool prefill = a.qo_indptr != nullptr;
    if (prefill && a.batch > 0) {
        if (a.qo_indptr[0] != 0)
            return fail(detail, "qo_indptr[0] != 0", PA_ERR_INVALID_ARG);
        for (int32_t b = 0; b < a.batch; b++) {
            if (a.qo_indptr[b + 1] < a.qo_indptr[b])
                return fail(detail, "qo_indptr decreases", PA_ERR_INVALID_ARG);
            if (a.qo_indptr[b + 1] - a.qo_indptr[b] > a.kv_indptr[b + 1] - a.kv_indptr[b])
                return fail(detail, "chunk longer than its slot list", PA_ERR_INVALID_ARG);
        }
    }

    std::vector<Unit> units;
    std::vector<pa_merge_unit> merges;
    int32_t n_partials = 0;

    if (!prefill) {
        int64_t S = 0;
        if (!forced) {
            int64_t total = a.batch > 0 ? a.kv_indptr[a.batch] : 0;
            int64_t work = total * Hkv;
            int64_t target = (int64_t)std::max(1, a.num_cu) * kTargetUnitsPerCu;
            S = std::max(ceil_div(work, target), min_unit_tokens(a.head_dim));
            S = ceil_div(S, kUnitGranule) * kUnitGranule;
            res->unit_tokens = (int32_t)S;
        }
        for (int32_t b = 0; b < a.batch; b++) {
            const int32_t beg = a.kv_indptr[b], L = a.kv_indptr[b + 1] - a.kv_indptr[b];
            const int32_t n = forced ? forced : (int32_t)std::max<int64_t>(1, ceil_div(L, S));
            for (int32_t h = 0; h < Hkv; h++) {
                int32_t first = n_partials;
                for (int32_t j = 0; j < n; j++) {
                    int64_t lo, hi;
                    if (forced) {
                        lo = (int64_t)L * j / n;
                        hi = (int64_t)L * (j + 1) / n;
                    } else {
                        lo = std::min<int64_t>(L, j * S);
                        hi = std::min<int64_t>(L, (j + 1) * S);
                    }
                    Unit x;
                    x.u.request = b;
                    x.u.kv_head = h;
                    x.u.kv_begin = beg + (int32_t)lo;
                    x.u.kv_end = beg + (int32_t)hi;
                    x.u.q_begin = b;
                    x.u.q_end = b + 1;
                    x.u.partial = n > 1 ? n_partials++ : -1;
                    x.u.diag = x.u.kv_end - 1;
                    x.part = j;
                    x.tokens = hi - lo;
                    units.push_back(x);
                }
                if (n > 1) {
                    pa_merge_unit m;
                    std::memset(&m, 0, sizeof m);
                    m.request = b;
                    m.kv_head = h;
                    m.q_begin = b;
                    m.q_end = b + 1;
                    m.first_partial = first;
                    m.n_parts = n;
                    merges.push_back(m);
                }
            }
        }
    } else {
        const int32_t qt = prefill_tile_tokens(g);
        // tiles: (request, head, chunk-row tile)
        int64_t n_tiles = 0;
        for (int32_t b = 0; b < a.batch; b++)
            n_tiles += (int64_t)Hkv * ceil_div(a.qo_indptr[b + 1] - a.qo_indptr[b], qt);
        // cut KV ranges only when the tiles alone cannot fill the GPU
        int64_t part_len = 0;  // 0 = no cut
        if (forced == 0 && n_tiles > 0 && n_tiles < 2LL * a.num_cu) {
            int64_t kv_work = 0;
            for (int32_t b = 0; b < a.batch; b++) {
                int64_t C = a.qo_indptr[b + 1] - a.qo_indptr[b];
                if (C > 0)
                    kv_work += (int64_t)Hkv * ceil_div(C, qt) * (a.kv_indptr[b + 1] - a.kv_indptr[b]);
            }
            part_len = std::max<int64_t>(256, ceil_div(kv_work, 4LL * a.num_cu));
            part_len = ceil_div(part_len, 64) * 64;
        }
        for (int32_t b = 0; b < a.batch; b++) {
            const int32_t kv0 = a.kv_indptr[b];
            const int32_t L = a.kv_indptr[b + 1] - kv0;
            const int32_t q0 = a.qo_indptr[b];
            const int32_t C = a.qo_indptr[b + 1] - q0;
            const int32_t P = L - C;
            for (int32_t h = 0; h < Hkv; h++) {
                for (int32_t t0 = 0; t0 < C; t0 += qt) {
                    const int32_t t1 = std::min(C, t0 + qt);
                    const int64_t visible = (int64_t)P + t1;  // list entries the last row sees
                    int32_t n = 1;
                    if (forced)
                        n = forced;
                    else if (part_len)
                        n = (int32_t)std::max<int64_t>(1, ceil_div(visible, part_len));
                    int32_t first = n_partials;
                    for (int32_t j = 0; j < n; j++) {
                        int64_t lo = visible * j / n, hi = visible * (j + 1) / n;
                        if (!forced && part_len) {
                            lo = std::min<int64_t>(visible, j * part_len);
                            hi = std::min<int64_t>(visible, (j + 1) * part_len);
                        }
                        Unit x;
                        x.u.request = b;
                        x.u.kv_head = h;
                        x.u.kv_begin = kv0 + (int32_t)lo;
                        x.u.kv_end = kv0 + (int32_t)hi;
                        x.u.q_begin = q0 + t0;
                        x.u.q_end = q0 + t1;
                        x.u.partial = n > 1 ? n_partials++ : -1;
                        x.u.diag = kv0 + P + t0;
                        x.part = j;
                        x.tokens = (hi - lo) * (t1 - t0);
                        units.push_back(x);
                    }
                    if (n > 1) {
                        pa_merge_unit m;
                        std::memset(&m, 0, sizeof m);
                        m.request = b;
                        m.kv_head = h;
                        m.q_begin = q0 + t0;
                        m.q_end = q0 + t1;
                        m.first_partial = first;
                        m.n_parts = n;
                        merges.push_back(m);
                    }
                }
            }
        }
    }

    std::vector<pa_work_unit> ordered;
    if ((a.flags & PA_PLAN_NO_XCD_ORDER) || a.num_xcd <= 1) {
        ordered.reserve(units.size());
        for (auto &x : units)
            ordered.push_back(x.u);
    } else {
        ordered = xcd_order(units, a.num_xcd);
    }

    res->n_units = (int32_t)ordered.size();
    res->n_merges = (int32_t)merges.size();
    res->n_partials = n_partials;
    if (res->n_units > unit_capacity || res->n_merges > merge_capacity)
        return fail(detail, "plan capacity exceeded", PA_ERR_CAPACITY);
    if (!ordered.empty())
        std::memcpy(units_out, ordered.data(), ordered.size() * sizeof(pa_work_unit));
    if (!merges.empty())
        std::memcpy(merges_out, merges.data(), merges.size() * sizeof(pa_merge_unit));
    return PA_OK;
}

}  // namespace pa
