// plan.cpp -- host-side split-KV partitioner of libpa.
//
// The plan is computed once per decode step and reused by every layer
// (Agent-Infer page, "Agent-Infer: 纯 Rust 编写的高性能 LLM 推理引擎", section
// "分页 KV 缓存", and stage 3 of the table in "优化历程").  How the work is cut
// is not on the pages; this file's policy is:
//
// Decode (automatic).  The work of request b is Hkv independent streams
// ("segments", one per KV head) of L_b list entries.  The launch holds exactly
// as many workgroups as the GPU keeps resident at once (kernel occupancy x
// compute units), so every workgroup starts at time zero and none waits for a
// free slot; each gets an equal budget of list entries (plus a fixed cost per
// piece of work it handles), scaled by its XCD's weight when the caller gives
// per-XCD or per-workgroup weights (the XCDs and compute units of one GPU do
// not run at equal speeds; see PA_PLAN_SPEED_FEEDBACK in pa.h).  Segments are taken in (KV head, request) order:
// the first piece of segment i opens workgroup i, so requests that sit next to
// each other in the batch -- those that share a prompt prefix under a radix
// prefix cache (Agent-Infer page, section "前缀缓存") -- read their common
// leading slots at the same moment; the rest of every segment is then streamed
// over the workgroups in order, cut where a workgroup's budget ends.  A
// workgroup runs its pieces one after another.  A segment cut into n > 1
// pieces writes n partial results that a merge unit combines by log-sum-exp
// weights.  Workgroups are laid out in contiguous blocks per XCD (workgroup id
// w runs on XCD w % 8, each XCD with its own L2), so neighbouring segments
// share an L2.
//
// Decode with forced splits, and prefill.  One unit per workgroup.  Prefill
// units are (request, KV head, tile of chunk rows); the tile stacks the
// group's query heads so it holds prefill_tile_rows(head_dim) rows, and its KV range ends
// at the causal window of its last row.  When the tiles alone cannot fill the
// GPU, KV ranges are also cut and merged.  Units are grouped into clusters
// (same part, same KV head, 16 consecutive requests) that are spread over the
// XCDs by token balance, largest first.
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

using Groups = std::vector<std::vector<pa_work_unit>>;  // workgroup id -> its units

int32_t forced_splits(uint32_t flags) {
    return (int32_t)((flags & PA_PLAN_FORCE_SPLITS_MASK) >> PA_PLAN_FORCE_SPLITS_SHIFT);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One unit per workgroup: place units on XCD queues by cluster and return the
// workgroups in id order (empty workgroups pad the queues to equal depth).
Groups xcd_order_single(const std::vector<Unit> &units, int num_xcd) {
    if (units.empty())
        return {};
    struct Cluster {
        int64_t tokens = 0;
        std::vector<int32_t> members;
        int32_t part, head, block;
    };
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
    Groups out(depth * num_xcd);
    for (int x = 0; x < num_xcd; x++)
        for (size_t p = 0; p < queue[x].size(); p++)
            out[p * num_xcd + x].push_back(units[queue[x][p]].u);
    return out;
}

Groups plain_single(const std::vector<Unit> &units) {
    Groups out(units.size());
    for (size_t i = 0; i < units.size(); i++)
        out[i].push_back(units[i].u);
    return out;
}

pa_status fail(const char **detail, const char *msg, pa_status s) {
    if (detail)
        *detail = msg;
    return s;
}

int64_t min_unit_tokens(int32_t head_dim) {
    // K and V rows of one head: 2 * head_dim bf16 values per token
    return std::max<int64_t>(kUnitGranule, kMinUnitBytes / (4 * (int64_t)head_dim));
}

int32_t prefill_tile_tokens(int32_t group, int32_t head_dim) { return prefill_tile_rows(head_dim) / group; }

// ---------------------------------------------------------------------------
// decode, automatic: balanced workgroup bins
// ---------------------------------------------------------------------------
// Segment s = h * B + b is KV head h of request b.  Bin i (one workgroup)
// holds the opening piece of segment i (i < number of segments), then a run
// of the "stream": the remainders of all segments in segment order, cut into
// pieces where a bin's budget ends.  Pass 1 cuts the stream; pass 2 numbers
// partial slots and merge units; pass 3 writes the units workgroup by
// workgroup.  Linear in segments + bins; the arrays live in the caller's
// workspace, which only grows.
pa_status decode_bins(const PartitionArgs &a, PartitionScratch &ws, int32_t *wg_offsets,
                      int32_t wg_capacity, pa_work_unit *units_out, int32_t unit_capacity,
                      pa_merge_unit *merges_out, int32_t merge_capacity, PartitionResult *res,
                      const char **detail) {
    const int32_t B = a.batch, Hkv = a.num_kv_heads;
    const int64_t n_seg = (int64_t)B * Hkv;
    // request of each segment, filled without divisions (segments are few,
    // but one integer division per piece would dominate the partition)
    ws.seg_request.resize(n_seg);
    for (int32_t h = 0, s = 0; h < Hkv; h++)
        for (int32_t b = 0; b < B; b++)
            ws.seg_request[s++] = b;
    // entries a request's decode units skip at the start of its list (the
    // shared prefix of a cascade plan, read by the prefix units)
    auto skip_of = [&](int32_t b) { return a.kv_skip ? a.kv_skip[b] : 0; };
    auto seg_len = [&](int64_t s) {
        const int32_t b = ws.seg_request[s];
        return a.kv_indptr[b + 1] - a.kv_indptr[b] - skip_of(b);
    };
    int64_t total = B > 0 ? (int64_t)a.kv_indptr[B] * Hkv : 0;
    if (a.kv_skip)
        for (int32_t b = 0; b < B; b++)
            total -= (int64_t)a.kv_skip[b] * Hkv;
    // a segment whose request has a cascade prefix always writes a partial:
    // its merge folds the prefix parts in
    auto must_merge = [&](int64_t s) { return skip_of(ws.seg_request[s]) > 0; };
    const int64_t max_wg = std::max(1, a.max_workgroups);
    const int64_t n = std::max<int64_t>(1, std::min(max_wg, ceil_div(total, min_unit_tokens(a.head_dim))));
    const double ov = kPieceOverheadTokens;
    const bool xcd = !(a.flags & PA_PLAN_NO_XCD_ORDER) && a.num_xcd > 1;
    const int64_t per_xcd = xcd ? ceil_div(n, a.num_xcd) : n;
    // Bin i runs as workgroup wg_of(i), on XCD i / per_xcd when placed by
    // XCD.  Its budget is base * (weight of that XCD) * (weight of that
    // workgroup id); the budgets add up to the whole work.
    auto wg_of = [&](int64_t i) {
        return xcd ? (i % per_xcd) * a.num_xcd + i / per_xcd : i;
    };
    auto weight_of = [&](int64_t i) {
        double w = (xcd && a.xcd_weights) ? a.xcd_weights[i / per_xcd] : 1.0;
        const int64_t id = wg_of(i);
        if (a.wg_weights && id < a.n_wg_weights)
            w *= a.wg_weights[id];
        return w;
    };
    const bool weighted = (xcd && a.xcd_weights) || a.wg_weights;
    double wsum = (double)n;
    if (weighted) {
        ws.bin_cap.resize(n);
        wsum = 0.0;
        for (int64_t i = 0; i < n; i++) {
            ws.bin_cap[i] = weight_of(i);
            wsum += ws.bin_cap[i];
        }
    }
    const double base = ((double)total + ov * (double)(n_seg + n)) / wsum;
    if (weighted)
        for (int64_t i = 0; i < n; i++)
            ws.bin_cap[i] *= base;
    auto cap_of = [&](int64_t i) { return weighted ? ws.bin_cap[i] : base; };
    // entries of the opening piece of segment s < n
    auto open_len = [&](int64_t s) {
        return (int32_t)std::min<double>(seg_len(s), std::max(0.0, cap_of(s) - ov));
    };

    ws.seg_pieces.assign(n_seg, 0);
    ws.seg_first.resize(n_seg);
    ws.seg_merge.resize(n_seg);
    ws.bin_stream.resize(n + 1);
    ws.stream.clear();

    // pass 1: cut the stream over the bins
    int64_t p = 0;
    double fill = (0 < n_seg) ? open_len(0) + ov : 0.0;  // fill of bin p
    double cap = cap_of(0);                               // its budget
    ws.bin_stream[0] = 0;
    auto advance = [&]() {
        p++;
        ws.bin_stream[p] = (int32_t)ws.stream.size();
        // bins 0 .. n-1 exist (p reaches n only to close bin_stream), and
        // only segments below n have an opening piece
        fill = (p < n && p < n_seg) ? open_len(p) + ov : 0.0;
        if (p < n)
            cap = cap_of(p);
    };
    for (int64_t s = 0; s < n_seg; s++) {
        const int32_t L = seg_len(s);
        int32_t off = 0;
        if (s < n) {
            ws.seg_pieces[s] = 1;  // the opening piece
            off = open_len(s);
            if (off >= L)
                continue;
        }
        if (L == 0) {  // an empty segment still writes its (empty) result
            while (p < n - 1 && fill + ov > cap)
                advance();
            ws.stream.push_back({(int32_t)s, 0, 0, ws.seg_pieces[s]++});
            fill += ov;
            continue;
        }
        while (off < L) {
            while (p < n - 1 && fill + ov + kMinPieceTokens > cap)
                advance();
            int32_t take = L - off;
            if (p < n - 1) {
                take = std::min<int32_t>(take, (int32_t)(cap - fill - ov));
                if (L - off - take < kMinPieceTokens)
                    take = L - off;  // no sliver left for another workgroup
            }
            ws.stream.push_back({(int32_t)s, off, off + take, ws.seg_pieces[s]++});
            fill += take + ov;
            off += take;
        }
    }
    while (p < n)
        advance();  // bin_stream[i] for the bins after the last used one, and [n]

    // pass 2: partial slots contiguous per segment in segment order; merge
    // units in (request, head) order
    int32_t np = 0;
    for (int64_t s = 0; s < n_seg; s++) {
        const bool merged = ws.seg_pieces[s] > 1 || must_merge(s);
        ws.seg_first[s] = merged ? np : -1;
        np += merged ? ws.seg_pieces[s] : 0;
    }
    int32_t n_merges = 0;
    for (int32_t b = 0; b < B; b++)
        for (int32_t h = 0; h < Hkv; h++) {
            const int64_t s = (int64_t)h * B + b;
            ws.seg_merge[s] = ws.seg_first[s] >= 0 ? n_merges++ : -1;
        }

    const int64_t n_wg = xcd ? per_xcd * a.num_xcd : n;
    const int64_t n_units = std::min<int64_t>(n, n_seg) + (int64_t)ws.stream.size();
    res->n_workgroups = (int32_t)n_wg;
    res->n_units = (int32_t)n_units;
    res->n_merges = n_merges;
    res->n_partials = np;
    if (n_wg + 1 > wg_capacity || n_units > unit_capacity || n_merges > merge_capacity)
        return fail(detail, "plan capacity exceeded", PA_ERR_CAPACITY);

    for (int32_t b = 0; b < B; b++)
        for (int32_t h = 0; h < Hkv; h++) {
            const int64_t s = (int64_t)h * B + b;
            if (ws.seg_merge[s] < 0)
                continue;
            pa_merge_unit &m = merges_out[ws.seg_merge[s]];
            std::memset(&m, 0, sizeof m);
            m.request = b;
            m.kv_head = h;
            m.q_begin = b;
            m.q_end = b + 1;
            m.first_partial = ws.seg_first[s];
            m.n_parts = ws.seg_pieces[s];
        }

    // pass 3: workgroup ids hold the bins in contiguous blocks per XCD
    // (bin i runs as workgroup (i % per_xcd) * num_xcd + i / per_xcd)
    auto emit = [&](pa_work_unit &u, int32_t seg, int32_t lo, int32_t hi, int32_t ordinal) {
        const int32_t b = ws.seg_request[seg];
        u.request = b;
        u.kv_head = (seg - b) / B;
        u.kv_begin = a.kv_indptr[b] + skip_of(b) + lo;
        u.kv_end = a.kv_indptr[b] + skip_of(b) + hi;
        u.q_begin = b;
        u.q_end = b + 1;
        u.partial = ws.seg_first[seg] >= 0 ? ws.seg_first[seg] + ordinal : -1;
        u.diag = u.kv_end - 1;
        u.merge = ws.seg_merge[seg];
        u.part_stride = u.reserved2 = 0;
        u.cached_end = a.kv_cached && a.kv_cached[b] > 0 ? a.kv_indptr[b] + a.kv_cached[b] : 0;
    };
    const int64_t stride = xcd ? a.num_xcd : 1;   // workgroup w = k * stride + x
    int32_t pos = 0;
    for (int64_t k = 0, w = 0; k < n_wg / stride; k++) {
        for (int64_t x = 0; x < stride; x++, w++) {
            wg_offsets[w] = pos;
            const int64_t i = x * per_xcd + k;
            if (i >= n)
                continue;  // padding workgroup
            if (i < n_seg)
                emit(units_out[pos++], (int32_t)i, 0, open_len(i), 0);
            for (int32_t j = ws.bin_stream[i]; j < ws.bin_stream[i + 1]; j++) {
                const PartitionScratch::Piece &pc = ws.stream[j];
                emit(units_out[pos++], pc.seg, pc.lo, pc.hi, pc.ordinal);
            }
        }
    }
    wg_offsets[n_wg] = pos;
    return PA_OK;
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

void partition_capacity(int32_t max_batch, int64_t max_kv_total, int32_t max_q_total,
                        int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t max_workgroups, int32_t num_xcd, int64_t *max_wg_entries,
                        int64_t *max_units, int64_t *max_merges, int64_t *max_partial_rows,
                        int64_t *max_prefix_units) {
    const int32_t g = num_qo_heads / num_kv_heads;
    const int64_t segs = (int64_t)num_kv_heads * max_batch;
    // decode, automatic: an opening piece per segment, one more piece where a
    // segment continues, one more per workgroup boundary
    const int64_t dec_auto = 2 * segs + std::max(1, max_workgroups);
    // decode, forced splits (documented guarantee)
    const int64_t dec_forced = (int64_t)num_kv_heads * (max_batch + max_kv_total / 256);
    const int64_t dec = std::max(dec_auto, dec_forced);
    // prefill: tiles, then at most ~4 units per CU after KV splitting
    int64_t tiles = 0, pre = 0;
    if (max_q_total > 0) {
        const int32_t qt = prefill_tile_tokens(g, head_dim);
        tiles = (int64_t)num_kv_heads * (ceil_div(max_q_total, qt) + max_batch);
        pre = 4LL * kNumCu + tiles;
    }
    *max_units = std::max(dec, pre);
    // one-unit workgroups may be padded up to the XCD count times
    *max_wg_entries = std::max<int64_t>(std::max(1, max_workgroups) + num_xcd,
                                        std::max(dec_forced, pre) * num_xcd) + 1;
    *max_merges = std::max(segs, tiles);
    // cascade: a (subgroup, KV head) pair has K prefix units and K slots per
    // member, K <= kMaxCascadeParts, and K > 1 only while the pairs number
    // fewer than the decode workgroups (K <= ceil(max_workgroups / pairs)):
    // so at most max(pairs, 2 * max_workgroups) units and max(segments,
    // 2 * (members per pair) * max_workgroups) slots, pairs <= segments
    const int64_t max_wg = std::max(1, max_workgroups);
    const int64_t prefix_slots =
        std::max(segs, std::min<int64_t>(segs * kMaxCascadeParts,
                                         2 * (int64_t)(prefill_tile_rows(head_dim) / g) * max_wg));
    *max_prefix_units = std::max(segs, std::min<int64_t>(segs * kMaxCascadeParts, 2 * max_wg));
    *max_partial_rows =
        std::max((dec + prefix_slots) * g, (max_q_total > 0) ? pre * prefill_tile_rows(head_dim) : 0);
}

pa_status cascade_partition(const PartitionArgs &a, const CascadeArgs &c, PartitionScratch *scratch,
                            int32_t *wg_offsets, int32_t wg_capacity, pa_work_unit *units,
                            int32_t unit_capacity, pa_merge_unit *merges, int32_t merge_capacity,
                            pa_work_unit *prefix_units, int32_t prefix_capacity,
                            PartitionResult *res, const char **detail) {
    *res = PartitionResult{};
    if (a.qo_indptr || forced_splits(a.flags))
        return fail(detail, "a cascade plan is an automatic decode plan", PA_ERR_INVALID_ARG);
    if (c.num_groups < 0 || (a.batch > 0 && (!c.group_indptr || !c.prefix_len)))
        return fail(detail, "group arrays are null or num_groups < 0", PA_ERR_INVALID_ARG);
    if (c.num_groups > 0 && !c.group_indptr)
        return fail(detail, "group_indptr is null", PA_ERR_INVALID_ARG);
    if ((c.num_groups > 0 || a.batch > 0) &&
        (c.group_indptr[0] != 0 || c.group_indptr[c.num_groups] != a.batch))
        return fail(detail, "group_indptr must run from 0 to batch", PA_ERR_INVALID_ARG);
    PartitionScratch local;
    PartitionScratch &ws = scratch ? *scratch : local;
    ws.kv_skip.assign(std::max(0, a.batch), 0);
    // the checks partition() makes, before the lists are read
    if (a.batch < 0)
        return fail(detail, "batch < 0", PA_ERR_INVALID_ARG);
    if (!supported_shape(a.num_qo_heads, a.num_kv_heads, a.head_dim))
        return fail(detail, "unsupported head shape (need Hq/Hkv in {1,2,4,8}, D in {128,256})",
                    PA_ERR_UNSUPPORTED);
    if ((a.flags & ~(PA_PLAN_NO_XCD_ORDER | PA_PLAN_SPEED_FEEDBACK | PA_PLAN_CASCADE_ALL | PA_PLAN_KV_FP8)) != 0)
        return fail(detail, "unknown flag bits", PA_ERR_INVALID_ARG);
    if (a.num_xcd < 1 || a.num_xcd > kMaxXcd)
        return fail(detail, "XCD count out of range", PA_ERR_INVALID_ARG);
    if (a.batch > 0) {
        if (!a.kv_indptr)
            return fail(detail, "kv_indptr is null", PA_ERR_INVALID_ARG);
        if (a.kv_indptr[0] != 0)
            return fail(detail, "kv_indptr[0] != 0", PA_ERR_INVALID_ARG);
        for (int32_t b = 0; b < a.batch; b++)
            if (a.kv_indptr[b + 1] < a.kv_indptr[b])
                return fail(detail, "kv_indptr decreases", PA_ERR_INVALID_ARG);
    }
    for (int32_t gi = 0; gi < c.num_groups; gi++) {
        const int32_t b0 = c.group_indptr[gi], b1 = c.group_indptr[gi + 1];
        if (b1 < b0)
            return fail(detail, "group_indptr decreases", PA_ERR_INVALID_ARG);
        const int32_t plen = c.prefix_len[gi];
        if (plen < 0)
            return fail(detail, "negative prefix length", PA_ERR_INVALID_ARG);
        if (plen > 0 && b1 == b0)
            return fail(detail, "a prefix for an empty group", PA_ERR_INVALID_ARG);
        for (int32_t b = b0; b < b1; b++)
            if (plen > a.kv_indptr[b + 1] - a.kv_indptr[b])
                return fail(detail, "prefix longer than a member's list", PA_ERR_INVALID_ARG);
    }
    // the prefixes that get prefix units
    const int32_t g = a.num_qo_heads / a.num_kv_heads, Hkv = a.num_kv_heads;
    auto used_prefix = [&](int32_t gi) {
        const int32_t members = c.group_indptr[gi + 1] - c.group_indptr[gi];
        const bool big = (int64_t)members * g >= kCascadeMinRows || (a.flags & PA_PLAN_CASCADE_ALL);
        return big ? c.prefix_len[gi] : 0;
    };
    // a shared prefix without prefix units is left to the L2: its members'
    // decode units read it with cached loads (they stream everything else)
    ws.kv_cached.assign(std::max(0, a.batch), 0);
    for (int32_t gi = 0; gi < c.num_groups; gi++) {
        const int32_t members = c.group_indptr[gi + 1] - c.group_indptr[gi];
        const bool shared_in_l2 = used_prefix(gi) == 0 && members > 1;
        for (int32_t b = c.group_indptr[gi]; b < c.group_indptr[gi + 1]; b++) {
            ws.kv_skip[b] = used_prefix(gi);
            ws.kv_cached[b] = shared_in_l2 ? c.prefix_len[gi] : 0;
        }
    }
    PartitionArgs d = a;
    d.kv_skip = ws.kv_skip.data();
    d.kv_cached = ws.kv_cached.data();
    // on PA_ERR_CAPACITY the counts are still wanted: go on counting
    pa_status st = decode_bins(d, ws, wg_offsets, wg_capacity, units, unit_capacity, merges,
                               merge_capacity, res, detail);
    if (st != PA_OK && st != PA_ERR_CAPACITY)
        return st;
    const bool decode_fits = st == PA_OK;
    if (!decode_fits)
        merge_capacity = 0;   // the merges were not written

    // prefix units: per group, subgroups of up to prefill_tile_rows / g members
    // (one query tile), per KV head, the prefix cut into K parts; part k of
    // member t of (subgroup, head) writes slot base + t * K + k
    const int32_t max_members = prefill_tile_rows(a.head_dim) / g;
    int64_t pairs = 0;   // (subgroup, KV head) pairs with a prefix
    for (int32_t gi = 0; gi < c.num_groups; gi++)
        if (used_prefix(gi) > 0)
            pairs += Hkv * ceil_div(c.group_indptr[gi + 1] - c.group_indptr[gi], max_members);
    const int64_t want_parts = pairs > 0 ? ceil_div(std::max(1, a.max_workgroups), pairs) : 1;
    int32_t n_prefix = 0, slot = res->n_partials;
    for (int32_t gi = 0; gi < c.num_groups; gi++) {
        const int32_t plen = used_prefix(gi);
        if (plen == 0)
            continue;
        const int32_t K = (int32_t)std::max<int64_t>(
            1, std::min<int64_t>({(int64_t)kMaxCascadeParts, want_parts,
                                  ceil_div(plen, kCascadeMinPartEntries)}));
        for (int32_t s0 = c.group_indptr[gi]; s0 < c.group_indptr[gi + 1]; s0 += max_members) {
            const int32_t m = std::min(max_members, c.group_indptr[gi + 1] - s0);
            for (int32_t h = 0; h < Hkv; h++) {
                const int32_t base = slot;
                slot += m * K;
                for (int32_t k = 0; k < K; k++) {
                    const int32_t lo = (int32_t)((int64_t)plen * k / K);
                    const int32_t hi = (int32_t)((int64_t)plen * (k + 1) / K);
                    if (n_prefix < prefix_capacity) {
                        pa_work_unit &u = prefix_units[n_prefix];
                        u.request = s0;
                        u.kv_head = h;
                        u.kv_begin = a.kv_indptr[s0] + lo;
                        u.kv_end = a.kv_indptr[s0] + hi;
                        u.q_begin = s0;
                        u.q_end = s0 + m;
                        u.partial = base + k;
                        u.diag = u.kv_end - 1;   // every member row sees the whole part
                        u.merge = -1;
                        u.part_stride = K;
                        u.cached_end = u.reserved2 = 0;
                    }
                    n_prefix++;
                }
                for (int32_t t = 0; t < m; t++) {
                    // with a prefix, every (request, head) segment has a merge
                    const int32_t mi = ws.seg_merge[(int64_t)h * a.batch + s0 + t];
                    if (mi >= 0 && mi < merge_capacity) {
                        merges[mi].prefix_first = base + t * K;
                        merges[mi].prefix_parts = K;
                    }
                }
            }
        }
    }
    res->n_prefix_units = n_prefix;
    res->n_partials = slot;
    if (!decode_fits)
        return st;
    if (n_prefix > prefix_capacity)
        return fail(detail, "plan capacity exceeded (prefix units)", PA_ERR_CAPACITY);
    return PA_OK;
}

pa_status partition(const PartitionArgs &a, PartitionScratch *scratch, int32_t *wg_offsets,
                    int32_t wg_capacity, pa_work_unit *units_out, int32_t unit_capacity,
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
    if ((a.flags & ~(PA_PLAN_FORCE_SPLITS_MASK | PA_PLAN_NO_XCD_ORDER | PA_PLAN_SPEED_FEEDBACK |
                     PA_PLAN_CASCADE_ALL | PA_PLAN_KV_FP8)) != 0)
        return fail(detail, "unknown flag bits", PA_ERR_INVALID_ARG);
    if (a.num_xcd < 1 || a.num_xcd > kMaxXcd)
        return fail(detail, "XCD count out of range", PA_ERR_INVALID_ARG);
    if (a.xcd_weights)
        for (int32_t x = 0; x < a.num_xcd; x++)
            if (!(a.xcd_weights[x] >= kMinXcdWeight && a.xcd_weights[x] <= kMaxXcdWeight))
                return fail(detail, "XCD weight outside [0.25, 4]", PA_ERR_INVALID_ARG);
    if (a.wg_weights)
        for (int32_t w = 0; w < a.n_wg_weights; w++)
            if (!(a.wg_weights[w] >= kMinXcdWeight && a.wg_weights[w] <= kMaxXcdWeight))
                return fail(detail, "workgroup weight outside [0.25, 4]", PA_ERR_INVALID_ARG);
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

    Groups groups;
    std::vector<pa_merge_unit> merges;
    int32_t n_partials = 0;
    const bool xcd = !(a.flags & PA_PLAN_NO_XCD_ORDER) && a.num_xcd > 1;

    if (!prefill && !forced) {
        PartitionScratch local;
        return decode_bins(a, scratch ? *scratch : local, wg_offsets, wg_capacity, units_out,
                           unit_capacity, merges_out, merge_capacity, res, detail);
    } else if (!prefill) {
        std::vector<Unit> units;
        for (int32_t b = 0; b < a.batch; b++) {
            const int32_t beg = a.kv_indptr[b], L = a.kv_indptr[b + 1] - a.kv_indptr[b];
            const int32_t n = forced;
            for (int32_t h = 0; h < Hkv; h++) {
                const int32_t first = n_partials;
                for (int32_t j = 0; j < n; j++) {
                    const int64_t lo = (int64_t)L * j / n, hi = (int64_t)L * (j + 1) / n;
                    Unit x;
                    x.u.request = b;
                    x.u.kv_head = h;
                    x.u.kv_begin = beg + (int32_t)lo;
                    x.u.kv_end = beg + (int32_t)hi;
                    x.u.q_begin = b;
                    x.u.q_end = b + 1;
                    x.u.partial = n > 1 ? n_partials++ : -1;
                    x.u.diag = x.u.kv_end - 1;
                    x.u.merge = n > 1 ? (int32_t)merges.size() : -1;
                    x.u.part_stride = x.u.cached_end = x.u.reserved2 = 0;
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
        groups = xcd ? xcd_order_single(units, a.num_xcd) : plain_single(units);
    } else {
        const int32_t qt = prefill_tile_tokens(g, a.head_dim);
        int64_t n_tiles = 0;
        for (int32_t b = 0; b < a.batch; b++)
            n_tiles += (int64_t)Hkv * ceil_div(a.qo_indptr[b + 1] - a.qo_indptr[b], qt);
        // Cut KV ranges only when the tiles alone cannot fill the GPU (one
        // prefill workgroup per compute unit), and then into about that many
        // parts: every part runs in the first round, and more parts only add
        // partial rows to write and merge.
        const int64_t resident = (int64_t)kPrefillWorkgroupsPerCu * kNumCu;
        int64_t part_len = 0;  // 0 = no cut
        if (forced == 0 && n_tiles > 0 && n_tiles < resident) {
            int64_t kv_work = 0;
            for (int32_t b = 0; b < a.batch; b++) {
                const int64_t C = a.qo_indptr[b + 1] - a.qo_indptr[b];
                if (C > 0)
                    kv_work += (int64_t)Hkv * ceil_div(C, qt) * (a.kv_indptr[b + 1] - a.kv_indptr[b]);
            }
            part_len = std::max<int64_t>(256, ceil_div(kv_work, resident));
            part_len = ceil_div(part_len, 64) * 64;
        }
        std::vector<Unit> units;
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
                    const int32_t first = n_partials;
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
                        x.u.merge = n > 1 ? (int32_t)merges.size() : -1;
                        x.u.part_stride = x.u.cached_end = x.u.reserved2 = 0;
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
        groups = xcd ? xcd_order_single(units, a.num_xcd) : plain_single(units);
    }

    int64_t n_units = 0;
    for (auto &gr : groups)
        n_units += (int64_t)gr.size();
    res->n_workgroups = (int32_t)groups.size();
    res->n_units = (int32_t)n_units;
    res->n_merges = (int32_t)merges.size();
    res->n_partials = n_partials;
    if ((int64_t)groups.size() + 1 > wg_capacity || n_units > unit_capacity ||
        (int64_t)merges.size() > merge_capacity)
        return fail(detail, "plan capacity exceeded", PA_ERR_CAPACITY);
    int32_t pos = 0;
    for (size_t w = 0; w < groups.size(); w++) {
        wg_offsets[w] = pos;
        for (const pa_work_unit &u : groups[w])
            units_out[pos++] = u;
    }
    wg_offsets[groups.size()] = pos;
    if (!merges.empty())
        std::memcpy(merges_out, merges.data(), merges.size() * sizeof(pa_merge_unit));
    return PA_OK;
}

}  // namespace pa
