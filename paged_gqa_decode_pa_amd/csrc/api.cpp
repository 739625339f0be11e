// api.cpp -- the C ABI of libpa (declared in include/pa.h): argument checking,
// the plan object (allocated once, reused every step), upload of the
// partition, and kernel launches on the caller's stream.
//
// Buffers are allocated once at plan creation and a plan is computed once per
// step and reused by every layer: Agent-Infer page ("Agent-Infer: 纯 Rust 编写的
// 高性能 LLM 推理引擎"), section "分页 KV 缓存" and stages 2-3 of the table in
// "优化历程".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pa_internal.h"

struct pa_plan {
    int device = -1;
    int32_t max_batch = 0;
    int64_t max_kv_total = 0;
    int32_t max_q_total = 0;
    int32_t num_qo_heads = 0, num_kv_heads = 0, head_dim = 0, group = 0;
    int32_t num_cu = pa::kNumCu, num_xcd = pa::kNumXcd;
    int32_t max_workgroups = 0;  // decode workgroups resident at once (bf16 pools)
    int32_t max_workgroups_fp8 = 0;  // the same for E4M3 pools (PA_PLAN_KV_FP8)
    int64_t wg_cap = 0, unit_cap = 0, merge_cap = 0, partial_rows_cap = 0;
    int64_t prefix_cap = 0;       // cascade prefix units
    // device: [workgroup offsets | units | merges] packed by the last pa_plan,
    // and partial storage
    void *d_table = nullptr;
    float *d_part_o = nullptr;
    float *d_part_lse = nullptr;
    int32_t *d_arrivals = nullptr;  // per merge unit, zero between launches
    // pinned staging, two alternating buffers holding a whole table
    void *h_stage[2] = {nullptr, nullptr};
    hipEvent_t stage_done[2] = {nullptr, nullptr};
    bool stage_pending[2] = {false, false};
    int next_stage = 0;
    // the last partition
    pa::PlanMode mode = pa::PlanMode::kNone;
    int32_t batch = 0;
    int64_t kv_total = 0;
    int32_t q_total = 0;
    int32_t n_workgroups = 0, n_units = 0, n_merges = 0, n_partials = 0;
    int32_t n_prefix_units = 0;   // cascade plan: prefix units after the merges
    pa::PartitionScratch scratch;  // host working arrays of the partition
    double plan_total_us = 0.0, plan_wait_us = 0.0;  // host time of the last pa_plan
    // work weights of the automatic decode split: per XCD (set by the
    // caller) and per workgroup id (PA_PLAN_SPEED_FEEDBACK).  With the
    // feedback the decode kernel adds each workgroup's run time to
    // d_wg_clock; pa_plan copies the counters to h_wg_clock and a later call
    // turns the difference of two copies into new workgroup weights
    float xcd_weight[pa::kMaxXcd];
    int32_t n_clock = 0;                 // workgroup ids with a counter
    std::vector<float> wg_weight;        // n_clock entries, from cu_weight
    std::vector<float> cu_weight;        // num_cu entries
    bool xcd_weighted = false, wg_weighted = false;   // some weight differs from 1
    std::vector<double> cu_busy;         // update_cu_weights' working array
    uint64_t *d_wg_clock = nullptr;      // device, n_clock counters, kClockStride apart
    uint64_t *h_wg_clock = nullptr;      // pinned copy
    hipEvent_t clock_done = nullptr;
    bool clock_pending = false;          // a copy is in flight or unread
    std::vector<uint64_t> clock_last;    // the counters of the copy read last
    std::vector<float> clock_weight;     // unit weights of the launches the pending copy covers
    std::vector<float> interval_weight;  // pa_plan's copy of the unit weights before it updates them
    bool clock_record = false;           // the last plan's decode launches record
    // kernel timing: event pairs recorded around the attention kernel
    std::vector<hipEvent_t> prof_events;   // 2 per pair
    mutable int32_t prof_used = 0;
    bool prof_on = false;
};

namespace {

thread_local std::string g_detail;

pa_status fail(pa_status s, const std::string &msg) {
    g_detail = msg;
    return s;
}

pa_status hip_fail(hipError_t e, const char *what) {
    g_detail = std::string(what) + ": " + hipGetErrorString(e);
    return PA_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr size_t kUnit = sizeof(pa_work_unit);
constexpr size_t kMerge = sizeof(pa_merge_unit);
static_assert(kUnit == 48 && kMerge == 32, "table entry sizes");

// Bytes of the workgroup-offset block of a table with n_workgroups
// workgroups (n + 1 offsets, rounded up to 64 bytes).
size_t offsets_bytes(int64_t n_workgroups) {
    return (size_t)((n_workgroups + 1 + 15) / 16) * 64;
}

// Table layout (device and staging): [workgroup offsets | merge units | work
// units | prefix workgroup offsets | prefix units], each region at a fixed
// offset sized by the plan's capacities (the prefix regions are used only by
// cascade plans).  A launch captured into a HIP graph keeps the region
// addresses it was given, so they must not move when a later pa_plan of the
// same plan cuts the lists into a different number of units or merges (the
// speed feedback does that from step to step).
struct TableLayout {
    size_t merges, units, prefix_offsets, prefix_units, end;
};
TableLayout table_layout(const pa_plan_t *p) {
    TableLayout t;
    t.merges = offsets_bytes(p->wg_cap);
    t.units = t.merges + (size_t)p->merge_cap * kMerge;
    t.prefix_offsets = t.units + (size_t)p->unit_cap * kUnit;
    t.prefix_units = t.prefix_offsets + offsets_bytes(p->prefix_cap);
    t.end = t.prefix_units + (size_t)p->prefix_cap * kUnit;
    return t;
}
size_t table_bytes(const pa_plan_t *p) { return table_layout(p).end; }

void drop_profile(pa_plan_t *p) {
    for (hipEvent_t e : p->prof_events)
        (void)hipEventDestroy(e);
    p->prof_events.clear();
    p->prof_used = 0;
    p->prof_on = false;
}

// Record the start (second = false) or end of a timed kernel.
hipError_t profile_mark(const pa_plan_t *p, hipStream_t s, bool end) {
    if (!p->prof_on || (size_t)p->prof_used * 2 >= p->prof_events.size())
        return hipSuccess;
    hipError_t e = hipEventRecord(p->prof_events[(size_t)p->prof_used * 2 + (end ? 1 : 0)], s);
    if (end)
        p->prof_used++;
    return e;
}

void release(pa_plan_t *p) {
    if (!p)
        return;
    drop_profile(p);
    if (p->clock_done) {
        if (p->clock_pending)
            (void)hipEventSynchronize(p->clock_done);
        (void)hipEventDestroy(p->clock_done);
    }
    if (p->h_wg_clock)
        (void)hipHostFree(p->h_wg_clock);
    if (p->d_wg_clock)
        (void)hipFree(p->d_wg_clock);
    for (int i = 0; i < 2; i++) {
        if (p->stage_done[i]) {
            if (p->stage_pending[i])
                (void)hipEventSynchronize(p->stage_done[i]);
            (void)hipEventDestroy(p->stage_done[i]);
        }
        if (p->h_stage[i])
            (void)hipHostFree(p->h_stage[i]);
    }
    if (p->d_table)
        (void)hipFree(p->d_table);
    if (p->d_part_o)
        (void)hipFree(p->d_part_o);
    if (p->d_part_lse)
        (void)hipFree(p->d_part_lse);
    if (p->d_arrivals)
        (void)hipFree(p->d_arrivals);
    delete p;
}

// Checks shared by the run entry points; fills the launch descriptor.
// Bounds of the weights the feedback moves to, and the fraction of the way
// from the current weights to the measured rates taken per update.
constexpr float kFeedbackMinWeight = 0.5f, kFeedbackMaxWeight = 1.5f;
constexpr double kFeedbackGain = 0.5;

// Rescale weights to average 1.
void normalise_weights(float *w, int n) {
    double sum = 0.0;
    for (int x = 0; x < n; x++)
        sum += w[x];
    for (int x = 0; x < n; x++)
        w[x] = (float)(w[x] * n / sum);
}

// Turn the counters of the completed clock copy into new weights.  A launch
// that fills the GPU places workgroup ids w, w + C, w + 2C, ... (C = compute
// units) on one compute unit, and the unit is done when the last of them is,
// so the weights are kept per unit: the launches since the copy before it
// gave unit c a budget proportional to clock_weight[c] and it was busy for
// busy_c = the largest mean run time of its workgroups, so it ran at
// clock_weight[c] / busy_c; an even finish gives each unit a share
// proportional to that rate.  Units whose workgroups recorded nothing keep
// their weights.  Workgroup id w then weighs cu_weight[w % C].
void update_cu_weights(pa_plan_t *p) {
    const uint64_t time_mask = (1ull << pa::kClockCountShift) - 1;
    const int32_t C = p->num_cu;
    std::vector<double> &busy = p->cu_busy;
    std::fill(busy.begin(), busy.end(), 0.0);
    for (int32_t w = 0; w < p->n_clock; w++) {
        const uint64_t now = p->h_wg_clock[(size_t)w * pa::kClockStride];
        const uint64_t diff = now - p->clock_last[w];
        p->clock_last[w] = now;
        const uint64_t count = diff >> pa::kClockCountShift, ticks = diff & time_mask;
        if (count > 0)
            busy[w % C] = std::max(busy[w % C], (double)ticks / (double)count);
    }
    double sum = 0.0;
    int active = 0;
    for (int32_t c = 0; c < C; c++)
        if (busy[c] > 0.0) {
            busy[c] = p->clock_weight[c] / busy[c];   // now the unit's rate
            sum += busy[c];
            active++;
        }
    if (active == 0)
        return;
    const double mean_rate = sum / active;
    double wsum = 0.0;
    for (int32_t c = 0; c < C; c++) {
        if (busy[c] == 0.0)
            continue;
        const double v = (1.0 - kFeedbackGain) * p->cu_weight[c] + kFeedbackGain * busy[c] / mean_rate;
        p->cu_weight[c] = std::min(kFeedbackMaxWeight, std::max(kFeedbackMinWeight, (float)v));
        wsum += p->cu_weight[c];
    }
    for (int32_t c = 0; c < C; c++)   // mean 1 over the units that ran
        if (busy[c] != 0.0)
            p->cu_weight[c] = (float)(p->cu_weight[c] * active / wsum);
    for (int32_t w = 0; w < p->n_clock; w++)
        p->wg_weight[w] = p->cu_weight[w % C];
    p->wg_weighted = true;
}

// The launch of a cascade plan's prefix units: the decode launch l with the
// prefix workgroup offsets and units of the table.
pa::DecodeLaunch prefix_launch(const pa_plan_t *p, const pa::DecodeLaunch &l) {
    pa::DecodeLaunch x = l;
    const char *tbl = static_cast<const char *>(p->d_table);
    const TableLayout t = table_layout(p);
    x.wg_offsets = reinterpret_cast<const int32_t *>(tbl + t.prefix_offsets);
    x.n_workgroups = p->n_prefix_units;
    x.units = reinterpret_cast<const pa_work_unit *>(tbl + t.prefix_units);
    x.n_units = p->n_prefix_units;
    x.merges = nullptr;
    x.n_merges = 0;
    x.wg_clock = nullptr;
    return x;
}

pa_status prepare_run(const pa_plan_t *p, pa::PlanMode want, const void *q, const void *k_pool,
                      const void *v_pool, int64_t num_slots, int64_t slot_stride,
                      const int32_t *kv_indices, float sm_scale, float *out, float *lse,
                      pa::DecodeLaunch *l) {
    if (!p)
        return fail(PA_ERR_INVALID_ARG, "plan is null");
    if (p->mode != want)
        return fail(PA_ERR_PLAN_MISMATCH, p->mode == pa::PlanMode::kNone
                                              ? "pa_plan has not been called on this plan"
                                              : "the last pa_plan was for the other mode "
                                                "(decode: qo_indptr NULL; prefill: non-NULL)");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev != p->device)
        return fail(PA_ERR_INVALID_ARG, "current HIP device differs from the plan's device");
    const bool has_rows = (want == pa::PlanMode::kDecode) ? p->batch > 0 : p->q_total > 0;
    if (has_rows && (!q || !out))
        return fail(PA_ERR_INVALID_ARG, "q or out is null");
    if (p->kv_total > 0 && (!k_pool || !v_pool || !kv_indices))
        return fail(PA_ERR_INVALID_ARG, "k_pool, v_pool or kv_indices is null");
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
        return fail(PA_ERR_INVALID_ARG, "q, k_pool and v_pool must be 16-byte aligned");
    if (!aligned(kv_indices, 4) || !aligned(out, 4) || !aligned(lse, 4))
        return fail(PA_ERR_INVALID_ARG, "kv_indices, out and lse must be 4-byte aligned");
    const int64_t row = (int64_t)p->num_kv_heads * p->head_dim;
    if (slot_stride == 0)
        slot_stride = row;
    if (slot_stride < row || slot_stride % 8 != 0)
        return fail(PA_ERR_INVALID_ARG, "slot_stride must be >= Hkv*D and a multiple of 8");
    if (slot_stride * 2 > 0x7fffffffLL)
        return fail(PA_ERR_INVALID_ARG, "slot_stride too large");
    if (num_slots < 0 || (p->kv_total > 0 && num_slots == 0))
        return fail(PA_ERR_INVALID_ARG, "num_slots must be positive");
    if (!std::isfinite(sm_scale))
        return fail(PA_ERR_INVALID_ARG, "sm_scale is not finite");
    const char *tbl = static_cast<const char *>(p->d_table);
    const TableLayout t = table_layout(p);
    l->wg_offsets = reinterpret_cast<const int32_t *>(tbl);
    l->n_workgroups = p->n_workgroups;
    l->units = reinterpret_cast<const pa_work_unit *>(tbl + t.units);
    l->n_units = p->n_units;
    l->merges = reinterpret_cast<const pa_merge_unit *>(tbl + t.merges);
    l->n_merges = p->n_merges;
    l->arrivals = p->d_arrivals;
    l->q = q;
    l->k_pool = k_pool;
    l->v_pool = v_pool;
    l->slot_stride = slot_stride;
    l->num_slots = num_slots;
    l->kv_indices = kv_indices;
    l->sm_scale = sm_scale;
    l->out = out;
    l->lse = lse;
    l->partial_o = p->d_part_o;
    l->partial_lse = p->d_part_lse;
    l->num_qo_heads = p->num_qo_heads;
    l->num_kv_heads = p->num_kv_heads;
    l->head_dim = p->head_dim;
    l->wg_clock = (want == pa::PlanMode::kDecode && p->clock_record) ? p->d_wg_clock : nullptr;
    return PA_OK;
}

}  // namespace

// pa_plan and pa_plan_cascade (casc != nullptr).
static pa_status plan_impl(pa_plan_t *p, const int32_t *kv_indptr_host, const int32_t *qo_indptr_host,
                           int32_t batch, uint32_t flags, pa_stream_t stream,
                           const pa::CascadeArgs *casc) {
    using clock = std::chrono::steady_clock;
    const clock::time_point t_start = clock::now();
    if (!p)
        return fail(PA_ERR_INVALID_ARG, "plan is null");
    if (batch < 0)
        return fail(PA_ERR_INVALID_ARG, "batch < 0");
    if (batch > 0 && !kv_indptr_host)
        return fail(PA_ERR_INVALID_ARG, "kv_indptr_host is null");
    if (batch > p->max_batch)
        return fail(PA_ERR_CAPACITY, "batch above the plan's max_batch");
    const int64_t kv_total = batch > 0 ? kv_indptr_host[batch] : 0;
    if (kv_total > p->max_kv_total)
        return fail(PA_ERR_CAPACITY, "total slot-list length above the plan's max_kv_total");
    int32_t q_total = 0;
    if (qo_indptr_host) {
        q_total = batch > 0 ? qo_indptr_host[batch] : 0;
        if (q_total > p->max_q_total)
            return fail(PA_ERR_CAPACITY, "total query rows above the plan's max_q_total");
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev != p->device)
        return fail(PA_ERR_INVALID_ARG, "current HIP device differs from the plan's device");

    const bool auto_decode = !qo_indptr_host &&
                             ((flags & PA_PLAN_FORCE_SPLITS_MASK) >> PA_PLAN_FORCE_SPLITS_SHIFT) == 0;
    const bool feedback = (flags & PA_PLAN_SPEED_FEEDBACK) && auto_decode;
    // the weights of the plans since the last clock copy (they change only
    // below, when a copy is read, and a copy is started only when none is
    // pending)
    if (feedback)
        std::copy(p->cu_weight.begin(), p->cu_weight.end(), p->interval_weight.begin());
    if (feedback && p->clock_pending) {
        const hipError_t before = hipPeekAtLastError();
        e = hipEventQuery(p->clock_done);
        if (e == hipSuccess) {
            p->clock_pending = false;
            update_cu_weights(p);
        } else if (e == hipErrorNotReady) {
            if (before == hipSuccess)
                (void)hipGetLastError();  // not an error: the copy is still in flight
        } else {
            return hip_fail(e, "clock copy");
        }
    }

    const int s = p->next_stage;
    const clock::time_point t_wait = clock::now();
    if (p->stage_pending[s]) {
        if ((e = hipEventSynchronize(p->stage_done[s])) != hipSuccess)
            return hip_fail(e, "waiting for an earlier plan upload");
        p->stage_pending[s] = false;
    }
    const clock::time_point t_waited = clock::now();
    // partition straight into the staging buffer at capacity offsets, then
    // pack the three lists together and upload them with one copy
    char *stage = static_cast<char *>(p->h_stage[s]);
    const TableLayout t = table_layout(p);
    int32_t *offsets = reinterpret_cast<int32_t *>(stage);
    pa_work_unit *units = reinterpret_cast<pa_work_unit *>(stage + t.units);
    pa_merge_unit *merges = reinterpret_cast<pa_merge_unit *>(stage + t.merges);
    // decode workgroups the GPU keeps resident for the pools' element type
    const bool kv_fp8 = (flags & PA_PLAN_KV_FP8) != 0;
    int32_t max_wg = kv_fp8 ? p->max_workgroups_fp8 : p->max_workgroups;
    if (auto_decode && p->num_cu > 0 && max_wg >= p->num_cu) {
        // as many workgroups per compute unit (1 .. resident) as the K/V
        // bytes need at about kWorkgroupTargetBytes each: a small step's
        // work in fewer, longer workgroups spends less on each one's fixed
        // latency chain and merge
        const int64_t bytes = kv_total * p->num_kv_heads * 2 * p->head_dim * (kv_fp8 ? 1 : 2);
        const int64_t per_cu = std::max<int64_t>(
            1, std::min<int64_t>(max_wg / p->num_cu, ceil_div64(bytes, (int64_t)p->num_cu * pa::kWorkgroupTargetBytes)));
        max_wg = (int32_t)(per_cu * p->num_cu);
    }
    pa::PartitionArgs a{kv_indptr_host, qo_indptr_host, batch, p->num_qo_heads, p->num_kv_heads,
                        p->head_dim, flags, max_wg, p->num_xcd,
                        p->xcd_weighted ? p->xcd_weight : nullptr,
                        p->wg_weighted ? p->wg_weight.data() : nullptr, p->n_clock};
    pa::PartitionResult r;
    const char *detail = "";
    auto clamp32 = [](int64_t v) { return (int32_t)std::min<int64_t>(v, 0x7fffffff); };
    pa_work_unit *prefix_units = reinterpret_cast<pa_work_unit *>(stage + t.prefix_units);
    pa_status st = casc ? pa::cascade_partition(a, *casc, &p->scratch, offsets, clamp32(p->wg_cap + 1),
                                                units, clamp32(p->unit_cap), merges,
                                                clamp32(p->merge_cap), prefix_units,
                                                clamp32(p->prefix_cap), &r, &detail)
                        : pa::partition(a, &p->scratch, offsets, clamp32(p->wg_cap + 1), units,
                                        clamp32(p->unit_cap), merges, clamp32(p->merge_cap), &r,
                                        &detail);
    if (st != PA_OK)
        return fail(st, detail);
    const int64_t rows_per_slot = qo_indptr_host ? pa::prefill_tile_rows(p->head_dim) : p->group;
    if ((int64_t)r.n_partials * rows_per_slot > p->partial_rows_cap)
        return fail(PA_ERR_CAPACITY, "partial storage of the plan exceeded");
    // upload the used part of each region (the unused capacity of a region
    // can be far larger than its used part, so each is copied on its own)
    if (r.n_prefix_units > 0) {
        // one prefix unit per workgroup
        int32_t *po = reinterpret_cast<int32_t *>(stage + t.prefix_offsets);
        for (int32_t w = 0; w <= r.n_prefix_units; w++)
            po[w] = w;
    }
    const size_t pieces[4][2] = {
        {0, offsets_bytes(r.n_workgroups)},
        {t.merges, (size_t)r.n_merges * kMerge},
        {t.units, (size_t)r.n_units * kUnit},
        {t.prefix_offsets, r.n_prefix_units > 0 ? t.prefix_units - t.prefix_offsets + (size_t)r.n_prefix_units * kUnit
                                                : 0},
    };
    char *dev_table = static_cast<char *>(p->d_table);
    for (const auto &pc : pieces)
        if (pc[1] > 0 && (e = hipMemcpyAsync(dev_table + pc[0], stage + pc[0], pc[1], hipMemcpyHostToDevice,
                                             (hipStream_t)stream)) != hipSuccess)
            return hip_fail(e, "plan upload");
    if ((e = hipEventRecord(p->stage_done[s], (hipStream_t)stream)) != hipSuccess)
        return hip_fail(e, "plan upload event");
    p->stage_pending[s] = true;
    p->next_stage = s ^ 1;
    if (feedback && !p->clock_pending) {
        // the counters as of the end of the launches enqueued so far: those
        // since the previous copy all used interval_weight
        if ((e = hipMemcpyAsync(p->h_wg_clock, p->d_wg_clock,
                                (size_t)p->n_clock * pa::kClockStride * sizeof(uint64_t),
                                hipMemcpyDeviceToHost, (hipStream_t)stream)) != hipSuccess ||
            (e = hipEventRecord(p->clock_done, (hipStream_t)stream)) != hipSuccess)
            return hip_fail(e, "clock copy");
        std::copy(p->interval_weight.begin(), p->interval_weight.end(), p->clock_weight.begin());
        p->clock_pending = true;
    }
    // only launches that fill the GPU measure the workgroups' speeds
    p->clock_record = feedback && r.n_workgroups >= max_wg &&
                      r.n_workgroups <= p->n_clock;
    p->mode = qo_indptr_host ? pa::PlanMode::kPrefill : pa::PlanMode::kDecode;
    p->batch = batch;
    p->kv_total = kv_total;
    p->q_total = q_total;
    p->n_workgroups = r.n_workgroups;
    p->n_units = r.n_units;
    p->n_merges = r.n_merges;
    p->n_partials = r.n_partials;
    p->n_prefix_units = r.n_prefix_units;
    p->plan_wait_us = std::chrono::duration<double, std::micro>(t_waited - t_wait).count();
    p->plan_total_us = std::chrono::duration<double, std::micro>(clock::now() - t_start).count();
    return PA_OK;
}

extern "C" {

const char *pa_strerror(pa_status s) {
    switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape";
    case PA_ERR_CAPACITY: return "plan capacity exceeded";
    case PA_ERR_PLAN_MISMATCH: return "run does not match the plan";
    case PA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *pa_last_error_detail(void) { return g_detail.c_str(); }

int32_t pa_version(void) { return 100; }

int32_t pa_prefill_tile_rows(int32_t head_dim) {
    return (head_dim == 128 || head_dim == 256) ? pa::prefill_tile_rows(head_dim) : 0;
}

pa_status pa_partition(const int32_t *kv_indptr_host, const int32_t *qo_indptr_host,
                       int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                       int32_t head_dim, uint32_t flags, int32_t max_workgroups,
                       int32_t *wg_offsets, int32_t wg_capacity, pa_work_unit *units,
                       int32_t unit_capacity, pa_merge_unit *merges, int32_t merge_capacity,
                       int32_t *n_workgroups, int32_t *n_units, int32_t *n_merges,
                       int32_t *n_partials) {
    return pa_partition_weighted(kv_indptr_host, qo_indptr_host, batch, num_qo_heads, num_kv_heads,
                                 head_dim, flags, max_workgroups, nullptr, 0, nullptr, 0, wg_offsets,
                                 wg_capacity, units, unit_capacity, merges, merge_capacity,
                                 n_workgroups, n_units, n_merges, n_partials);
}

pa_status pa_partition_weighted(const int32_t *kv_indptr_host, const int32_t *qo_indptr_host,
                                int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                int32_t head_dim, uint32_t flags, int32_t max_workgroups,
                                const float *xcd_weights, int32_t n_xcd_weights,
                                const float *wg_weights, int32_t n_wg_weights,
                                int32_t *wg_offsets, int32_t wg_capacity, pa_work_unit *units,
                                int32_t unit_capacity, pa_merge_unit *merges,
                                int32_t merge_capacity, int32_t *n_workgroups, int32_t *n_units,
                                int32_t *n_merges, int32_t *n_partials) {
    if (xcd_weights && n_xcd_weights != pa::kNumXcd)
        return fail(PA_ERR_INVALID_ARG, "n_xcd_weights must equal the XCD count (8)");
    if (n_wg_weights < 0 || (n_wg_weights > 0 && !wg_weights))
        return fail(PA_ERR_INVALID_ARG, "bad workgroup weights");
    if (!n_workgroups || !n_units || !n_merges || !n_partials)
        return fail(PA_ERR_INVALID_ARG, "count pointers must not be null");
    if ((wg_capacity > 0 && !wg_offsets) || (unit_capacity > 0 && !units) ||
        (merge_capacity > 0 && !merges) || wg_capacity < 0 || unit_capacity < 0 ||
        merge_capacity < 0)
        return fail(PA_ERR_INVALID_ARG, "bad output arrays");
    if (max_workgroups <= 0)
        max_workgroups = pa::kNumCu * pa::kDefaultWorkgroupsPerCu;
    pa::PartitionArgs a{kv_indptr_host, qo_indptr_host, batch, num_qo_heads, num_kv_heads,
                        head_dim, flags, max_workgroups, pa::kNumXcd, xcd_weights,
                        n_wg_weights > 0 ? wg_weights : nullptr, n_wg_weights};
    pa::PartitionResult r;
    const char *detail = "";
    pa_status s = pa::partition(a, nullptr, wg_offsets, wg_capacity, units, unit_capacity, merges,
                                merge_capacity, &r, &detail);
    *n_workgroups = r.n_workgroups;
    *n_units = r.n_units;
    *n_merges = r.n_merges;
    *n_partials = r.n_partials;
    if (s != PA_OK)
        return fail(s, detail);
    return PA_OK;
}

pa_status pa_partition_cascade(const int32_t *kv_indptr_host, int32_t batch,
                               const int32_t *group_indptr_host, int32_t num_groups,
                               const int32_t *prefix_len_host, int32_t num_qo_heads,
                               int32_t num_kv_heads, int32_t head_dim, uint32_t flags,
                               int32_t max_workgroups, int32_t *wg_offsets, int32_t wg_capacity,
                               pa_work_unit *units, int32_t unit_capacity, pa_merge_unit *merges,
                               int32_t merge_capacity, pa_work_unit *prefix_units,
                               int32_t prefix_capacity, int32_t *n_workgroups, int32_t *n_units,
                               int32_t *n_merges, int32_t *n_partials, int32_t *n_prefix_units) {
    if (!n_workgroups || !n_units || !n_merges || !n_partials || !n_prefix_units)
        return fail(PA_ERR_INVALID_ARG, "count pointers must not be null");
    if ((wg_capacity > 0 && !wg_offsets) || (unit_capacity > 0 && !units) ||
        (merge_capacity > 0 && !merges) || (prefix_capacity > 0 && !prefix_units) ||
        wg_capacity < 0 || unit_capacity < 0 || merge_capacity < 0 || prefix_capacity < 0)
        return fail(PA_ERR_INVALID_ARG, "bad output arrays");
    if (num_groups < 0 || (num_groups > 0 && (!group_indptr_host || !prefix_len_host)) ||
        (batch > 0 && !group_indptr_host))
        return fail(PA_ERR_INVALID_ARG, "group arrays are null or num_groups < 0");
    if (max_workgroups <= 0)
        max_workgroups = pa::kNumCu * pa::kDefaultWorkgroupsPerCu;
    pa::PartitionArgs a{kv_indptr_host, nullptr, batch, num_qo_heads, num_kv_heads,
                        head_dim, flags, max_workgroups, pa::kNumXcd};
    const pa::CascadeArgs c{group_indptr_host, num_groups, prefix_len_host};
    pa::PartitionResult r;
    const char *detail = "";
    pa_status s = pa::cascade_partition(a, c, nullptr, wg_offsets, wg_capacity, units,
                                        unit_capacity, merges, merge_capacity, prefix_units,
                                        prefix_capacity, &r, &detail);
    *n_workgroups = r.n_workgroups;
    *n_units = r.n_units;
    *n_merges = r.n_merges;
    *n_partials = r.n_partials;
    *n_prefix_units = r.n_prefix_units;
    if (s != PA_OK)
        return fail(s, detail);
    return PA_OK;
}

pa_status pa_plan_xcd_weights(const pa_plan_t *p, float *weights, int32_t capacity,
                              int32_t *n_xcd) {
    if (!p || !n_xcd || capacity < 0 || (capacity > 0 && !weights))
        return fail(PA_ERR_INVALID_ARG, "null argument or negative capacity");
    *n_xcd = p->num_xcd;
    for (int32_t x = 0; x < std::min(capacity, p->num_xcd); x++)
        weights[x] = p->xcd_weight[x];
    return PA_OK;
}

pa_status pa_plan_workgroup_weights(const pa_plan_t *p, float *weights, int32_t capacity,
                                    int32_t *n) {
    if (!p || !n || capacity < 0 || (capacity > 0 && !weights))
        return fail(PA_ERR_INVALID_ARG, "null argument or negative capacity");
    *n = p->n_clock;
    for (int32_t w = 0; w < std::min(capacity, p->n_clock); w++)
        weights[w] = p->wg_weight[w];
    return PA_OK;
}

pa_status pa_plan_set_xcd_weights(pa_plan_t *p, const float *weights, int32_t n) {
    if (!p || !weights)
        return fail(PA_ERR_INVALID_ARG, "null argument");
    if (n != p->num_xcd)
        return fail(PA_ERR_INVALID_ARG, "n must equal the plan's XCD count");
    for (int32_t x = 0; x < n; x++)
        if (!(weights[x] >= pa::kMinXcdWeight && weights[x] <= pa::kMaxXcdWeight))
            return fail(PA_ERR_INVALID_ARG, "XCD weight not finite or outside [0.25, 4]");
    float w[pa::kMaxXcd];
    std::memcpy(w, weights, sizeof(float) * (size_t)n);
    normalise_weights(w, n);
    for (int32_t x = 0; x < n; x++)   // the rescaled set must still be accepted
        w[x] = std::min(pa::kMaxXcdWeight, std::max(pa::kMinXcdWeight, w[x]));
    std::memcpy(p->xcd_weight, w, sizeof(float) * (size_t)n);
    p->xcd_weighted = false;
    for (int32_t x = 0; x < n; x++)
        p->xcd_weighted |= w[x] != 1.0f;
    return PA_OK;
}

pa_status pa_plan_create(pa_plan_t **out, int32_t max_batch, int64_t max_kv_total,
                         int32_t max_q_total, int32_t num_qo_heads, int32_t num_kv_heads,
                         int32_t head_dim) {
    if (!out)
        return fail(PA_ERR_INVALID_ARG, "out is null");
    if (max_batch < 0 || max_kv_total < 0 || max_q_total < 0)
        return fail(PA_ERR_INVALID_ARG, "negative capacity");
    if (max_kv_total > PA_MAX_KV_TOTAL)
        return fail(PA_ERR_INVALID_ARG, "max_kv_total above PA_MAX_KV_TOTAL");
    if (num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return fail(PA_ERR_INVALID_ARG, "head counts and head_dim must be positive");
    if (!pa::supported_shape(num_qo_heads, num_kv_heads, head_dim))
        return fail(PA_ERR_UNSUPPORTED,
                    "unsupported head shape (need Hq/Hkv in {1,2,4,8} and D in {128,256})");
    pa_plan_t *p = new (std::nothrow) pa_plan_t;
    if (!p)
        return fail(PA_ERR_INVALID_ARG, "host allocation failed");
    for (int x = 0; x < pa::kMaxXcd; x++)
        p->xcd_weight[x] = 1.0f;
    p->max_batch = max_batch;
    p->max_kv_total = max_kv_total;
    p->max_q_total = max_q_total;
    p->num_qo_heads = num_qo_heads;
    p->num_kv_heads = num_kv_heads;
    p->head_dim = head_dim;
    p->group = num_qo_heads / num_kv_heads;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        release(p);
        return hip_fail(e, "hipGetDevice");
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) == hipSuccess &&
        cus > 0)
        p->num_cu = cus;
    int per_cu = pa::decode_workgroups_per_cu(head_dim, p->group, false);
    if (per_cu <= 0)
        per_cu = pa::kDefaultWorkgroupsPerCu;
    p->max_workgroups = p->num_cu * per_cu;
    // E4M3 pools: as many workgroups as that kernel keeps resident (never
    // more than the bf16 count the capacities below are sized for)
    const int per_cu_fp8 = pa::decode_workgroups_per_cu(head_dim, p->group, true);
    p->max_workgroups_fp8 = per_cu_fp8 > 0 ? std::min(p->max_workgroups, p->num_cu * per_cu_fp8) : p->max_workgroups;
    pa::partition_capacity(max_batch, max_kv_total, max_q_total, num_qo_heads, num_kv_heads,
                           head_dim, p->max_workgroups, p->num_xcd, &p->wg_cap, &p->unit_cap,
                           &p->merge_cap, &p->partial_rows_cap, &p->prefix_cap);
    const size_t tbytes = table_bytes(p);
    const size_t part_o_bytes = (size_t)std::max<int64_t>(1, p->partial_rows_cap) * head_dim * sizeof(float);
    const size_t part_lse_bytes = (size_t)std::max<int64_t>(1, p->partial_rows_cap) * sizeof(float);
    const size_t arrivals_bytes = (size_t)std::max<int64_t>(1, p->merge_cap) * sizeof(int32_t);
    p->n_clock = p->max_workgroups + pa::kMaxXcd;   // ids of the automatic decode split
    try {
        p->wg_weight.assign((size_t)p->n_clock, 1.0f);
        p->cu_weight.assign((size_t)p->num_cu, 1.0f);
        p->cu_busy.assign((size_t)p->num_cu, 0.0);
        p->clock_weight.assign((size_t)p->num_cu, 1.0f);
        p->interval_weight.assign((size_t)p->num_cu, 1.0f);
        p->clock_last.assign((size_t)p->n_clock, 0);
    } catch (...) {
        release(p);
        return fail(PA_ERR_INVALID_ARG, "host allocation failed");
    }
    const size_t clock_bytes = (size_t)p->n_clock * pa::kClockStride * sizeof(uint64_t);
    if ((e = hipMalloc(&p->d_table, tbytes)) != hipSuccess ||
        (e = hipMalloc((void **)&p->d_part_o, part_o_bytes)) != hipSuccess ||
        (e = hipMalloc((void **)&p->d_part_lse, part_lse_bytes)) != hipSuccess ||
        (e = hipMalloc((void **)&p->d_arrivals, arrivals_bytes)) != hipSuccess ||
        (e = hipMalloc((void **)&p->d_wg_clock, clock_bytes)) != hipSuccess) {
        release(p);
        return hip_fail(e, "hipMalloc (plan workspace)");
    }
    // arrival counts start at zero; every launch leaves them at zero again.
    // The clock counters only grow (readers take differences).
    if ((e = hipMemset(p->d_arrivals, 0, arrivals_bytes)) != hipSuccess ||
        (e = hipMemset(p->d_wg_clock, 0, clock_bytes)) != hipSuccess ||
        (e = hipDeviceSynchronize()) != hipSuccess) {
        release(p);
        return hip_fail(e, "clearing the arrival counts");
    }
    for (int i = 0; i < 2; i++) {
        if ((e = hipHostMalloc(&p->h_stage[i], tbytes, hipHostMallocDefault)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&p->stage_done[i], hipEventDisableTiming)) != hipSuccess) {
            release(p);
            return hip_fail(e, "pinned staging / event");
        }
    }
    if ((e = hipHostMalloc((void **)&p->h_wg_clock, clock_bytes, hipHostMallocDefault)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&p->clock_done, hipEventDisableTiming)) != hipSuccess) {
        release(p);
        return hip_fail(e, "pinned clock copy / event");
    }
    *out = p;
    return PA_OK;
}

void pa_plan_destroy(pa_plan_t *plan) { release(plan); }

pa_status pa_plan(pa_plan_t *p, const int32_t *kv_indptr_host, const int32_t *qo_indptr_host,
                  int32_t batch, uint32_t flags, pa_stream_t stream) {
    return plan_impl(p, kv_indptr_host, qo_indptr_host, batch, flags, stream, nullptr);
}

pa_status pa_plan_cascade(pa_plan_t *p, const int32_t *kv_indptr_host, int32_t batch,
                          const int32_t *group_indptr_host, int32_t num_groups,
                          const int32_t *prefix_len_host, uint32_t flags, pa_stream_t stream) {
    if (num_groups < 0 || (num_groups > 0 && (!group_indptr_host || !prefix_len_host)) ||
        (batch > 0 && !group_indptr_host))
        return fail(PA_ERR_INVALID_ARG, "group arrays are null or num_groups < 0");
    if (p && num_groups > std::max(p->max_batch, 1))
        return fail(PA_ERR_CAPACITY, "more groups than the plan's max_batch");
    const pa::CascadeArgs c{group_indptr_host, num_groups, prefix_len_host};
    return plan_impl(p, kv_indptr_host, nullptr, batch, flags, stream, &c);
}

static pa_status append_impl(const void *k_new, const void *v_new, void *q, const int32_t *positions,
                             const int32_t *out_loc, int32_t num_tokens, int32_t num_qo_heads,
                             int32_t num_kv_heads, int32_t head_dim, float rope_theta, void *k_pool,
                             void *v_pool, int64_t num_slots, int64_t slot_stride, pa_stream_t stream,
                             bool kv_fp8, float k_scale, float v_scale) {
    if (kv_fp8 && !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
    if (num_tokens < 0 || num_qo_heads <= 0 || num_kv_heads <= 0)
        return fail(PA_ERR_INVALID_ARG, "bad token or head count");
    if (head_dim != 128 && head_dim != 256)
        return fail(PA_ERR_UNSUPPORTED, "head_dim must be 128 or 256");
    if (!std::isfinite(rope_theta))
        return fail(PA_ERR_INVALID_ARG, "rope_theta is not finite");
    if (num_tokens == 0)
        return PA_OK;
    const bool rotate = rope_theta > 0.f;
    if (!k_new || !v_new || !out_loc || !k_pool || !v_pool || (rotate && !positions))
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
        !aligned(q, 4) || !aligned(positions, 4) || !aligned(out_loc, 4))
        return fail(PA_ERR_INVALID_ARG, "k_new, v_new and the pools must be 16-byte aligned");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (slot_stride == 0)
        slot_stride = row;
    if (slot_stride < row || slot_stride % 8 != 0)
        return fail(PA_ERR_INVALID_ARG, "slot_stride must be >= Hkv*D and a multiple of 8");
    if (num_slots <= 0)
        return fail(PA_ERR_INVALID_ARG, "num_slots must be positive");
    pa::AppendLaunch l;
    l.k_new = k_new;
    l.v_new = v_new;
    l.q = q;
    l.positions = positions;
    l.out_loc = out_loc;
    l.num_tokens = num_tokens;
    l.num_qo_heads = num_qo_heads;
    l.num_kv_heads = num_kv_heads;
    l.head_dim = head_dim;
    l.rope_theta = rope_theta;
    l.k_pool = k_pool;
    l.v_pool = v_pool;
    l.num_slots = num_slots;
    l.slot_stride = slot_stride;
    l.kv_fp8 = kv_fp8;
    l.k_scale = k_scale;
    l.v_scale = v_scale;
    const int rc = pa::launch_append(l, stream);
    if (rc != 0)
        return hip_fail((hipError_t)rc, "append kernel launch");
    return PA_OK;
}

pa_status pa_kv_append(const void *k_new, const void *v_new, void *q, const int32_t *positions,
                       const int32_t *out_loc, int32_t num_tokens, int32_t num_qo_heads,
                       int32_t num_kv_heads, int32_t head_dim, float rope_theta, void *k_pool,
                       void *v_pool, int64_t num_slots, int64_t slot_stride, pa_stream_t stream) {
    return append_impl(k_new, v_new, q, positions, out_loc, num_tokens, num_qo_heads, num_kv_heads,
                       head_dim, rope_theta, k_pool, v_pool, num_slots, slot_stride, stream, false, 1.f,
                       1.f);
}

pa_status pa_kv_append_fp8(const void *k_new, const void *v_new, void *q, const int32_t *positions,
                           const int32_t *out_loc, int32_t num_tokens, int32_t num_qo_heads,
                           int32_t num_kv_heads, int32_t head_dim, float rope_theta, float k_scale,
                           float v_scale, void *k_pool, void *v_pool, int64_t num_slots,
                           int64_t slot_stride, pa_stream_t stream) {
    return append_impl(k_new, v_new, q, positions, out_loc, num_tokens, num_qo_heads, num_kv_heads,
                       head_dim, rope_theta, k_pool, v_pool, num_slots, slot_stride, stream, true, k_scale,
                       v_scale);
}

pa_status pa_plan_launch_shape(const pa_plan_t *p, int32_t *n_workgroups, int32_t *n_prefix_units) {
    if (!p)
        return fail(PA_ERR_INVALID_ARG, "plan is null");
    if (n_workgroups)
        *n_workgroups = p->mode == pa::PlanMode::kNone ? 0 : p->n_workgroups;
    if (n_prefix_units)
        *n_prefix_units = p->mode == pa::PlanMode::kNone ? 0 : p->n_prefix_units;
    return PA_OK;
}

pa_status pa_plan_info(const pa_plan_t *p, int32_t *mode, int32_t *rows, int32_t *num_qo_heads,
                       int32_t *num_kv_heads, int32_t *head_dim) {
    if (!p)
        return fail(PA_ERR_INVALID_ARG, "plan is null");
    if (mode)
        *mode = (int32_t)p->mode;
    if (rows)
        *rows = p->mode == pa::PlanMode::kPrefill ? p->q_total
                                                   : (p->mode == pa::PlanMode::kDecode ? p->batch : 0);
    if (num_qo_heads)
        *num_qo_heads = p->num_qo_heads;
    if (num_kv_heads)
        *num_kv_heads = p->num_kv_heads;
    if (head_dim)
        *head_dim = p->head_dim;
    return PA_OK;
}

pa_status pa_check_kv_indices(const int32_t *kv_indptr_host, int32_t batch,
                              const int32_t *kv_indices_host, int64_t num_slots,
                              int64_t *first_bad) {
    if (first_bad)
        *first_bad = -1;
    if (batch < 0 || num_slots < 0)
        return fail(PA_ERR_INVALID_ARG, "batch and num_slots must be >= 0");
    if (batch == 0)
        return PA_OK;
    if (!kv_indptr_host)
        return fail(PA_ERR_INVALID_ARG, "kv_indptr_host is null");
    if (kv_indptr_host[0] != 0)
        return fail(PA_ERR_INVALID_ARG, "kv_indptr[0] is not 0");
    for (int32_t b = 0; b < batch; b++)
        if (kv_indptr_host[b + 1] < kv_indptr_host[b])
            return fail(PA_ERR_INVALID_ARG,
                        "kv_indptr decreases at request " + std::to_string(b));
    if (kv_indptr_host[batch] > 0 && !kv_indices_host)
        return fail(PA_ERR_INVALID_ARG, "kv_indices_host is null");
    for (int32_t b = 0; b < batch; b++)
        for (int32_t j = kv_indptr_host[b]; j < kv_indptr_host[b + 1]; j++) {
            const int32_t id = kv_indices_host[j];
            if (id < 0 || (int64_t)id >= num_slots) {
                if (first_bad)
                    *first_bad = j;
                return fail(PA_ERR_INVALID_ARG,
                            "slot id " + std::to_string(id) + " at kv_indices[" + std::to_string(j) +
                                "] (request " + std::to_string(b) + ") is outside [0, " +
                                std::to_string(num_slots) + ")");
            }
        }
    return PA_OK;
}

pa_status pa_plan_host_timing(const pa_plan_t *p, double *total_us, double *wait_us) {
    if (!p || !total_us || !wait_us)
        return fail(PA_ERR_INVALID_ARG, "null argument");
    *total_us = p->plan_total_us;
    *wait_us = p->plan_wait_us;
    return PA_OK;
}

// One decode layer: a cascade plan's prefix units first (the shared prefixes,
// on the matrix cores; their partials are complete when the decode kernel's
// merges read them, same stream), then the decode kernel.  Both kernels take
// bf16 pools or, with kv_fp8, E4M3 pools and their scales.
static pa_status decode_run_impl(const pa_plan_t *p, const void *q, const void *k_pool,
                                 const void *v_pool, int64_t num_slots, int64_t slot_stride,
                                 const int32_t *kv_indices, float sm_scale, float *out, float *lse,
                                 pa_stream_t stream, bool kv_fp8, float k_scale, float v_scale) {
    pa::DecodeLaunch l;
    pa_status st = prepare_run(p, pa::PlanMode::kDecode, q, k_pool, v_pool, num_slots, slot_stride,
                               kv_indices, sm_scale, out, lse, &l);
    if (st != PA_OK)
        return st;
    if (kv_fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite");
    // the E4M3 decode reads up to 16 codes (16 bytes) a lane in one load, so
    // every slot's rows must start 16-byte aligned
    if (kv_fp8 && l.slot_stride % 16 != 0)
        return fail(PA_ERR_INVALID_ARG, "E4M3 pools need a slot_stride that is a multiple of 16 bytes");
    l.kv_fp8 = kv_fp8;
    l.k_scale = k_scale;
    l.v_scale = v_scale;
    hipError_t e = profile_mark(p, (hipStream_t)stream, false);
    if (e != hipSuccess)
        return hip_fail(e, "profile event");
    if (p->n_prefix_units > 0) {
        int rc = pa::launch_prefill(prefix_launch(p, l), stream);
        if (rc == (int)hipErrorNotSupported)
            return fail(PA_ERR_UNSUPPORTED, "prefill kernel not available in this build");
        if (rc != 0)
            return hip_fail((hipError_t)rc, "cascade prefix kernel launch");
    }
    int rc = pa::launch_decode(l, stream);
    if (rc != 0)
        return hip_fail((hipError_t)rc, "decode kernel launch");
    if ((e = profile_mark(p, (hipStream_t)stream, true)) != hipSuccess)
        return hip_fail(e, "profile event");
    return PA_OK;
}

pa_status pa_decode_run(const pa_plan_t *p, const void *q, const void *k_pool, const void *v_pool,
                        int64_t num_slots, int64_t slot_stride, const int32_t *kv_indices,
                        float sm_scale, float *out, float *lse, pa_stream_t stream) {
    return decode_run_impl(p, q, k_pool, v_pool, num_slots, slot_stride, kv_indices, sm_scale, out, lse,
                           stream, false, 1.f, 1.f);
}

pa_status pa_decode_run_fp8(const pa_plan_t *p, const void *q, const void *k_pool, const void *v_pool,
                            int64_t num_slots, int64_t slot_stride, const int32_t *kv_indices,
                            float sm_scale, float k_scale, float v_scale, float *out, float *lse,
                            pa_stream_t stream) {
    return decode_run_impl(p, q, k_pool, v_pool, num_slots, slot_stride, kv_indices, sm_scale, out, lse,
                           stream, true, k_scale, v_scale);
}

// One chunked-prefill layer over bf16 pools or, with kv_fp8, E4M3 pools.
static pa_status prefill_run_impl(const pa_plan_t *p, const void *q, const void *k_pool,
                                  const void *v_pool, int64_t num_slots, int64_t slot_stride,
                                  const int32_t *kv_indices, float sm_scale, float *out, float *lse,
                                  pa_stream_t stream, bool kv_fp8, float k_scale, float v_scale) {
    pa::DecodeLaunch l;
    pa_status st = prepare_run(p, pa::PlanMode::kPrefill, q, k_pool, v_pool, num_slots,
                               slot_stride, kv_indices, sm_scale, out, lse, &l);
    if (st != PA_OK)
        return st;
    // the prefill kernel writes each row's outputs four floats at a time
    if (!aligned(out, 16))
        return fail(PA_ERR_INVALID_ARG, "out must be 16-byte aligned for chunked prefill");
    if (kv_fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite");
    l.kv_fp8 = kv_fp8;
    l.k_scale = k_scale;
    l.v_scale = v_scale;
    hipError_t e = profile_mark(p, (hipStream_t)stream, false);
    if (e != hipSuccess)
        return hip_fail(e, "profile event");
    int rc = pa::launch_prefill(l, stream);
    if (rc == (int)hipErrorNotSupported)
        return fail(PA_ERR_UNSUPPORTED, "prefill kernel not available in this build");
    if (rc != 0)
        return hip_fail((hipError_t)rc, "prefill kernel launch");
    if ((e = profile_mark(p, (hipStream_t)stream, true)) != hipSuccess)
        return hip_fail(e, "profile event");
    return PA_OK;
}

pa_status pa_prefill_chunk_run(const pa_plan_t *p, const void *q, const void *k_pool,
                               const void *v_pool, int64_t num_slots, int64_t slot_stride,
                               const int32_t *kv_indices, float sm_scale, float *out, float *lse,
                               pa_stream_t stream) {
    return prefill_run_impl(p, q, k_pool, v_pool, num_slots, slot_stride, kv_indices, sm_scale, out, lse,
                            stream, false, 1.f, 1.f);
}

pa_status pa_prefill_chunk_run_fp8(const pa_plan_t *p, const void *q, const void *k_pool,
                                   const void *v_pool, int64_t num_slots, int64_t slot_stride,
                                   const int32_t *kv_indices, float sm_scale, float k_scale,
                                   float v_scale, float *out, float *lse, pa_stream_t stream) {
    return prefill_run_impl(p, q, k_pool, v_pool, num_slots, slot_stride, kv_indices, sm_scale, out, lse,
                            stream, true, k_scale, v_scale);
}

pa_status pa_decode_run_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                int64_t num_slots, int64_t slot_stride, const int32_t *kv_indptr,
                                const int32_t *kv_indices, int32_t batch, int32_t num_qo_heads,
                                int32_t num_kv_heads, int32_t head_dim, float sm_scale, float *out,
                                float *lse, pa_stream_t stream) {
    if (num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return fail(PA_ERR_INVALID_ARG, "head counts and head_dim must be positive");
    if (!pa::supported_shape(num_qo_heads, num_kv_heads, head_dim))
        return fail(PA_ERR_UNSUPPORTED,
                    "unsupported head shape (need Hq/Hkv in {1,2,4,8} and D in {128,256})");
    if (batch < 0)
        return fail(PA_ERR_INVALID_ARG, "batch < 0");
    if (batch > pa::kNoAllocMaxBatch || (int64_t)batch * num_kv_heads > pa::kNoAllocMaxSegments)
        return fail(PA_ERR_CAPACITY, "batch above " + std::to_string(pa::kNoAllocMaxBatch) +
                                         " or batch * num_kv_heads above " +
                                         std::to_string(pa::kNoAllocMaxSegments));
    if (batch == 0)
        return PA_OK;
    if (!q || !out || !k_pool || !v_pool || !kv_indices || !kv_indptr)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
        return fail(PA_ERR_INVALID_ARG, "q, k_pool and v_pool must be 16-byte aligned");
    if (!aligned(kv_indices, 4) || !aligned(kv_indptr, 4) || !aligned(out, 4) || !aligned(lse, 4))
        return fail(PA_ERR_INVALID_ARG, "kv_indptr, kv_indices, out and lse must be 4-byte aligned");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (slot_stride == 0)
        slot_stride = row;
    if (slot_stride < row || slot_stride % 8 != 0)
        return fail(PA_ERR_INVALID_ARG, "slot_stride must be >= Hkv*D and a multiple of 8");
    if (slot_stride * 2 > 0x7fffffffLL)
        return fail(PA_ERR_INVALID_ARG, "slot_stride too large");
    if (num_slots <= 0)
        return fail(PA_ERR_INVALID_ARG, "num_slots must be positive");
    if (!std::isfinite(sm_scale))
        return fail(PA_ERR_INVALID_ARG, "sm_scale is not finite");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    const int32_t group = num_qo_heads / num_kv_heads;
    pa::NoAllocLaunch a;
    int rc = pa::noalloc_setup(dev, head_dim, group, &a.scratch, &a.workgroups);
    if (rc != 0)
        return hip_fail((hipError_t)rc, "workspace set-up (hipGetSymbolAddress)");
    if (a.workgroups > pa::kNoAllocMaxWorkgroups ||
        2LL * a.workgroups * group * head_dim > pa::kNoAllocPartialFloats ||
        2LL * a.workgroups * group > pa::kNoAllocPartialLseFloats)
        return fail(PA_ERR_CAPACITY, "this GPU's decode workgroups (" + std::to_string(a.workgroups) +
                                         ") need more partial storage than the workspace holds");
    a.kv_indptr = kv_indptr;
    a.kv_indices = kv_indices;
    a.batch = batch;
    a.num_qo_heads = num_qo_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.num_slots = num_slots;
    a.slot_stride = slot_stride;
    a.sm_scale = sm_scale;
    a.out = out;
    a.lse = lse;
    rc = pa::launch_decode_noalloc(a, stream);
    if (rc != 0)
        return hip_fail((hipError_t)rc, "no-allocation decode launch");
    return PA_OK;
}

pa_status pa_profile_begin(pa_plan_t *p, int32_t capacity) {
    if (!p || capacity <= 0)
        return fail(PA_ERR_INVALID_ARG, "plan is null or capacity <= 0");
    drop_profile(p);
    p->prof_events.assign((size_t)capacity * 2, nullptr);
    for (auto &ev : p->prof_events) {
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) {
            ev = nullptr;
            drop_profile(p);
            return hip_fail(e, "hipEventCreate");
        }
    }
    p->prof_on = true;
    return PA_OK;
}

pa_status pa_profile_end(pa_plan_t *p, double *total_ms, int32_t *n_launches) {
    if (!p || !total_ms || !n_launches)
        return fail(PA_ERR_INVALID_ARG, "null argument");
    double total = 0.0;
    for (int32_t i = 0; i < p->prof_used; i++) {
        hipError_t e = hipEventSynchronize(p->prof_events[(size_t)i * 2 + 1]);
        float ms = 0.f;
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, p->prof_events[(size_t)i * 2], p->prof_events[(size_t)i * 2 + 1]);
        if (e != hipSuccess) {
            drop_profile(p);
            return hip_fail(e, "reading profile events");
        }
        total += ms;
    }
    *total_ms = total;
    *n_launches = p->prof_used;
    drop_profile(p);
    return PA_OK;
}

}  // extern "C"
