// pa_internal.h -- definitions shared by the host plan, the C ABI and the
// HIP kernels of libpa.  Not installed; the public contract is include/pa.h.
#pragma once

#include <stdint.h>
#include <stddef.h>

#include <vector>

#include "pa.h"

namespace pa {

// MI355X geometry the partition is tuned for: 256 compute units in 8 XCDs;
// workgroups are handed to the XCDs round-robin by workgroup id.
constexpr int kNumXcd = 8;
constexpr int kNumCu = 256;
// Largest XCD count a plan handles.
constexpr int kMaxXcd = 64;
// Accepted range of the per-XCD work weights of the automatic decode split.
constexpr float kMinXcdWeight = 0.25f, kMaxXcdWeight = 4.0f;

// Per-workgroup run-time record of the decode kernel (PA_PLAN_SPEED_FEEDBACK):
// one 64-bit counter per workgroup id, each in a 64-byte line of its own, to
// which the workgroup adds (1 << kClockCountShift) + its run time in ticks of
// the 100 MHz real-time counter.  The count bits and the time bits are
// separated by subtracting two readings: the time added between them must
// stay below 2^40 ticks (about three hours of workgroup time).
constexpr int kClockStride = 8;   // uint64_t per counter
constexpr int kClockCountShift = 40;

// Decode kernel geometry: 4 waves of 64 lanes per workgroup; a wave walks its
// share of a work unit in tiles of kTileTokens tokens.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * 64;
constexpr int kTileTokens = 16;
// Work units hold a multiple of this many tokens (one tile per wave).
constexpr int kUnitGranule = kDecodeWaves * kTileTokens;

// Automatic decode split: as many workgroups as the GPU holds at once, each
// with an equal share of the list entries, never less than kMinUnitBytes of
// K+V per workgroup.  A piece costs about kPieceOverheadTokens tokens of
// work beyond its list entries (state setup, the end-of-piece combine and
// its partial write); pieces are not cut shorter than kMinPieceTokens.
constexpr int64_t kMinUnitBytes = 128 * 1024;
constexpr int kPieceOverheadTokens = 128;
constexpr int kMinPieceTokens = 64;
// Workgroups per compute unit assumed when the occupancy is not known.
constexpr int kDefaultWorkgroupsPerCu = 3;
// pa_plan's automatic decode split gives each compute unit between one and
// as many workgroups as it holds at once, about this many K+V bytes each
// (measured on batch 8 x 512-4096 tokens: 24.0 us per layer with one
// workgroup per unit against 26.0 us with three; batch 64 keeps three).
constexpr int64_t kWorkgroupTargetBytes = 512 * 1024;

// Prefill kernel geometry: rows of one query tile (chunk tokens x group), one
// wave per 32 rows; 8 waves (2 per SIMD, one workgroup per compute unit) at
// head_dim 128, 4 (1 per SIMD) at head_dim 256.
constexpr int prefill_tile_rows(int head_dim) { return head_dim == 256 ? 128 : 256; }
// Prefill workgroups one compute unit holds.
constexpr int kPrefillWorkgroupsPerCu = 1;

enum class PlanMode : int32_t { kNone = 0, kDecode = 1, kPrefill = 2 };

struct PartitionArgs {
    const int32_t *kv_indptr;
    const int32_t *qo_indptr;   // nullptr: decode
    int32_t batch;
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    uint32_t flags;
    int32_t max_workgroups;  // decode workgroups resident at once
    int32_t num_xcd;
    // automatic decode: share of the work of each XCD's workgroups relative
    // to an equal split (num_xcd entries, positive); nullptr = equal
    const float *xcd_weights = nullptr;
    // and of each workgroup id (n_wg_weights entries, positive; ids beyond
    // them weigh 1), multiplied with its XCD's weight
    const float *wg_weights = nullptr;
    int32_t n_wg_weights = 0;
    // automatic decode: entries at the start of each request's list that its
    // decode units skip (read by cascade prefix units); nullptr = none
    const int32_t *kv_skip = nullptr;
    // automatic decode: entries at the start of each request's list that its
    // decode units read with cached loads (a shared prefix left to the L2);
    // nullptr = none
    const int32_t *kv_cached = nullptr;
};

// Shared-prefix groups of a cascade decode plan (pa_plan_cascade).
struct CascadeArgs {
    const int32_t *group_indptr;   // [num_groups + 1] over requests
    int32_t num_groups;
    const int32_t *prefix_len;     // [num_groups]
};

// Cascade prefix units: a prefix is cut into parts of at least
// kCascadeMinPartEntries entries, at most kMaxCascadeParts of them, as many as
// it takes for the prefix units to number about as many as the decode
// workgroups (they run one per workgroup, and short ones are latency bound).
constexpr int kCascadeMinPartEntries = 64;
// Groups with fewer member query rows than this get no prefix units unless
// PA_PLAN_CASCADE_ALL is set.
constexpr int kCascadeMinRows = 64;
constexpr int kMaxCascadeParts = 16;

struct PartitionResult {
    int32_t n_workgroups = 0;  // including empty padding workgroups
    int32_t n_units = 0;
    int32_t n_merges = 0;
    int32_t n_partials = 0;    // partial slots used (cascade: decode and prefix slots)
    int32_t n_prefix_units = 0;   // cascade: prefix units, one workgroup each
};

// Working arrays of the automatic decode partition, kept by a plan between
// steps so that a step's partition allocates nothing once they have grown.
struct PartitionScratch {
    struct Piece {
        int32_t seg, lo, hi;  // segment (KV head * batch + request), list range
        int32_t ordinal;      // index of the piece within its segment
    };
    std::vector<int32_t> seg_request, seg_pieces, seg_first, seg_merge, bin_stream;
    std::vector<Piece> stream;
    std::vector<double> bin_cap;   // budget of each bin when weighted
    std::vector<int32_t> kv_skip;  // cascade: per request, entries of its group's prefix
    std::vector<int32_t> kv_cached;  // cascade: per request, shared entries read cached
};

// Validates the arguments; fills wg_offsets (n_workgroups + 1 entries), units
// and merges up to the capacities.  Returns PA_ERR_CAPACITY (with the counts
// filled) if a capacity is too small.  scratch may be null (then a temporary
// one is used).
pa_status partition(const PartitionArgs &a, PartitionScratch *scratch, int32_t *wg_offsets,
                    int32_t wg_capacity, pa_work_unit *units, int32_t unit_capacity,
                    pa_merge_unit *merges, int32_t merge_capacity, PartitionResult *res,
                    const char **detail);

// Cascade decode partition: the automatic decode split of every list after
// its group's shared prefix (with a merge for every request that has one),
// then the prefix units into prefix_units[prefix_capacity]; merges carry the
// prefix slots.  Returns PA_ERR_CAPACITY if an array is too small.
pa_status cascade_partition(const PartitionArgs &a, const CascadeArgs &c, PartitionScratch *scratch,
                            int32_t *wg_offsets, int32_t wg_capacity, pa_work_unit *units,
                            int32_t unit_capacity, pa_merge_unit *merges, int32_t merge_capacity,
                            pa_work_unit *prefix_units, int32_t prefix_capacity,
                            PartitionResult *res, const char **detail);

// Upper bounds on what a plan created with these limits can need: workgroup
// offsets (entries), work and merge units, and partial storage in rows of
// head_dim floats (a decode partial slot holds `group` rows, a prefill slot
// prefill_tile_rows(head_dim) rows).
void partition_capacity(int32_t max_batch, int64_t max_kv_total, int32_t max_q_total,
                        int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t max_workgroups, int32_t num_xcd, int64_t *max_wg_entries,
                        int64_t *max_units, int64_t *max_merges, int64_t *max_partial_rows,
                        int64_t *max_prefix_units);

bool supported_shape(int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim);

// Kernel launchers (decode.hip / prefill.hip).  All asynchronous on `stream`.
struct DecodeLaunch {
    const int32_t *wg_offsets;      // device, n_workgroups + 1 entries
    int32_t n_workgroups;
    const pa_work_unit *units;      // device
    int32_t n_units;
    const pa_merge_unit *merges;    // device
    int32_t n_merges;
    const void *q;
    const void *k_pool;
    const void *v_pool;
    int64_t slot_stride;            // elements
    int64_t num_slots;
    const int32_t *kv_indices;
    float sm_scale;
    float *out;
    float *lse;                     // may be null
    float *partial_o;               // decode: [slots, group, D]; prefill: [slots, tile rows x D] in register order
    float *partial_lse;             // decode: [slots, group];    prefill: [slots, tile rows]
    int32_t *arrivals;              // per merge unit: parts finished in this launch (zero between launches)
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    bool kv_fp8 = false;             // pools of OCP FP8 E4M3 codes (decode and prefill kernels)
    float k_scale = 1.f, v_scale = 1.f;   // their per-pool scales
    uint64_t *wg_clock = nullptr;    // decode: per-workgroup run-time record, or null
};

int launch_decode(const DecodeLaunch &l, void *stream);   // returns hipError_t
// Whether a pool of num_slots slots of stride_bytes bytes can be addressed
// with 32-bit row offsets (every offset below 2^31).
bool row_offsets_fit_32(int64_t num_slots, uint32_t stride_bytes);
// Decode workgroups one compute unit holds at once, for bf16 or E4M3 pools
// (0 if unknown).
int decode_workgroups_per_cu(int32_t head_dim, int32_t group, bool kv_fp8);
int launch_prefill(const DecodeLaunch &l, void *stream);

// Decode without allocation (pa_decode_run_noalloc): the work table,
// partial results and arrival counters live in a file-scope device array of
// kNoAllocScratchBytes per GPU.  Limits: batch <= kNoAllocMaxBatch, batch *
// Hkv <= kNoAllocMaxSegments, the GPU's decode workgroups (occupancy x
// compute units) <= kNoAllocMaxWorkgroups, and 2 x workgroups x G x D <=
// kNoAllocPartialFloats (2 partial slots per workgroup at most).
constexpr int kNoAllocMaxBatch = 4096;
constexpr int kNoAllocMaxSegments = 16384;
constexpr int kNoAllocMaxWorkgroups = 1024;
constexpr int64_t kNoAllocPartialFloats = 1 << 21;
constexpr int64_t kNoAllocPartialLseFloats = 2 * kNoAllocMaxWorkgroups * 8;
constexpr size_t noalloc_round256(size_t x) { return (x + 255) / 256 * 256; }
constexpr size_t kNoAllocScratchBytes =
    noalloc_round256((size_t)(kNoAllocMaxWorkgroups + 1) * 4) +
    noalloc_round256((size_t)(kNoAllocMaxWorkgroups + kNoAllocMaxSegments) * sizeof(pa_work_unit)) +
    noalloc_round256((size_t)kNoAllocMaxSegments * sizeof(pa_merge_unit)) +
    noalloc_round256((size_t)kNoAllocMaxSegments * 4) + noalloc_round256((size_t)kNoAllocPartialLseFloats * 4) +
    (size_t)kNoAllocPartialFloats * 4;

struct NoAllocLaunch {
    void *scratch;                  // device address of the workspace array
    int32_t workgroups;             // decode workgroups launched (bins)
    const int32_t *kv_indptr;       // device [batch + 1]
    const int32_t *kv_indices;      // device
    int32_t batch, num_qo_heads, num_kv_heads, head_dim;
    const void *q, *k_pool, *v_pool;
    int64_t num_slots, slot_stride;
    float sm_scale;
    float *out, *lse;
};
// Once per device (later calls return the cached values): the device address
// of the workspace and the decode workgroups the device holds at once for
// this head shape.  Returns a hipError_t.
int noalloc_setup(int device, int32_t head_dim, int32_t group, void **scratch_ptr, int32_t *workgroups);
// The planner kernel, then the decode kernel, on `stream`.  Returns a hipError_t.
int launch_decode_noalloc(const NoAllocLaunch &a, void *stream);

// The append step: new tokens' K/V rows written to their slots, K (and the
// query rows, in place, if q is not null) rotated by RoPE when rope_theta > 0.
struct AppendLaunch {
    const void *k_new;          // bf16 [tokens, Hkv, D]
    const void *v_new;          // bf16 [tokens, Hkv, D]
    void *q;                    // bf16 [tokens, Hq, D] or null
    const int32_t *positions;   // device [tokens] (unused when rope_theta <= 0)
    const int32_t *out_loc;     // device [tokens]
    int32_t num_tokens, num_qo_heads, num_kv_heads, head_dim;
    float rope_theta;
    void *k_pool, *v_pool;            // bf16, or E4M3 codes when kv_fp8
    int64_t num_slots, slot_stride;   // elements
    bool kv_fp8 = false;
    float k_scale = 1.f, v_scale = 1.f;   // E4M3 pools: value = scale * code's value
};
int launch_append(const AppendLaunch &l, void *stream);   // returns hipError_t

}  // namespace pa
