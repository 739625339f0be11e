// pa_internal.h -- definitions shared by the host plan, the C ABI and the
// HIP kernels of libpa.  Not installed; the public contract is include/pa.h.
#pragma once

#include <stdint.h>
#include <stddef.h>

#include "pa.h"

namespace pa {

// MI355X geometry the partition is tuned for: 256 compute units in 8 XCDs;
// workgroups are handed to the XCDs round-robin by workgroup id.
constexpr int kNumXcd = 8;
constexpr int kNumCu = 256;

// Decode kernel geometry: 4 waves of 64 lanes per workgroup; a wave walks its
// share of a work unit in tiles of kTileTokens tokens.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * 64;
constexpr int kTileTokens = 16;
// Work units hold a multiple of this many tokens (one tile per wave).
constexpr int kUnitGranule = kDecodeWaves * kTileTokens;

// Automatic split: aim for about this many workgroups per compute unit over
// the launch, with units of at least this many bytes of K+V.
constexpr int kTargetUnitsPerCu = 8;
constexpr int64_t kMinUnitBytes = 128 * 1024;

// Prefill kernel geometry (rows of one query tile = chunk tokens x group).
constexpr int kPrefillTileRows = 128;

enum class PlanMode : int32_t { kNone = 0, kDecode = 1, kPrefill = 2 };

struct PartitionArgs {
    const int32_t *kv_indptr;
    const int32_t *qo_indptr;   // nullptr: decode
    int32_t batch;
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    uint32_t flags;
    int32_t num_cu;
    int32_t num_xcd;
};

struct PartitionResult {
    int32_t n_units = 0;     // including padding units
    int32_t n_merges = 0;
    int32_t n_partials = 0;  // partial slots used
    int32_t unit_tokens = 0; // automatic split length (tokens per unit), 0 if forced
};

// Validates the arguments; fills units/merges up to the capacities.  Returns
// PA_ERR_CAPACITY (with the counts filled) if a capacity is too small.
pa_status partition(const PartitionArgs &a, pa_work_unit *units, int32_t unit_capacity,
                    pa_merge_unit *merges, int32_t merge_capacity, PartitionResult *res,
                    const char **detail);

// Upper bounds on what a plan created with these limits can need: work and
// merge units, and partial storage in rows of head_dim floats (a decode
// partial slot holds `group` rows, a prefill slot kPrefillTileRows rows).
void partition_capacity(int32_t max_batch, int64_t max_kv_total, int32_t max_q_total,
                        int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t num_xcd, int64_t *max_units, int64_t *max_merges,
                        int64_t *max_partial_rows);

bool supported_shape(int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim);

// Kernel launchers (decode.hip / prefill.hip).  All asynchronous on `stream`.
struct DecodeLaunch {
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
    float *partial_o;               // decode: [slots, group, D]; prefill: [slots, tile rows, D]
    float *partial_lse;             // decode: [slots, group];    prefill: [slots, tile rows]
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
};

int launch_decode(const DecodeLaunch &l, void *stream);   // returns hipError_t
int launch_merge(const DecodeLaunch &l, void *stream);
int launch_prefill(const DecodeLaunch &l, void *stream);

}  // namespace pa
