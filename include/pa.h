/*
 * pa.h -- C ABI of libpa: batched grouped-query decode attention over a
 * token-granular paged KV pool on AMD Instinct MI355X (gfx950), with a
 * chunked-prefill variant over the same pool.
 *
 * Sources.  The pool follows the Agent-Infer page ("Agent-Infer: 纯 Rust 编写的
 * 高性能 LLM 推理引擎"), section "分页 KV 缓存": one pool slot per token (page
 * size 1), shared by every request so that decode batches across requests,
 * with a plan computed once per decode step and reused by every layer, over
 * buffers allocated up front (same section, and stages 2-3 of the table in
 * "优化历程").  The head geometry follows the Pegainfer page ("Pegainfer:
 * 纯Rust+CUDA构建的LLM推理引擎"), section "关键技术实现", items 1-2 (GQA with
 * 32 query heads over 8 KV heads and head_dim 128; head_dim 256 for Qwen3.5's
 * full-attention layers).  Chunked prefill follows the Agent-Infer page,
 * section "连续批处理" (chunks of 512 tokens, 64 while decodes run).  The pages
 * call the kernels through a plain C FFI (Pegainfer page, "核心组件概览",
 * ffi.rs); this header is that kind of boundary.
 *
 * What is computed (the pages name the operation but do not write it out;
 * this is the textbook reading):
 *   g = Hq / Hkv; query head h reads KV head h / g.
 *   For request b, S = kv_indices[kv_indptr[b] .. kv_indptr[b+1]) in list order.
 *   s_j = sm_scale * <q[b,h,:], K[S_j, h/g, :]>
 *   out[b,h,:] = sum_j exp(s_j - m) V[S_j, h/g, :] / sum_j exp(s_j - m),  m = max_j s_j
 *   lse[b,h]   = m + ln(sum_j exp(s_j - m))
 *   An empty list gives out = 0 and lse = -inf.  A slot listed twice counts
 *   twice.  Lists of different requests may share slots.
 *   Prefill: request b brings C_b = qo_indptr[b+1]-qo_indptr[b] query rows,
 *   which are the last C_b entries of its slot list (L_b >= C_b); chunk row i
 *   attends to list positions 0 .. (L_b - C_b) + i (causal inside the chunk).
 *
 * Data layout (all device pointers unless said otherwise):
 *   q        bf16, [B, Hq, D] for decode, [T, Hq, D] for prefill, contiguous,
 *            16-byte aligned.
 *   k_pool,  bf16; the row of slot s and KV head kh starts at element
 *   v_pool   s * slot_stride + kh * D and holds D contiguous values.
 *            slot_stride (elements) is >= Hkv*D and a multiple of 8, so a
 *            [slots, Hkv, D] pool has slot_stride = Hkv*D (pass 0 for that),
 *            and a fused [slots, 2, Hkv, D] buffer passes 2*Hkv*D with
 *            v_pool = k_pool + Hkv*D.  Both pools 16-byte aligned.  Pools may
 *            exceed 4 GiB; offsets are computed in 64 bits when they do.
 *   kv_indices int32 slot ids, 0 <= id < num_slots; read on the device.
 *   kv_indptr / qo_indptr int32 CSR offsets, read on the HOST by pa_plan.
 *   out      fp32, [B, Hq, D] (decode) or [T, Hq, D] (prefill), contiguous.
 *   lse      fp32, [B, Hq] or [T, Hq], natural log; may be NULL.
 *
 * Precision: bf16 inputs, fp32 arithmetic (the prefill variant multiplies
 * bf16 tiles on the matrix cores with fp32 accumulation), fp32 outputs.
 *
 * Streams: every entry point that touches the GPU takes a hipStream_t passed
 * as pa_stream_t (NULL = the null stream) and is asynchronous on it.  The run
 * entry points never allocate and never synchronise, so they can be captured
 * into a HIP graph.  Runs must be ordered after the pa_plan call whose
 * result they read (same stream, or an event); kv_indices must not change
 * between that pa_plan and the last run of the step.  A captured run keeps
 * the launch size of the plan current at capture and reads the plan's device
 * tables, which stay at the same addresses for the life of the plan: its
 * replays after a later pa_plan of the same plan are valid while that
 * pa_plan yields the same number of workgroups and of cascade prefix units
 * (pa_plan_launch_shape), as the same lists with the same flags do, and as a
 * decode step whose work fills the GPU does whatever its lengths; otherwise
 * capture again.
 *
 * Errors: every call returns a pa_status; no exception crosses the ABI.
 * Argument errors are detected on the host before any GPU work is enqueued,
 * and then nothing is enqueued.  A HIP failure returns PA_ERR_HIP; faults of
 * kernels already enqueued surface from a later call or at the caller's
 * synchronisation.  pa_last_error_detail() describes the last failure of the
 * calling thread.  Slot ids outside [0, num_slots) are not checked on the
 * device: they are the caller's error and their result is undefined.
 */
#ifndef PA_H
#define PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_plan pa_plan_t;
typedef void *pa_stream_t; /* a hipStream_t */

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad CSR offsets, bad sizes */
    PA_ERR_UNSUPPORTED = 2,   /* head_dim not in {128, 256}, Hq/Hkv not in {1, 2, 4, 8} */
    PA_ERR_CAPACITY = 3,      /* more requests / tokens than the plan was created for */
    PA_ERR_PLAN_MISMATCH = 4, /* a run that does not match the last pa_plan (mode, heads) */
    PA_ERR_HIP = 5            /* a HIP runtime call failed */
} pa_status;

/* pa_plan flags */
#define PA_PLAN_FORCE_SPLITS_SHIFT 8
#define PA_PLAN_FORCE_SPLITS_MASK (0xffffu << PA_PLAN_FORCE_SPLITS_SHIFT)
/* Cut every request's KV list (per KV head) into exactly n parts (1 <= n <=
 * PA_MAX_FORCED_SPLITS), instead of the automatic split.  Parts may be empty.
 * Used to test that the result does not depend on the partition.  Each part
 * is then a workgroup of its own.  Forced parts count against the plan's
 * capacity: a plan holds at least num_kv_heads * (max_batch + max_kv_total /
 * 256) work units, and pa_plan returns PA_ERR_CAPACITY when batch * n exceeds
 * max_batch + max_kv_total / 256.  In prefill mode every (request, KV head,
 * row tile) is cut into n parts: the n * num_kv_heads * sum_b ceil(C_b / t)
 * units (t = 256 / (Hq/Hkv) chunk tokens per tile at head_dim 128, 128 /
 * (Hq/Hkv) at 256) always fit when they number at most 1024 + num_kv_heads *
 * (ceil(max_q_total / t) + max_batch) (a larger max_q_total makes room); a
 * call that needs more units than the plan holds returns PA_ERR_CAPACITY. */
#define PA_PLAN_FORCE_SPLITS(n) (((uint32_t)(n) & 0xffffu) << PA_PLAN_FORCE_SPLITS_SHIFT)
#define PA_MAX_FORCED_SPLITS 256
/* Keep the automatic split but place workgroups in plain order instead of
 * grouping neighbouring requests on one XCD. */
#define PA_PLAN_NO_XCD_ORDER 0x1u
/* Balance the automatic decode partition by the measured speed of the
 * compute units.  The decode launches of a plan computed with this flag (when
 * they fill the GPU) record how long each workgroup ran (one atomic add per
 * workgroup).  A later pa_plan call with the flag reads those records without
 * waiting (each call starts an asynchronous copy that a following call
 * consumes once it has completed) and moves each compute unit's share of the
 * next partition towards the rate it achieved.  A launch that fills the GPU
 * places workgroup ids w, w + C, w + 2C, ... on one compute unit (C = compute
 * units), every launch alike, and the units of one GPU do not run at equal
 * speeds (which are slow changes from run to run, and between XCDs), so an
 * equal split leaves the fast ones idle while the slowest finish.  Ignored for
 * prefill and forced splits.  For a fixed plan the results are deterministic;
 * two steps with identical inputs may be cut differently and so differ by
 * rounding (within the usual tolerance).  The weights in use are read with
 * pa_plan_workgroup_weights. */
#define PA_PLAN_SPEED_FEEDBACK 0x2u
/* pa_plan_cascade: give every group with a prefix its prefix units.  Without
 * it, groups whose member query rows (members x Hq/Hkv) number fewer than 64
 * get no prefix units: the plain split decodes their lists, the members read
 * the shared slots at the same moment, and those rows are loaded so that
 * they stay in the L2 cache for the other members (every other row is
 * streamed), which measured faster than a separate prefix pass over so few
 * rows. */
#define PA_PLAN_CASCADE_ALL 0x4u
/* Size the decode partition for pa_decode_run_fp8: its kernel keeps fewer
 * workgroups resident per compute unit than the bf16 one, and the automatic
 * split cuts the lists for as many workgroups as run at once.  Either run
 * call accepts a plan made with or without it (the result is the same up to
 * rounding); a mismatched plan only balances the work less well. */
#define PA_PLAN_KV_FP8 0x8u

/* Largest max_kv_total a plan accepts: list entries are addressed with 32-bit
 * byte offsets. */
#define PA_MAX_KV_TOTAL (1LL << 29)

/*
 * pa_plan_create: allocate a plan object for up to max_batch requests whose
 * slot lists hold at most max_kv_total (<= PA_MAX_KV_TOTAL) entries in total,
 * and (prefill) at most
 * max_q_total query rows.  All device and pinned-host memory the plan and its
 * runs need is allocated here, on the current HIP device, once.
 *   num_qo_heads % num_kv_heads == 0, group Hq/Hkv in {1, 2, 4, 8};
 *   head_dim in {128, 256}.
 * Returns PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED for bad sizes, PA_ERR_HIP if
 * an allocation fails.  *out is set only on success.
 */
pa_status pa_plan_create(pa_plan_t **out, int32_t max_batch, int64_t max_kv_total,
                         int32_t max_q_total, int32_t num_qo_heads,
                         int32_t num_kv_heads, int32_t head_dim);

/*
 * pa_plan: partition one step's work; called once per decode (or prefill)
 * step and reused by every layer's run.
 *   kv_indptr_host [batch+1], host memory, non-decreasing, kv_indptr[0] = 0,
 *     kv_indptr[batch] <= max_kv_total.
 *   qo_indptr_host NULL for a decode plan; for a prefill plan, [batch+1] host
 *     offsets of each request's chunk rows, non-decreasing, starting at 0, with
 *     qo_indptr[b+1]-qo_indptr[b] <= kv_indptr[b+1]-kv_indptr[b] and total rows
 *     <= max_q_total.
 *   flags: PA_PLAN_* bits.
 * The partition is computed on the host and uploaded with one asynchronous
 * copy on `stream` from pinned staging memory owned by the plan (two staging
 * buffers alternate; a call waits only if the copy of the call before the
 * previous one has not finished).  The host arrays may be reused as soon as
 * this returns.
 */
pa_status pa_plan(pa_plan_t *plan, const int32_t *kv_indptr_host,
                  const int32_t *qo_indptr_host, int32_t batch, uint32_t flags,
                  pa_stream_t stream);

/*
 * pa_plan_cascade: a decode plan that reads each group's shared prompt prefix
 * once for the whole group (cascade decode; the radix prefix cache that makes
 * requests share leading slots is on the Agent-Infer page, section "前缀缓存").
 *   kv_indptr_host, batch, flags, stream: as in pa_plan (decode);
 *   group_indptr_host [num_groups + 1]: group g is requests
 *     [group_indptr[g], group_indptr[g+1]); group_indptr[0] = 0,
 *     nondecreasing, group_indptr[num_groups] = batch;
 *   prefix_len_host [num_groups]: the first prefix_len[g] entries of every
 *     member's list are the same slot ids (the caller guarantees it; they are
 *     read from the first member's list), 0 <= prefix_len[g] <= the shortest
 *     member list.
 * pa_decode_run under this plan launches two kernels: the prefix units
 * (matrix-core attention of all member query rows over the shared prefix,
 * at most 128 / (Hq/Hkv) requests per unit, the prefix cut into up to 16
 * parts) writing partial results, then the decode kernel over the rest of
 * every list, whose merges fold the prefix partials in.  The result equals
 * pa_decode_run under pa_plan up to summation order.  Groups with
 * prefix_len 0 and singleton groups cost nothing extra.  Errors: as pa_plan,
 * plus PA_ERR_INVALID_ARG for inconsistent groups or prefix lengths.
 * pa_decode_run_fp8 runs cascade plans the same way over E4M3 pools (the
 * prefix units read the codes as pa_prefill_chunk_run_fp8 does; add
 * PA_PLAN_KV_FP8 to the flags to size the decode part for its kernel).
 */
pa_status pa_plan_cascade(pa_plan_t *plan, const int32_t *kv_indptr_host, int32_t batch,
                          const int32_t *group_indptr_host, int32_t num_groups,
                          const int32_t *prefix_len_host, uint32_t flags, pa_stream_t stream);

/*
 * pa_decode_run: decode attention of one layer under a decode plan.
 *   q [batch, Hq, D] bf16; k_pool / v_pool as above with num_slots slots;
 *   kv_indices int32 device array with kv_indptr[batch] entries;
 *   sm_scale: softmax scale (e.g. 1/sqrt(D) as a float);
 *   out [batch, Hq, D] fp32; lse [batch, Hq] fp32 or NULL.
 * One kernel launch.  Where a list was split, each part writes a partial
 * result into the plan's workspace and counts its arrival; the part that
 * arrives last merges them and resets the count.  So two runs of one plan
 * must not execute concurrently (runs on one stream are fine).
 */
pa_status pa_decode_run(const pa_plan_t *plan, const void *q, const void *k_pool,
                        const void *v_pool, int64_t num_slots, int64_t slot_stride,
                        const int32_t *kv_indices, float sm_scale, float *out,
                        float *lse, pa_stream_t stream);

/*
 * pa_decode_run_fp8: pa_decode_run over 8-bit pools.  The pools hold OCP FP8
 * E4M3 codes (1 byte per element, same [slots, Hkv, D] layout and slot
 * stride in elements = bytes), and the row values are k_scale * code and
 * v_scale * code (one scale per pool).  Quantised KV is on the Agent-Infer
 * page's roadmap (section "模型支持与发展路线图": FP8 among the quantisation
 * formats); the
 * format and the per-pool scales are this library's reading.  Same plan,
 * arguments, output and errors as pa_decode_run, plus PA_ERR_INVALID_ARG for
 * a non-finite scale or a slot_stride that is not a multiple of 16 (bytes:
 * rows are read 16 codes at a time).  Code 0x7F / 0xFF (NaN) in a referenced
 * row makes the results NaN; unreferenced rows are never read.
 */
pa_status pa_decode_run_fp8(const pa_plan_t *plan, const void *q, const void *k_pool,
                            const void *v_pool, int64_t num_slots, int64_t slot_stride,
                            const int32_t *kv_indices, float sm_scale, float k_scale,
                            float v_scale, float *out, float *lse, pa_stream_t stream);

/*
 * pa_prefill_chunk_run: chunked-prefill attention of one layer under a
 * prefill plan (pa_plan with qo_indptr_host != NULL).
 *   q [T, Hq, D] bf16 with T = qo_indptr[batch]; pools and kv_indices as in
 *   decode (each request's chunk tokens are the last entries of its list,
 *   already written into the pool); out [T, Hq, D] fp32, 16-byte aligned
 *   (rows are written four floats at a time); lse [T, Hq] or NULL.
 */
pa_status pa_prefill_chunk_run(const pa_plan_t *plan, const void *q, const void *k_pool,
                               const void *v_pool, int64_t num_slots, int64_t slot_stride,
                               const int32_t *kv_indices, float sm_scale, float *out,
                               float *lse, pa_stream_t stream);

/*
 * pa_prefill_chunk_run_fp8: pa_prefill_chunk_run over 8-bit pools (the
 * pools of pa_decode_run_fp8: OCP FP8 E4M3 codes, 1 byte per element, row
 * values k_scale * code and v_scale * code).  Same plan (any prefill plan;
 * PA_PLAN_KV_FP8 is not needed), arguments, output and errors as
 * pa_prefill_chunk_run, plus PA_ERR_INVALID_ARG for a non-finite scale.  The
 * codes are widened exactly on the way into the matrix cores (every E4M3
 * value is a bf16 and an fp16 value); a NaN code in a row a query token sees
 * makes that token's results NaN.
 */
pa_status pa_prefill_chunk_run_fp8(const pa_plan_t *plan, const void *q, const void *k_pool,
                                   const void *v_pool, int64_t num_slots, int64_t slot_stride,
                                   const int32_t *kv_indices, float sm_scale, float k_scale,
                                   float v_scale, float *out, float *lse, pa_stream_t stream);

/*
 * pa_decode_run_noalloc: pa_decode_run without a plan object and without any
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split of the lists over workgroups is computed on the device on every call
 * (an equal split of the (KV head, request) entries, no XCD placement or
 * speed feedback), and the work table, partial results and arrival counters
 * live in a workspace inside the library: a device array of about 9.4 MiB
 * that each GPU the library runs on holds until the process ends.
 *   q, k_pool, v_pool, num_slots, slot_stride, kv_indices, sm_scale, out,
 *   lse: as in pa_decode_run (same layout, same result up to summation
 *   order, out and lse written for every request);
 *   kv_indptr: DEVICE int32 [batch + 1] CSR offsets (kv_indptr[0] = 0,
 *   non-decreasing, kv_indptr[batch] <= PA_MAX_KV_TOTAL); offsets that break
 *   these rules are detected on the device and give NaN in out and lse;
 *   batch <= 4096, batch * num_kv_heads <= 16384; head shapes as in
 *   pa_plan_create.
 * Two kernels on `stream`; nothing is allocated, freed or synchronised.
 * Every call on one GPU uses that GPU's single workspace, so calls that can
 * run at the same time on one GPU (other streams, or other host threads) race
 * and must be ordered by the caller; calls on one stream are fine.  Errors:
 * PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED as pa_plan_create and
 * pa_decode_run, PA_ERR_CAPACITY above the limits (nothing is enqueued),
 * PA_ERR_HIP if the workspace cannot be located on the current device.
 */
pa_status pa_decode_run_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                int64_t num_slots, int64_t slot_stride, const int32_t *kv_indptr,
                                const int32_t *kv_indices, int32_t batch, int32_t num_qo_heads,
                                int32_t num_kv_heads, int32_t head_dim, float sm_scale, float *out,
                                float *lse, pa_stream_t stream);

/* Release everything pa_plan_create allocated.  Waits for the plan's pending
 * uploads; the caller must not destroy a plan that enqueued runs still use. */
void pa_plan_destroy(pa_plan_t *plan);

/* Static description of a status code. */
const char *pa_strerror(pa_status status);

/* Description of the calling thread's last failure ("" if none). */
const char *pa_last_error_detail(void);

/*
 * Host-only inspection of the partition (no GPU needed).
 *
 * A plan is a list of workgroups; workgroup w processes the work units
 * units[wg_offsets[w] .. wg_offsets[w+1]) one after the other.  Workgroup w is
 * launched as workgroup id w, which the hardware places on XCD w % 8.
 *
 * pa_work_unit is one piece of work as the kernels read it: KV head kv_head of
 * request `request`, list entries [kv_begin, kv_end) (absolute offsets into
 * kv_indices), query rows [q_begin, q_end) (prefill; decode: q_begin =
 * request, q_end = request + 1), and where the result goes: partial < 0 writes
 * the final output, partial >= 0 writes partial slot `partial`, later merged.
 * diag (prefill): query row q_begin + r sees list entries up to offset
 * diag + r inclusive (the causal window); decode units set diag = kv_end - 1.
 * merge: index of the pa_merge_unit that combines this unit's partial with
 * the other parts of its range (-1 when partial < 0).  part_stride (prefix
 * units of a cascade plan, see pa_plan_cascade): query row q_begin + t of the
 * unit writes partial slot partial + t * part_stride; 0 for every other unit
 * (a prefill unit's rows then fill slot `partial` of the prefill layout).
 * cached_end (decode units): list entries before this absolute offset are
 * read with ordinary loads that stay in the L2 for other requests (the shared
 * prefix of a small group in a cascade plan); the rest are streamed
 * (non-temporal loads).  0 in every other unit.
 *
 * pa_merge_unit: the partial slots [first_partial, first_partial + n_parts)
 * that make up query rows [q_begin, q_end) of KV head kv_head, plus, in a
 * cascade plan, the slots [prefix_first, prefix_first + prefix_parts) written
 * by the prefix units of the request's group before the decode kernel runs
 * (prefix_parts = 0 otherwise).  Decode and prefix partial slots hold one row
 * per query head of the KV head's group.
 */
typedef struct pa_work_unit {
    int32_t request;
    int32_t kv_head;
    int32_t kv_begin;
    int32_t kv_end;
    int32_t q_begin;
    int32_t q_end;
    int32_t partial;
    int32_t diag;
    int32_t merge;
    int32_t part_stride;
    int32_t cached_end;
    int32_t reserved2;
} pa_work_unit;

typedef struct pa_merge_unit {
    int32_t request;
    int32_t kv_head;
    int32_t q_begin;
    int32_t q_end;
    int32_t first_partial;
    int32_t n_parts;
    int32_t prefix_first;
    int32_t prefix_parts;
} pa_merge_unit;

/*
 * pa_kv_append: the step before attention.  Writes the K and V rows of
 * num_tokens new tokens into their slots of the token-granular pool (one slot
 * per token: Agent-Infer page, section "分页 KV 缓存"), rotating K by rotary
 * position embedding (an operator named on the Pegainfer page, section
 * "核心组件概览") when rope_theta > 0, and, if q is not NULL, rotating the
 * tokens' query rows in place with the same positions.  Rotation: pair
 * i < D/2 couples elements i and i + D/2 and turns them by the angle
 * positions[t] * rope_theta^(-2i/D) (computed in double precision, rounded
 * once to bf16, nearest-even).  rope_theta <= 0: K is copied unrotated and q
 * is left alone.
 *   k_new, v_new   device bf16 [num_tokens, num_kv_heads, head_dim], 16-byte aligned
 *   q              device bf16 [num_tokens, num_qo_heads, head_dim] or NULL
 *   positions      device int32 [num_tokens] (may be NULL when rope_theta <= 0)
 *   out_loc        device int32 [num_tokens]: the slot of each token, distinct;
 *                  a token whose slot is outside [0, num_slots) is not written
 *   k_pool, v_pool device bf16 pools as for the runs (slot_stride 0 = Hkv*D)
 * Asynchronous on `stream`; allocates nothing.  Overlapping slots between
 * tokens of one call race.  PA_ERR_INVALID_ARG for null or misaligned
 * pointers and bad sizes, PA_ERR_UNSUPPORTED for head_dim not in {128, 256}.
 */
pa_status pa_kv_append(const void *k_new, const void *v_new, void *q, const int32_t *positions,
                       const int32_t *out_loc, int32_t num_tokens, int32_t num_qo_heads,
                       int32_t num_kv_heads, int32_t head_dim, float rope_theta, void *k_pool,
                       void *v_pool, int64_t num_slots, int64_t slot_stride, pa_stream_t stream);

/*
 * pa_kv_append_fp8: pa_kv_append into 8-bit pools (the pools of
 * pa_decode_run_fp8: OCP FP8 E4M3 codes, 1 byte per element, one scale per
 * pool; quantised KV is on the Agent-Infer page's roadmap, section
 * "模型支持与发展路线图", the format and its rounding are this library's
 * reading).  K is rotated as by pa_kv_append, in double precision, and each
 * rotated value y is stored as the E4M3 code nearest to y / k_scale; each V
 * value x (bf16) as the code nearest to x / v_scale.  Nearest: the quotient
 * is formed in double and rounded once to nearest, ties to even, among the
 * finite codes, so magnitudes at or beyond 448 store +-448 (0x7E / 0xFE),
 * NaN stores 0x7F, and a zero result keeps the input's sign.  q, if given,
 * is rotated in place and stays bf16.
 *   k_pool, v_pool  device E4M3 codes [slots, Hkv, D] (slot_stride in bytes,
 *                   0 = Hkv*D, a multiple of 8), 16-byte aligned
 *   k_scale, v_scale  finite and > 0
 * Other arguments, ownership and errors as pa_kv_append, plus
 * PA_ERR_INVALID_ARG for a scale that is not finite and positive.
 */
pa_status pa_kv_append_fp8(const void *k_new, const void *v_new, void *q, const int32_t *positions,
                           const int32_t *out_loc, int32_t num_tokens, int32_t num_qo_heads,
                           int32_t num_kv_heads, int32_t head_dim, float rope_theta, float k_scale,
                           float v_scale, void *k_pool, void *v_pool, int64_t num_slots,
                           int64_t slot_stride, pa_stream_t stream);

/*
 * pa_partition: compute the partition pa_plan would upload, into host arrays.
 *   Arguments as in pa_plan_create / pa_plan; max_workgroups is the number of
 *   decode workgroups the GPU holds at once (pa_plan uses the kernel's
 *   occupancy times the compute-unit count; <= 0 here means 768, three per
 *   compute unit of an MI355X).
 *   wg_offsets[wg_capacity], units[unit_capacity] and merges[merge_capacity]
 *   receive the lists; *n_workgroups, *n_units, *n_merges and *n_partials their
 *   lengths (wg_offsets holds *n_workgroups + 1 entries).  PA_ERR_CAPACITY if
 *   an array is too small (the counts are still written).
 */
pa_status pa_partition(const int32_t *kv_indptr_host, const int32_t *qo_indptr_host,
                       int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                       int32_t head_dim, uint32_t flags, int32_t max_workgroups,
                       int32_t *wg_offsets, int32_t wg_capacity, pa_work_unit *units,
                       int32_t unit_capacity, pa_merge_unit *merges, int32_t merge_capacity,
                       int32_t *n_workgroups, int32_t *n_units, int32_t *n_merges,
                       int32_t *n_partials);

/*
 * pa_partition_weighted: pa_partition with work weights for the automatic
 * decode split: the workgroup that bin i runs as (id w, on XCD w % 8) gets
 * xcd_weights[w % 8] * wg_weights[w] times the budget of an equal split
 * (ids at or beyond n_wg_weights weigh 1).  n_xcd_weights must be 8 (the XCDs
 * of an MI355X); every weight must be in [0.25, 4]; they need not average 1
 * (the budgets are rescaled to the work).  NULL weights weigh 1; both NULL is
 * pa_partition.  XCD weights apply only to the XCD-ordered placement; other
 * modes (prefill, forced splits) ignore all weights.
 */
pa_status pa_partition_weighted(const int32_t *kv_indptr_host, const int32_t *qo_indptr_host,
                                int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                                int32_t head_dim, uint32_t flags, int32_t max_workgroups,
                                const float *xcd_weights, int32_t n_xcd_weights,
                                const float *wg_weights, int32_t n_wg_weights,
                                int32_t *wg_offsets, int32_t wg_capacity, pa_work_unit *units,
                                int32_t unit_capacity, pa_merge_unit *merges,
                                int32_t merge_capacity, int32_t *n_workgroups, int32_t *n_units,
                                int32_t *n_merges, int32_t *n_partials);

/*
 * pa_partition_cascade: the partition pa_plan_cascade would upload, into host
 * arrays (arguments as in pa_plan_cascade and pa_partition).  The decode part
 * is returned as by pa_partition; prefix_units[prefix_capacity] receives the
 * prefix units (*n_prefix_units of them; prefix unit i runs as workgroup i of
 * the prefix launch).  *n_partials counts decode and prefix slots.
 * PA_ERR_CAPACITY if an array is too small (the counts are still written).
 */
pa_status pa_partition_cascade(const int32_t *kv_indptr_host, int32_t batch,
                               const int32_t *group_indptr_host, int32_t num_groups,
                               const int32_t *prefix_len_host, int32_t num_qo_heads,
                               int32_t num_kv_heads, int32_t head_dim, uint32_t flags,
                               int32_t max_workgroups, int32_t *wg_offsets, int32_t wg_capacity,
                               pa_work_unit *units, int32_t unit_capacity, pa_merge_unit *merges,
                               int32_t merge_capacity, pa_work_unit *prefix_units,
                               int32_t prefix_capacity, int32_t *n_workgroups, int32_t *n_units,
                               int32_t *n_merges, int32_t *n_partials, int32_t *n_prefix_units);

/*
 * pa_plan_xcd_weights: the per-XCD weights the plan's next automatic decode
 * partition will use (share of an XCD's workgroups relative to an equal
 * split; they average 1).  *n_xcd receives the XCD count and
 * min(capacity, *n_xcd) weights are written to `weights` (which may be NULL
 * when capacity is 0).  They start at 1 and change only through
 * pa_plan_set_xcd_weights.
 *
 * pa_plan_set_xcd_weights: set them.  n must equal the XCD count and every
 * weight be finite and in [0.25, 4]; they are rescaled to average 1.  Used by
 * callers that know their XCDs' speeds, or to pin a partition.
 */
pa_status pa_plan_xcd_weights(const pa_plan_t *plan, float *weights, int32_t capacity,
                              int32_t *n_xcd);
pa_status pa_plan_set_xcd_weights(pa_plan_t *plan, const float *weights, int32_t n);

/*
 * pa_plan_workgroup_weights: the per-workgroup-id weights that
 * PA_PLAN_SPEED_FEEDBACK has measured (1 until it has; id w weighs what its
 * compute unit w % C does; they multiply the XCD weights and average 1 over
 * the units that recorded).  *n receives their number and min(capacity, *n)
 * are written to `weights` (which may be NULL when capacity is 0).
 */
pa_status pa_plan_workgroup_weights(const pa_plan_t *plan, float *weights, int32_t capacity,
                                    int32_t *n);

/*
 * Kernel timing (instrumentation for benchmarks).  pa_profile_begin creates
 * `capacity` pairs of HIP events (it allocates; call it outside timed or
 * captured regions) and makes the following runs of this plan record one
 * pair around their attention kernel, on the run's stream, until the pairs are
 * used up.  pa_profile_end waits for the recorded events, returns the summed
 * kernel time in milliseconds and the number of timed launches, and stops
 * recording.  A pair spans every kernel of its run (with a cascade plan, the
 * prefix units and the decode kernel; splits are merged inside the kernels).
 * Not for concurrent use.
 */
pa_status pa_profile_begin(pa_plan_t *plan, int32_t capacity);
pa_status pa_profile_end(pa_plan_t *plan, double *total_ms, int32_t *n_launches);

/*
 * Host time of the last successful pa_plan call on this plan, measured inside
 * the library with a steady clock: *total_us is the whole call, *wait_us the
 * part spent waiting for the upload of two calls back to finish (its pinned
 * staging buffer is reused).  PA_ERR_INVALID_ARG for null pointers.
 */
pa_status pa_plan_host_timing(const pa_plan_t *plan, double *total_us, double *wait_us);

/*
 * pa_plan_launch_shape: the launch sizes of the runs under the last
 * successful pa_plan / pa_plan_cascade call on this plan: *n_workgroups, the
 * grid of the attention kernel, and *n_prefix_units, the grid of a cascade
 * plan's prefix launch (0 without one).  A run captured into a HIP graph
 * keeps the sizes current at capture, so its replays stay valid after a
 * later pa_plan of the same plan while both are unchanged: a caller that
 * keeps one graph per batch size compares them after each pa_plan and
 * captures again when they differ.  Host only; any output pointer may be
 * NULL.  PA_ERR_INVALID_ARG for a null plan.
 */
pa_status pa_plan_launch_shape(const pa_plan_t *plan, int32_t *n_workgroups, int32_t *n_prefix_units);

/*
 * pa_plan_info: what the last successful pa_plan / pa_plan_cascade call on
 * this plan set up, so that a caller can size its tensors for the runs.
 *   *mode: 0 no plan yet, 1 decode, 2 prefill;
 *   *rows: query rows a run reads and writes (decode: batch; prefill: the
 *          total chunk rows qo_indptr[batch]);
 *   *num_qo_heads, *num_kv_heads, *head_dim: as given to pa_plan_create.
 * A run reads q [rows, Hq, D] and writes out [rows, Hq, D] and lse [rows, Hq].
 * Any output pointer may be NULL.  PA_ERR_INVALID_ARG for a null plan.
 */
pa_status pa_plan_info(const pa_plan_t *plan, int32_t *mode, int32_t *rows,
                       int32_t *num_qo_heads, int32_t *num_kv_heads, int32_t *head_dim);

/*
 * pa_check_kv_indices: opt-in bounds check of a step's slot lists on the
 * host (the runs do not check slot ids on the device: an id outside
 * [0, num_slots) is undefined behaviour there).  For callers that keep a host
 * copy of the lists, or debug runs that copy them back.
 *   kv_indptr_host [batch+1] and kv_indices_host [kv_indptr[batch]], host
 *   memory, as passed to pa_plan and the runs; num_slots as for the runs.
 * Returns PA_OK when kv_indptr is a valid CSR offset array (starts at 0,
 * non-decreasing) and every id is in [0, num_slots).  Otherwise
 * PA_ERR_INVALID_ARG, with *first_bad (if not NULL) set to the position in
 * kv_indices of the first out-of-range id (-1 for a bad kv_indptr), and
 * pa_last_error_detail() naming the request, the position and the id.
 * Reads only its arguments; no GPU work.
 */
pa_status pa_check_kv_indices(const int32_t *kv_indptr_host, int32_t batch,
                              const int32_t *kv_indices_host, int64_t num_slots,
                              int64_t *first_bad);

/*
 * pa_prefill_tile_rows: query rows (chunk tokens x Hq/Hkv) of one prefill
 * work unit at this head_dim, i.e. the tile height pa_partition uses to cut
 * chunk rows (0 for an unsupported head_dim).  Host-only.
 */
int32_t pa_prefill_tile_rows(int32_t head_dim);

/* Library version as major*10000 + minor*100 + patch. */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
