// prefill.hip -- gfx950 chunked-prefill kernel of libpa (matrix-core path).
//
// Operation: a request whose prompt is processed in chunks (Agent-Infer page,
// "Agent-Infer: 纯 Rust 编写的高性能 LLM 推理引擎", section "连续批处理":
// chunks of 512 tokens, 64 while decodes run) has a slot list of
// L entries whose last C entries are the chunk's own tokens, already written
// into the pool; chunk token i (0-based) attends to list entries 0 .. L-C+i
// (its cached prefix plus the chunk up to itself).  Scores, softmax and the
// weighted sum are the textbook ones, in the base-2 exponent domain as in the
// decode kernel.
//
// One workgroup runs one work unit at a time: one request, one KV head, a
// tile of chunk tokens whose G query heads are stacked into the tile's rows
// (row r = token * G + head; 256 rows over 8 waves at head_dim 128, 128 rows
// over 4 waves at 256; wave w owns rows 32w .. 32w+31), and a contiguous
// range of the list.  Per tile of KT list entries:
//   * all threads gather the KT K rows and V rows of the KV head (16-byte
//     loads, one slot id per row) into registers two tiles ahead, and write
//     them into one of four LDS stages (row-major, rows padded so that the
//     reads below hit distinct banks; one barrier per two tiles); K stays
//     bf16, V is converted to fp16 (exact for bf16 magnitudes in [2^-14,
//     65520));
//   * each wave computes its 32 x KT score block transposed, S^T = K Q^T,
//     with v_mfma_f32_32x32x16_bf16 (K rows from LDS as the A operand, the
//     wave's 32 query rows held in registers as the B operand for the whole
//     unit), so every lane ends up owning 16 x (KT/32) scores of ONE query
//     row and the row statistics need a single cross-half exchange;
//   * online softmax in fp32 with a lazily moved maximum (as in decode);
//   * the weights P are rounded once to fp16 and O^T += V^T P^T runs on
//     v_mfma_f32_32x32x16_f16; the row sum adds the same rounded weights, so
//     the result is the exact weighted mean of V under them; the V^T operand
//     is read straight from the row-major LDS tile with the transposing read
//     ds_read_b64_tr_b16, in the order of list entries in which each lane
//     already holds its row's weights, so the weights are the P^T operand
//     as they stand (no exchange between lanes);
//   * O^T accumulates in the MFMA's fp32 registers: a lane holds D/2 values
//     of its own row, so rescaling is a per-lane multiply.
// A unit whose V holds a finite value that fp16 cannot represent runs again
// with V scaled by a power of two.  A unit over a whole range writes the
// final rows; the parts of a cut range publish normalised rows and their
// log2-sum-exp, and the last part to finish merges them (no second launch);
// cascade prefix units write partial rows that the decode kernel merges.
//
// Pools of OCP FP8 E4M3 codes with one scale per pool (quantised KV is on the
// Agent-Infer page's roadmap, section "模型支持与发展路线图") take the same
// path: a staging thread gathers 8 codes (8 bytes) of a row instead of 8 bf16
// values and widens them exactly, K to bf16 and V to fp16, into the same LDS
// tiles; k_scale joins the score scale and v_scale multiplies the output rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNoMax = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;
// Waves of a prefill workgroup: one per 32 rows of its query tile (8 at
// head_dim 128, 4 at 256); they share every staged K/V tile.
template <int D>
constexpr int prefill_waves() {
    return prefill_tile_rows(D) / 32;
}

template <int D>
struct PrefillGeo {
    static constexpr int KT = D == 128 ? 64 : 32;     // list entries per tile
    // LDS row pitches (64 banks of 4 bytes).  K rows are read 16 bytes per
    // lane down a column of rows; a 16-byte pad moves each row by 4 banks, so
    // 16 consecutive rows hit distinct banks.  V rows are read by the
    // transposing read, 8 bytes per lane, 4 rows x 32 bytes per 16 lanes and
    // two column blocks per 32 lanes; a 64-byte pad moves each row by 16
    // banks, so the 32 lanes of a read cycle hit 64 distinct banks (a 32-byte
    // pad left 25% of the LDS cycles in bank conflicts, rocprofv3
    // SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; this one none).
    static constexpr int KROW = D * 2 + 16;
    static constexpr int VROW = D * 2 + 64;
    static constexpr int STAGE = KT * (KROW + VROW);  // one buffer: K tile then V tile
    static constexpr int TPR = D / 8;                  // staging threads per row (16 B each)
    static constexpr int THREADS = 64 * prefill_waves<D>();
    static constexpr int RPP = THREADS / TPR;          // rows per staging pass
    static constexpr int PASSES = KT / RPP;
    static constexpr int DS = D / 16;                  // MFMA k-steps over D (QK^T)
    static constexpr int DB = D / 32;                  // 32-wide column blocks of O
    static constexpr int SB = KT / 32;                 // 32-entry score blocks
    static constexpr int KS = KT / 16;                 // MFMA k-steps over entries (PV)
    static_assert(PASSES * RPP == KT, "staging passes must cover the tile");
};

template <int D>
constexpr int prefill_waves_per_simd() {
    return D == 128 ? 2 : 1;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of x held by lane (l + 32) % 64.
__device__ __forceinline__ float other_half(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(__lane_id() < 32 ? p[1] : p[0]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
// A bf16 pair as an fp16 pair (exact for magnitudes in [2^-14, 65520); below,
// fp16's subnormals keep an absolute error under 2^-25; from 65520 up, inf).
__device__ __forceinline__ uint32_t bf16_pair_to_f16(uint32_t u) {
    return pack_f16(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
// The same, with both values multiplied by 2^-shift first (exact unless the
// product falls below fp16's normal range).
__device__ __forceinline__ uint32_t bf16_pair_to_f16_scaled(uint32_t u, int shift) {
    const float a = __uint_as_float(u << 16), b = __uint_as_float(u & 0xffff0000u);
    return pack_f16(__builtin_amdgcn_ldexpf(a, -shift), __builtin_amdgcn_ldexpf(b, -shift));
}
// Smallest magnitude that fp16 rounds to infinity.
constexpr float kF16Overflow = 65520.0f;

// s_waitcnt vmcnt(0): every vector-memory access of this wave has completed.
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Agent-scope (all XCDs) coherent accesses: relaxed atomics, which the
// compiler emits as plain loads and stores with the coherence bits set, so
// that they bypass the non-shared L2 of the issuing XCD.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same coherence for pairs of floats, as raw buffer accesses with the
// instruction's sc1 bit (cache-policy operand 16), over a descriptor of one
// partial slot: byte offset = voff (per lane) + soff (uniform).  One 32-bit
// lane offset instead of a 64-bit address per access keeps the merge's
// registers within the tile loop's budget.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kCoherentPolicy = 16;
constexpr int32_t kBufferWord3 = 0x00020000;   // 32-bit data format, no swizzle or stride
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(float *p, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, bytes, kBufferWord3);
}
__device__ __forceinline__ void store_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float a,
                                                float b) {
    const u32x2_t v = {__float_as_uint(a), __float_as_uint(b)};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, kCoherentPolicy);
}
__device__ __forceinline__ f32x2_t load_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCoherentPolicy));
}

// Eight E4M3 codes (one 8-byte chunk of a row) widened exactly: every E4M3
// value is a bf16 value and an fp16 value (3 mantissa bits, exponents
// 2^-9 .. 2^8), so the K operand goes to the bf16 matrix core and the V
// operand to the fp16 one unchanged; element order is kept.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(u32x2_t c) {
    return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true))};
}
__device__ __forceinline__ u32x4_t e4m3x8_to_f16(u32x2_t c) {
    return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[0], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[0], 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[1], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[1], 1.0f, true))};
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_f16(f16x8_t a, f16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// KV8: pools of OCP FP8 E4M3 codes (one byte per element); the scores carry
// k_scale inside scale_log2 and the outputs are multiplied by out_scale
// (v_scale); bf16 pools pass out_scale = 1 and never use it.
template <int D, int G, bool WIDE, bool KV8>
__global__ __launch_bounds__(64 * prefill_waves<D>())
__attribute__((amdgpu_waves_per_eu(prefill_waves_per_simd<D>(), prefill_waves_per_simd<D>()))) void
prefill_kernel(const int32_t *__restrict__ wg_offsets, const pa_work_unit *__restrict__ units,
               const uint16_t *__restrict__ q, const char *__restrict__ k_pool,
               const char *__restrict__ v_pool, uint64_t stride_bytes,
               const int32_t *__restrict__ kv_indices, float scale_log2, float *__restrict__ out,
               float *__restrict__ lse, float *__restrict__ part_o, float *__restrict__ part_lse,
               const pa_merge_unit *__restrict__ merges, int32_t *__restrict__ arrivals,
               int32_t num_qo_heads, float out_scale) {
    using Geo = PrefillGeo<D>;
    // a staging thread's 8 elements of a row: 16 bytes of bf16 or 8 of codes
    using Chunk = std::conditional_t<KV8, u32x2_t, u32x4_t>;
    constexpr int EB = KV8 ? 1 : 2;   // bytes per pool element
    constexpr int KT = Geo::KT, KROW = Geo::KROW, VROW = Geo::VROW, STAGE = Geo::STAGE;
    constexpr int TPR = Geo::TPR, RPP = Geo::RPP, PASSES = Geo::PASSES;
    constexpr int DS = Geo::DS, DB = Geo::DB, SB = Geo::SB, KS = Geo::KS;
    constexpr int WAVES = prefill_waves<D>(), TILE_ROWS = prefill_tile_rows(D);

    __shared__ __attribute__((aligned(16))) char smem[4 * STAGE];
    __shared__ float flag_lds[WAVES];
    __shared__ int32_t arrived_lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int row = wave * 32 + col;       // tile row of this lane's scores and output
    const int tt = row / G, g = row % G;   // its chunk token (within the tile) and head
    // staging: this thread moves 16-byte chunk `chunk` of rows srow + p*RPP
    const int srow = tid / TPR, chunk = tid % TPR;
    // LDS byte offsets of this lane's MFMA operands within a stage
    const int k_lane = col * KROW + half * 16;
    // V^T operand of a k-step over 16 list entries: the matrix core pairs
    // the 8 k-values of lane half h of its A operand with the 8 of its B
    // operand, in order.  A lane of half h holds its row's weights of entries
    // 4h..4h+3 and 8+4h..8+4h+3 of the k-step (the score layout), so the two
    // transposing reads take V rows 4h+e4 and 8+4h+e4 (e4 = 0..3, the row
    // within a read's 4-row group), and the weights are the B operand as they are.
    const int gi = lane >> 4, e4 = (lane & 15) >> 2, q4 = lane & 3;
    const int v_lane = KT * KROW + (4 * (gi >> 1) + e4) * VROW + (16 * (gi & 1) + 4 * q4) * 2;
    // Scores are scaled after taking their maximum, which needs a positive
    // scale: a negative scale is applied as |scale| to -q (bf16 negation is
    // exact), a zero scale as 1 to q = 0 (every score 0, as it should be).
    const uint32_t q_sign = scale_log2 < 0.f ? 0x80008000u : 0u;
    const bool q_zero = scale_log2 == 0.f;
    const float c_exp = q_zero ? 1.f : fabsf(scale_log2);

    const int32_t unit_begin = wg_offsets[blockIdx.x], unit_end = wg_offsets[blockIdx.x + 1];
    for (int32_t ui = unit_begin; ui < unit_end; ui++) {
        const pa_work_unit unit = units[ui];
        if (unit.request < 0)
            continue;  // padding unit (uniform over the workgroup)

        const int32_t n_tok = unit.q_end - unit.q_begin;
        const bool row_valid = tt < n_tok;
        bf16x8_t qf[DS];
        {
            const int64_t qrow = ((int64_t)(unit.q_begin + tt) * num_qo_heads + unit.kv_head * G + g) * D;
            const uint4 *qp = reinterpret_cast<const uint4 *>(q + qrow + 8 * half);
#pragma unroll
            for (int s = 0; s < DS; s++) {
                uint4 v = (row_valid && !q_zero) ? qp[2 * s] : uint4{0, 0, 0, 0};
                v.x ^= q_sign;
                v.y ^= q_sign;
                v.z ^= q_sign;
                v.w ^= q_sign;
                qf[s] = __builtin_bit_cast(bf16x8_t, v);
            }
        }
        const int32_t kv0 = unit.kv_begin, kv1 = unit.kv_end;
        const int32_t n_tiles = (kv1 - kv0 + KT - 1) / KT;
        // Entries at or past kv1 (the tail of the last tile) are clamped to the
        // range's last entry, so every row read is one the unit references and
        // the loads need no branch; the causal mask gives those entries weight
        // 0 (their row limit is at most kv1 - 1).
        const int32_t *const unit_ids = kv_indices + kv0;   // the unit's entries, uniform base
        int32_t slot[PASSES];
        auto load_slots = [&](int32_t tile) {
#pragma unroll
            for (int p = 0; p < PASSES; p++)
                slot[p] = unit_ids[(uint32_t)min(tile * KT + p * RPP + srow, kv1 - kv0 - 1)];
        };
        // the first tile's slot ids travel with the query loads: one memory
        // round trip fewer before the first tile
        if (n_tiles > 0)
            load_slots(0);
        // the query operand stays in registers for the whole unit; waiting for
        // it here keeps the tile loop from waiting on every load in flight
        wait_vector_memory();

        const uint64_t head_off = (uint64_t)unit.kv_head * D * EB + chunk * 8 * EB;
        // row limit: the last list entry (absolute offset) this row may see
        const int32_t row_last = min(kv1 - 1, unit.diag + tt);
        const int32_t unit_last = min(kv1 - 1, unit.diag);  // smallest row limit of the unit
        // tiles that lie entirely within every row's window need no mask
        const int32_t n_open = max(0, min(n_tiles, (unit_last - kv0 + 1) / KT));

        // One pass over the unit, V staged in fp16 as V * 2^-vshift.  The
        // first pass takes vshift = 0.  If its result is not finite, a V
        // value may have overflowed fp16 (or V holds an infinity or NaN): the
        // unit's largest finite |V| is found by reading its V rows again, and
        // if it is 65520 or more the pass writes nothing and returns true with
        // *retry the power of two that brings every V of the unit below 2^15;
        // the unit then runs again with it (the result scaled back by
        // 2^vshift).  Otherwise the non-finite result is the right one
        // (infinite or NaN V make the result infinite or NaN either way).
        auto run_unit = [&](const int vshift, int *retry) -> bool {
            __syncthreads();  // the previous unit's (or pass's) last tile is no longer read

            Chunk kreg[PASSES], vreg[PASSES];
            auto load_rows = [&]() {
#pragma unroll
                for (int p = 0; p < PASSES; p++) {
                    // pools whose byte offsets stay below 2^31 (the host
                    // checks) take a 32-bit offset, shared by the K and V loads
                    if constexpr (WIDE) {
                        const uint64_t off = (uint64_t)(uint32_t)slot[p] * stride_bytes + head_off;
                        kreg[p] = *reinterpret_cast<const Chunk *>(k_pool + off);
                        vreg[p] = *reinterpret_cast<const Chunk *>(v_pool + off);
                    } else {
                        const uint32_t off =
                            __umul24((uint32_t)slot[p], (uint32_t)stride_bytes) + (uint32_t)head_off;
                        kreg[p] = *reinterpret_cast<const Chunk *>(k_pool + off);
                        vreg[p] = *reinterpret_cast<const Chunk *>(v_pool + off);
                    }
                }
            };
            // K rows as they are (bf16), V rows converted to fp16 (one uniform
            // branch for the whole stage: the scaled form is the rare retry);
            // E4M3 codes widened to the same two forms
            auto store_rows = [&](int buf) {
                char *st = smem + buf * STAGE;
                if constexpr (KV8) {
#pragma unroll
                    for (int p = 0; p < PASSES; p++) {
                        const int r = p * RPP + srow;
                        *reinterpret_cast<u32x4_t *>(st + r * KROW + chunk * 16) = e4m3x8_to_bf16(kreg[p]);
                        *reinterpret_cast<u32x4_t *>(st + KT * KROW + r * VROW + chunk * 16) = e4m3x8_to_f16(vreg[p]);
                    }
                } else {
                    u32x4_t v[PASSES];
                    if (vshift == 0) {
#pragma unroll
                        for (int p = 0; p < PASSES; p++)
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                v[p][j] = bf16_pair_to_f16(vreg[p][j]);
                    } else {
#pragma unroll
                        for (int p = 0; p < PASSES; p++)
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                v[p][j] = bf16_pair_to_f16_scaled(vreg[p][j], vshift);
                    }
#pragma unroll
                    for (int p = 0; p < PASSES; p++) {
                        const int r = p * RPP + srow;
                        *reinterpret_cast<u32x4_t *>(st + r * KROW + chunk * 16) = kreg[p];
                        *reinterpret_cast<u32x4_t *>(st + KT * KROW + r * VROW + chunk * 16) = v[p];
                    }
                }
            };

            float m = kNoMax, l = 0.f;
            f32x16_t o[DB];
#pragma unroll
            for (int b = 0; b < DB; b++)
                o[b] = f32x16_t{};

            // Four LDS stages, tile t in stage t % 4.  Rows are gathered two
            // tiles ahead and stored at the end of the tile before, so the
            // barrier before tile t (t even) covers the stores of tiles t and
            // t+1, and no stage is rewritten while a wave may still read it:
            // one barrier per two tiles.
            if (n_tiles > 0) {
                if (vshift != 0)
                    load_slots(0);   // a second pass: the first one moved on
                load_rows();
                if (n_tiles > 1)
                    load_slots(1);
                store_rows(0);
                if (n_tiles > 1) {
                    load_rows();
                    if (n_tiles > 2)
                        load_slots(2);
                    store_rows(1);
                }
            }

            // one tile: entries kv0 + it*KT ...; MASK: some entry lies beyond a row's limit
            auto step = [&](int32_t it, auto mask_tag) {
                constexpr bool MASK = decltype(mask_tag)::value;
                const int buf = it & 3;
                if (it + 2 < n_tiles) {
                    load_rows();  // tile it+2, slots fetched one iteration earlier
                    if (it + 3 < n_tiles)
                        load_slots(it + 3);
                }
                if ((it & 1) == 0)
                    __syncthreads();  // stages of tiles it, it+1 written by every thread

                const char *st = smem + buf * STAGE;
                // S^T = K Q^T, one 32x32 block per 32 entries; entry of s[b][i]:
                // b*32 + 8*(i/4) + 4*half + i%4 within the tile
                f32x16_t s[SB];
#pragma unroll
                for (int b = 0; b < SB; b++) {
                    uint4 ka[DS];
#pragma unroll
                    for (int d = 0; d < DS; d++)
                        ka[d] = *reinterpret_cast<const uint4 *>(st + k_lane + b * 32 * KROW + d * 32);
                    s[b] = mfma(__builtin_bit_cast(bf16x8_t, ka[0]), qf[0], f32x16_t{});
#pragma unroll
                    for (int d = 1; d < DS; d++)
                        s[b] = mfma(__builtin_bit_cast(bf16x8_t, ka[d]), qf[d], s[b]);
                }
                if (MASK) {
                    const int32_t lim = row_last - (kv0 + it * KT) - 4 * half;
#pragma unroll
                    for (int b = 0; b < SB; b++)
#pragma unroll
                        for (int i = 0; i < 16; i++)
                            if (b * 32 + 8 * (i / 4) + (i % 4) > lim)
                                s[b][i] = -INFINITY;
                }
                // Weights relative to the running maximum as it stands, rounded
                // once to fp16; the row sum adds the rounded weights, so the
                // result is the exact weighted mean of V under them.  The tile's
                // own maximum is only needed when a weight does not fit fp16
                // (a score 16 or more above the running maximum in log2 units,
                // and always on a unit's first tile): the sum then comes out
                // infinite (or NaN), and the tile is weighed again after the
                // maximum has moved, as in the online softmax, to any score that
                // exceeds it by more than the slack.  Weights stay below 65520.
                const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
                uint32_t ph[SB][8];
                auto weigh = [&](float lsum) {
#pragma unroll
                    for (int b = 0; b < SB; b++)
#pragma unroll
                        for (int i = 0; i < 16; i += 2) {
                            const float p0 = fast_exp2(fmaf(s[b][i], c_exp, -m));
                            const float p1 = fast_exp2(fmaf(s[b][i + 1], c_exp, -m));
                            ph[b][i / 2] = pack_f16(p0, p1);
                            lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, ph[b][i / 2]), ones, lsum,
                                                          false);
                        }
                    return lsum;
                };
                float l_new = weigh(l);
                if (__builtin_amdgcn_ballot_w64(!(l_new <= 3.4028235e38f))) {
                    float tmax = -INFINITY;
#pragma unroll
                    for (int b = 0; b < SB; b++)
#pragma unroll
                        for (int i = 0; i < 16; i++)
                            tmax = fmaxf(tmax, s[b][i]);
                    tmax *= c_exp;
                    tmax = fmaxf(tmax, other_half(tmax));
                    const bool move = tmax > m + kRescaleSlack;
                    const float m_new = move ? tmax : m;
                    const float alpha = fast_exp2(m - m_new);
                    l *= alpha;
#pragma unroll
                    for (int b = 0; b < DB; b++)
#pragma unroll
                        for (int i = 0; i < 16; i++)
                            o[b][i] *= alpha;
                    m = m_new;
                    l_new = weigh(l);
                }
                l = l_new;
                // O^T += V^T P^T, 16 entries per k-step
#pragma unroll
                for (int k = 0; k < KS; k++) {
                    const int b = k / 2, w0 = 4 * (k % 2);  // dword index of entries 16*(k%2) + 4*half
                    const f16x8_t bh = __builtin_bit_cast(
                        f16x8_t, uint4{ph[b][w0], ph[b][w0 + 1], ph[b][w0 + 2], ph[b][w0 + 3]});
#pragma unroll
                    for (int db = 0; db < DB; db++) {
                        const int off = v_lane + k * 16 * VROW + db * 64;
                        const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(st + off));
                        const i16x4_t hi4 =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(st + off + 8 * VROW));
                        const f16x8_t a = __builtin_bit_cast(
                            f16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
                        o[db] = mfma_f16(a, bh, o[db]);
                    }
                }
                if (it + 2 < n_tiles)
                    store_rows((it + 2) & 3);
            };
            for (int32_t it = 0; it < n_open; it++)
                step(it, std::false_type{});
            for (int32_t it = n_open; it < n_tiles; it++)
                step(it, std::true_type{});

            // (E4M3 values stay below 448: fp16 holds every V, so a non-finite
            // result of an 8-bit pool is the right one and needs no check)
            if constexpr (!KV8) {
                if (vshift == 0) {
                    // a non-finite O or row sum anywhere in the workgroup?
                    float chk = l;
#pragma unroll
                    for (int db = 0; db < DB; db++)
#pragma unroll
                        for (int i = 0; i < 16; i++)
                            chk += o[db][i];
                    const bool bad = !(fabsf(chk) <= 3.4028235e38f);
                    if (lane == 0)
                        flag_lds[wave] = __builtin_amdgcn_ballot_w64(bad) != 0 ? 1.f : 0.f;
                    __syncthreads();
                    float any_bad = 0.f;
#pragma unroll
                    for (int w = 0; w < WAVES; w++)
                        any_bad += flag_lds[w];
                    if (any_bad != 0.f) {
                        // the unit's largest finite |V| (read again: a rare path)
                        float vm = 0.f;
                        for (int32_t tile = 0; tile < n_tiles; tile++) {
                            load_slots(tile);
                            load_rows();
#pragma unroll
                            for (int p = 0; p < PASSES; p++)
#pragma unroll
                                for (int j = 0; j < 4; j++) {
                                    const float a = fabsf(__uint_as_float(vreg[p][j] << 16));
                                    const float b = fabsf(__uint_as_float(vreg[p][j] & 0xffff0000u));
                                    vm = fmaxf(vm, fmaxf(a <= 3.4028235e38f ? a : 0.f, b <= 3.4028235e38f ? b : 0.f));
                                }
                        }
#pragma unroll
                        for (int off = 32; off > 0; off >>= 1)
                            vm = fmaxf(vm, __shfl_xor(vm, off));
                        __syncthreads();   // every wave has read the flags
                        if (lane == 0)
                            flag_lds[wave] = vm;
                        __syncthreads();
                        float wmax = 0.f;
#pragma unroll
                        for (int w = 0; w < WAVES; w++)
                            wmax = fmaxf(wmax, flag_lds[w]);
                        if (wmax >= kF16Overflow) {
                            // 2^e <= wmax < 2^(e+1): wmax * 2^-(e-14) < 2^15
                            *retry = __builtin_amdgcn_readfirstlane((int)((__float_as_uint(wmax) >> 23) & 0xff) - 127 - 14);
                            return true;
                        }
                    }
                }
            }

            // the two lanes of a row hold disjoint halves of its entries
            const float l_row = l + other_half(l);
            const float inv = l_row > 0.f ? __builtin_amdgcn_ldexpf(1.f / l_row, vshift) : 0.f;
            const float lse2 = l_row > 0.f ? m + fast_log2(l_row) : -INFINITY;
            // O^T element i of block db: column db*32 + 8*(i/4) + 4*half + i%4
            auto write_row = [&](float *dst, float f) {
#pragma unroll
                for (int db = 0; db < DB; db++)
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const float4 v = {o[db][4 * j] * f, o[db][4 * j + 1] * f, o[db][4 * j + 2] * f,
                                          o[db][4 * j + 3] * f};
                        *reinterpret_cast<float4 *>(dst + db * 32 + 8 * j + 4 * half) = v;
                    }
            };
            if (unit.partial < 0) {
                if (!row_valid)
                    return false;
                const int64_t orow = (int64_t)(unit.q_begin + tt) * num_qo_heads + unit.kv_head * G + g;
                if (lse && half == 0)
                    lse[orow] = lse2 * kLn2;
                write_row(out + orow * D, KV8 ? inv * out_scale : inv);
                return false;
            }
            if (unit.part_stride > 0) {
                // a cascade prefix unit: query token tt's rows go to slot
                // partial + tt * part_stride (G rows per slot, the decode
                // layout), merged by the decode kernel
                if (!row_valid)
                    return false;
                const int64_t prow = ((int64_t)unit.partial + (int64_t)tt * unit.part_stride) * G + g;
                if (half == 0)
                    part_lse[prow] = lse2;
                write_row(part_o + prow * D, KV8 ? inv * out_scale : inv);
                return false;
            }

            // One of the parts of a cut KV range.  It publishes its normalised
            // rows in fp16 and their log2-sum-exp in its partial slot, the rows
            // in register order (wave w's block of 32 rows, then 8-byte piece k
            // of every lane in turn, four values a piece: each store and load
            // below is one contiguous 512-byte run).  The rows are stored as
            // O * 2^-vshift (below 2^15 when vshift > 0, below 65520 otherwise:
            // fp16 holds them), and vshift after them; fp16 rounds them to
            // 2^-12 of their size, 8 times finer than the bf16 inputs, and
            // halves the bytes written here and read back by the merge.  The
            // stores are agent-scope coherent stores, which write through the
            // compute unit's own L2 (the 8 XCDs do not share one); once they
            // have completed (s_waitcnt vmcnt(0) in every wave, then the
            // barrier) it counts itself in.  The part that arrives last reads
            // every part back with agent-scope coherent loads, issued after it
            // has seen the count, merges them, and clears the counter for the
            // next launch.  As in the decode kernel's merge, the ordering
            // rests on gfx950's coherence of sc1 accesses, not on the C++
            // memory model alone: re-check it on another architecture or
            // compiler (an acquire-release counter would order it formally,
            // at the cost of whole-L2 write-back and invalidation).
            constexpr int32_t SLOT_BYTES = TILE_ROWS * D * 4;
            // The lane id passes through an empty asm statement, so that the
            // offsets derived from it are computed here and not hoisted to the
            // kernel's start, where they would hold registers through the
            // tile loop.
            uint32_t lid = lane;
            asm volatile("" : "+v"(lid));
            // this lane's byte offset within a slot: its wave's block, its 8 bytes of a piece
            const uint32_t lane_off = (uint32_t)(wave * (32 * D * 2)) + lid * 8;
            constexpr int32_t SHIFT_FLOAT = TILE_ROWS * D / 2;   // vshift, after the fp16 rows
            {
                float *const base = part_o + (int64_t)unit.partial * (TILE_ROWS * D);
                const __amdgpu_buffer_rsrc_t slot = slot_rsrc(base, SLOT_BYTES);
                if (half == 0)
                    store_coherent(part_lse + (int64_t)unit.partial * TILE_ROWS + row, lse2);
                if (tid == 0)
                    store_coherent(base + SHIFT_FLOAT, __int_as_float(vshift));
                const float f = __builtin_amdgcn_ldexpf(inv, -vshift);
#pragma unroll
                for (int db = 0; db < DB; db++)
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        store_coherent2(slot, lane_off + (db * 4 + k) * 512, 0,
                                        __uint_as_float(pack_f16(o[db][4 * k] * f, o[db][4 * k + 1] * f)),
                                        __uint_as_float(pack_f16(o[db][4 * k + 2] * f, o[db][4 * k + 3] * f)));
            }
            wait_vector_memory();
            __syncthreads();
            if (tid == 0)
                arrived_lds = __hip_atomic_fetch_add(arrivals + unit.merge, 1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int32_t first = merges[unit.merge].first_partial, n_parts = merges[unit.merge].n_parts;
            if (arrived_lds != n_parts - 1)
                return false;
            // log-sum-exp merge of the parts in index order with a running
            // maximum, acc = sum_p 2^(lse_p - M) O_p, wsum = sum_p 2^(lse_p -
            // M), every part (this one too) read back from its slot: the same
            // sums whichever part arrives last
            float M = -INFINITY, wsum = 0.f;
#pragma unroll
            for (int db = 0; db < DB; db++)
                o[db] = f32x16_t{};
            for (int32_t pi = first; pi < first + n_parts; pi++) {
                float *const base = part_o + (int64_t)pi * (TILE_ROWS * D);
                const float lp = load_coherent(part_lse + (int64_t)pi * TILE_ROWS + row);
                const int shift = __float_as_int(load_coherent(base + SHIFT_FLOAT));
                const __amdgpu_buffer_rsrc_t src = slot_rsrc(base, SLOT_BYTES);
                const float mx = fmaxf(M, lp);
                const bool live = mx != -INFINITY;      // some part so far is not empty
                const float a = live ? fast_exp2(M - mx) : 1.f;   // 0 while M is -inf
                const float w = live ? fast_exp2(lp - mx) : 0.f;
                const float wv = __builtin_amdgcn_ldexpf(w, shift);   // weight of the stored rows
                // two column blocks (32 values of the row) per round trip
#pragma unroll
                for (int dp = 0; dp < DB; dp += 2) {
                    f32x2_t v[8];
#pragma unroll
                    for (int k = 0; k < 8; k++)
                        v[k] = load_coherent2(src, lane_off + (dp * 4 + k) * 512, 0);
#pragma unroll
                    for (int j = 0; j < 2; j++)
#pragma unroll
                        for (int i = 0; i < 16; i++) {
                            // the element is copied out before the bit cast: the
                            // ROCm 7.2 compiler reads element 0 for a bit cast of a
                            // vector element written in place
                            const float x = v[4 * j + i / 4][(i / 2) % 2];
                            const f16x2_t h = __builtin_bit_cast(f16x2_t, x);
                            o[dp + j][i] = fmaf(wv, (float)h[i % 2], o[dp + j][i] * a);
                        }
                }
                wsum = fmaf(wsum, a, w);
                M = live ? mx : M;
            }
            if (tid == 0)
                __hip_atomic_store(arrivals + unit.merge, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (!row_valid)
                return false;
            const int64_t orow = (int64_t)(unit.q_begin + tt) * num_qo_heads + unit.kv_head * G + g;
            if (lse && half == 0)
                lse[orow] = wsum > 0.f ? (M + fast_log2(wsum)) * kLn2 : -INFINITY;
            // (8-bit pools: the parts hold rows of code values, below 448 and
            // so within fp16; v_scale is applied here, after the merge)
            write_row(out + orow * D, wsum > 0.f ? (KV8 ? out_scale / wsum : 1.f / wsum) : 0.f);
            return false;
        };
        // one call site (a loop) keeps the pass inlined once; vshift is
        // uniform over the workgroup
        int vshift = 0;
        for (int pass = 0; pass < 2 && run_unit(vshift, &vshift); pass++) {
        }
    }
}

template <int D, int G, bool KV8>
int launch_prefill_dgk(const DecodeLaunch &l, hipStream_t stream) {
    const uint64_t stride_bytes = (uint64_t)l.slot_stride * (KV8 ? 1 : 2);
    const bool wide = stride_bytes >= (1u << 24) || !row_offsets_fit_32(l.num_slots, (uint32_t)stride_bytes);
    // 8-bit pools: K = k_scale * code enters the scores, V = v_scale * code the output
    const float scale_log2 = (KV8 ? l.sm_scale * l.k_scale : l.sm_scale) * kLog2e;
    const float out_scale = KV8 ? l.v_scale : 1.0f;
    if (wide)
        hipLaunchKernelGGL((prefill_kernel<D, G, true, KV8>), dim3(l.n_workgroups), dim3(PrefillGeo<D>::THREADS), 0,
                           stream, l.wg_offsets, l.units, (const uint16_t *)l.q, (const char *)l.k_pool,
                           (const char *)l.v_pool, stride_bytes, l.kv_indices, scale_log2, l.out, l.lse,
                           l.partial_o, l.partial_lse, l.merges, l.arrivals, l.num_qo_heads, out_scale);
    else
        hipLaunchKernelGGL((prefill_kernel<D, G, false, KV8>), dim3(l.n_workgroups), dim3(PrefillGeo<D>::THREADS), 0,
                           stream, l.wg_offsets, l.units, (const uint16_t *)l.q, (const char *)l.k_pool,
                           (const char *)l.v_pool, stride_bytes, l.kv_indices, scale_log2, l.out, l.lse,
                           l.partial_o, l.partial_lse, l.merges, l.arrivals, l.num_qo_heads, out_scale);
    return (int)hipGetLastError();
}

template <int D, int G>
int launch_prefill_dg(const DecodeLaunch &l, hipStream_t stream) {
    return l.kv_fp8 ? launch_prefill_dgk<D, G, true>(l, stream) : launch_prefill_dgk<D, G, false>(l, stream);
}

}  // namespace

int launch_prefill(const DecodeLaunch &l, void *stream) {
    if (l.n_workgroups == 0)
        return 0;
    hipStream_t s = (hipStream_t)stream;
    const int G = l.num_qo_heads / l.num_kv_heads;
    if (l.head_dim == 128) {
        switch (G) {
        case 1: return launch_prefill_dg<128, 1>(l, s);
        case 2: return launch_prefill_dg<128, 2>(l, s);
        case 4: return launch_prefill_dg<128, 4>(l, s);
        case 8: return launch_prefill_dg<128, 8>(l, s);
        }
    } else if (l.head_dim == 256) {
        switch (G) {
        case 1: return launch_prefill_dg<256, 1>(l, s);
        case 2: return launch_prefill_dg<256, 2>(l, s);
        case 4: return launch_prefill_dg<256, 4>(l, s);
        case 8: return launch_prefill_dg<256, 8>(l, s);
        }
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace pa
