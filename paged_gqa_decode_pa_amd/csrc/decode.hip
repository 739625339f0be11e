// decode.hip -- gfx950 kernels of libpa's decode path: split-KV paged GQA
// decode attention and the log-sum-exp merge of split partitions.
//
// Operation: batched decode attention over a token-granular KV pool (one slot
// per token, shared by all requests), Agent-Infer page ("Agent-Infer: 纯 Rust
// 编写的高性能 LLM 推理引擎"), section "分页 KV 缓存"; grouped-query heads,
// Pegainfer page ("Pegainfer: 纯Rust+CUDA构建的LLM推理引擎"), section
// "关键技术实现" items 1-2.  The arithmetic is the textbook softmax attention,
// computed online in the base-2 exponent domain:
//     s = <q, k> * scale * log2(e);  p = exp2(s - m);  o = sum p v / sum p
// which gives the same result as exp(<q,k>*scale - m') with m' = m * ln 2.
//
// Lane layout of the decode kernel (one workgroup = 4 waves; it runs the work
// units of its list one after another, each unit being one request, one KV
// head and a contiguous part of its slot list):
//   * a K or V row of one head is D bf16 = D*2 bytes; LPR = D/8 lanes load it
//     with one 16-byte load each (lane chunk c = lane % LPR holds elements
//     8c..8c+7), so one wave-wide load instruction fetches RPI = 64/LPR whole
//     rows (4 rows at D = 128, 2 at D = 256): fully coalesced 128-bit loads,
//     each lane gathering through its own slot id;
//     E4M3 pools (one byte per element) take 16 elements a lane for groups of
//     up to 4 query heads (LPR = D/16; a row of 8 lanes is two quads 8 lanes
//     apart) and 8 for groups of 8;
//   * a wave walks the unit in tiles of NI instructions (NI*RPI tokens); the
//     four waves take every fourth tile; tiles alternate between two register
//     sets, so one tile's K and V rows are in flight while the other's are
//     used;
//   * slot ids are read through a buffer descriptor whose range ends at the
//     unit's last entry: an id past it reads as 0 (a valid slot, whose row
//     the masked scores ignore), so the loads of the look-ahead need no
//     clamping;
//   * each K row is used by all G query heads of its group straight from the
//     registers it was loaded into (dot2 bf16 products, fp32 accumulation);
//     the partial dot products are reduced across the row's lanes with DPP
//     and the reduction is "transposed": G values per lane go in, and lane c
//     comes out holding the full score of head c % G, so each (token, head)
//     exponential is computed by LPR/G lanes instead of LPR.  Lane c keeps
//     its query heads in the order h ^ (c % G), so that at every exchange
//     step a lane adds its partner's value at a fixed register index (no
//     per-lane selects);
//   * softmax is online per (lane row, head) with a lazily moved running
//     maximum (it moves only when a score exceeds it by more than 8 in the
//     log2 domain, so weights stay <= 256 and rescaling is rare);
//   * V rows accumulate into fp32 o[G][8] per lane; at the end the rows of a
//     wave are combined with cross-lane shuffles, then the four waves through
//     LDS, and the unit writes either the final output or a partial result
//     (normalised o and its log2-sum-exp);
//   * a unit that wrote a partial counts its arrival on its merge unit; the
//     unit that arrives last merges the parts by log-sum-exp weights, writes
//     the final output and resets the count to zero for the next launch.
//     Partials are stored and loaded with agent-scope atomic accesses, which
//     are coherent across the XCDs' separate L2s, and every store has
//     completed (vmcnt 0) before the arrival is counted.  The C++ memory
//     model does not order relaxed stores before a relaxed counter update by
//     itself: this relies on gfx950's sc1 stores having reached the
//     device-coherent level once vmcnt reports them complete, and on sc1
//     loads issued after the count was seen reading that level.  Re-check it
//     on any other architecture or compiler (the merge-protocol, forced-split
//     and determinism tests guard it).  An acquire-release counter at agent
//     scope would order it formally, through a write-back and invalidation of
//     the whole L2 around every arrival: +25% on batch 64, +82% on batch 8.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima start here instead of -inf so that exp2(s - m) is never
// exp2(-inf - -inf); any real score is far above it.
constexpr float kNoMax = -1.0e30f;
// Lazy rescale threshold (log2 domain): weights stay below 2^8.
constexpr float kRescaleSlack = 8.0f;
// Word 3 of a raw buffer descriptor: 32-bit data format, no swizzle, no
// index stride.
constexpr int32_t kBufferWord3 = 0x00020000;


__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane moves inside 16-lane rows (all sources valid: permutations).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf,
                                                              true));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;   // row_ror:4
constexpr int kRowRor8 = 0x128;   // row_ror:8 (== lane ^ 8 within a row)

// Cross-row exchanges without lane-index arithmetic.  v_permlane16_swap
// (v_permlane32_swap) with both operands x returns, in its two results, the
// lane's own x and that of lane ^ 16 (lane ^ 32), in an order that depends
// on the lane; sums and maxima do not care about the order.
__device__ __forceinline__ float sum_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
// ds_swizzle in bit mode inside 32-lane halves: source lane =
// ((lane & AND) | OR) ^ XOR.
template <int AND, int OR, int XOR>
__device__ __forceinline__ float swizzle(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), AND | (OR << 5) | (XOR << 10)));
}
// Sum (max) over the rows of a wave instruction: lanes that hold the same
// chunk of different rows (lane ^ 16, lane ^ 32 at 16 lanes per row; lane ^
// 32 at 32; lane ^ 4, ^ 16, ^ 32 at 8, where a row is two quads 8 lanes
// apart).
template <int LPR>
__device__ __forceinline__ float sum_rows(float x) {
    if constexpr (LPR == 8)
        x += swizzle<0x1f, 0, 4>(x);
    if constexpr (LPR <= 16)
        x = sum_xor16(x);
    return sum_xor32(x);
}
template <int LPR>
__device__ __forceinline__ float max_rows(float x) {
    if constexpr (LPR == 8)
        x = fmaxf(x, swizzle<0x1f, 0, 4>(x));
    if constexpr (LPR <= 16)
        x = max_xor16(x);
    return max_xor32(x);
}

// Agent-scope (all XCDs) coherent 32-bit accesses.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every vector memory access this wave issued has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left free).
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32):
// exp2(-inf) = 0, exp2(0) = 1.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane `h` of this lane's G-lane group (G <= 4: inside the quad;
// G = 8: a swizzle over groups of 8 lanes).
template <int G>
__device__ __forceinline__ float group_bcast(float x, int h, int lane) {
    if constexpr (G == 1) {
        return x;
    } else if constexpr (G == 2) {
        // quad_perm [h, h, 2+h, 2+h]
        return h == 0 ? dpp_mov<0xA0>(x) : dpp_mov<0xF5>(x);
    } else if constexpr (G == 4) {
        switch (h) {
        case 0: return dpp_mov<0x00>(x);
        case 1: return dpp_mov<0x55>(x);
        case 2: return dpp_mov<0xAA>(x);
        default: return dpp_mov<0xFF>(x);
        }
    } else {
        switch (h) {
        case 0: return swizzle<0x18, 0, 0>(x);
        case 1: return swizzle<0x18, 1, 0>(x);
        case 2: return swizzle<0x18, 2, 0>(x);
        case 3: return swizzle<0x18, 3, 0>(x);
        case 4: return swizzle<0x18, 4, 0>(x);
        case 5: return swizzle<0x18, 5, 0>(x);
        case 6: return swizzle<0x18, 6, 0>(x);
        default: return swizzle<0x18, 7, 0>(x);
        }
    }
}

// Score partials of one K row for the G heads, reduced across the row's LPR
// lanes (the reduction is "transposed": lane c returns the full dot product
// of head c % G).  Lane c holds, at index j, the query of head j ^ (c % G).
// Exchange step k pairs lane c with c ^ 2^k: the partner's value at index
// 2m+1 belongs to the same head as this lane's value at 2m, so
// v[m] = v[2m] + partner(v[2m+1]) halves the values while keeping the head of
// index m equal to (m << (k+1)) ^ (c % G); after log2(G) steps lane c holds
// head c % G, and the remaining steps add the lanes of the row that hold the
// same head.  In the first step the partner's value is the starting value of
// the dot-product chain of index 2m, which saves the add and the zeroing of
// that chain's accumulator.
template <int G, int LPR, int NQ>
__device__ __forceinline__ float row_scores(const uint32_t (&qv)[G][NQ], const uint32_t (&k)[NQ]) {
    auto chain = [&](int j, float c) {
        float a = c;
#pragma unroll
        for (int w = 0; w < NQ; w++)
            a = dot2_bf16(qv[j][w], k[w], a);
        return a;
    };
    float x;
    if constexpr (G == 1) {
        x = chain(0, 0.f);
        x += dpp_mov<kQuadXor1>(x);
        x += dpp_mov<kQuadXor2>(x);
    } else {
        float v[G / 2];
#pragma unroll
        for (int m = 0; m < G / 2; m++)
            v[m] = chain(2 * m, dpp_mov<kQuadXor1>(chain(2 * m + 1, 0.f)));
        if constexpr (G >= 4) {
#pragma unroll
            for (int m = 0; m < G / 4; m++)
                v[m] = v[2 * m] + dpp_mov<kQuadXor2>(v[2 * m + 1]);
        }
        if constexpr (G >= 8)
            v[0] = v[0] + swizzle<0x1f, 0, 4>(v[1]);
        x = v[0];
        if constexpr (G == 2)
            x += dpp_mov<kQuadXor2>(x);
    }
    if constexpr (LPR == 8) {
        // the row's other quad holds the same heads 8 lanes away
        x += dpp_mov<kRowRor8>(x);
    } else {
        if constexpr (G <= 4)
            x += dpp_mov<kRowRor4>(x);
        x += dpp_mov<kRowRor8>(x);
        if constexpr (LPR == 32)
            x = sum_xor16(x);
    }
    return x;
}

// The plan tables are read-only during a launch.  Reading them through the
// constant address space lets the compiler use scalar loads even after the
// kernel's own stores and atomics (with generic pointers those would be
// vector loads, whose waits also wait for the K/V rows in flight).
using ConstantI32 = const __attribute__((address_space(4))) int32_t *;
__device__ __forceinline__ ConstantI32 constant_view(const int32_t *p) { return (ConstantI32)p; }
__device__ __forceinline__ pa_work_unit load_unit(const pa_work_unit *units, int32_t i) {
    const ConstantI32 w = (ConstantI32)(units + i);
    pa_work_unit u;
    u.request = w[0]; u.kv_head = w[1]; u.kv_begin = w[2]; u.kv_end = w[3];
    u.q_begin = w[4]; u.q_end = w[5]; u.partial = w[6]; u.diag = w[7];
    u.merge = w[8]; u.part_stride = w[9]; u.cached_end = w[10]; u.reserved2 = 0;
    return u;
}
__device__ __forceinline__ pa_merge_unit load_merge(const pa_merge_unit *merges, int32_t i) {
    const ConstantI32 w = (ConstantI32)(merges + i);
    pa_merge_unit m;
    m.request = w[0]; m.kv_head = w[1]; m.q_begin = w[2]; m.q_end = w[3];
    m.first_partial = w[4]; m.n_parts = w[5]; m.prefix_first = w[6]; m.prefix_parts = w[7];
    return m;
}

// Buffer descriptor over 4-byte elements [0, n) of p.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t index_rsrc(const int32_t *p, int32_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(p), (short)0, n * 4, kBufferWord3);
}

// Load of a gathered K or V row, marked non-temporal (the instruction's nt
// bit: the L2 keeps the line at the eviction end of its set).  A pool row is
// read once per launch, or by a prefix group's few requests at about the
// same moment; marking the stream keeps it from evicting the lines that are
// still in use (slot ids, shared-prefix rows, partials).  Measured on the
// batch-64 workload: 195.9-199.5 us per layer against 205.5-208.4 us with
// ordinary loads.
template <typename T>
__device__ __forceinline__ T load_streamed(const T *p) {
    typedef unsigned int V __attribute__((ext_vector_type(sizeof(T) / 4)));
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const V *>(p)));
}

// Lane layout of K/V rows: EPL elements of a row per lane (16 bytes of bf16,
// 8 or 16 bytes of E4M3 codes).
template <int D, int EPL, int NI_>
struct Geometry {
    static constexpr int LPR = D / EPL;        // lanes per row
    static constexpr int RPI = 64 / LPR;       // rows per wave instruction
    static constexpr int NI = NI_;             // instructions per tile
    static constexpr int TILE = NI * RPI;      // tokens per wave tile
    // Row (within an instruction) and chunk of a lane.  Rows of 16 or 32
    // lanes are contiguous.  A row of 8 lanes is two quads 8 lanes apart
    // (lanes 16a + 4b .. +3 and 16a + 4b + 8 .. +11 for row 2a + b), so
    // that every exchange of the score reduction stays a DPP move inside a
    // 16-lane row (quad permutations, then lane ^ 8).
    static __device__ __forceinline__ int row(int lane) {
        if constexpr (LPR == 8)
            return 2 * (lane >> 4) + ((lane >> 2) & 1);
        else
            return lane / LPR;
    }
    static __device__ __forceinline__ int chunk(int lane) {
        if constexpr (LPR == 8)
            return (lane & 3) + ((lane >> 1) & 4);
        else
            return lane % LPR;
    }
};

// Byte offset of a pool row: 32-bit form or 64-bit form.  The 32-bit form
// is only used when every row offset is below 2^31: the compiler widens the
// 24-bit product with a sign extension, so offsets of 2 GiB and more must
// take the 64-bit form.
template <bool WIDE>
struct RowAddr;
template <>
struct RowAddr<false> {
    static __device__ __forceinline__ const char *at(const char *base, int32_t slot,
                                                     uint32_t stride_bytes, uint32_t lane_off) {
        uint32_t off = __umul24((uint32_t)slot, stride_bytes) + lane_off;
        return base + off;
    }
};
template <>
struct RowAddr<true> {
    static __device__ __forceinline__ const char *at(const char *base, int32_t slot,
                                                     uint32_t stride_bytes, uint32_t lane_off) {
        uint64_t off = (uint64_t)(uint32_t)slot * stride_bytes + lane_off;
        return base + off;
    }
};

// Element type of the pools and the lane's part of a row.
//   * bf16: a lane's 8 elements of a row are one 16-byte load, already in
//     the dot-product and FMA operand formats.
//   * OCP FP8 E4M3: 16 codes a lane (one 16-byte load) for groups of up to
//     4 query heads, 8 (one 8-byte load) for groups of 8, whose 8 x 16 fp32
//     accumulators would not fit.  K codes are widened to bf16 pairs (exact:
//     every E4M3 value is a bf16 value, v_cvt_scalef32_pk_bf16_fp8) for the
//     dot products.  The weighted sum runs on fp16 dot products over two
//     tokens at once (PAIRED): element e of the lane's rows i, i+1 becomes
//     one fp16 pair (bytes interleaved with v_perm_b32, then
//     v_cvt_scalef32_pk_f16_fp8: E4M3 -> fp16 is exact), the two rows'
//     weights (<= 2^8) are rounded once to an fp16 pair, and one
//     v_dot2_f32_f16 adds both products with fp32 accumulation: half the
//     multiply-adds of the fp32 form.  The row sums add the same rounded
//     weights, so the result is the exact weighted mean of V under them.
// Scale 1 in the conversions: the pools' scales are applied to the softmax
// scale and to the output.
template <bool KV8, int EPL>
struct PoolRow;
template <>
struct PoolRow<false, 8> {
    using T = uint4;
    static constexpr uint32_t kElemBytes = 2;
    static constexpr int NQ = 4;               // bf16 pairs of the lane's elements
    static constexpr bool PAIRED = false;
    static __device__ __forceinline__ void k_words(const uint4 &x, uint32_t (&w)[4]) {
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    }
    static __device__ __forceinline__ void v_f32(const uint4 &x, float (&f)[8]) {
        // a bf16 value is the upper half of the fp32 with the same value
        f[0] = __uint_as_float(x.x << 16); f[1] = __uint_as_float(x.x & 0xffff0000u);
        f[2] = __uint_as_float(x.y << 16); f[3] = __uint_as_float(x.y & 0xffff0000u);
        f[4] = __uint_as_float(x.z << 16); f[5] = __uint_as_float(x.z & 0xffff0000u);
        f[6] = __uint_as_float(x.w << 16); f[7] = __uint_as_float(x.w & 0xffff0000u);
    }
};
// two E4M3 codes (the low or high half of w) as a bf16 pair
__device__ __forceinline__ uint32_t e4m3_pair_bf16(uint32_t w, bool hi) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <>
struct PoolRow<true, 8> {
    using T = uint2;
    static constexpr uint32_t kElemBytes = 1;
    static constexpr int NQ = 4;
    static constexpr bool PAIRED = true;
    static __device__ __forceinline__ void v_pairs(const uint2 &a, const uint2 &b, f16x2_t (&f)[8]) {
        const uint32_t wa[2] = {a.x, a.y}, wb[2] = {b.x, b.y};
#pragma unroll
        for (int w = 0; w < 2; w++) {
            const uint32_t lo = __builtin_amdgcn_perm(wb[w], wa[w], 0x05010400u);   // a0 b0 a1 b1
            const uint32_t hi = __builtin_amdgcn_perm(wb[w], wa[w], 0x07030602u);   // a2 b2 a3 b3
            f[4 * w] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
            f[4 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
            f[4 * w + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
            f[4 * w + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
        }
    }
    static __device__ __forceinline__ void k_words(const uint2 &x, uint32_t (&w)[4]) {
        w[0] = e4m3_pair_bf16(x.x, false); w[1] = e4m3_pair_bf16(x.x, true);
        w[2] = e4m3_pair_bf16(x.y, false); w[3] = e4m3_pair_bf16(x.y, true);
    }
};
template <>
struct PoolRow<true, 16> {
    using T = uint4;
    static constexpr uint32_t kElemBytes = 1;
    static constexpr int NQ = 8;
    static constexpr bool PAIRED = true;
    static __device__ __forceinline__ void k_words(const uint4 &x, uint32_t (&w)[8]) {
        w[0] = e4m3_pair_bf16(x.x, false); w[1] = e4m3_pair_bf16(x.x, true);
        w[2] = e4m3_pair_bf16(x.y, false); w[3] = e4m3_pair_bf16(x.y, true);
        w[4] = e4m3_pair_bf16(x.z, false); w[5] = e4m3_pair_bf16(x.z, true);
        w[6] = e4m3_pair_bf16(x.w, false); w[7] = e4m3_pair_bf16(x.w, true);
    }
    // f[e] = (element e of row a, element e of row b) as an fp16 pair:
    // bytes of the two rows interleaved (v_perm_b32), then widened two at a
    // time.
    static __device__ __forceinline__ void v_pairs(const uint4 &a, const uint4 &b, f16x2_t (&f)[16]) {
        const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int w = 0; w < 4; w++) {
            // byte k of the result = byte sel[k] of {wb (4..7), wa (0..3)}
            const uint32_t lo = __builtin_amdgcn_perm(wb[w], wa[w], 0x05010400u);   // a0 b0 a1 b1
            const uint32_t hi = __builtin_amdgcn_perm(wb[w], wa[w], 0x07030602u);   // a2 b2 a3 b3
            f[4 * w] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
            f[4 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
            f[4 * w + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
            f[4 * w + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
        }
    }
};
// Elements of a row per lane: 16 E4M3 codes for groups of up to 4 query
// heads, else 8.
template <bool KV8, int G>
constexpr int lane_elems() {
    return KV8 && G <= 4 ? 16 : 8;
}
// Instructions per wave tile: 4 (bf16), 4 (E4M3, 16 codes a lane: 32 tokens)
// or 8 (E4M3, 8 codes a lane: 32 tokens).  The E4M3 tiles move as many bytes
// per wave as the bf16 ones, so that as many are in flight.
template <bool KV8, int G>
constexpr int tile_instructions() {
    return KV8 && lane_elems<KV8, G>() == 8 ? 8 : 4;
}

// Log-sum-exp merge of one merge unit: partial slots [first, first+n) of
// query rows [q_begin, q_end) of one KV head.  Each slot holds rows_per_slot
// rows of D floats (row = (q - q_begin)*G + h) and their log2-sum-exp values.
// Threads tid, tid+nthreads, ... of the caller each produce output elements.
// COHERENT: read the partials with agent-scope coherent loads (partials
// written by other workgroups of the running kernel).
// The parts are read kMergeBatch at a time (all loads of a batch in flight
// together, one memory round trip per batch) and folded in with a running
// maximum; for up to kMergeBatch parts this is the plain two-pass formula
// o = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M), M = max_i lse_i.
constexpr int kMergeBatch = 8;

template <int D, int G, bool COHERENT>
__device__ __forceinline__ void merge_rows(const pa_merge_unit &mu, const float *__restrict__ part_o,
                                           const float *__restrict__ part_lse, int32_t rows_per_slot,
                                           float *__restrict__ out, float *__restrict__ lse,
                                           int32_t num_qo_heads, int tid, int nthreads) {
    const int32_t rows = (mu.q_end - mu.q_begin) * G;
    // the parts: slots first_partial .. + n_parts, then (cascade) the prefix
    // slots prefix_first .. + prefix_parts
    const int32_t n_own = mu.n_parts, n = mu.n_parts + mu.prefix_parts;
    const int32_t prefix_shift = mu.prefix_first - n_own;
    for (int32_t idx = tid; idx < rows * D; idx += nthreads) {
        const int32_t row = idx / D, d = idx % D;
        float M = -INFINITY, o = 0.f, wsum = 0.f;
        for (int32_t i0 = 0; i0 < n; i0 += kMergeBatch) {
            float l[kMergeBatch], v[kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; j++) {
                const int32_t i = min(i0 + j, n - 1);   // past the end: re-read the last part
                const int32_t slot = i < n_own ? mu.first_partial + i : prefix_shift + i;
                const int64_t slot_row = (int64_t)slot * rows_per_slot + row;
                l[j] = COHERENT ? load_coherent(part_lse + slot_row) : part_lse[slot_row];
                v[j] = COHERENT ? load_coherent(part_o + slot_row * D + d) : part_o[slot_row * D + d];
            }
            float m = M;
#pragma unroll
            for (int j = 0; j < kMergeBatch; j++) {
                if (i0 + j >= n)
                    l[j] = -INFINITY;
                m = fmaxf(m, l[j]);
            }
            if (m == -INFINITY)
                continue;  // only empty parts so far
            const float a = fast_exp2(M - m);  // 0 while M is -inf
            o *= a;
            wsum *= a;
#pragma unroll
            for (int j = 0; j < kMergeBatch; j++) {
                const float w = fast_exp2(l[j] - m);
                o = fmaf(w, v[j], o);
                wsum += w;
            }
            M = m;
        }
        const int32_t qtok = mu.q_begin + row / G, h = mu.kv_head * G + row % G;
        const int64_t orow = (int64_t)qtok * num_qo_heads + h;
        if (M == -INFINITY) {
            out[orow * D + d] = 0.f;
            if (lse && d == 0)
                lse[orow] = -INFINITY;
        } else {
            out[orow * D + d] = o / wsum;
            if (lse && d == 0)
                lse[orow] = (M + fast_log2(wsum)) * kLn2;
        }
    }
}

// Waves per SIMD the decode kernel is compiled for: three (at most 168
// VGPRs, room for the rotating K/V registers without spills) for bf16 pools
// and groups of up to four query heads; two for groups of eight and for E4M3
// pools, whose tiles hold twice the tokens (measured on the batch-64
// workload: 114-115 us per layer against 125-129 us with three waves and
// half the tokens per tile, and 118-119 us with 6 instructions a tile).
template <int G, bool KV8>
constexpr int decode_waves_per_simd() {
    return G <= 4 && !KV8 ? 3 : 2;
}

template <int D, int G, bool WIDE, bool KV8>
__global__ __launch_bounds__(kDecodeThreads)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<G, KV8>(), 8))) void decode_kernel(
    const int32_t *__restrict__ wg_offsets, const pa_work_unit *__restrict__ units,
    const pa_merge_unit *__restrict__ merges, int32_t *__restrict__ arrivals,
    const uint16_t *__restrict__ q, const char *__restrict__ k_pool,
    const char *__restrict__ v_pool, uint32_t stride_bytes,
    const int32_t *__restrict__ kv_indices, float scale_log2, float out_scale, float *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ part_o, float *__restrict__ part_lse,
    int32_t num_qo_heads, uint64_t *__restrict__ wg_clock) {
    constexpr int EPL = lane_elems<KV8, G>();
    using Geo = Geometry<D, EPL, tile_instructions<KV8, G>()>;
    using PR = PoolRow<KV8, EPL>;
    using Row = typename PR::T;
    constexpr int LPR = Geo::LPR, RPI = Geo::RPI, NI = Geo::NI, TILE = Geo::TILE, NQ = PR::NQ;
    constexpr int WAVES = kDecodeWaves;

    __shared__ float lds_o[WAVES][G][D];
    __shared__ float lds_m[WAVES][G];
    __shared__ float lds_l[WAVES][G];
    __shared__ int32_t lds_arrived;

    // start of the workgroup's run on the 100 MHz real-time counter
    const uint64_t t_begin = wg_clock ? __builtin_amdgcn_s_memrealtime() : 0;
    const int32_t unit_begin = constant_view(wg_offsets)[blockIdx.x];
    const int32_t unit_end = constant_view(wg_offsets)[blockIdx.x + 1];

    // Issue priority by remaining work.  Workgroups that share a compute unit
    // start with equal budgets, but the instruction arbiter prefers older
    // waves, so without this the first workgroup placed on a unit runs ahead
    // and the last one is left alone at the end.  A wave's priority is the
    // number of quarters of its workgroup's list entries still ahead of it
    // (3 .. 0): a wave that has run ahead yields issue slots to those behind.
    int32_t wg_total = 0;
    for (int32_t ui = unit_begin; ui < unit_end; ui++) {
        const pa_work_unit u = load_unit(units, ui);
        if (u.request >= 0)
            wg_total += u.kv_end - u.kv_begin;
    }
    const int32_t quarter1 = wg_total / 4, quarter2 = wg_total / 2, quarter3 = wg_total - wg_total / 4;
    int32_t done_before = 0;   // entries of the units finished
    int priority = -1;
    auto set_priority = [&](int32_t remaining) {
        const int level = (remaining > quarter1) + (remaining > quarter2) + (remaining > quarter3);
        if (level != priority) {
            priority = level;
            switch (level) {
            case 0: __builtin_amdgcn_s_setprio(0); break;
            case 1: __builtin_amdgcn_s_setprio(1); break;
            case 2: __builtin_amdgcn_s_setprio(2); break;
            default: __builtin_amdgcn_s_setprio(3); break;
            }
        }
    };

    for (int32_t ui = unit_begin; ui < unit_end; ui++) {
    const pa_work_unit unit = load_unit(units, ui);
    if (unit.request < 0)
        continue;  // padding unit (uniform over the workgroup)

    const int tid = threadIdx.x;
    // wave index as a scalar: the tile loop below is uniform per wave
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = Geo::row(lane);     // row within an instruction
    const int c = Geo::chunk(lane);   // chunk of the row (elements EPL*c ..)
    const int hsel = lane % G;     // head whose score this lane holds after reduction

    // query rows of the group: qv[j] = q[b, kvh*G + (j ^ hsel), EPL*c .. EPL*c + EPL-1]
    uint32_t qv[G][NQ];
    {
        const uint16_t *qrow = q + ((int64_t)unit.request * num_qo_heads + (int64_t)unit.kv_head * G) * D + c * EPL;
#pragma unroll
        for (int j = 0; j < G; j++)
#pragma unroll
            for (int u = 0; u < NQ / 4; u++) {
                const uint4 t = *reinterpret_cast<const uint4 *>(qrow + (int64_t)(j ^ hsel) * D + 8 * u);
                qv[j][4 * u] = t.x; qv[j][4 * u + 1] = t.y; qv[j][4 * u + 2] = t.z; qv[j][4 * u + 3] = t.w;
            }
    }

    const uint32_t lane_off = (uint32_t)(unit.kv_head * D + c * EPL) * PR::kElemBytes;
    const int32_t kv_begin = unit.kv_begin, kv_end = unit.kv_end;
    const int32_t n_tiles = (kv_end - kv_begin + TILE - 1) / TILE;

    float m_run = kNoMax, l_run = 0.f;
    float acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int e = 0; e < EPL; e++)
            acc[h][e] = 0.f;

    // slot ids of a tile: entries kv_begin + tile*TILE + r + i*RPI of the
    // list.  Entries at or past kv_end (the tail of the last tile and the
    // tiles the look-ahead requests past the end) are clamped to the unit's
    // last entry, so every row read is one the unit references.  In bytes:
    // min(e + 4*i*RPI, last) = min(e, last - 4*i*RPI) + 4*i*RPI, whose
    // constant term goes into the load's immediate offset.
    const __amdgpu_buffer_rsrc_t slot_rsrc = index_rsrc(kv_indices + kv_begin, kv_end - kv_begin);
    const int32_t last4 = (kv_end - kv_begin - 1) * 4;
    auto load_slots = [&](int32_t(&slot)[NI], int tile) {
        const int32_t e4 = (tile * TILE + r) * 4;
#pragma unroll
        for (int i = 0; i < NI; i++)
            slot[i] = __builtin_amdgcn_raw_buffer_load_b32(
                slot_rsrc, min(e4, last4 - i * RPI * 4) + i * RPI * 4, 0, 0);
    };
    // rows of the streamed range: non-temporal; of the cached range (a shared
    // prefix other requests read too): ordinary loads
    auto load_rows = [&](auto stream, Row(&x)[NI], const char *pool, const int32_t(&slot)[NI]) {
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const Row *p = reinterpret_cast<const Row *>(RowAddr<WIDE>::at(pool, slot[i], stride_bytes, lane_off));
            if constexpr (decltype(stream)::value)
                x[i] = load_streamed(p);
            else
                x[i] = *p;
        }
    };
    // scores of this lane's head (lane % G) for the tile's tokens, log2 domain
    auto qk = [&](const Row(&k)[NI], float(&s)[NI], int tile) {
        // entries of the tile left in the unit (uniform)
        const int32_t left = kv_end - kv_begin - tile * TILE;
#pragma unroll
        for (int i = 0; i < NI; i++) {
            uint32_t kw[NQ];
            PR::k_words(k[i], kw);
            const float sc = row_scores<G, LPR, NQ>(qv, kw) * scale_log2;
            s[i] = (r + i * RPI < left) ? sc : -INFINITY;
        }
    };
    // online softmax: scores -> weights, running max / sum, accumulator rescale
    auto softmax = [&](const float(&s)[NI], float(&p)[NI]) {
        float tmax = s[0];
#pragma unroll
        for (int i = 1; i < NI; i++)
            tmax = fmaxf(tmax, s[i]);
        const bool move = tmax > m_run + kRescaleSlack;
        if (__any(move)) {
            const float m_new = move ? tmax : m_run;
            const float alpha = fast_exp2(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float ah = group_bcast<G>(alpha, h, lane);
#pragma unroll
                for (int e = 0; e < EPL; e++)
                    acc[h][e] *= ah;
            }
        }
#pragma unroll
        for (int i = 0; i < NI; i++) {
            p[i] = fast_exp2(s[i] - m_run);
            if constexpr (!PR::PAIRED)
                l_run += p[i];   // (paired: the rounded weights, in pv)
        }
    };
    auto pv = [&](const Row(&v)[NI], const float(&p)[NI]) {
        if constexpr (PR::PAIRED) {
            const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int i = 0; i < NI; i += 2) {
                f16x2_t vp[EPL];
                PR::v_pairs(v[i], v[i + 1], vp);
                // weights of rows i, i+1 (<= 2^8) rounded once to fp16
                const f16x2_t pp = __builtin_convertvector(f32x2_t{p[i], p[i + 1]}, f16x2_t);
                l_run = __builtin_amdgcn_fdot2(pp, ones, l_run, false);
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const f16x2_t ph =
                        __builtin_bit_cast(f16x2_t, group_bcast<G>(__builtin_bit_cast(float, pp), h, lane));
#pragma unroll
                    for (int e = 0; e < EPL; e++)
                        acc[h][e] = __builtin_amdgcn_fdot2(ph, vp[e], acc[h][e], false);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NI; i++) {
                float vf[8];
                PR::v_f32(v[i], vf);
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float ph = group_bcast<G>(p[i], h, lane);
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
                }
            }
        }
    };

    // Tiles wave, wave+4, wave+8, ... (t0, t1, ...) alternate between two
    // register sets A and B: while the tile in one set is computed, the next
    // tile's K and V rows are in flight into the other, and a set is refilled
    // (two tiles ahead) as soon as its tile is done.  Slot ids are fetched two
    // tiles ahead of their rows.  Every load is unconditional (slot ids of
    // tiles past the end are clamped to the last entry and re-read one row),
    // so each set is refilled in place.
    // The wave's tiles t_first, t_first + WAVES, ... below t_end, in the same
    // order in either range.  The look-ahead runs two tiles past t_end: in
    // the cached range those are the streamed range's first tiles (which
    // then find them in the L2), past the unit's end the slot ids clamp to
    // its last entry.
    auto run_tiles = [&](auto stream, int tile, int t_end) {
        if (tile >= t_end)
            return;
        auto ahead = [](int t) { return t; };
        int32_t sa[NI], sb[NI];
        Row ka[NI], va[NI], kb[NI], vb[NI];
        load_slots(sa, tile);
        load_slots(sb, ahead(tile + WAVES));
        load_rows(stream, ka, k_pool, sa);
        load_rows(stream, va, v_pool, sa);
        load_rows(stream, kb, k_pool, sb);
        load_rows(stream, vb, v_pool, sb);
        load_slots(sa, ahead(tile + 2 * WAVES));
        load_slots(sb, ahead(tile + 3 * WAVES));
        auto compute = [&](const Row(&k)[NI], const Row(&v)[NI]) {
            float sc[NI], pw[NI];
            qk(k, sc, tile);
            softmax(sc, pw);
            pv(v, pw);
        };
        while (true) {
            set_priority(wg_total - done_before - tile * TILE);
            compute(ka, va);
            // refills stay behind the last use of the registers they overwrite
            __builtin_amdgcn_sched_barrier(0);
            load_rows(stream, ka, k_pool, sa);
            load_rows(stream, va, v_pool, sa);
            load_slots(sa, ahead(tile + 4 * WAVES));
            tile += WAVES;
            if (tile >= t_end)
                break;
            compute(kb, vb);
            __builtin_amdgcn_sched_barrier(0);
            load_rows(stream, kb, k_pool, sb);
            load_rows(stream, vb, v_pool, sb);
            load_slots(sb, ahead(tile + 4 * WAVES));
            tile += WAVES;
            if (tile >= t_end)
                break;
        }
    };
    // tiles that hold entries before cached_end: cached loads; the rest streamed
    const int32_t n_cached =
        unit.cached_end > kv_begin ? min(n_tiles, (unit.cached_end - kv_begin + TILE - 1) / TILE) : 0;
    if (n_cached > 0) {
        run_tiles(std::false_type{}, wave, n_cached);
        // the wave's first tile of the streamed range
        const int first = wave + (n_cached - wave + WAVES - 1) / WAVES * WAVES;
        run_tiles(std::true_type{}, first, n_tiles);
    } else {
        run_tiles(std::true_type{}, wave, n_tiles);
    }

    // ---- combine the rows of this wave (same head: lanes with equal lane % G)
    const float mm = max_rows<LPR>(m_run);
    const float f = fast_exp2(m_run - mm);
    const float lsum = sum_rows<LPR>(l_run * f);
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float fh = group_bcast<G>(f, h, lane);
#pragma unroll
        for (int e = 0; e < EPL; e++)
            acc[h][e] = sum_rows<LPR>(acc[h][e] * fh);
    }
    // ---- combine the waves through LDS
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; h++) {
            float4 *dst = reinterpret_cast<float4 *>(&lds_o[wave][h][c * EPL]);
#pragma unroll
            for (int u = 0; u < EPL / 4; u++)
                dst[u] = make_float4(acc[h][4 * u], acc[h][4 * u + 1], acc[h][4 * u + 2], acc[h][4 * u + 3]);
        }
        if (c < G) {
            lds_m[wave][c] = mm;
            lds_l[wave][c] = lsum;
        }
    }
    __syncthreads();

    const int32_t qrow0 = unit.request * num_qo_heads + unit.kv_head * G;
    for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
        const int h = idx / D, d = idx % D;
        float M = lds_m[0][h];
#pragma unroll
        for (int w = 1; w < WAVES; w++)
            M = fmaxf(M, lds_m[w][h]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; w++) {
            const float wgt = fast_exp2(lds_m[w][h] - M);
            o = fmaf(wgt, lds_o[w][h][d], o);
            l = fmaf(wgt, lds_l[w][h], l);
        }
        const bool empty = !(l > 0.f);
        const float res = empty ? 0.f : o / l * out_scale;
        const float lse2 = empty ? -INFINITY : M + fast_log2(l);
        if (unit.partial < 0) {
            out[(int64_t)(qrow0 + h) * D + d] = res;
            if (lse && d == 0)
                lse[qrow0 + h] = lse2 * kLn2;
        } else {
            store_coherent(part_o + ((int64_t)unit.partial * G + h) * D + d, res);
            if (d == 0)
                store_coherent(part_lse + (int64_t)unit.partial * G + h, lse2);
        }
    }
    if (unit.partial >= 0) {
        // count this part once its stores have completed; the last to arrive merges
        wait_vector_memory();
        __syncthreads();
        if (tid == 0)
            lds_arrived = __hip_atomic_fetch_add(arrivals + unit.merge, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const pa_merge_unit mu = load_merge(merges, unit.merge);
        if (lds_arrived == mu.n_parts - 1) {
            merge_rows<D, G, true>(mu, part_o, part_lse, G, out, lse, num_qo_heads, tid, kDecodeThreads);
            if (tid == 0)
                __hip_atomic_store(arrivals + unit.merge, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    done_before += kv_end - kv_begin;
    if (ui + 1 < unit_end)
        __syncthreads();  // the next unit rewrites the LDS just read
    }
    // add this workgroup's run time and a count of one to its record (wave 0
    // leaves after the last combine, which waits for every wave)
    if (wg_clock && wg_total > 0 && threadIdx.x == 0) {
        const uint64_t ticks = __builtin_amdgcn_s_memrealtime() - t_begin;
        __hip_atomic_fetch_add(wg_clock + (size_t)blockIdx.x * kClockStride,
                               (1ull << kClockCountShift) + ticks, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

bool row_offsets_fit_32(int64_t num_slots, uint32_t stride_bytes) {
    // largest offset: (num_slots - 1) * stride + (row start within the slot
    // + 16-byte chunk), all below num_slots * stride
    const uint64_t span = (uint64_t)num_slots * stride_bytes;
    return span <= 0x80000000ull && num_slots <= (1 << 24) && stride_bytes < (1u << 24);
}

namespace {

template <int D, int G, bool KV8>
int launch_decode_dgk(const DecodeLaunch &l, hipStream_t stream) {
    const uint32_t stride_bytes = (uint32_t)(l.slot_stride * (KV8 ? 1 : 2));
    // the 32-bit row address needs every byte offset below 2^31 (it is
    // sign-extended into the address) and 24-bit multiply operands
    const bool wide = !row_offsets_fit_32(l.num_slots, stride_bytes);
    // 8-bit pools: K = k_scale * code enters the scores, V = v_scale * code the output
    const float scale_log2 = (KV8 ? l.sm_scale * l.k_scale : l.sm_scale) * kLog2e;
    const float out_scale = KV8 ? l.v_scale : 1.0f;
    dim3 grid(l.n_workgroups), block(kDecodeThreads);
    if (wide)
        hipLaunchKernelGGL((decode_kernel<D, G, true, KV8>), grid, block, 0, stream, l.wg_offsets, l.units,
                           l.merges, l.arrivals,
                           (const uint16_t *)l.q, (const char *)l.k_pool, (const char *)l.v_pool,
                           stride_bytes, l.kv_indices, scale_log2, out_scale, l.out, l.lse, l.partial_o,
                           l.partial_lse, l.num_qo_heads, l.wg_clock);
    else
        hipLaunchKernelGGL((decode_kernel<D, G, false, KV8>), grid, block, 0, stream, l.wg_offsets, l.units,
                           l.merges, l.arrivals,
                           (const uint16_t *)l.q, (const char *)l.k_pool, (const char *)l.v_pool,
                           stride_bytes, l.kv_indices, scale_log2, out_scale, l.out, l.lse, l.partial_o,
                           l.partial_lse, l.num_qo_heads, l.wg_clock);
    return (int)hipGetLastError();
}

template <int D, int G>
int launch_decode_dg(const DecodeLaunch &l, hipStream_t stream) {
    return l.kv_fp8 ? launch_decode_dgk<D, G, true>(l, stream) : launch_decode_dgk<D, G, false>(l, stream);
}

template <int D, int G>
int occupancy_dg(bool kv_fp8) {
    int n = 0;
    const hipError_t e =
        kv_fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, G, false, true>, kDecodeThreads, 0)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, G, false, false>, kDecodeThreads, 0);
    return e == hipSuccess ? n : 0;
}

}  // namespace

int decode_workgroups_per_cu(int32_t head_dim, int32_t group, bool kv_fp8) {
    if (head_dim == 128) {
        switch (group) {
        case 1: return occupancy_dg<128, 1>(kv_fp8);
        case 2: return occupancy_dg<128, 2>(kv_fp8);
        case 4: return occupancy_dg<128, 4>(kv_fp8);
        case 8: return occupancy_dg<128, 8>(kv_fp8);
        }
    } else if (head_dim == 256) {
        switch (group) {
        case 1: return occupancy_dg<256, 1>(kv_fp8);
        case 2: return occupancy_dg<256, 2>(kv_fp8);
        case 4: return occupancy_dg<256, 4>(kv_fp8);
        case 8: return occupancy_dg<256, 8>(kv_fp8);
        }
    }
    return 0;
}

int launch_decode(const DecodeLaunch &l, void *stream) {
    if (l.n_workgroups == 0)
        return 0;
    hipStream_t s = (hipStream_t)stream;
    const int G = l.num_qo_heads / l.num_kv_heads;
    if (l.head_dim == 128) {
        switch (G) {
        case 1: return launch_decode_dg<128, 1>(l, s);
        case 2: return launch_decode_dg<128, 2>(l, s);
        case 4: return launch_decode_dg<128, 4>(l, s);
        case 8: return launch_decode_dg<128, 8>(l, s);
        }
    } else if (l.head_dim == 256) {
        switch (G) {
        case 1: return launch_decode_dg<256, 1>(l, s);
        case 2: return launch_decode_dg<256, 2>(l, s);
        case 4: return launch_decode_dg<256, 4>(l, s);
        case 8: return launch_decode_dg<256, 8>(l, s);
        }
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace pa
