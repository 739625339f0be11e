// append.hip -- gfx950 kernel of libpa's append step: the new tokens' K and V
// rows are written to their slots of the token-granular pool (Agent-Infer
// page, "Agent-Infer: 纯 Rust 编写的高性能 LLM 推理引擎", section "分页 KV 缓存":
// each token owns one slot), with rotary position embedding applied to K (and,
// if given, to the query rows in place) on the way (RoPE is one of the GPU
// operators listed on the Pegainfer page, "Pegainfer: 纯Rust+CUDA构建的LLM推理引擎",
// section "核心组件概览"; the pages do not write it out).  Rotation used
// (rotate-half pairs): pair i < D/2 couples elements i and i + D/2 and turns
// them by the angle pos * theta^(-2i/D):
//     y[i]       = x[i] cos(a) - x[i + D/2] sin(a)
//     y[i + D/2] = x[i + D/2] cos(a) + x[i] sin(a)
// The angle and the rotation are computed in double precision (positions of
// tens of thousands make a float angle lose ~1e-3 rad) and rounded once to
// bf16 (nearest-even, through a round-to-odd float so there is no double
// rounding).  V rows are copied bit for bit.  A token whose slot id is out of
// [0, num_slots) writes nothing.
//
// 8-bit pools (OCP FP8 E4M3 codes with one scale per pool; quantised KV is on
// the Agent-Infer page's roadmap, section "模型支持与发展路线图"): the rotated K
// value y (double) is stored as the code nearest to y / k_scale, a V value x
// as the code nearest to x / v_scale, the quotient formed in double and
// rounded once: to nearest, ties to even, among the finite codes, so that
// magnitudes at or beyond the largest finite value 448 store +-448; NaN
// stores 0x7F.
//
// One thread per rotated pair (K, then Q) and one per 16-byte chunk of a V
// row (8 values); consecutive threads take consecutive pairs of a row, so
// every load and store of a wave is one contiguous run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kAppendThreads = 256;

__device__ __forceinline__ double widen_bf16(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

// Round a double to bf16, nearest-even: truncate to float, mark inexact results
// in the lowest bit (round to odd: 16 guard bits remain below bf16's last bit,
// so the second rounding cannot land on a false tie), then round the float.
__device__ __forceinline__ uint16_t bf16_from_double(double y) {
    const float f = __double2float_rz(y);
    uint32_t u = __float_as_uint(f);
    if ((double)f != y)
        u |= 1u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// E4M3 code of a double: nearest among the finite codes, ties to even, NaN
// to 0x7F, a zero result signed as the input.  At or beyond 448 (the largest
// finite value, infinities included) the nearest finite code is 448 itself.
// From 2^-6 up, a = q * 2^(E-3) with E = floor(log2 a) in [-6, 8] and the
// code is (E + 7) << 3 | (rint(q) - 8); rint(q) = 16 carries into the next
// exponent by the addition.  Below 2^-6 the codes step by 2^-9 (code 8 is
// 2^-6 again).  rint rounds half to even; the scalings are exact.
__device__ __forceinline__ uint32_t e4m3_from_double(double y) {
    if (__builtin_isnan(y))
        return 0x7Fu;
    const uint32_t sign = __builtin_signbit(y) ? 0x80u : 0u;
    const double a = fabs(y);
    uint32_t mag;
    if (a >= 448.0) {
        mag = 0x7Eu;
    } else if (a < 0x1p-6) {
        mag = (uint32_t)rint(a * 0x1p9);
    } else {
        int e;
        (void)frexp(a, &e);           // a = f * 2^e, f in [0.5, 1): E = e - 1
        const int E = e - 1;
        mag = (uint32_t)((E + 7) << 3) + ((uint32_t)rint(ldexp(a, 3 - E)) - 8u);
    }
    return sign | mag;
}

struct AppendArgs {
    const uint16_t *k_new, *v_new;
    uint16_t *q;                      // null: no query rotation
    const int32_t *positions, *out_loc;
    int32_t tokens, hq, hkv, d;
    double log2_theta;                // log2(rope_theta), when rotating
    bool rotate;                      // rope_theta > 0
    void *k_pool, *v_pool;            // bf16, or E4M3 codes (1 byte)
    double k_scale, v_scale;          // E4M3 pools: the pool scales
    int64_t num_slots, slot_stride;   // elements
    int64_t k_pairs, v_chunks, q_pairs;
};

// Rotation of pair i of token t: inverse frequency theta^(-2i/D) and angle
// pos * inv_freq, all in double.
__device__ __forceinline__ void rotate_pair(const AppendArgs &a, int64_t t, int i, uint16_t x1b, uint16_t x2b,
                                            double *y1, double *y2) {
    const double inv_freq = exp2(a.log2_theta * (-2.0 * (double)i / (double)a.d));
    double s, c;
    sincos((double)a.positions[t] * inv_freq, &s, &c);
    const double x1 = widen_bf16(x1b), x2 = widen_bf16(x2b);
    *y1 = x1 * c - x2 * s;
    *y2 = x2 * c + x1 * s;
}

template <bool KV8>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
    int64_t g = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    const int half = a.d / 2;
    if (g < a.k_pairs) {
        // K: pair i of row (t, h)
        const int64_t row = g / half;
        const int i = (int)(g % half);
        const int64_t t = row / a.hkv;
        const int h = (int)(row % a.hkv);
        const int32_t slot = a.out_loc[t];
        if (slot < 0 || slot >= a.num_slots)
            return;
        const uint16_t *x = a.k_new + row * a.d;
        const int64_t off = (int64_t)slot * a.slot_stride + (int64_t)h * a.d;
        if constexpr (KV8) {
            double y1 = widen_bf16(x[i]), y2 = widen_bf16(x[i + half]);
            if (a.rotate)
                rotate_pair(a, t, i, x[i], x[i + half], &y1, &y2);
            uint8_t *dst = static_cast<uint8_t *>(a.k_pool) + off;
            dst[i] = (uint8_t)e4m3_from_double(y1 / a.k_scale);
            dst[i + half] = (uint8_t)e4m3_from_double(y2 / a.k_scale);
        } else {
            uint16_t *dst = static_cast<uint16_t *>(a.k_pool) + off;
            if (a.rotate) {
                double y1, y2;
                rotate_pair(a, t, i, x[i], x[i + half], &y1, &y2);
                dst[i] = bf16_from_double(y1);
                dst[i + half] = bf16_from_double(y2);
            } else {
                dst[i] = x[i];
                dst[i + half] = x[i + half];
            }
        }
        return;
    }
    g -= a.k_pairs;
    if (g < a.v_chunks) {
        // V: 16-byte chunk c of row (t, h), copied
        const int per_row = a.d / 8;
        const int64_t row = g / per_row;
        const int c = (int)(g % per_row);
        const int64_t t = row / a.hkv;
        const int h = (int)(row % a.hkv);
        const int32_t slot = a.out_loc[t];
        if (slot < 0 || slot >= a.num_slots)
            return;
        const uint4 v = *reinterpret_cast<const uint4 *>(a.v_new + row * a.d + c * 8);
        const int64_t off = (int64_t)slot * a.slot_stride + (int64_t)h * a.d + c * 8;
        if constexpr (KV8) {
            // eight bf16 values -> eight codes, one 8-byte store
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t packed[2] = {0u, 0u};
            for (int e = 0; e < 8; e++) {
                const uint16_t b = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                packed[e >> 2] |= e4m3_from_double(widen_bf16(b) / a.v_scale) << (8 * (e & 3));
            }
            *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(a.v_pool) + off) = make_uint2(packed[0], packed[1]);
        } else {
            *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.v_pool) + off) = v;
        }
        return;
    }
    g -= a.v_chunks;
    if (g < a.q_pairs) {
        // Q: pair i of row (t, h), rotated in place
        const int64_t row = g / half;
        const int i = (int)(g % half);
        const int64_t t = row / a.hq;
        uint16_t *x = a.q + row * a.d;
        double y1, y2;
        rotate_pair(a, t, i, x[i], x[i + half], &y1, &y2);
        x[i] = bf16_from_double(y1);
        x[i + half] = bf16_from_double(y2);
    }
}

}  // namespace

int launch_append(const AppendLaunch &l, void *stream) {
    if (l.num_tokens == 0)
        return 0;
    AppendArgs a;
    a.k_new = static_cast<const uint16_t *>(l.k_new);
    a.v_new = static_cast<const uint16_t *>(l.v_new);
    a.q = static_cast<uint16_t *>(l.q);
    a.positions = l.positions;
    a.out_loc = l.out_loc;
    a.tokens = l.num_tokens;
    a.hq = l.num_qo_heads;
    a.hkv = l.num_kv_heads;
    a.d = l.head_dim;
    a.rotate = l.rope_theta > 0.f;
    a.log2_theta = a.rotate ? log2((double)l.rope_theta) : 0.0;
    a.k_pool = l.k_pool;
    a.v_pool = l.v_pool;
    a.k_scale = l.kv_fp8 ? (double)l.k_scale : 1.0;
    a.v_scale = l.kv_fp8 ? (double)l.v_scale : 1.0;
    a.num_slots = l.num_slots;
    a.slot_stride = l.slot_stride;
    const int64_t rows_kv = (int64_t)l.num_tokens * l.num_kv_heads;
    a.k_pairs = rows_kv * (l.head_dim / 2);
    a.v_chunks = rows_kv * (l.head_dim / 8);
    a.q_pairs = (a.q && a.rotate) ? (int64_t)l.num_tokens * l.num_qo_heads * (l.head_dim / 2) : 0;
    const int64_t total = a.k_pairs + a.v_chunks + a.q_pairs;
    const int64_t blocks = (total + kAppendThreads - 1) / kAppendThreads;
    if (blocks > 0x7fffffffLL)
        return (int)hipErrorInvalidValue;
    if (l.kv_fp8)
        hipLaunchKernelGGL(append_kernel<true>, dim3((uint32_t)blocks), dim3(kAppendThreads), 0,
                           (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(append_kernel<false>, dim3((uint32_t)blocks), dim3(kAppendThreads), 0,
                           (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

}  // namespace pa
