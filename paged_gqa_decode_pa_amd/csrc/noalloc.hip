// noalloc.hip -- decode attention that allocates nothing: the device-side
// partition behind pa_decode_run_noalloc and the workspace it uses, a
// file-scope device array.
//
// The split-KV decode of pa_decode_run needs a work table, partial results
// and arrival counters, which a plan object allocates once.  Callers that may
// not allocate at all (code under graph capture, serving loops or harnesses
// that forbid it) get the same decode kernel over a table that a one-
// workgroup planner kernel writes into `scratch` on every call, from the
// slot-list offsets already on the device:
//   * the (KV head, request) segments are laid end to end, KV head major
//     (segment s = kvh * B + b covers positions kvh*T + kv_indptr[b] ..
//     kvh*T + kv_indptr[b+1], T = kv_indptr[B]), and the E = Hkv*T positions
//     are cut into W equal bins, W = the decode workgroups the GPU holds at
//     once: bin w covers [floor(w E / W), floor((w+1) E / W));
//   * bin w becomes workgroup w, whose work units are the pieces of the
//     segments it overlaps; a segment cut over bins w0..w1 has parts in
//     partial slots P(s) .. P(s) + w1 - w0, numbered in segment order (a bin
//     holds at most two cut pieces, its first and its last, so at most 2W
//     slots are used), and one merge unit (index s);
//   * requests with empty lists are written (out = 0, lse = -inf) by the
//     planner itself.
// The decode kernel then merges cut segments exactly as under a plan (the
// part that arrives last), and leaves every arrival counter at zero; the
// planner also clears the counters it will use before each call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Byte offsets of the parts of the workspace.
constexpr size_t kNaOffsetsAt = 0;
constexpr size_t kNaUnitsAt = kNaOffsetsAt + round256((size_t)(kNoAllocMaxWorkgroups + 1) * 4);
constexpr size_t kNaMergesAt =
    kNaUnitsAt + round256((size_t)(kNoAllocMaxWorkgroups + kNoAllocMaxSegments) * sizeof(pa_work_unit));
constexpr size_t kNaArrivalsAt = kNaMergesAt + round256((size_t)kNoAllocMaxSegments * sizeof(pa_merge_unit));
constexpr size_t kNaPartLseAt = kNaArrivalsAt + round256((size_t)kNoAllocMaxSegments * 4);
constexpr size_t kNaPartOAt = kNaPartLseAt + round256((size_t)kNoAllocPartialLseFloats * 4);
constexpr size_t kNaBytes = kNaPartOAt + (size_t)kNoAllocPartialFloats * 4;
static_assert(kNaBytes == kNoAllocScratchBytes, "scratch layout and its published size differ");

constexpr int kPlanThreads = 1024;

}  // namespace
}  // namespace pa

// The workspace of pa_decode_run_noalloc, one copy per GPU the library runs
// on, kept until the process ends.  Host code never passes this name to a
// kernel (on the host it is only a handle of the symbol): it takes the
// device address from hipGetSymbolAddress once per device.
static __device__ __align__(256) unsigned char scratch[pa::kNoAllocScratchBytes];

namespace pa {
namespace {

// Invalid offsets (kv_indptr[0] != 0, decreasing, or a total above
// PA_MAX_KV_TOTAL) give no work units and NaN outputs: the planner must not
// loop on them, and the result must not look valid.
__global__ __launch_bounds__(kPlanThreads) void noalloc_plan_kernel(
    const int32_t *__restrict__ kv_indptr, int32_t B, int32_t Hkv, int32_t Hq, int32_t D, int32_t W,
    int32_t *__restrict__ wg_offsets, pa_work_unit *__restrict__ units, pa_merge_unit *__restrict__ merges,
    int32_t *__restrict__ arrivals, float *__restrict__ out, float *__restrict__ lse) {
    __shared__ int32_t ip[kNoAllocMaxBatch + 1];
    __shared__ int32_t scan[kPlanThreads];
    __shared__ int32_t chunk_first[kPlanThreads];
    __shared__ int32_t bad;
    const int tid = threadIdx.x;
    const int32_t S = B * Hkv;

    if (tid == 0)
        bad = 0;
    __syncthreads();
    for (int i = tid; i <= B; i += kPlanThreads) {
        const int32_t v = kv_indptr[i];
        ip[i] = v;
        if ((i == 0 && v != 0) || (i > 0 && v < kv_indptr[i - 1]) || v > (int32_t)PA_MAX_KV_TOTAL)
            bad = 1;   // every writer stores the same value
    }
    for (int s = tid; s < S; s += kPlanThreads)
        arrivals[s] = 0;
    __syncthreads();
    if (bad) {
        for (int64_t i = tid; i < (int64_t)B * Hq * D; i += kPlanThreads)
            out[i] = __builtin_nanf("");
        if (lse)
            for (int64_t i = tid; i < (int64_t)B * Hq; i += kPlanThreads)
                lse[i] = __builtin_nanf("");
        for (int w = tid; w <= W; w += kPlanThreads)
            wg_offsets[w] = 0;
        return;
    }

    const int64_t T = ip[B];
    const uint64_t E = (uint64_t)Hkv * (uint64_t)T;
    // bins: W, or one per position when there are fewer positions (so that
    // no bin is empty and a segment cut over bins w0..w1 has a piece in each)
    const int32_t Wb = E < (uint64_t)W ? (int32_t)E : W;
    // requests with empty lists
    for (int32_t b = 0; b < B; b++) {
        if (ip[b + 1] != ip[b])
            continue;
        for (int i = tid; i < Hq * D; i += kPlanThreads)
            out[(int64_t)b * Hq * D + i] = 0.f;
        if (lse)
            for (int i = tid; i < Hq; i += kPlanThreads)
                lse[(int64_t)b * Hq + i] = -INFINITY;
    }

    // bin w covers positions [lo(w), lo(w+1)); bin_of(x) is the bin holding x
    auto lo_of = [&](int64_t w) -> uint64_t { return (uint64_t)w * E / (uint64_t)Wb; };
    auto bin_of = [&](uint64_t x) -> int32_t { return (int32_t)(((x + 1) * (uint64_t)Wb - 1) / E); };
    // request holding list position p (0 <= p < T): ip[b] <= p < ip[b+1]
    auto request_at = [&](int32_t p) {
        int32_t a = 0, z = B;
        while (z - a > 1) {
            const int32_t mid = (a + z) >> 1;
            if (ip[mid] <= p)
                a = mid;
            else
                z = mid;
        }
        return a;
    };
    // parts of segment s when it is cut over several bins, else 0
    auto nparts_of = [&](int32_t s) -> int32_t {
        const int32_t kvh = s / B, b = s - kvh * B;
        if (ip[b + 1] == ip[b])
            return 0;
        const uint64_t start = (uint64_t)kvh * T + ip[b], end = (uint64_t)kvh * T + ip[b + 1];
        const int32_t w0 = bin_of(start), w1 = bin_of(end - 1);
        return w1 > w0 ? w1 - w0 + 1 : 0;
    };
    auto inclusive_scan = [&](int32_t v) {
        scan[tid] = v;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            const int32_t add = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        return scan[tid];
    };
    // the pieces of bin w, in position order: f(kvh, b, piece lo, piece hi)
    // with positions relative to the start of the segment
    auto for_pieces = [&](int32_t w, auto f) {
        uint64_t x = lo_of(w);
        const uint64_t hi = lo_of(w + 1);
        while (x < hi) {
            const int32_t kvh = (int32_t)(x / (uint64_t)T);
            const uint64_t seg0 = (uint64_t)kvh * T;
            const int32_t b = request_at((int32_t)(x - seg0));
            const uint64_t seg_start = seg0 + ip[b], seg_end = seg0 + ip[b + 1];
            const uint64_t e = seg_end < hi ? seg_end : hi;
            f(kvh, b, (int32_t)(x - seg_start), (int32_t)(e - seg_start), seg_start);
            x = e;
        }
    };

    // workgroup offsets: bin w's piece count, scanned (workgroups Wb .. W-1
    // get no units)
    int32_t count = 0;
    if (tid < Wb)
        for_pieces(tid, [&](int32_t, int32_t, int32_t, int32_t, uint64_t) { count++; });
    const int32_t units_end = inclusive_scan(count);
    const int32_t unit_base = units_end - count;
    if (tid < W)
        wg_offsets[tid] = unit_base;
    if (tid == W - 1)
        wg_offsets[W] = units_end;
    __syncthreads();

    // partial slots: segment s's parts start at P(s), numbered in segment
    // order; thread t numbers the segments of chunk t and keeps the chunk's
    // first slot
    const int32_t C = (S + kPlanThreads - 1) / kPlanThreads;
    const int32_t s_lo = min(S, tid * C), s_hi = min(S, s_lo + C);
    int32_t local = 0;
    for (int32_t s = s_lo; s < s_hi; s++)
        local += nparts_of(s);
    const int32_t chunk_end = inclusive_scan(local);
    chunk_first[tid] = chunk_end - local;
    int32_t first = chunk_end - local;
    for (int32_t s = s_lo; s < s_hi; s++) {
        const int32_t n = nparts_of(s);
        if (n > 0) {
            const int32_t kvh = s / B, b = s - kvh * B;
            pa_merge_unit m;
            m.request = b;
            m.kv_head = kvh;
            m.q_begin = b;
            m.q_end = b + 1;
            m.first_partial = first;
            m.n_parts = n;
            m.prefix_first = 0;
            m.prefix_parts = 0;
            merges[s] = m;
        }
        first += n;
    }
    __syncthreads();

    // the units of bin w
    if (tid < Wb) {
        int32_t at = unit_base;
        for_pieces(tid, [&](int32_t kvh, int32_t b, int32_t plo, int32_t phi, uint64_t seg_start) {
            const int32_t s = kvh * B + b;
            const int32_t len = ip[b + 1] - ip[b];
            pa_work_unit u;
            u.request = b;
            u.kv_head = kvh;
            u.kv_begin = ip[b] + plo;
            u.kv_end = ip[b] + phi;
            u.q_begin = b;
            u.q_end = b + 1;
            u.diag = u.kv_end - 1;
            u.part_stride = 0;
            u.cached_end = 0;
            u.reserved2 = 0;
            if (plo == 0 && phi == len) {
                u.partial = -1;
                u.merge = -1;
            } else {
                // P(s): the first slot of s's chunk plus the parts of the
                // chunk's segments before s
                const int32_t c = s / C;
                int32_t p = chunk_first[c];
                for (int32_t s2 = c * C; s2 < s; s2++)
                    p += nparts_of(s2);
                u.partial = p + (tid - bin_of(seg_start));
                u.merge = s;
            }
            units[at++] = u;
        });
    }
}

// Device address of `scratch` for each device (looked up once per device),
// and the decode workgroups each device holds at once per (D, G).
constexpr int kMaxDevices = 64;
std::mutex g_setup_mutex;
void *g_scratch[kMaxDevices];
int32_t g_workgroups[kMaxDevices][2][4];   // [device][D == 256][log2 G]; 0 = not known yet

int log2_group(int32_t g) { return g == 1 ? 0 : g == 2 ? 1 : g == 4 ? 2 : 3; }

}  // namespace

int noalloc_setup(int device, int32_t head_dim, int32_t group, void **scratch_ptr, int32_t *workgroups) {
    if (device < 0 || device >= kMaxDevices)
        return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_setup_mutex);
    if (!g_scratch[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return (int)e;
        if (!p)
            return (int)hipErrorInvalidSymbol;
        g_scratch[device] = p;
    }
    int32_t &w = g_workgroups[device][head_dim == 256 ? 1 : 0][log2_group(group)];
    if (w == 0) {
        int cus = 0;
        const hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
        if (e != hipSuccess)
            return (int)e;
        int per_cu = decode_workgroups_per_cu(head_dim, group, false);
        if (per_cu <= 0)
            per_cu = kDefaultWorkgroupsPerCu;
        w = cus * per_cu;
    }
    *scratch_ptr = g_scratch[device];
    *workgroups = w;
    return 0;
}

int launch_decode_noalloc(const NoAllocLaunch &a, void *stream) {
    char *base = static_cast<char *>(a.scratch);
    int32_t *wg_offsets = reinterpret_cast<int32_t *>(base + kNaOffsetsAt);
    pa_work_unit *units = reinterpret_cast<pa_work_unit *>(base + kNaUnitsAt);
    pa_merge_unit *merges = reinterpret_cast<pa_merge_unit *>(base + kNaMergesAt);
    int32_t *arrivals = reinterpret_cast<int32_t *>(base + kNaArrivalsAt);
    float *part_lse = reinterpret_cast<float *>(base + kNaPartLseAt);
    float *part_o = reinterpret_cast<float *>(base + kNaPartOAt);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(noalloc_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a.kv_indptr, a.batch,
                       a.num_kv_heads, a.num_qo_heads, a.head_dim, a.workgroups, wg_offsets, units, merges,
                       arrivals, a.out, a.lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return (int)e;
    DecodeLaunch l;
    l.wg_offsets = wg_offsets;
    l.n_workgroups = a.workgroups;
    l.units = units;
    l.n_units = a.workgroups + a.batch * a.num_kv_heads;
    l.merges = merges;
    l.n_merges = a.batch * a.num_kv_heads;
    l.q = a.q;
    l.k_pool = a.k_pool;
    l.v_pool = a.v_pool;
    l.slot_stride = a.slot_stride;
    l.num_slots = a.num_slots;
    l.kv_indices = a.kv_indices;
    l.sm_scale = a.sm_scale;
    l.out = a.out;
    l.lse = a.lse;
    l.partial_o = part_o;
    l.partial_lse = part_lse;
    l.arrivals = arrivals;
    l.num_qo_heads = a.num_qo_heads;
    l.num_kv_heads = a.num_kv_heads;
    l.head_dim = a.head_dim;
    return launch_decode(l, stream);
}

}  // namespace pa
