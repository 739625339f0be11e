// partition_fuzz.cpp -- the host partitioner (plan.cpp and the pa_partition
// entry points of api.cpp) driven with random step shapes, built for the host
// with AddressSanitizer and UBSan by tests/test_partition_sanitized.py.
// Cases: decode with the automatic split, with XCD and workgroup weights and
// with forced splits; chunked prefill; cascade groups; invalid offsets and
// group arrays; and output arrays sized exactly to the counts a first call
// reports (so any write past them is caught), or one entry short (which must
// give PA_ERR_CAPACITY).  Every decode partition is checked to cover each
// (request, KV head) list exactly once.  With a second argument N the cases
// run on N threads at once (each with its own random sequence), for a build
// with ThreadSanitizer.  Test infrastructure, host only: the GPU launchers are
// stubs that report "not supported".  Exit 0 when every case holds; a failing
// case is named on stderr.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace pa {
// stand-ins for the HIP translation units (never called by the partitioner)
constexpr int kNotSupported = 801;   // hipErrorNotSupported
int launch_decode(const DecodeLaunch &, void *) { return kNotSupported; }
int launch_prefill(const DecodeLaunch &, void *) { return kNotSupported; }
int launch_append(const AppendLaunch &, void *) { return kNotSupported; }
int launch_decode_noalloc(const NoAllocLaunch &, void *) { return kNotSupported; }
int noalloc_setup(int, int32_t, int32_t, void **, int32_t *) { return kNotSupported; }
int decode_workgroups_per_cu(int32_t, int32_t, bool) { return 3; }
}  // namespace pa

namespace {

thread_local uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {   // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
int32_t uniform(int32_t lo, int32_t hi) { return lo + (int32_t)(next_u32() % (uint32_t)(hi - lo + 1)); }

std::atomic<int> failures{0};
#define EXPECT(cond, ...)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            std::fprintf(stderr, "case %d: ", case_id);     \
            std::fprintf(stderr, __VA_ARGS__);              \
            std::fprintf(stderr, "\n");                     \
            failures++;                                     \
            return;                                         \
        }                                                   \
    } while (0)

std::vector<int32_t> draw_lengths(int32_t batch, bool allow_empty) {
    std::vector<int32_t> len(batch);
    const int mix = uniform(0, 2);
    for (auto &l : len) {
        l = mix == 0 ? uniform(1, 80) : mix == 1 ? uniform(1, 3000) : uniform(1000, 20000);
        if (allow_empty && uniform(0, 9) == 0)
            l = 0;
    }
    return len;
}

std::vector<int32_t> offsets(const std::vector<int32_t> &len) {
    std::vector<int32_t> ip(len.size() + 1, 0);
    for (size_t b = 0; b < len.size(); b++)
        ip[b + 1] = ip[b] + len[b];
    return ip;
}

// Each (request, KV head) range [ip[b], ip[b+1]) covered by the units exactly once.
bool covers_exactly(const std::vector<int32_t> &ip, int32_t hkv, const std::vector<pa_work_unit> &units,
                    int32_t first_entry_of_list_offset = 0) {
    (void)first_entry_of_list_offset;
    const int32_t batch = (int32_t)ip.size() - 1;
    std::vector<int32_t> hits((size_t)ip[batch] * hkv, 0);
    for (const auto &u : units) {
        if (u.request < 0)
            continue;   // padding
        if (u.request >= batch || u.kv_head < 0 || u.kv_head >= hkv || u.kv_begin < ip[u.request] ||
            u.kv_end > ip[u.request + 1] || u.kv_begin > u.kv_end)
            return false;
        for (int32_t e = u.kv_begin; e < u.kv_end; e++)
            hits[(size_t)e * hkv + u.kv_head]++;
    }
    for (int32_t h : hits)
        if (h != 1)
            return false;
    return true;
}

void decode_case(int case_id) {
    const int32_t batch = uniform(0, 70);
    const int32_t hkv = uniform(1, 8), g = 1 << uniform(0, 3), d = uniform(0, 1) ? 128 : 256;
    const auto len = draw_lengths(batch, true);
    const auto ip = offsets(len);
    uint32_t flags = uniform(0, 3) == 0 ? PA_PLAN_NO_XCD_ORDER : 0;
    const bool forced = uniform(0, 3) == 0;
    const int32_t n_forced = uniform(1, 300);
    if (forced)
        flags |= PA_PLAN_FORCE_SPLITS(n_forced);
    const int32_t mw_choice[] = {-1, 0, 1, 7, 256, 512, 768, 1024};
    const int32_t max_wg = mw_choice[uniform(0, 7)];
    const bool weighted = uniform(0, 2) == 0;
    std::vector<float> xw(8), ww(uniform(0, 800));
    for (auto &w : xw)
        w = 0.25f + 3.75f * (float)(next_u32() % 1000) / 999.f;
    for (auto &w : ww)
        w = 0.25f + 3.75f * (float)(next_u32() % 1000) / 999.f;
    auto call = [&](int32_t wcap, int32_t ucap, int32_t mcap, int32_t *wgo, pa_work_unit *un, pa_merge_unit *me,
                    int32_t *nw, int32_t *nu, int32_t *nm, int32_t *np) {
        if (weighted)
            return pa_partition_weighted(ip.data(), nullptr, batch, g * hkv, hkv, d, flags, max_wg, xw.data(), 8,
                                         ww.data(), (int32_t)ww.size(), wgo, wcap, un, ucap, me, mcap, nw, nu, nm,
                                         np);
        return pa_partition(ip.data(), nullptr, batch, g * hkv, hkv, d, flags, max_wg, wgo, wcap, un, ucap, me,
                            mcap, nw, nu, nm, np);
    };
    int32_t nw = -1, nu = -1, nm = -1, np = -1;
    pa_status st = call(0, 0, 0, nullptr, nullptr, nullptr, &nw, &nu, &nm, &np);
    if (forced && n_forced > PA_MAX_FORCED_SPLITS) {
        EXPECT(st == PA_ERR_INVALID_ARG, "forced %d splits: status %d, want invalid", n_forced, (int)st);
        return;
    }
    if (batch == 0 || ip[batch] == 0) {
        EXPECT(st == PA_OK || st == PA_ERR_CAPACITY, "empty step: status %d", (int)st);
        if (st == PA_OK)
            return;
    } else {
        EXPECT(st == PA_ERR_CAPACITY, "zero capacity: status %d", (int)st);
    }
    EXPECT(nw >= 0 && nu >= 0 && nm >= 0 && np >= 0, "counts not written: %d %d %d %d", nw, nu, nm, np);
    std::vector<int32_t> wgo(nw + 1);
    std::vector<pa_work_unit> units(nu);
    std::vector<pa_merge_unit> merges(nm);
    int32_t nw2, nu2, nm2, np2;
    st = call(nw + 1, nu, nm, wgo.data(), units.data(), merges.data(), &nw2, &nu2, &nm2, &np2);
    EXPECT(st == PA_OK, "exact capacity: status %d (%s)", (int)st, pa_last_error_detail());
    EXPECT(nw2 == nw && nu2 == nu && nm2 == nm && np2 == np, "counts changed between calls");
    EXPECT(wgo[0] == 0 && wgo[nw] == nu, "workgroup offsets do not span the units");
    for (int32_t w = 0; w < nw; w++)
        EXPECT(wgo[w] <= wgo[w + 1], "workgroup offsets decrease at %d", w);
    EXPECT(covers_exactly(ip, hkv, units), "decode lists not covered exactly once (batch %d, hkv %d)", batch, hkv);
    for (const auto &u : units)
        if (u.request >= 0 && u.partial >= 0)
            EXPECT(u.partial < np && u.merge >= 0 && u.merge < nm, "partial or merge index out of range");
    if (nu > 0) {   // one unit short
        std::vector<pa_work_unit> short_units(nu - 1);
        st = call(nw + 1, nu - 1, nm, wgo.data(), short_units.data(), merges.data(), &nw2, &nu2, &nm2, &np2);
        EXPECT(st == PA_ERR_CAPACITY, "one unit short: status %d", (int)st);
    }
}

void prefill_case(int case_id) {
    const int32_t batch = uniform(1, 12);
    const int32_t hkv = uniform(1, 8), g = 1 << uniform(0, 3), d = uniform(0, 1) ? 128 : 256;
    const auto len = draw_lengths(batch, false);
    std::vector<int32_t> chunk(batch);
    for (int32_t b = 0; b < batch; b++)
        chunk[b] = uniform(0, len[b] < 600 ? len[b] : 600);
    const auto ip = offsets(len), qo = offsets(chunk);
    uint32_t flags = uniform(0, 2) == 0 ? PA_PLAN_FORCE_SPLITS(uniform(1, 20)) : 0;
    int32_t nw = -1, nu = -1, nm = -1, np = -1;
    pa_status st = pa_partition(ip.data(), qo.data(), batch, g * hkv, hkv, d, flags, 768, nullptr, 0, nullptr, 0,
                                nullptr, 0, &nw, &nu, &nm, &np);
    if (st == PA_OK)
        return;   // nothing to place
    EXPECT(st == PA_ERR_CAPACITY, "prefill zero capacity: status %d (%s)", (int)st, pa_last_error_detail());
    std::vector<int32_t> wgo(nw + 1);
    std::vector<pa_work_unit> units(nu);
    std::vector<pa_merge_unit> merges(nm);
    int32_t nw2, nu2, nm2, np2;
    st = pa_partition(ip.data(), qo.data(), batch, g * hkv, hkv, d, flags, 768, wgo.data(), nw + 1, units.data(), nu,
                      merges.data(), nm, &nw2, &nu2, &nm2, &np2);
    EXPECT(st == PA_OK, "prefill exact capacity: status %d (%s)", (int)st, pa_last_error_detail());
    for (const auto &u : units) {
        if (u.request < 0)
            continue;
        EXPECT(u.request < batch && u.q_begin >= qo[u.request] && u.q_end <= qo[u.request + 1] &&
                   u.q_begin < u.q_end && u.kv_begin >= ip[u.request] && u.kv_end <= ip[u.request + 1],
               "prefill unit outside its request");
    }
    // a chunk longer than its list is refused
    std::vector<int32_t> bad_chunk = chunk;
    bad_chunk[0] = len[0] + 1;
    const auto bad_qo = offsets(bad_chunk);
    st = pa_partition(ip.data(), bad_qo.data(), batch, g * hkv, hkv, d, 0, 768, nullptr, 0, nullptr, 0, nullptr, 0,
                      &nw, &nu, &nm, &np);
    EXPECT(st == PA_ERR_INVALID_ARG, "chunk longer than its list: status %d", (int)st);
}

void cascade_case(int case_id) {
    const int32_t batch = uniform(1, 80);
    const int32_t hkv = uniform(1, 8), g = 1 << uniform(0, 3), d = uniform(0, 1) ? 128 : 256;
    auto len = draw_lengths(batch, false);
    std::vector<int32_t> gi{0};
    while (gi.back() < batch)
        gi.push_back(gi.back() + uniform(1, batch - gi.back()));
    const int32_t ng = (int32_t)gi.size() - 1;
    std::vector<int32_t> pl(ng);
    const bool bad = uniform(0, 5) == 0;
    for (int32_t k = 0; k < ng; k++) {
        int32_t shortest = len[gi[k]];
        for (int32_t b = gi[k]; b < gi[k + 1]; b++)
            shortest = len[b] < shortest ? len[b] : shortest;
        pl[k] = uniform(0, shortest);
        if (bad && k == 0)
            pl[k] = shortest + 1;   // longer than a member's list
    }
    const auto ip = offsets(len);
    const uint32_t flags = uniform(0, 1) ? PA_PLAN_CASCADE_ALL : 0;
    int32_t nw = -1, nu = -1, nm = -1, np = -1, npre = -1;
    pa_status st = pa_partition_cascade(ip.data(), batch, gi.data(), ng, pl.data(), g * hkv, hkv, d, flags, 768,
                                        nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0, &nw, &nu, &nm, &np, &npre);
    if (bad) {
        EXPECT(st == PA_ERR_INVALID_ARG, "prefix longer than a list: status %d", (int)st);
        return;
    }
    EXPECT(st == PA_ERR_CAPACITY, "cascade zero capacity: status %d (%s)", (int)st, pa_last_error_detail());
    std::vector<int32_t> wgo(nw + 1);
    std::vector<pa_work_unit> units(nu), pre(npre);
    std::vector<pa_merge_unit> merges(nm);
    int32_t nw2, nu2, nm2, np2, npre2;
    st = pa_partition_cascade(ip.data(), batch, gi.data(), ng, pl.data(), g * hkv, hkv, d, flags, 768, wgo.data(),
                              nw + 1, units.data(), nu, merges.data(), nm, pre.data(), npre, &nw2, &nu2, &nm2, &np2,
                              &npre2);
    EXPECT(st == PA_OK, "cascade exact capacity: status %d (%s)", (int)st, pa_last_error_detail());
    EXPECT(nw2 == nw && nu2 == nu && nm2 == nm && npre2 == npre, "cascade counts changed between calls");
}

void bad_offsets_case(int case_id) {
    std::vector<int32_t> ip{0, 5, 3, 9};
    int32_t nw, nu, nm, np;
    pa_status st = pa_partition(ip.data(), nullptr, 3, 8, 2, 128, 0, 768, nullptr, 0, nullptr, 0, nullptr, 0, &nw,
                                &nu, &nm, &np);
    EXPECT(st == PA_ERR_INVALID_ARG, "decreasing offsets: status %d", (int)st);
    ip = {1, 5, 9};
    st = pa_partition(ip.data(), nullptr, 2, 8, 2, 128, 0, 768, nullptr, 0, nullptr, 0, nullptr, 0, &nw, &nu, &nm,
                      &np);
    EXPECT(st == PA_ERR_INVALID_ARG, "offsets not starting at 0: status %d", (int)st);
}

void run_cases(int cases, uint64_t seed) {
    rng_state ^= seed * 0xD1B54A32D192ED03ull;
    for (int c = 0; c < cases; c++) {
        switch (c % 3) {
        case 0: decode_case(c); break;
        case 1: prefill_case(c); break;
        default: cascade_case(c); break;
        }
    }
    bad_offsets_case(cases);
}

}  // namespace

int main(int argc, char **argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 1500;
    const int threads = argc > 2 ? std::atoi(argv[2]) : 0;
    if (threads <= 0) {
        run_cases(cases, 0);
    } else {
        std::vector<std::thread> pool;
        for (int t = 0; t < threads; t++)
            pool.emplace_back(run_cases, cases, (uint64_t)t + 1);
        for (auto &th : pool)
            th.join();
    }
    std::printf("partition_fuzz: %d cases, %d failures\n", (cases + 1) * (threads > 0 ? threads : 1),
                failures.load());
    return failures == 0 ? 0 : 1;
}
