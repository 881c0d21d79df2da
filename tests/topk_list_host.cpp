// Host build of the top-K candidate list's bookkeeping (TopKAcc in
// speculative_sampling_verification_04_amd/csrc/specv_topk_list.hpp),
// compiled with g++ against an emulated 64-lane wave: one std::thread per
// lane, and every wave-wide primitive (ballot, maximum) is a rendezvous of
// the 64 threads. Each lane owns its TopKAcc copy, as each lane does on the
// GPU, and the list lives in a shared array with a guard region past
// kCandCap, so an overflow is seen by the checks instead of corrupting
// memory.
//
// For each steps-per-iteration U up to 8 (U = 1 also covers the tail's one()), each
// K and each row shape, one wave is fed a row the way stream_chunk feeds it
// (lane l of wave 0 sees step it * 256 * U + u * 256 + l of 8 elements, then
// the tail one element per lane) and after every block() / one() the list's
// count must be <= kCandCap (with the guard region untouched). After the
// final compaction the wave's gathered keys (the keys of its kept entries
// that reach its threshold) must number <= kLaneElems * K, i.e. the four
// waves' together <= topf_keys<K>(), and they must hold the K largest keys
// of what the wave saw. Prints "ok" and exits 0, or names the failure.
#include <barrier>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <random>
#include <string>
#include <thread>
#include <vector>

#define __device__
#define __forceinline__ inline

namespace specv {

constexpr int kThreads = 256;
constexpr int kWaveSize = 64;
constexpr int kWaves = kThreads / kWaveSize;
constexpr int kLaneElems = 8;

thread_local int t_lane = 0;
std::barrier<>* g_bar = nullptr;
uint64_t g_vals[kWaveSize];

inline int lane_id() { return t_lane; }

// The 64 values of one wave-wide step: every lane writes, all meet, each
// reads, all meet again before the array is reused.
template <class F>
inline uint64_t wave_reduce(uint64_t mine, F f) {
    g_vals[t_lane] = mine;
    g_bar->arrive_and_wait();
    uint64_t r = 0;
    for (int i = 0; i < kWaveSize; ++i) r = f(r, g_vals[i], i);
    g_bar->arrive_and_wait();
    return r;
}

inline uint64_t wave_max_u64(uint64_t x) {
    return wave_reduce(x, [](uint64_t r, uint64_t v, int) { return v > r ? v : r; });
}

inline int lanes_below(uint64_t m) {
    return __builtin_popcountll(m & ((t_lane == 0) ? 0ull : (~0ull >> (64 - t_lane))));
}

inline float max8(const float v[kLaneElems]) {
    float m = v[0];
    for (int e = 1; e < kLaneElems; ++e) m = std::max(m, v[e]);
    return m;
}

inline uint32_t f2u(float v) { uint32_t u; std::memcpy(&u, &v, 4); return u; }
inline float u2f(uint32_t u) { float v; std::memcpy(&v, &u, 4); return v; }

// The device's order-preserving logit key and its inverse.
inline uint32_t logit_key(float v) {
    uint32_t u = f2u(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
inline float key_logit(uint32_t k) { return u2f((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }
inline uint64_t full_key(float v, int64_t j) { return (uint64_t(logit_key(v)) << 32) | uint64_t(~uint32_t(j)); }

}  // namespace specv

inline uint64_t __ballot(int pred) {
    return specv::wave_reduce(pred ? 1ull : 0ull,
                              [](uint64_t r, uint64_t v, int i) { return v ? (r | (1ull << i)) : r; });
}
inline int __popcll(uint64_t m) { return __builtin_popcountll(m); }

#include "specv_topk_list.hpp"

using namespace specv;

constexpr int kGuard = 1024;
int32_t g_ent[kCandCap + kGuard];
uint64_t g_key[kCandCap + kGuard];
bool g_failed = false;
std::string g_why;

void fail(const std::string& why) {
    if (!g_failed) { g_failed = true; g_why = why; }
}

bool guard_clean() {
    for (int i = kCandCap; i < kCandCap + kGuard; ++i)
        if (g_ent[i] != -7 || g_key[i] != 7ull) return false;
    return true;
}

// One wave streams `row` (n elements) as stream_chunk does, with U steps per
// iteration; checks the invariants. Returns the gathered keys (lane 0's view).
template <int U, int K>
void run_wave(const std::vector<float>& row, const std::string& name) {
    const int64_t n = int64_t(row.size());
    const int64_t nstep = n / kLaneElems;
    const int64_t kStride = int64_t(kThreads) * U;
    const int64_t nit = (nstep + kStride - 1) / kStride;
    for (int i = 0; i < kCandCap + kGuard; ++i) { g_ent[i] = -7; g_key[i] = 7ull; }
    std::barrier<> bar(kWaveSize);
    g_bar = &bar;
    std::vector<uint64_t> seen;        // every key wave 0 was shown (lane 0 collects after the run)
    std::vector<std::vector<uint64_t>> lane_seen(kWaveSize);
    std::vector<uint64_t> gathered;
    int max_count = 0;
    auto lane_main = [&](int lane) {
        t_lane = lane;
        TopKAcc<0, K> acc;
        acc.init(g_ent, g_key);
        auto check = [&](const char* where) {
            bar.arrive_and_wait();
            if (lane == 0) {
                max_count = std::max(max_count, acc.count);
                if (acc.count > kCandCap || !guard_clean())
                    fail(name + ": list overflow after " + where + " (count " + std::to_string(acc.count) + ")");
            }
            bar.arrive_and_wait();
        };
        for (int64_t it = 0; it < nit; ++it) {
            float v[U][kLaneElems];
            int64_t base[U];
            bool valid[U];
            for (int u = 0; u < U; ++u) {
                const int64_t s = it * kStride + int64_t(u) * kThreads + lane;   // wave 0: threads 0..63
                valid[u] = s < nstep;
                base[u] = s * kLaneElems;
                for (int e = 0; e < kLaneElems; ++e) {
                    v[u][e] = valid[u] ? row[s * kLaneElems + e] : -INFINITY;
                    if (valid[u]) lane_seen[lane].push_back(full_key(v[u][e], s * kLaneElems + e));
                }
            }
            acc.template block<U>(v, base, valid);
            check("block");
        }
        for (int64_t j0 = nstep * kLaneElems; j0 < n; j0 += kThreads) {
            const int64_t j = j0 + lane;
            const bool ok = j < n;
            if (ok) lane_seen[lane].push_back(full_key(row[j], j));
            acc.one(ok ? row[j] : -INFINITY, j, ok);
            check("one");
        }
        acc.compact();
        check("the final compaction");
        if (lane == 0) {
            if (acc.count > K && acc.count > 0) fail(name + ": more than K entries after the final compaction");
            const uint64_t th = acc.theta & 0xffffffff00000000ull;
            for (int e = 0; e < acc.count; ++e) {
                const int32_t ent = acc.ent[e];
                const int64_t j0 = ent & ~kSingle;
                const int m = (ent & kSingle) ? 1 : kLaneElems;
                for (int q = 0; q < m && j0 + q < n; ++q) {
                    const uint64_t key = full_key(row[j0 + q], j0 + q);
                    if (key >= th) gathered.push_back(key);
                }
            }
        }
    };
    std::vector<std::thread> lanes;
    for (int l = 0; l < kWaveSize; ++l) lanes.emplace_back(lane_main, l);
    for (auto& t : lanes) t.join();
    for (auto& ls : lane_seen) seen.insert(seen.end(), ls.begin(), ls.end());
    if ((int64_t)gathered.size() > int64_t(kLaneElems) * K)
        fail(name + ": " + std::to_string(gathered.size()) + " gathered keys, more than kLaneElems * K");
    if (int64_t(kWaves) * kLaneElems * K != topf_keys<K>()) fail("topf_keys<K>() is not kWaves * kLaneElems * K");
    std::sort(seen.rbegin(), seen.rend());
    std::sort(gathered.rbegin(), gathered.rend());
    for (int r = 0; r < K && r < int(seen.size()); ++r)
        if (!std::binary_search(gathered.rbegin(), gathered.rend(), seen[r]))
            fail(name + ": the " + std::to_string(r) + "-th largest key was not gathered");
    std::printf("%-40s U=%d K=%2d max count %3d gathered %3zu\n", name.c_str(), U, K, max_count, gathered.size());
}

template <int U, int K>
void all_rows() {
    std::mt19937 gen(1234 + U * 100 + K);
    std::normal_distribution<float> nd(0.0f, 3.0f);
    const int64_t n = int64_t(kThreads) * U * kLaneElems * 6 + 8 * 37 + 5;   // six iterations, a ragged tail
    std::vector<float> eq(n, 1.0f), asc(n), desc(n), rnd(n), neg(n);
    for (int64_t i = 0; i < n; ++i) {
        asc[i] = float(i);
        desc[i] = float(n - i);
        rnd[i] = nd(gen);
        neg[i] = (i % 3 == 0) ? -INFINITY : (i % 3 == 1 ? -0.0f : 0.0f);
    }
    // Ascending within each lane's stream: every new group beats theta, the
    // most pushes the list can see.
    std::vector<float> lane_asc(n);
    for (int64_t i = 0; i < n; ++i) lane_asc[i] = float(i / kLaneElems) + 0.001f * float(i % kLaneElems);
    run_wave<U, K>(eq, "all equal");
    run_wave<U, K>(asc, "strictly ascending");
    run_wave<U, K>(lane_asc, "ascending by step");
    run_wave<U, K>(desc, "strictly descending");
    run_wave<U, K>(rnd, "random");
    run_wave<U, K>(neg, "-inf, -0 and +0");
}

template <int U>
void all_k() {
    all_rows<U, 2>();
    all_rows<U, 4>();
    all_rows<U, 8>();
    all_rows<U, 16>();
    all_rows<U, 32>();
}

int main() {
    all_k<1>();   // one() and single-step blocks
    all_k<2>();   // draft-row and top-F streaming shapes
    all_k<4>();
    all_k<8>();
    if (g_failed) {
        std::printf("FAILED: %s\n", g_why.c_str());
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
