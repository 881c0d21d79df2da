// Streaming selection of the K largest (logit, -index) keys of a row, for the
// SSD/Saguaro bonus-token candidates [Speculative Speculative Decoding, sec.
// 4.1.1].
//
// Keys: (order-preserving logit key << 32) | ~index, so a larger key is a
// larger logit, or an equal logit at a lower index. Each lane tracks only its
// running maximum (value and lowest index). Once per streaming iteration the
// wave forms a lower bound theta on the K-th largest key seen so far: the
// minimum, over K groups of lanes, of each group's largest lane maximum (K
// distinct elements are >= theta). An 8-element group whose maximum reaches
// theta is recorded as a candidate (its start index) in the wave's LDS list;
// every other group cannot hold one of the K largest keys. When the list runs
// full, and at the end of the chunk, it is compacted exactly: the K groups
// with the largest maxima are kept and theta becomes the K-th of those maxima.
// The K largest keys of the chunk then lie in the kept groups.
#pragma once

#include <limits.h>

#include "specv_sample.hpp"

namespace specv {

constexpr int kCandCap = 512;                  // candidate groups per wave
constexpr int32_t kSingle = 0x40000000;       // candidate holds one element, not 8

__device__ __forceinline__ int lanes_below(uint64_t m) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Largest key of a candidate's elements (8 from its start, or one), < hi.
template <int DT>
__device__ uint64_t candidate_max_key(const void* row, int32_t ent, int64_t hi) {
    const int64_t j0 = ent & ~kSingle;
    const int n = (ent & kSingle) ? 1 : kLaneElems;
    uint64_t best = 0;
    for (int e = 0; e < n; ++e)
        if (j0 + e < hi) best = umax64(best, full_key(load_elem<DT>(row, j0 + e), j0 + e));
    return best;
}

template <int DT, int K>
struct TopKAcc {
    static_assert(K >= 1 && K <= 32 && (K & (K - 1)) == 0, "K is a power of two <= 32");
    static constexpr int kGroupLanes = kWaveSize / K;

    const void* row;
    int64_t hi;          // elements at or past hi are not part of the chunk
    int32_t* buf;        // this wave's candidate list (LDS, kCandCap entries)
    int count;           // wave-uniform
    float lm;            // lane maximum and its lowest index (-1: none yet)
    int32_t li;
    uint64_t theta;      // wave-uniform lower bound on the K-th largest key (0: none)
    float th_val;
    int32_t th_idx;

    __device__ void init(const void* r, int64_t h, int32_t* b) {
        row = r; hi = h; buf = b; count = 0;
        lm = -INFINITY; li = -1;
        theta = 0; th_val = -INFINITY; th_idx = INT_MAX;
    }

    // theta's logit and index; an index part of 0 (key lo) stands for "any
    // index", i.e. th_idx = INT_MAX.
    __device__ __forceinline__ void raise_theta(uint64_t k) {
        if (k > theta) {
            theta = k;
            th_val = key_logit(uint32_t(k >> 32));
            th_idx = uint32_t(k) == 0u ? INT_MAX : int32_t(~uint32_t(k));
        }
    }

    // Min over K groups of the group's largest lane maximum (wave-uniform
    // result), on logit keys only: (key << 32 | 0) is below every full key with
    // that logit, so it is still a lower bound on the K-th largest full key.
    __device__ __forceinline__ void refresh() {
        uint32_t k = li >= 0 ? logit_key(lm) : 0u;
#pragma unroll
        for (int o = 1; o < kGroupLanes; o <<= 1) k = max(k, uint32_t(__shfl_xor(k, o)));
#pragma unroll
        for (int o = kGroupLanes; o < kWaveSize; o <<= 1) k = min(k, uint32_t(__shfl_xor(k, o)));
        raise_theta(uint64_t(k) << 32);
    }

    // A group with maximum vm starting at `start` may hold a key >= theta.
    __device__ __forceinline__ bool reaches(float vm, int64_t start) const {
        return vm > th_val || (vm == th_val && start <= th_idx);
    }

    __device__ __forceinline__ void push(bool pass, int32_t ent) {
        const uint64_t m = __ballot(pass);
        if (pass) buf[count + lanes_below(m)] = ent;
        count += __popcll(m);
    }

    // Exact compaction: keep the K candidates with the largest maxima and
    // raise theta to the K-th of them (only when at least K candidates exist).
    __device__ void compact() {
        constexpr int R = kCandCap / kWaveSize;
        int32_t ent[R];
        uint64_t mk[R], tmp[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = lane_id() + r * kWaveSize;
            ent[r] = e < count ? buf[e] : -1;
            mk[r] = ent[r] >= 0 ? candidate_max_key<DT>(row, ent[r], hi) : 0;
            tmp[r] = mk[r];
        }
        uint64_t kth = 0;
        int got = 0;
        for (int k = 0; k < K; ++k) {
            uint64_t l = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) l = umax64(l, tmp[r]);
            const uint64_t w = wave_max_u64(l);
            if (w == 0) break;
            kth = w;
            ++got;
#pragma unroll
            for (int r = 0; r < R; ++r) tmp[r] = (tmp[r] == w) ? 0 : tmp[r];
        }
        if (got < K) return;  // fewer than K candidates: nothing to drop
        raise_theta(kth);
        int n = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool keep = ent[r] >= 0 && mk[r] >= kth;
            const uint64_t m = __ballot(keep);
            if (keep) buf[n + lanes_below(m)] = ent[r];
            n += __popcll(m);
        }
        count = n;
    }

    template <int U>
    __device__ __forceinline__ void block(const float (&v)[U][kLaneElems], const int64_t* base, const bool* valid) {
        float vm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            vm[u] = max8(v[u]);
            if (valid[u] && (vm[u] > lm || li < 0)) {
                int e = kLaneElems - 1;
#pragma unroll
                for (int k = kLaneElems - 2; k >= 0; --k) e = (v[u][k] == vm[u]) ? k : e;
                lm = vm[u];
                li = int32_t(base[u] + e);
            }
        }
        refresh();
        if (count > kCandCap - kWaveSize * U) compact();
#pragma unroll
        for (int u = 0; u < U; ++u) push(valid[u] && reaches(vm[u], base[u]), int32_t(base[u]));
    }

    __device__ __forceinline__ void one(float z, int64_t j, bool ok) {
        if (ok && (z > lm || li < 0)) { lm = z; li = int32_t(j); }
        refresh();
        if (count > kCandCap - kWaveSize) compact();
        push(ok && reaches(z, j), int32_t(j) | kSingle);
    }
};

}  // namespace specv
