// Streaming selection of the K largest (logit, -index) keys of a row, for the
// SSD/Saguaro bonus-token candidates [Speculative Speculative Decoding, sec.
// 4.1.1].
//
// Keys: (order-preserving logit key << 32) | ~index, so a larger key is a
// larger logit, or an equal logit at a lower index. The row is seen in
// 8-element groups, and a group's key is (its maximum's logit key << 32) |
// ~(its start): groups do not overlap, so group keys order groups exactly as
// the keys of their largest elements do. Each wave records the groups whose
// maximum reaches a threshold theta in an LDS list (start, group key). When
// the list runs full, and at the end of the chunk, it is compacted exactly:
// the K groups with the largest keys are kept and theta becomes the K-th of
// them. A group whose maximum is below theta's logit cannot hold one of the K
// largest elements (each of the K kept groups holds an element at least that
// large), so the K largest keys of the chunk lie in the kept groups. While
// streaming, a group costs one compare against theta; recording is rare once
// theta has settled.
#pragma once

#include "specv_sample.hpp"
#include "specv_topk_list.hpp"

namespace specv {

// The `need` <= K largest keys of what acc streamed, largest first, in LDS
// (0 = none): every wave compacts its candidates to at most K groups, the
// keys that reach the largest wave threshold are gathered and wave 0 pops the
// largest. Whole workgroup.
template <int DT, int K>
__device__ __forceinline__ const uint64_t* topf_pick(TopKAcc<DT, K>& acc, const void* rp, int64_t V, int need,
                                                     uint64_t* keys) {
    __shared__ uint64_t s_theta[kWaves];
    __shared__ uint64_t s_pick[K];
    __shared__ int s_nkeys;

    acc.compact();
    if (lane_id() == 0) s_theta[wave_id()] = acc.theta;
    if (threadIdx.x == 0) s_nkeys = 0;
    __syncthreads();
    uint64_t th = s_theta[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) th = umax64(th, s_theta[w]);
    // The logit part only: every element of the workgroup's K largest has a
    // logit at least that of every wave's K-th group maximum.
    th &= 0xffffffff00000000ull;

    // Keys that reach the workgroup threshold: at most 8 per kept group.
    for (int e = lane_id(); e < acc.count; e += kWaveSize) {
        const int32_t ent = acc.ent[e];
        const int64_t j0 = ent & ~kSingle;
        const int n = (ent & kSingle) ? 1 : kLaneElems;
        for (int q = 0; q < n; ++q) {
            if (j0 + q >= V) break;
            const uint64_t key = full_key(load_elem<DT>(rp, j0 + q), j0 + q);
            if (key >= th) keys[atomicAdd(&s_nkeys, 1)] = key;
        }
    }
    __syncthreads();

    if (wave_id() == 0) {
        const int n = s_nkeys;
        for (int r = 0; r < need; ++r) {
            uint64_t l = 0;
            for (int i = lane_id(); i < n; i += kWaveSize) l = umax64(l, keys[i]);
            const uint64_t w = wave_max_u64(l);
            for (int i = lane_id(); i < n; i += kWaveSize)
                if (keys[i] == w) keys[i] = 0;   // keys are unique: one owner
            if (lane_id() == 0) s_pick[r] = w;
        }
    }
    __syncthreads();
    return s_pick;
}

// Writes the first F of the `need` picked keys that are not `excl` (ids and
// logits), then -1 up to Fmax entries. One thread.
__device__ __forceinline__ void topf_write(const uint64_t* pick, int need, int F, int Fmax, int32_t excl,
                                           int32_t* out_ids, float* out_logits) {
    int n = 0;
    for (int r = 0; r < need && n < F; ++r) {
        const uint64_t key = pick[r];
        if (key == 0) break;
        const int32_t idx = int32_t(~uint32_t(key));
        if (idx == excl) continue;
        out_ids[n] = idx;
        if (out_logits) out_logits[n] = key_logit(uint32_t(key >> 32));
        ++n;
    }
    for (; n < Fmax; ++n) {  // unused entries (and fewer candidates than F, only when vocab <= F)
        out_ids[n] = -1;
        if (out_logits) out_logits[n] = -INFINITY;
    }
}

// The F1 largest keys of a row searched in chunks, from the chunks' published
// lists (n pairs at kw: each chunk's F1 largest keys, 0 for none), which the
// caller has seen published (ok; if not, nothing is read): loads them into mk
// (LDS, n words) and pops the F1 largest, which are the row's own (each of
// them is among its chunk's F1 largest). Returns them in LDS, largest first
// (0 = none; all 0 without ok). Whole workgroup.
template <int kMaxKeys>
__device__ __forceinline__ const uint64_t* topf_merge_chunks(const uint64_t* kw, int n, int F1, uint64_t* mk,
                                                             bool ok) {
    __shared__ uint64_t s_pick[kMaxKeys];
    for (int i = threadIdx.x; i < n; i += kThreads) mk[i] = ok ? read_pair(kw, i) : 0ull;
    __syncthreads();
    if (wave_id() == 0) {
        for (int r = 0; r < F1; ++r) {
            uint64_t l = 0;
            for (int i = lane_id(); i < n; i += kWaveSize) l = umax64(l, mk[i]);
            const uint64_t w = wave_max_u64(l);
            for (int i = lane_id(); i < n; i += kWaveSize)
                if (w != 0 && mk[i] == w) mk[i] = 0;   // keys are unique: one owner
            if (lane_id() == 0) s_pick[r] = w;
        }
    }
    __syncthreads();
    return s_pick;
}

// Ends a row's selection (whole workgroup, after streaming; keys: LDS of
// topf_keys<K>() words): every wave compacts its candidates to at most K
// groups, the keys that reach the largest wave threshold are gathered, wave 0
// pops the F + 1 largest, and thread 0 writes the first F ids (and logits)
// that are not `excl`, then -1 up to Fmax entries. Returns the F + 1 largest
// keys of the row in LDS (0 = none), before the exclusion; they stay valid
// until the caller's next barrier.
template <int DT, int K>
__device__ __forceinline__ const uint64_t* topf_finish(TopKAcc<DT, K>& acc, const void* rp, int64_t V, int F,
                                                       int Fmax, int32_t excl, int32_t* out_ids, float* out_logits,
                                                       uint64_t* keys) {
    const uint64_t* pick = topf_pick<DT, K>(acc, rp, V, F + 1, keys);
    if (threadIdx.x == 0) topf_write(pick, F + 1, F, Fmax, excl, out_ids, out_logits);
    __syncthreads();
    return pick;
}

// The F-th largest key of the row (no exclusion), or ~0 (reached by no key)
// when F = 0: a key is among the row's top F iff it is >= this.
__device__ __forceinline__ uint64_t topf_sigma_key(const uint64_t* pick, int F) { return F > 0 ? pick[F - 1] : ~0ull; }

// The F-th largest key once `excl` is dropped, or ~0 when F = 0: a key other
// than excl's is a cache candidate iff it is >= this (0 when the row has
// fewer than F other elements: then every one is).
__device__ __forceinline__ uint64_t topf_cache_key(const uint64_t* pick, int F, int32_t excl) {
    if (F == 0) return ~0ull;
    int n = 0;
    for (int r = 0; r <= F && n < F; ++r) {
        const uint64_t key = pick[r];
        if (key == 0) break;
        if (int32_t(~uint32_t(key)) == excl) continue;
        if (++n == F) return key;
    }
    return 0ull;
}

}  // namespace specv
