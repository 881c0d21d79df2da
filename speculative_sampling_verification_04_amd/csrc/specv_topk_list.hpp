// The per-wave candidate list of the streaming top-K selection (TopKAcc;
// the selection itself is described in specv_topk.hpp) [Speculative
// Speculative Decoding, sec. 4.1.1].
//
// This header only needs, from its includer, the wave primitives lane_id,
// __ballot, __popcll, lanes_below and wave_max_u64, the key functions
// logit_key, key_logit, full_key and max8, and kWaveSize, kLaneElems and
// kWaves (with __device__ and __forceinline__ defined), so that the list's
// bookkeeping can also be compiled on the host against an emulated wave.
//
// Bookkeeping invariant: a wave's list never holds more than kCandCap
// entries. Each step (of a block, or one()) pushes at most kWaveSize
// entries; it first compacts a list holding more than kCandCap - kWaveSize
// down to K (keys are unique, so exactly K are kept), so after the step the
// list holds at most max(kCandCap - kWaveSize, K) + kWaveSize <= kCandCap
// entries, which the static_assert in block() requires (kWaveSize + K <=
// kCandCap), whatever the number of steps per block. After the final compaction a wave keeps at most K
// entries of at most kLaneElems elements each, so the keys gathered from all
// waves fit topf_keys<K>().
#pragma once

namespace specv {

constexpr int kCandCap = 256;                  // candidate groups per wave
constexpr int32_t kSingle = 0x40000000;       // candidate holds one element, not 8


__device__ __forceinline__ uint64_t group_key(float vm, int64_t start) {
    return (uint64_t(logit_key(vm)) << 32) | uint64_t(~uint32_t(start));
}

template <int DT, int K>
struct TopKAcc {
    static_assert(K >= 1 && K <= 32 && (K & (K - 1)) == 0, "K is a power of two <= 32");

    int32_t* ent;        // this wave's candidates (LDS, kCandCap each): start
    uint64_t* mkey;      //   index (| kSingle for one element) and group key
    int count;           // wave-uniform
    uint64_t theta;      // wave-uniform: K-th largest group key at the last compaction (0: none)
    float th_val;        // its logit (-inf: none)

    __device__ void init(int32_t* e, uint64_t* k) {
        ent = e; mkey = k; count = 0;
        theta = 0; th_val = -INFINITY;
    }

    __device__ __forceinline__ void push(bool pass, int32_t e, uint64_t key) {
        const uint64_t m = __ballot(pass);
        if (pass) {
            const int pos = count + lanes_below(m);
            ent[pos] = e;
            mkey[pos] = key;
        }
        count += __popcll(m);
    }

    // Exact compaction from LDS: the K-th largest recorded group key becomes
    // theta and only the groups whose key reaches it are kept (nothing
    // changes while fewer than K candidates exist).
    __device__ void compact() {
        if (count < K) return;
        // Keys are unique: round k finds the largest key below round k-1's.
        uint64_t kth = ~0ull;
        for (int k = 0; k < K; ++k) {
            uint64_t l = 0;
            for (int i = lane_id(); i < count; i += kWaveSize) {
                const uint64_t x = mkey[i];
                if (x < kth && x > l) l = x;
            }
            kth = wave_max_u64(l);
        }
        if (kth > theta) {
            theta = kth;
            th_val = key_logit(uint32_t(kth >> 32));
        }
        int n = 0;
        for (int base = 0; base < count; base += kWaveSize) {
            const int i = base + lane_id();
            const bool keep = i < count && mkey[i] >= kth;
            const int32_t e = keep ? ent[i] : 0;
            const uint64_t x = keep ? mkey[i] : 0;
            const uint64_t m = __ballot(keep);
            if (keep) {
                const int pos = n + lanes_below(m);
                ent[pos] = e;
                mkey[pos] = x;
            }
            n += __popcll(m);
        }
        count = n;
    }

    // Each step of a block pushes up to kWaveSize groups, onto at most
    // kCandCap - kWaveSize (before a compaction) or K (after one): both fit
    // the list, whatever the number of steps U.
    template <int U>
    __device__ __forceinline__ void block(const float (&v)[U][kLaneElems], const int64_t* base, const bool* valid) {
        static_assert(kWaveSize + K <= kCandCap, "a step's candidates must fit the per-wave list after a compaction");
        float vm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) vm[u] = max8(v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (count > kCandCap - kWaveSize) compact();
            const bool pass = valid[u] && vm[u] >= th_val;
            push(pass, int32_t(base[u]), pass ? group_key(vm[u], base[u]) : 0ull);
        }
    }

    __device__ __forceinline__ void one(float z, int64_t j, bool ok) {
        if (count > kCandCap - kWaveSize) compact();
        const bool pass = ok && z >= th_val;
        push(pass, int32_t(j) | kSingle, pass ? full_key(z, j) : 0ull);
    }
};

// LDS words that topf_pick (and topf_finish) need for their key list.
template <int K>
constexpr int topf_keys() { return kWaves * kLaneElems * K; }

}  // namespace specv
