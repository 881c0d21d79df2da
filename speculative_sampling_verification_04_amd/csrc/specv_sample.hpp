// Workgroup-level pieces of the resolve step of the verification kernels:
// collecting the published row statistics, block merges, and inverse-CDF
// sampling from a row of non-negative weights.
//
// Inverse CDF [reading of Lecture 5: Speculative Decoding and SpecInfer, sec.
// 2.2 step 4 / Speculative Decoding (dl-note), sec. 2.3]: the sample is the
// smallest index j with w_0 + ... + w_j >= v * W, W = sum of all weights.
// Two passes over the row: (A) the waves sum 512-element tiles (64 lanes x 8
// consecutive elements), several tiles in flight per wave, into LDS; (B) wave 0
// scans the tile sums in fp64 to find the tile that holds v*W, recomputes that
// tile's weights (bit-identical to pass A) and scans them for the index. Only
// the one row (pair) that needs a sample is read a second time.
#pragma once

#include "specv_device.hpp"

namespace specv {

constexpr int kTilesInFlight = 4;      // residual pass: tiles per wave per iteration

// Bound on every wait for another workgroup's word, in ticks of the
// constant-rate clock read by wall_clock64 (100 MHz): by default 2^27 ticks,
// about 1.3 s, kMaxWaitTicks (the launches pass it in their arguments). A
// wait that reaches it gives up and its call reports failure (-1) instead of
// hanging.
struct WaitBound {
    uint64_t t0, ticks;
    __device__ explicit WaitBound(uint64_t n) : t0(wall_clock64()), ticks(n) {}
    __device__ bool expired() const { return wall_clock64() - t0 > ticks; }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWaveSize - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWaveSize; }

__device__ __forceinline__ void block_merge_softmax(float& m, float& mc, double& s) {
    __shared__ float sm[kWaves], smc[kWaves];
    __shared__ double ss[kWaves];
    wave_merge_softmax(m, mc, s);
    if (lane_id() == 0) { sm[wave_id()] = m; smc[wave_id()] = mc; ss[wave_id()] = s; }
    __syncthreads();
    m = sm[0]; mc = smc[0]; s = ss[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) merge_softmax(m, mc, s, sm[w], smc[w], ss[w]);
    __syncthreads();
}

__device__ __forceinline__ void block_merge_argmax(float& v, int32_t& i) {
    __shared__ float sv[kWaves];
    __shared__ int32_t si[kWaves];
    wave_merge_argmax(v, i);
    if (lane_id() == 0) { sv[wave_id()] = v; si[wave_id()] = i; }
    __syncthreads();
    v = sv[0]; i = si[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        if (argmax_better(sv[w], si[w], v, i)) { v = sv[w]; i = si[w]; }
    __syncthreads();
}

constexpr int kMaxOrderedBatch = 4096;

// Where a workgroup of a chain launch sits: its sequence slot, its index in
// that slot's tasks, and the sequence in the slot.
struct Placement {
    int sidx;
    int64_t w;
    int b;
};

// Placement of workgroup g. Sequences are dispatched T > 0 first, then the
// greedy ones, each group by increasing index (identity when B >
// kMaxOrderedBatch): only T > 0 sequences re-read a row to draw the bonus, so
// their bonus workgroups start early and overlap the greedy sequences' rows.
// decode(nS, sidx, w) maps g to its slot given the number nS of T > 0
// sequences. Wave 0 computes everything (one round trip for the
// temperatures, ballots, no serial search); whole workgroup, one barrier.
template <class Decode>
__device__ __forceinline__ Placement place(const float* temperature, int B, Decode decode) {
    __shared__ uint64_t masks[kMaxOrderedBatch / kWaveSize];
    __shared__ Placement s_pl;
    if (wave_id() == 0) {
        const int lane = lane_id();
        const int nm = (B + kWaveSize - 1) / kWaveSize;
        const bool ordered = B <= kMaxOrderedBatch;
        int nS = B;
        if (ordered) {
            nS = 0;
            for (int c = 0; c < nm; ++c) {
                const int i = c * kWaveSize + lane;
                const uint64_t m = __ballot(i < B && temperature[i] > 0.0f);
                if (lane == 0) masks[c] = m;
                nS += __popcll(m);
            }
        }
        int sidx;
        int64_t w;
        decode(nS, sidx, w);
        int b = sidx;
        if (ordered) {
            const bool sampled = sidx < nS;
            int k = sampled ? sidx : sidx - nS;
            for (int c = 0; c < nm; ++c) {
                uint64_t m = sampled ? masks[c] : ~masks[c];
                const int valid = min(kWaveSize, B - c * kWaveSize);
                if (valid < kWaveSize) m &= (1ull << valid) - 1ull;
                const int cnt = __popcll(m);
                if (k < cnt) {   // the k-th set bit of m
                    const bool bit = (m >> lane) & 1ull;
                    const uint64_t hit = __ballot(bit && lanes_below(m) == k);
                    b = c * kWaveSize + __builtin_ctzll(hit);
                    break;
                }
                k -= cnt;
            }
        }
        if (lane == 0) s_pl = Placement{sidx, w, b};
    }
    __syncthreads();
    return s_pl;
}

// Waits until the n slots are all published (wave 0 polls with agent-scope
// atomic loads). Every slot's writer is a workgroup with a lower index, which
// is dispatched before the caller and never waits itself, so the wait ends;
// the spin is bounded anyway. Returns false if the bound was reached.
__device__ bool wait_slots(const uint64_t* slots, int64_t n, uint64_t ticks) {
    __shared__ int s_ok;
    if (wave_id() == 0) {
        int ok = 0;
        for (const WaitBound t(ticks); !t.expired();) {
            // Four loads in flight per lane per step (no short-circuit, so
            // that no load waits for another).
            bool mine = true;
            int64_t i = lane_id();
            for (; i + 3 * kWaveSize < n; i += 4 * kWaveSize) {
                const uint64_t a0 = peek(slots + i), a1 = peek(slots + i + kWaveSize);
                const uint64_t a2 = peek(slots + i + 2 * kWaveSize), a3 = peek(slots + i + 3 * kWaveSize);
                mine &= slot_ready(a0) & slot_ready(a1) & slot_ready(a2) & slot_ready(a3);
            }
            for (; i < n; i += kWaveSize) mine &= slot_ready(peek(slots + i));
            if (__all(mine)) { ok = 1; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane_id() == 0) s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

// Returns the n slots to zero (the workspace's resting state).
__device__ __forceinline__ void zero_slots(uint64_t* slots, int64_t n) {
    for (int64_t i = threadIdx.x; i < n; i += kThreads) publish(slots + i, 0ull);
}

// Merged statistics of one row (all chunks).
struct RowStats {
    float m;     // max logit (greedy: best logit)
    float mc;    // fp32 m * c
    int32_t idx; // greedy argmax
    double Z;    // sum of 2^(z*c - mc)
};

// A row's statistics from its one word (S = 1): what merging that word alone
// gives. Any thread.
__device__ __forceinline__ RowStats stats_of_word(uint64_t w, bool greedy, float c) {
    RowStats r{-INFINITY, -INFINITY, -1, 0.0};
    const float v = slot_hi(w);
    if (greedy) {
        const int32_t i = slot_idx(w);
        if (i >= 0) { r.m = v; r.idx = i; }
    } else if (v != -INFINITY) {
        r.m = v;
        r.mc = v * c;
        r.Z = double(slot_s(w));
    }
    return r;
}

// A row's statistics from its S <= 64 chunk words, chunk j's word in lane j
// (the words of lanes >= S are ignored). Greedy: the largest (value, lowest
// index) over the chunks, an order-free maximum. Softmax: the largest chunk
// maximum m, then the chunks' sums rescaled to it, 2^(m_j c - m c), and added
// in the wave's fixed order, so that every workgroup that merges the same
// words gets the same bits. Whole wave (every lane active); the result is
// the same in every lane. The S loads are one round trip, issued by the
// caller.
__device__ __forceinline__ RowStats merge_chunk_words(uint64_t w, int S, bool greedy, float c) {
    const bool mine = lane_id() < S;
    RowStats r;
    if (greedy) {
        const int32_t i = slot_idx(w);
        const uint64_t key = (mine && i >= 0) ? full_key(slot_hi(w), i) : 0ull;
        const uint64_t best = wave_max_u64(key);
        r.m = best ? key_logit(uint32_t(best >> 32)) : -INFINITY;
        r.idx = best ? int32_t(~uint32_t(best)) : -1;
        r.mc = -INFINITY;
        r.Z = 0.0;
        return r;
    }
    const float m = mine ? slot_hi(w) : -INFINITY;
    const uint64_t top = wave_max_u64(uint64_t(logit_key(m)) << 32);
    r.m = key_logit(uint32_t(top >> 32));
    r.mc = r.m * c;
    r.idx = -1;
    const double part = (m == -INFINITY) ? 0.0 : double(slot_s(w)) * exp2(double(m * c) - double(r.mc));
    r.Z = wave_sum(part);
    return r;
}

// p(x) = 2^(z*c - mc) / Z in fp64, the same reference the streaming pass used.
__device__ __forceinline__ double prob_of(float z, float c, const RowStats& st) {
    if (z == -INFINITY) return 0.0;
    return exp2(double(z) * double(c) - double(st.mc)) / st.Z;
}

// Raw bits of 8 consecutive elements [j0, j0+8): one or two 16-byte loads when
// the row start is 16-byte aligned (`vec`) and the group is whole; element
// loads otherwise, -inf past the end of the row.
template <int DT>
__device__ __forceinline__ void load_group(const void* row, int64_t j0, int64_t V, bool vec, Raw8<DT>& r) {
    if (vec && j0 + kLaneElems <= V) {
        load_raw8<DT>(r, static_cast<const char*>(row) + j0 * ElemT<DT>::kBytes);
        return;
    }
    uint32_t h[kLaneElems];
    if constexpr (DT == DT_BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(row);
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) h[e] = (j0 + e < V) ? uint32_t(p[j0 + e]) : 0xFF80u;
        r.w[0] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    } else {
        const uint32_t* p = static_cast<const uint32_t*>(row);
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) h[e] = (j0 + e < V) ? p[j0 + e] : 0xFF800000u;
        r.w[0] = make_uint4(h[0], h[1], h[2], h[3]);
        r.w[1] = make_uint4(h[4], h[5], h[6], h[7]);
    }
}

// Probabilities p = 2^(z*c - mc) / Z of one row (fp32). With a threshold key
// (Saguaro sampling), the elements whose key reaches it (the row's top F) are
// scaled by `scale` and Z is the correspondingly reduced normaliser.
template <int DT, bool kScaled = false>
struct ProbRow {
    const void* row;
    float c, nmc, invZ;
    bool vec;
    float scale;          // factor on the top-F elements (kScaled only)
    uint64_t top_word;    // threshold key + 1 (0: no scaling; kScaled only)
    __device__ void init(const void* r, float c_, const RowStats& st) {
        row = r; c = c_; nmc = -st.mc; invZ = float(1.0 / st.Z);
        vec = (reinterpret_cast<uintptr_t>(r) & 15u) == 0;
        scale = 1.0f; top_word = 0ull;
    }
    // Elements j0 .. j0 + 7.
    __device__ __forceinline__ void probs(const Raw8<DT>& raw, int64_t j0, float p[kLaneElems]) const {
        float z[kLaneElems];
        unpack8<DT>(raw, z);
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(z[e], c, nmc)) * invZ;
        if (kScaled && top_word != 0ull) {
#pragma unroll
            for (int e = 0; e < kLaneElems; ++e)
                if (full_key(z[e], j0 + e) + 1ull >= top_word) p[e] *= scale;
        }
    }
};

// Weights p of one row (the bonus after every draft was accepted, a leaf).
template <int DT>
struct TargetWeights {
    struct Raw { Raw8<DT> p; };
    ProbRow<DT> p;
    int64_t V;
    __device__ __forceinline__ void load(int64_t j0, Raw& r) const { load_group<DT>(p.row, j0, V, p.vec, r.p); }
    __device__ __forceinline__ void weights(const Raw& r, int64_t j0, float w[kLaneElems]) const { p.probs(r.p, j0, w); }
};

// Weights of p with one token removed: max(p - onehot(x), 0), the residual
// when the draft has no probabilities and q is the point mass at the drafted
// token x [Speculative Decoding (dl-note), Appendix "Implementation Details"].
template <int DT>
struct ExcludeWeights {
    struct Raw { Raw8<DT> p; };
    ProbRow<DT> p;
    int64_t V;
    int64_t x;
    __device__ __forceinline__ void load(int64_t j0, Raw& r) const { load_group<DT>(p.row, j0, V, p.vec, r.p); }
    __device__ __forceinline__ void weights(const Raw& r, int64_t j0, float w[kLaneElems]) const {
        p.probs(r.p, j0, w);
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e)
            if (j0 + e == x) w[e] = 0.0f;
    }
};

// Weights max(p - coef * q, 0): the chain residual (coef = 1) and the MSS
// residual after rejections (coef = c_j of the tree kernel's recurrence).
template <int DT, bool kScaledQ = false>
struct ResidualWeights {
    struct Raw { Raw8<DT> p, q; };
    ProbRow<DT> p;
    ProbRow<DT, kScaledQ> q;
    float coef;
    int64_t V;
    __device__ __forceinline__ void load(int64_t j0, Raw& r) const {
        load_group<DT>(p.row, j0, V, p.vec, r.p);
        load_group<DT>(q.row, j0, V, q.vec, r.q);
    }
    __device__ __forceinline__ void weights(const Raw& r, int64_t j0, float w[kLaneElems]) const {
        float a[kLaneElems], b[kLaneElems];
        p.probs(r.p, j0, a);
        q.probs(r.q, j0, b);
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) w[e] = fmaxf(fmaf(-coef, b[e], a[e]), 0.0f);
    }
};

// Pass A over tiles [t_lo, t_hi): per-tile sums of the weights (fp32), handed
// to sink(t, sum) by lane 0 of the wave that summed the tile. Every wave keeps
// TIF tiles' loads in flight (more is faster for a lone workgroup; fewer keeps
// the registers of a kernel that also streams rows low).
template <int TIF = kTilesInFlight, class WFn, class Sink>
__device__ __forceinline__ void weight_tile_range(const WFn& f, int t_lo, int t_hi, Sink sink) {
    for (int t0 = t_lo + wave_id() * TIF; t0 < t_hi; t0 += kWaves * TIF) {
        typename WFn::Raw raw[TIF];
#pragma unroll
        for (int u = 0; u < TIF; ++u)
            if (t0 + u < t_hi) f.load(int64_t(t0 + u) * kTileElems + lane_id() * kLaneElems, raw[u]);
#pragma unroll
        for (int u = 0; u < TIF; ++u) {
            if (t0 + u >= t_hi) break;
            float w[kLaneElems];
            f.weights(raw[u], int64_t(t0 + u) * kTileElems + lane_id() * kLaneElems, w);
            const float ls = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
            const float ts = wave_sum(ls);
            if (lane_id() == 0) sink(t0 + u, ts);
        }
    }
}

// Total of the tile sums in fp64 (whole workgroup; tile_sum in LDS).
__device__ __forceinline__ double tiles_total(const float* tile_sum, int ntiles) {
    __shared__ double s_total;
    __syncthreads();
    if (wave_id() == 0) {
        double ps = 0.0;
        for (int t = lane_id(); t < ntiles; t += kWaveSize) ps += tile_sum[t];
        ps = wave_sum(ps);
        if (lane_id() == 0) s_total = ps;
    }
    __syncthreads();
    return s_total;
}

// Pass A over the whole row by one workgroup: tile sums into LDS, and their
// total.
template <int TIF = kTilesInFlight, class WFn>
__device__ __forceinline__ double weight_tiles(const WFn& f, int64_t V, float* tile_sum) {
    const int ntiles = int((V + kTileElems - 1) / kTileElems);
    weight_tile_range<TIF>(f, 0, ntiles, [&](int t, float ts) { tile_sum[t] = ts; });
    return tiles_total(tile_sum, ntiles);
}

// A tile sum published to another workgroup: one 64-bit word, hi = 1 so that
// a published word is never 0 (0 = not yet written), lo = the fp32 bits.
__device__ __forceinline__ uint64_t pack_tile(float ts) { return (1ull << 32) | uint64_t(__float_as_uint(ts)); }
__device__ __forceinline__ float tile_of(uint64_t w) { return __uint_as_float(uint32_t(w)); }

// The element of tile `tile` at which the running sum of f's weights over the
// tile first reaches tin; rounding past the tile's scanned total takes its
// last positive element. Wave 0 computes; whole workgroup.
template <class WFn>
__device__ __forceinline__ int32_t sample_in_tile(const WFn& f, int tile, double tin) {
    __shared__ int32_t s_idx;
    const int lane = lane_id();
    if (wave_id() == 0) {
        typename WFn::Raw raw;
        f.load(int64_t(tile) * kTileElems + lane * kLaneElems, raw);
        float w[kLaneElems];
        f.weights(raw, int64_t(tile) * kTileElems + lane * kLaneElems, w);
        double ls = 0.0;
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) ls += double(w[e]);
        const double incl = wave_inclusive_scan(ls);
        double acc = __shfl_up(incl, 1);
        if (lane == 0) acc = 0.0;
        int fe = -1, le = -1;
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) {
            acc += double(w[e]);
            if (fe < 0 && w[e] > 0.0f && acc >= tin) fe = e;
            if (w[e] > 0.0f) le = e;
        }
        const uint64_t m = __ballot(fe >= 0);
        int32_t idx;
        if (m != 0) {
            const int L = __builtin_ctzll(m);
            idx = tile * kTileElems + L * kLaneElems + __shfl(fe, L);
        } else {  // rounding: v*W fell past the tile's scanned total; take its last positive element
            const uint64_t m2 = __ballot(le >= 0);
            const int L = 63 - __builtin_clzll(m2);
            idx = tile * kTileElems + L * kLaneElems + __shfl(le, L);
        }
        if (lane == 0) s_idx = idx;
    }
    __syncthreads();
    return s_idx;
}

// The tile of tile_sum[0..n) (fp32 sums of consecutive tiles) at which a
// running fp64 sum that starts at `base` first reaches `target`, counting
// positive tiles only, and the remainder of the target inside it (*tin).
// Rounding that leaves the target past the last tile takes the last positive
// tile. -1 when no tile is positive. Wave 0 computes; whole workgroup.
__device__ __forceinline__ int find_tile(const float* tile_sum, int n, double base, double target, double* tin) {
    __shared__ int32_t s_tile;
    __shared__ double s_tin;
    const int lane = lane_id();
    if (wave_id() == 0) {
        const int seg = (n + kWaveSize - 1) / kWaveSize;
        const int t0 = lane * seg;
        const int t1 = min(n, t0 + seg);
        double ps = 0.0;
        bool pos = false;
        for (int t = t0; t < t1; ++t) { ps += tile_sum[t]; pos = pos || tile_sum[t] > 0.0f; }
        const double incl = base + wave_inclusive_scan(ps);
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = base;
        const uint64_t m = __ballot(pos && incl >= target);
        const uint64_t mp = __ballot(pos);
        int tile = -1;
        double rem = 0.0;
        if (mp != 0) {
            const int L = m != 0 ? __builtin_ctzll(m) : 63 - __builtin_clzll(mp);
            if (lane == L) {
                double acc = excl;
                for (int t = t0; t < t1; ++t) {
                    const float ts = tile_sum[t];
                    const double nx = acc + double(ts);
                    if (ts > 0.0f && nx >= target) { tile = t; rem = target - acc; break; }
                    acc = nx;
                }
                if (tile < 0) {  // rounding left the target past this segment: its last positive tile
                    for (int t = t1 - 1; t >= t0; --t)
                        if (tile_sum[t] > 0.0f) { tile = t; rem = double(tile_sum[t]); break; }
                }
            }
            tile = __shfl(tile, L);
            rem = __shfl(rem, L);
        }
        if (lane == 0) { s_tile = tile; s_tin = rem; }
    }
    __syncthreads();
    *tin = s_tin;
    return s_tile;
}

// Pass B: given the tile sums of pass A, the smallest j with S_j >= v * W.
// Returns -1 when the total is 0.
template <class WFn>
__device__ __forceinline__ int32_t sample_from_tiles(const WFn& f, int64_t V, float v, const float* tile_sum) {
    const int ntiles = int((V + kTileElems - 1) / kTileElems);
    const int lane = lane_id();
    __shared__ int32_t s_tile;
    __shared__ double s_tin;
    if (wave_id() == 0) {
        const int seg = (ntiles + kWaveSize - 1) / kWaveSize;
        const int t0 = lane * seg;
        const int t1 = min(ntiles, t0 + seg);
        double ps = 0.0;
        for (int t = t0; t < t1; ++t) ps += tile_sum[t];
        const double incl = wave_inclusive_scan(ps);
        const double W = __shfl(incl, kWaveSize - 1);
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0;
        const double target = double(v) * W;
        const uint64_t m = __ballot(W > 0.0 && incl >= target);
        int tile = -1;
        double tin = 0.0;
        if (m != 0) {
            const int L = __builtin_ctzll(m);
            if (lane == L) {
                double acc = excl;
                for (int t = t0; t < t1; ++t) {
                    const float ts = tile_sum[t];
                    const double nx = acc + double(ts);
                    if (ts > 0.0f && nx >= target) { tile = t; tin = target - acc; break; }
                    acc = nx;
                }
                if (tile < 0) {  // rounding left v*W past this segment: take its last positive tile
                    for (int t = t1 - 1; t >= t0; --t)
                        if (tile_sum[t] > 0.0f) { tile = t; tin = double(tile_sum[t]); break; }
                }
            }
            tile = __shfl(tile, L);
            tin = __shfl(tin, L);
        }
        if (lane == 0) { s_tile = tile; s_tin = tin; }
    }
    __syncthreads();
    const int tile = s_tile;
    return tile >= 0 ? sample_in_tile(f, tile, s_tin) : -1;
}

}  // namespace specv
