// Workgroup-level pieces of the resolve step of the verification kernels:
// collecting the published row statistics, block merges, and inverse-CDF
// sampling from a row of non-negative weights.
//
// Inverse CDF [reading of Lecture 5: Speculative Decoding and SpecInfer, sec.
// 2.2 step 4 / Speculative Decoding (dl-note), sec. 2.3]: the sample is the
// smallest index j with w_0 + ... + w_j >= v * W, W = sum of all weights.
// Two passes over the row: (A) the waves sum 512-element tiles (64 lanes x 8
// consecutive elements), several tiles in flight per wave, in fp64; (B) wave
// 0 scans the tile sums in fp64 to find the tile that holds v*W, recomputes
// that tile's weights (the same values as pass A) and scans them for the
// index. Only the one row (pair) that needs a sample is read a second time.
//
// Accuracy. A draw agrees with the exact one unless v*W lies within the
// weights' relative error of a bucket edge, so every weight is computed with
// an error relative to itself of a few 1e-7, whatever the row:
//  * p = 2^(z*c - B) with t = z*c - B formed in fp64 and split as n + f,
//    |f| <= 1/2, so the fp32 exponential sees a small argument;
//  * the residual max(p - q, 0) = p * max(0, 1 - 2^h), h = log2(q/p), is
//    never formed as a difference of two probabilities: h is formed in fp64
//    from the two logits, and 1 - 2^h by a series where |h| < 1;
//  * the ratio of the two rows' normalisers, which enters every h, is known
//    from the streaming pass only to ~1e-7 relative (fp32 terms), an error
//    that would shift W by ~1e-7 absolute, far above 1e-7 * W when W is
//    small. Pass A therefore also measures the correction: with the
//    streaming normalisers, sum_x p(x) 2^h(x) = 2^kappa should be 1, and
//    kappa = log2(1 + sum p (2^h - 1)) is accumulated from terms p * (2^h -
//    1) whose errors are relative to |p - q|, hence bounded by ~1e-7 * W.
//    The corrected weights are p * max(0, 1 - 2^(h - kappa)), i.e. for every
//    element with h < 0: w~ + a * q~ with w~ = p (1 - 2^h), q~ = p 2^h and
//    a = 1 - 2^-kappa (exact, not a linearisation), so the pass keeps the
//    tile sums of w~ and q~ and applies a once kappa is known. Elements whose
//    sign of h - kappa differs from that of h (|h| < |kappa| ~ 1e-7) are off
//    by at most p * |kappa|.
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

// ------------------------------------------------------------ scheduling
//
// Two launch disciplines, neither of which depends on the order in which the
// hardware starts workgroups or on what else runs on the GPU.
//
// Chain launches (verify, fused top-F, ragged): workgroup g runs task g of a
// fixed map (decode_chain, decode_fused) that puts a sequence's bonus tasks
// after the row tasks whose words they read, so in practice their waits are
// short. Every wait is bounded (kRescueTicks); a bonus task whose wait runs
// out gives up and marks its sequence deferred, and a second launch on the
// same stream (the finisher) resolves the deferred sequences. By then every
// workgroup of the first launch has finished, so the finisher never waits.
// No workgroup ever needs another one to start: the first launch drains in
// bounded time, the finisher has nothing to wait for, and the outcome is the
// same as without the deferral. The launch needs no shared counter, which
// would be one atomic per workgroup on one address, all of them at once
// when the launch starts.
//
// Tree launches: the walkers of a tree exchange totals on every pass and
// cannot stand in for one another, so they need each other running. Each
// workgroup takes its task number from a ticket counter in the workspace
// when it starts (TaskQueue), so tasks are numbered in the order in which
// workgroups actually start. A task waits only for tasks with smaller
// numbers, which a running workgroup has claimed, or for the other walkers
// of its tree, whose numbers are consecutive: by induction from the
// smallest unfinished task, the launch drains whatever the start order.

struct TaskQueue {
    uint64_t* ticket;
    int64_t n;          // tasks (n >= 1)
    // Claim by thread 0 (the caller broadcasts it). The wrapping increment
    // hands out old and stores (old >= n - 1 ? 0 : old + 1): the claim of
    // n - 1 leaves the counter at zero for the next launch, with no store
    // that could race a claim. A counter found at n or above (a workspace
    // that was not zeroed) is wrapped to zero by that same claim, which then
    // claims again; from then on every stored value is below n, so the
    // second claim is in range. The result is clamped all the same: a task
    // number is always in [0, n).
    __device__ __forceinline__ int64_t claim() const {
        const uint64_t last = uint64_t(n - 1);
        uint64_t t = __builtin_amdgcn_atomic_inc64(ticket, last, __ATOMIC_RELAXED, "agent");
        if (t > last) t = __builtin_amdgcn_atomic_inc64(ticket, last, __ATOMIC_RELAXED, "agent");
        return int64_t(t < last ? t : last);
    }
};

// One task per workgroup of a tree launch, its number taken from the ticket
// counter when the workgroup starts: the launch has exactly n workgroups, so
// its claims are 0 .. n - 1 and leave the counter at zero.
__device__ __forceinline__ int64_t claim_one(uint64_t* ticket, int64_t n) {
    __shared__ int64_t s_task;
    if (threadIdx.x == 0) s_task = TaskQueue{ticket, n}.claim();
    __syncthreads();
    return uniform_i64(s_task);
}

// Dispatch order of the sequences of a chain launch: T > 0 first, then the
// greedy ones, each group by increasing index (identity when B >
// kMaxOrderedBatch): only T > 0 sequences re-read a row to draw the bonus, so
// their bonus tasks come early and overlap the greedy sequences' rows. A
// workgroup builds the order once (one ballot per 64 temperatures) and maps
// each task's sequence slot to its sequence.
struct SeqOrder {
    static constexpr int kKeptTemps = 256;          // batches up to this keep their temperatures here
    uint64_t masks[kMaxOrderedBatch / kWaveSize];   // bit b: sequence b has T > 0
    float temps[kKeptTemps];
    int nS;                                          // T > 0 sequences (B when not ordered)
    int B;
    bool ordered;
    // Whole workgroup (wave 0 reads the temperatures). Up to kKeptTemps
    // sequences, every lane issues its kKeptTemps / 64 loads before any is
    // used, so the placement costs one memory round trip (a loop that used
    // each chunk before loading the next took one round trip per 64
    // sequences); larger batches take the loop. `pre` runs in wave 0 after
    // those loads are issued and before they are used: a caller's own loads
    // issued there share the round trip.
    template <class Pre>
    __device__ __forceinline__ void init(const float* temperature, int B_, Pre pre) {
        if (wave_id() == 0) {
            const int lane = lane_id();
            const bool ord = B_ <= kMaxOrderedBatch;
            int nseq = B_;
            if (ord && B_ <= kKeptTemps) {
                constexpr int kChunks = kKeptTemps / kWaveSize;
                float t[kChunks];
#pragma unroll
                for (int c = 0; c < kChunks; ++c) {   // unconditional loads, clamped index
                    const int i = c * kWaveSize + lane;
                    t[c] = temperature[i < B_ ? i : B_ - 1];
                }
                pre();
                nseq = 0;
#pragma unroll
                for (int c = 0; c < kChunks; ++c) {
                    const int i = c * kWaveSize + lane;
                    const float tc = i < B_ ? t[c] : 0.0f;
                    if (i < B_) temps[i] = tc;
                    const uint64_t m = __ballot(tc > 0.0f);
                    if (lane == 0) masks[c] = m;
                    nseq += __popcll(m);
                }
            } else {
                pre();
                if (ord) {
                    nseq = 0;
                    const int nm = (B_ + kWaveSize - 1) / kWaveSize;
                    for (int c = 0; c < nm; ++c) {
                        const int i = c * kWaveSize + lane;
                        const float t = i < B_ ? temperature[i] : 0.0f;
                        const uint64_t m = __ballot(t > 0.0f);
                        if (lane == 0) masks[c] = m;
                        nseq += __popcll(m);
                    }
                }
            }
            if (lane == 0) { nS = nseq; B = B_; ordered = ord; }
        }
        __syncthreads();
    }
    __device__ __forceinline__ void init(const float* temperature, int B_) {
        init(temperature, B_, [] {});
    }
    // Sequence b's temperature: from LDS when init kept it (no second
    // round trip to memory before the task can start), else from memory.
    __device__ __forceinline__ float temperature_of(const float* temperature, int b) const {
        const float t = (ordered && B <= kKeptTemps) ? temps[b] : temperature[b];
        return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t)));
    }
    // The sequence in slot sidx. Whole wave (the same in every lane).
    __device__ __forceinline__ int seq_wave(int sidx) const {
        if (!ordered) return sidx;
        const bool sampled = sidx < nS;
        int k = sampled ? sidx : sidx - nS;
        const int nm = (B + kWaveSize - 1) / kWaveSize;
        for (int c = 0; c < nm; ++c) {
            uint64_t m = sampled ? masks[c] : ~masks[c];
            const int valid = min(kWaveSize, B - c * kWaveSize);
            if (valid < kWaveSize) m &= (1ull << valid) - 1ull;
            const int cnt = __popcll(m);
            if (k < cnt) {   // the k-th set bit of m
                const bool bit = (m >> lane_id()) & 1ull;
                const uint64_t hit = __ballot(bit && lanes_below(m) == k);
                return c * kWaveSize + __builtin_ctzll(hit);
            }
            k -= cnt;
        }
        return sidx;
    }
};

// Where a task of a chain launch sits: its sequence slot, its index in that
// slot's tasks, and the sequence in the slot.
struct Placement {
    int sidx;
    int64_t w;
    int b;
};

// Placement of task t given decode(nS, sidx, w); wave 0 computes, the
// workgroup gets it through LDS (one barrier), as wave-uniform values (so
// that what is derived from them stays in scalar registers).
template <class Decode>
__device__ __forceinline__ Placement place_task(const SeqOrder& ord, Decode decode) {
    __shared__ Placement s_pl;
    if (wave_id() == 0) {
        int sidx;
        int64_t w;
        decode(ord.nS, sidx, w);
        const int b = ord.seq_wave(sidx);
        if (lane_id() == 0) s_pl = Placement{sidx, w, b};
    }
    __syncthreads();
    return Placement{__builtin_amdgcn_readfirstlane(s_pl.sidx), uniform_i64(s_pl.w),
                     __builtin_amdgcn_readfirstlane(s_pl.b)};
}

// Waits until the n pairs at p (2n words) all carry `tag` (wave 0 polls with
// agent-scope atomic loads, four loads per lane in flight), for at most
// `ticks`. Returns false if the bound was reached. Whole workgroup.
__device__ bool wait_pairs(const uint64_t* p, int64_t n, uint32_t tag, uint64_t ticks) {
    __shared__ int s_ok;
    if (wave_id() == 0) {
        int ok = 0;
        const int64_t nw = 2 * n;
        for (const WaitBound t(ticks); !t.expired();) {
            bool mine = true;
            int64_t i = 2 * lane_id();
            for (; i + 2 * kWaveSize < nw; i += 4 * kWaveSize) {
                const uint64_t a0 = peek(p + i), a1 = peek(p + i + 1);
                const uint64_t a2 = peek(p + i + 2 * kWaveSize), a3 = peek(p + i + 2 * kWaveSize + 1);
                mine &= pair_ok(a0, a1, tag) & pair_ok(a2, a3, tag);
            }
            for (; i < nw; i += 2 * kWaveSize) mine &= pair_ok(peek(p + i), peek(p + i + 1), tag);
            if (__all(mine)) { ok = 1; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane_id() == 0) s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

// wait_pairs for a few pairs (n <= kWaveSize) whose values are wanted too:
// lane i of wave 0 polls pair i, and the poll that finds them all tagged
// leaves their values in out[0, n) (LDS). A loop that read them one at a time
// afterwards would wait one memory round trip per pair. Whole workgroup;
// false if the bound was reached.
__device__ bool gather_pairs(const uint64_t* p, int n, uint32_t tag, uint64_t ticks, uint64_t* out) {
    __shared__ int s_ok;
    if (wave_id() == 0) {
        int ok = 0;
        const int i = lane_id();
        for (const WaitBound t(ticks); !t.expired();) {
            const uint64_t hi = i < n ? peek(p + 2 * i) : 0ull;
            const uint64_t lo = i < n ? peek(p + 2 * i + 1) : 0ull;
            if (__all(i >= n || pair_ok(hi, lo, tag))) {
                if (i < n) out[i] = pair_value(hi, lo);
                ok = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (i == 0) s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

// Returns n pairs (2n words) to zero, the workspace's resting state.
__device__ __forceinline__ void zero_pairs(uint64_t* p, int64_t n) {
    for (int64_t i = threadIdx.x; i < 2 * n; i += kThreads) clear_word(p + i);
}

// Merged statistics of one row (all chunks).
struct RowStats {
    float m;     // max logit (greedy: best logit)
    float mc;    // fp32 m * c
    int32_t idx; // greedy argmax
    double Z;    // sum of 2^(z*c - mc)
};

// A row's statistics from its one value (S = 1): what merging that value
// alone gives. Any thread.
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

// A row's statistics from its S <= 64 chunk values, chunk j's in lane j (the
// values of lanes >= S are ignored). Greedy: the largest (value, lowest
// index) over the chunks, an order-free maximum. Softmax: the largest chunk
// maximum m, then the chunks' sums rescaled to it, 2^(m_j c - m c), and added
// in the wave's fixed order, so that every workgroup that merges the same
// values gets the same bits. Whole wave (every lane active); the result is
// the same in every lane.
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

// log2 of a row's normaliser in the streaming pass's reference: p(x) =
// 2^(z*c - log2_norm).
__device__ __forceinline__ double log2_norm(const RowStats& st) { return double(st.mc) + log2(st.Z); }

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

// ------------------------------------------------------------ weights
//
// 2^t in fp32 for t <= ~1 with a relative error of about one fp32 rounding
// whatever |t|: t = n + f, n = rint(t), |f| <= 1/2, 2^t = 2^f * 2^n. (Formed
// as fp32 fma(z, c, -m c), t itself would carry an absolute rounding error
// of up to |t| * 2^-24, i.e. a relative error of |t| * 4e-8 in 2^t.)
__device__ __forceinline__ float exp2_reduced(double t) {
    t = fmax(t, -300.0);                   // 2^-300 is 0 in fp32 (keeps -inf out of rint)
    const double n = rint(t);
    return ldexpf(__builtin_amdgcn_exp2f(float(t - n)), int(n));
}

// 2^h - 1 with an error relative to itself of a few fp32 roundings: for
// |h| < 1 the series of e^x - 1 at x = h ln 2 (terms up to x^9 / 9!, a
// truncation below 1e-8 relative for |x| < ln 2); beyond, 2^h - 1 directly
// (|2^h - 1| >= 1/2 there). -inf gives -1.
__device__ __forceinline__ float exp2m1(float h) {
    const float x = h * 0.69314718055994531f;
    float s = 1.0f / 362880.0f;                 // 1/9!
    s = fmaf(s, x, 1.0f / 40320.0f);
    s = fmaf(s, x, 1.0f / 5040.0f);
    s = fmaf(s, x, 1.0f / 720.0f);
    s = fmaf(s, x, 1.0f / 120.0f);
    s = fmaf(s, x, 1.0f / 24.0f);
    s = fmaf(s, x, 1.0f / 6.0f);
    s = fmaf(s, x, 0.5f);
    s = fmaf(s, x, 1.0f);
    const float big = __builtin_amdgcn_exp2f(h) - 1.0f;
    return fabsf(h) < 1.0f ? x * s : big;
}

// Lane sums of one 8-element group as pass A needs them: of the weights w,
// of q (the residual's second term, 0 unless a correction is pending), and
// the lane's contributions to the correction sums p and pg.
struct GroupSums {
    float w = 0.0f, q = 0.0f, p = 0.0f, pg = 0.0f;
};

// Weights p of one row (the bonus after every draft was accepted, a leaf):
// p(x) = 2^(z*c - B), B = log2 of the row's normaliser. With `excl` >= 0 that
// token's weight is 0: the residual when the draft has no probabilities and q
// is the point mass at the drafted token [Speculative Decoding (dl-note),
// Appendix "Implementation Details"].
template <int DT>
struct TargetWeights {
    static constexpr bool kCorrected = false;
    struct Raw { Raw8<DT> p; };
    const void* row;
    double c, B;
    int64_t V;
    int64_t excl;
    bool vec;
    __device__ void init(const void* r, double c64, const RowStats& st, int64_t V_, int64_t excl_ = -1) {
        row = r; c = c64; B = log2_norm(st); V = V_; excl = excl_;
        vec = (reinterpret_cast<uintptr_t>(r) & 15u) == 0;
    }
    __device__ __forceinline__ void load(int64_t j0, Raw& r) const { load_group<DT>(row, j0, V, vec, r.p); }
    __device__ __forceinline__ void weights(const Raw& r, int64_t j0, float w[kLaneElems]) const {
        float z[kLaneElems];
        unpack8<DT>(r.p, z);
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) {
            const float p = exp2_reduced(fma(double(z[e]), c, -B));   // 0 for z = -inf
            w[e] = (j0 + e == excl) ? 0.0f : p;
        }
    }
    __device__ __forceinline__ void sums(const Raw& r, int64_t j0, GroupSums& g) const {
        float w[kLaneElems];
        weights(r, j0, w);
        g.w = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
    }
};

// Residual weights max(0, p - coef * q) = p * max(0, 1 - 2^h) with
// h = log2(coef * q / p) = (zq - zp) c + [top] log2 C - Hk: the chain residual
// (coef = 1) and the multi-step residual after rejections (coef = c_j of the
// tree walk's recurrence), q optionally Saguaro's sigma_{F,C} (its top-F
// elements, key >= top_key, carry C). Hk = B_q - B_p - log2(coef) (+ kappa,
// once known), B = log2 of each row's normaliser. With a pending correction
// (kCorrected use: a != 0 after kappa is known) the weight of an element with
// h < 0 is w~ + a q~ (see the file comment); pass A returns w~ and q~.
// kMeasure = false: the weights of a pass whose correction is already folded
// into Hk (a = 0): only w~, the same values bit for bit, without the terms of
// the correction sums and q~.
template <int DT, bool kTop = false, bool kMeasure = true>
struct ResidualWeights {
    static constexpr bool kCorrected = kMeasure;
    struct Raw { Raw8<DT> p, q; };
    const void* prow;
    const void* qrow;
    double c, Bp, Hk, log2C;
    uint64_t top_key;      // elements of q whose full key is >= this carry C (~0: none)
    int64_t V;
    bool pvec, qvec;
    float a;               // 1 - 2^-kappa: the correction applied to the weights (0: none)
    __device__ void init(const void* pr, const void* qr, double c64, const RowStats& sp, double Bq, double coef,
                         int64_t V_) {
        prow = pr; qrow = qr; c = c64; Bp = log2_norm(sp);
        Hk = Bq - Bp - log2(coef);
        log2C = 0.0; top_key = ~0ull; V = V_; a = 0.0f;
        pvec = (reinterpret_cast<uintptr_t>(pr) & 15u) == 0;
        qvec = (reinterpret_cast<uintptr_t>(qr) & 15u) == 0;
    }
    __device__ __forceinline__ void load(int64_t j0, Raw& r) const {
        load_group<DT>(prow, j0, V, pvec, r.p);
        load_group<DT>(qrow, j0, V, qvec, r.q);
    }
    // Element e of a group: w~ and q~ (0 unless h < 0), and its terms of the
    // correction sums, p and p (2^h - 1).
    __device__ __forceinline__ void element(float zp, float zq, int64_t j, double nq, float& wt, float& qt, float& p,
                                            float& pg) const {
        const bool top = kTop && full_key(zq, j) >= top_key;
        const double tp = fma(double(zp), c, -Bp);                   // log2 p~
        p = exp2_reduced(tp);                                         // 0 for zp = -inf
        double h = fma(double(zq) - double(zp), c, -Hk);             // log2(coef q / p)
        if (top) h += log2C;
        const float em1 = exp2m1(float(h));                          // 2^h - 1 (relative accuracy)
        wt = fmaxf(p * -em1, 0.0f);                                   // p (1 - 2^h) where h < 0
        qt = wt > 0.0f ? p - wt : 0.0f;
        pg = p * em1;                                                 // p (2^h - 1) = coef q~ - p
        // Where p is 0 (a -inf target logit, or below fp32's range) or 2^h
        // leaves fp32's range, p (2^h - 1) is coef q~ - p with q~ = 2^tq
        // formed directly (q's mass where p vanishes). Rare: a wave takes
        // this branch only if one of its lanes needs it.
        if (!(p > 0.0f && h < 120.0)) {
            double tq = fma(double(zq), c, nq);                       // log2 of coef q~
            if (top) tq += log2C;
            pg = exp2_reduced(tq) - p;
            if (!(p > 0.0f)) wt = qt = 0.0f;
        }
    }
    // w~ alone: p (1 - 2^h) where h < 0, else 0. Where p is 0 or 2^h leaves
    // fp32's range the product is 0 or not a number and fmaxf returns 0, as
    // element() does.
    __device__ __forceinline__ float light(float zp, float zq, int64_t j) const {
        const bool top = kTop && full_key(zq, j) >= top_key;
        const float p = exp2_reduced(fma(double(zp), c, -Bp));
        double h = fma(double(zq) - double(zp), c, -Hk);
        if (top) h += log2C;
        return fmaxf(p * -exp2m1(float(h)), 0.0f);
    }
    __device__ __forceinline__ void sums(const Raw& r, int64_t j0, GroupSums& g) const {
        float zp[kLaneElems], zq[kLaneElems];
        unpack8<DT>(r.p, zp);
        unpack8<DT>(r.q, zq);
        if constexpr (!kMeasure) {   // the same sum, in the same order, as below
#pragma unroll
            for (int e = 0; e < kLaneElems; ++e) g.w += light(zp[e], zq[e], j0 + e);
            return;
        }
        const double nq = -(Hk + Bp);                                // log2 q~ = zq c [+ log2 C] + nq
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) {
            float wt, qt, p, pg;
            element(zp[e], zq[e], j0 + e, nq, wt, qt, p, pg);
            g.w += wt;
            g.q += qt;
            g.p += p;
            g.pg += pg;
        }
    }
    // The weights of a pass B tile scan: w~ + a q~ on the elements with h < 0.
    __device__ __forceinline__ void weights(const Raw& r, int64_t j0, float w[kLaneElems]) const {
        float zp[kLaneElems], zq[kLaneElems];
        unpack8<DT>(r.p, zp);
        unpack8<DT>(r.q, zq);
        const double nq = -(Hk + Bp);
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) {
            float wt, qt, p, pg;
            element(zp[e], zq[e], j0 + e, nq, wt, qt, p, pg);
            w[e] = fmaxf(fmaf(a, qt, wt), 0.0f);
        }
    }
};

// Pass A over tiles [t_lo, t_hi): per tile the fp64 sums of w~ and q~,
// handed to sink(t, w_sum, q_sum) by lane 0 of the wave that summed the tile;
// the lane's contributions to sum p and sum p (2^h - 1) are added to psum and
// pgsum (fp64, per thread; corrected weights only). Every wave keeps TIF
// tiles' loads in flight (more is faster for a lone workgroup; fewer keeps
// the registers of a kernel that also streams rows low).
template <int TIF = kTilesInFlight, class WFn, class Sink>
__device__ __forceinline__ void weight_tile_range(const WFn& f, int t_lo, int t_hi, Sink sink, double& psum,
                                                  double& pgsum) {
    for (int t0 = t_lo + wave_id() * TIF; t0 < t_hi; t0 += kWaves * TIF) {
        typename WFn::Raw raw[TIF];
#pragma unroll
        for (int u = 0; u < TIF; ++u)
            if (t0 + u < t_hi) f.load(int64_t(t0 + u) * kTileElems + lane_id() * kLaneElems, raw[u]);
#pragma unroll
        for (int u = 0; u < TIF; ++u) {
            if (t0 + u >= t_hi) break;
            GroupSums g;
            f.sums(raw[u], int64_t(t0 + u) * kTileElems + lane_id() * kLaneElems, g);
            const double tw = wave_sum(double(g.w));
            double tq = 0.0;
            if (WFn::kCorrected) {
                tq = wave_sum(double(g.q));
                psum += double(g.p);
                pgsum += double(g.pg);
            }
            if (lane_id() == 0) sink(t0 + u, tw, tq);
        }
    }
}

// Workgroup totals (in a fixed order: wave sums, then the waves in order) of
// two per-thread fp64 values. Whole workgroup.
__device__ __forceinline__ void block_sum2(double& x, double& y) {
    __shared__ double sx[kWaves], sy[kWaves];
    x = wave_sum(x);
    y = wave_sum(y);
    if (lane_id() == 0) { sx[wave_id()] = x; sy[wave_id()] = y; }
    __syncthreads();
    x = sx[0];
    y = sy[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) { x += sx[w]; y += sy[w]; }
    __syncthreads();
}

// The correction of the file comment from the totals of sum p and
// sum p (2^h - 1): a = 1 - 2^-kappa, kappa = log2(1 + pg / p).
__device__ __forceinline__ double correction_kappa(double psum, double pgsum) {
    const double r = psum > 0.0 ? 1.0 + pgsum / psum : 0.0;
    return r > 0.0 ? log2(r) : 0.0;
}
__device__ __forceinline__ double correction_a(double kappa) { return 1.0 - exp2(-kappa); }

// Total of the tile sums in fp64 (whole workgroup; tile_sum in LDS).
__device__ __forceinline__ double tiles_total(const double* tile_sum, int ntiles) {
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
            if (m2 != 0) {
                const int L = 63 - __builtin_clzll(m2);
                idx = tile * kTileElems + L * kLaneElems + __shfl(le, L);
            } else {
                idx = -1;
            }
        }
        if (lane == 0) s_idx = idx;
    }
    __syncthreads();
    return s_idx;
}

// The tile of tile_sum[0..n) (fp64 sums of consecutive tiles) at which a
// running fp64 sum that starts at `base` first reaches `target`, counting
// positive tiles only, and the remainder of the target inside it (*tin).
// Rounding that leaves the target past the last tile takes the last positive
// tile. -1 when no tile is positive. Wave 0 computes; whole workgroup.
__device__ __forceinline__ int find_tile(const double* tile_sum, int n, double base, double target, double* tin) {
    __shared__ int32_t s_tile;
    __shared__ double s_tin;
    const int lane = lane_id();
    if (wave_id() == 0) {
        const int seg = (n + kWaveSize - 1) / kWaveSize;
        const int t0 = lane * seg;
        const int t1 = min(n, t0 + seg);
        double ps = 0.0;
        bool pos = false;
        for (int t = t0; t < t1; ++t) { ps += tile_sum[t]; pos = pos || tile_sum[t] > 0.0; }
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
                    const double ts = tile_sum[t];
                    const double nx = acc + ts;
                    if (ts > 0.0 && nx >= target) { tile = t; rem = target - acc; break; }
                    acc = nx;
                }
                if (tile < 0) {  // rounding left the target past this segment: its last positive tile
                    for (int t = t1 - 1; t >= t0; --t)
                        if (tile_sum[t] > 0.0) { tile = t; rem = tile_sum[t]; break; }
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

// Pass B: given the tile sums of pass A (total W), the smallest j with
// S_j >= v * W. Returns -1 when W is not positive.
template <class WFn>
__device__ __forceinline__ int32_t sample_from_tiles(const WFn& f, int64_t V, float v, const double* tile_sum,
                                                     double W) {
    if (!(W > 0.0)) return -1;
    const int ntiles = int((V + kTileElems - 1) / kTileElems);
    double tin = 0.0;
    const int tile = find_tile(tile_sum, ntiles, 0.0, double(v) * W, &tin);
    return tile >= 0 ? sample_in_tile(f, tile, tin) : -1;
}

}  // namespace specv
