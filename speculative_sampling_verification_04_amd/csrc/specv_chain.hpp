// Chain verification pieces shared by the verify kernel, the fused
// verify + top-F kernel and the ragged kernel [Lecture 5: Speculative Decoding
// and SpecInfer, sec. 2.2, 2.7, 3.1; Speculative Decoding (dl-note), sec.
// 2.2-2.3 and Appendix "Implementation Details"].
//
// After a sequence's row workgroups, H bonus workgroups are dispatched
// (h = 0 .. H-1). Each waits for the row statistics and decides the accepted
// prefix k on its own (the same arithmetic on the same words, so they agree).
// For a T > 0 sequence the bonus needs one more pass over a row pair (the
// residual max(p_t - p_d, 0) of row k) or a row (p_t of row gamma): with
// H > 1 workgroup h sums tiles [h*n/H, (h+1)*n/H) of it and publishes each
// tile sum as a self-validating word, so the pass runs H-wide instead of on
// one workgroup. The last one (h = H-1) collects the tile sums, draws the
// bonus, writes the outcome and returns the words it consumed to zero.
//
// Every wait is bounded. In the main launch a wait that runs out makes the
// last bonus workgroup mark the sequence deferred (its other workgroups just
// stop), and the finisher launch, which runs after every workgroup of the
// main launch has finished, resolves it with the same code (Finish = true):
// one workgroup that computes every helper's tiles itself, with the same
// arithmetic, so the outcome is the one the main launch would have given.

#pragma once

#include <type_traits>

#include "specv_launch.hpp"
#include "specv_sample.hpp"

namespace specv {

// Tiles in flight per wave in the bonus pass: the pass is spread over H
// workgroups, and it shares the kernel's register allocation with the
// streaming code, so one tile per wave keeps the streaming occupancy.
constexpr int kBonusTiles = 2;

__device__ __forceinline__ const void* row_ptr(const RowView& v, int esz, int64_t b, int64_t r) {
    return static_cast<const char*>(v.data) + (b * v.stride_seq + r * v.stride_row) * esz;
}

__device__ __forceinline__ float log2e_over(float T) { return float(1.4426950408889634 / double(T)); }

// One sequence as the resolve step sees it.
struct SeqView {
    int b;                   // sequence index: Philox counter and per-sequence outputs
    int gamma;               // its number of draft tokens
    int G;                   // layout: target rows at words 0..G, draft rows at G+1+i
    const int32_t* tokens;   // its gamma draft tokens
    const char* trow;        // target row i at trow + i * tstride (bytes)
    int64_t tstride;
    const char* drow;        // draft row i at drow + i * dstride (null: no draft probabilities)
    int64_t dstride;
    int32_t* out_tokens;     // out_len entries: accepted tokens, the bonus, then -1
    int out_len;
    float* out_probs;        // gamma x 2, or null
    __device__ __forceinline__ const void* target(int i) const { return trow + i * tstride; }
    __device__ __forceinline__ const void* draft(int i) const { return drow + i * dstride; }
};

// The view of sequence b in the dense [B][rows][V] layout of specv_verify and
// specv_verify_topk.
template <int DT>
__device__ __forceinline__ SeqView dense_seq(const ChainArgs& a, int b) {
    constexpr int esz = ElemT<DT>::kBytes;
    SeqView q;
    q.b = b;
    q.gamma = a.gamma;
    q.G = a.gamma;
    q.tokens = a.tokens + int64_t(b) * a.gamma;
    q.trow = static_cast<const char*>(row_ptr(a.target, esz, b, 0));
    q.tstride = a.target.stride_row * esz;
    q.drow = static_cast<const char*>(row_ptr(a.draft, esz, b, 0));
    q.dstride = a.draft.stride_row * esz;
    q.out_tokens = a.out_tokens + int64_t(b) * (a.gamma + 1);
    q.out_len = a.gamma + 1;
    q.out_probs = a.out_probs ? a.out_probs + int64_t(b) * a.gamma * 2 : nullptr;
    return q;
}

// LDS of one bonus workgroup. A kernel whose row workgroups need LDS of their
// own may overlay the two (a workgroup is one or the other). The tile sums
// live in the launch's dynamic LDS (TileLds), sized by the vocabulary.
struct ResolveLds {
    RowStats st[2 * 64 + 1];
};

// Per-tile sums of the bonus pass in dynamic LDS: w (fp64, the corrected
// tile sums in the end) and q (the residual's second term, fp32: it only
// carries the correction, ~1e-7 of a tile, so its own rounding is
// immaterial).
struct TileLds {
    double* w;
    float* q;
};

extern __shared__ __align__(16) char specv_dyn_lds[];

// The dynamic LDS bytes a chain launch needs for `ntiles` tiles.
inline size_t tile_lds_bytes(int64_t ntiles) { return size_t(ntiles) * (sizeof(double) + sizeof(float)) + 16; }

__device__ __forceinline__ TileLds tile_lds(int ntiles) {
    double* w = reinterpret_cast<double*>(specv_dyn_lds);
    return TileLds{w, reinterpret_cast<float*>(w + ntiles)};
}

// Bonus workgroup h of a sequence. slots: the sequence's nslots pairs (row r
// chunk j at pair r * S + j: target row r for r <= G, draft row r - G - 1
// after that; then, with a.cache_words, three cache pairs per draft row from
// pair (2G + 2) * S). tiles: its tile pairs (two per tile: the sums of w~ and
// q~) and parts: its helpers' pairs (two per helper: sum p and sum p (2^h -
// 1)), used when H > 1. mark: the sequence's deferral pair. NoDraft: the
// draft has no probabilities (q is the point mass at the drafted token).
// Cache: the cache pairs exist (a.cache_words; specv_verify_cache only).
// Finish: the finisher's resolve of a deferred sequence (h = H - 1; every
// word it reads is already published).
template <int DT, bool NoDraft = false, bool Cache = false, bool Finish = false>
__device__ __forceinline__ void chain_resolve(const ChainArgs& a, const SeqView& q, float T, uint64_t* slots,
                                              int64_t nslots, uint64_t* tiles, uint64_t* parts, uint64_t* mark,
                                              int h, ResolveLds& lds) {
    const int b = q.b;
    const int gamma = q.gamma;
    const int G = q.G;
    const int R = NoDraft ? G + 1 : 2 * G + 1;   // rows to merge
    const bool greedy = !(T > 0.0f);
    const bool last = h == a.H - 1;
    const float c = greedy ? 0.0f : log2e_over(T);
    const double c64 = greedy ? 0.0 : 1.4426950408889634 / double(T);   // the bonus weights' exponent scale
    const uint32_t ep = a.epoch;
    const uint64_t* extra = slots + 2 * int64_t(2 * G + 2) * a.S;  // the cache pairs, when a.cache_words

    if (greedy && !last) return;  // the greedy bonus is an argmax: nothing to share

    RowStats* st = lds.st;
    const int ntiles = int((int64_t(a.V) + kTileElems - 1) / kTileElems);
    const TileLds tl = tile_lds(ntiles);
    __shared__ int32_t s_k;
    __shared__ int32_t s_bonus;
    __shared__ float s_mass;
    __shared__ uint64_t s_cache_word;

    const uint64_t ticks = Finish ? kMaxWaitTicks : a.wait_ticks;
    // A wait that ran out: the main launch defers the sequence; the
    // finisher, for which every word is already published, reports -1 (not
    // expected) and returns the words to zero.
    auto give_up = [&]() {
        if (!last) return;
        if (Finish) {
            if (threadIdx.x == 0) a.out_nacc[b] = -1;
            zero_pairs(slots, nslots);
            if (tiles) zero_pairs(tiles, 2 * int64_t(ntiles));
            if (parts) zero_pairs(parts, 2 * int64_t(a.H));
        } else if (threadIdx.x == 0) {
            publish_pair(mark, 1ull, ep);
        }
    };
    // The accept tests' inputs that the caller provides (the drafted tokens
    // and the logits at them) are loaded before the wait for the rows'
    // words, by the lanes that use them, so the two dependent round trips
    // overlap the wait instead of following it.
    int32_t pre_x = -1;
    float pre_zt = -INFINITY, pre_zd = -INFINITY;
    if (wave_id() == 0 && lane_id() < gamma) {
        pre_x = q.tokens[lane_id()];
        if (!greedy && pre_x >= 0 && pre_x < a.V) {
            pre_zt = load_elem<DT>(q.target(lane_id()), pre_x);
            if (!NoDraft) pre_zd = load_elem<DT>(q.draft(lane_id()), pre_x);
        }
    }
    if (!wait_pairs(slots, nslots, ep, ticks)) {
        give_up();
        return;
    }
    // One value per row: thread r reads row r's. Several: row r's S chunk
    // values are merged by one wave, four rows per wave at a time, with all
    // their loads in flight together.
    constexpr int kRowsPerStep = 4;
    if (a.S == 1) {
        for (int r = threadIdx.x; r < R; r += kThreads)
            st[r] = (greedy && r > G) ? RowStats{-INFINITY, -INFINITY, -1, 0.0} : stats_of_word(read_pair(slots, r), greedy, c);
    }
    for (int r0 = wave_id(); a.S > 1 && r0 < R; r0 += kRowsPerStep * kWaves) {
        uint64_t wv[kRowsPerStep];
#pragma unroll
        for (int j = 0; j < kRowsPerStep; ++j) {
            const int r = r0 + j * kWaves;
            const bool need = r < R && !(greedy && r > G) && lane_id() < a.S;
            wv[j] = need ? read_pair(slots, int64_t(r) * a.S + lane_id()) : 0ull;
        }
#pragma unroll
        for (int j = 0; j < kRowsPerStep; ++j) {
            const int r = r0 + j * kWaves;
            if (r >= R) break;
            const RowStats x = (greedy && r > G) ? RowStats{-INFINITY, -INFINITY, -1, 0.0}
                                                 : merge_chunk_words(wv[j], a.S, greedy, c);
            if (lane_id() == 0) st[r] = x;
        }
    }
    __syncthreads();

    // Accept tests: lane i of wave 0 takes position i.
    if (wave_id() == 0) {
        const int i = lane_id();
        bool reject = false;
        if (i < gamma) {
            const int32_t x = pre_x;
            const bool in_range = x >= 0 && x < a.V;
            float pt_out = 0.0f, pd_out = 1.0f;
            if (greedy) {
                const bool acc = in_range && x == st[i].idx;
                pt_out = acc ? 1.0f : 0.0f;
                reject = !acc;
            } else {
                double pt = 0.0, pd = 0.0;
                if (in_range) {
                    pt = prob_of(pre_zt, c, st[i]);
                    if (NoDraft) {
                        pd = 1.0;
                    } else {
                        const float zd = pre_zd;
                        RowStats qs = st[G + 1 + i];
                        double scale = 1.0;
                        if (Cache) {  // Saguaro sampling: q = sigma_{F_i,C}(draft_i / T)
                            const uint64_t zw = read_pair(extra, 3 * i);
                            if ((zw >> 32) == 1ull) {
                                qs.Z = double(__uint_as_float(uint32_t(zw)));
                                if (full_key(zd, x) >= read_pair(extra, 3 * i + 1)) scale = double(a.C);
                            }
                        }
                        pd = scale * prob_of(zd, c, qs);
                    }
                }
                const float u = stream_uniform(a.seed, a.offset, uint32_t(b), 0u, uint32_t(i));
                reject = !(pd > 0.0 && double(u) <= pt / (double(a.lenience) * pd));
                pt_out = float(pt);
                pd_out = float(pd);
            }
            if (last && q.out_probs) {
                q.out_probs[i * 2 + 0] = pt_out;
                q.out_probs[i * 2 + 1] = pd_out;
            }
        }
        const uint64_t rej = __ballot(reject);
        if (lane_id() == 0) s_k = rej ? __builtin_ctzll(rej) : gamma;
    }
    __syncthreads();
    const int k = s_k;

    if (greedy) {
        if (threadIdx.x == 0) { s_bonus = st[k].idx; s_mass = 1.0f; }
    } else {
        const float v = stream_uniform(a.seed, a.offset, uint32_t(b), 0u, uint32_t(gamma));
        // The bonus weights: the residual of row k (corrected, see
        // specv_sample.hpp), p_t of row k without the drafted token (no draft
        // probabilities), or p_t of row gamma when every draft was accepted.
        const bool resid = k < gamma && !NoDraft;
        TargetWeights<DT> tgt;
        tgt.init(q.target(k), c64, st[k], a.V, (NoDraft && k < gamma) ? int64_t(q.tokens[k]) : int64_t(-1));
        ResidualWeights<DT, Cache> res;
        if (resid) {
            if constexpr (!NoDraft) {
                const RowStats& qs = st[G + 1 + k];
                double Bq = log2_norm(qs);
                uint64_t top_key = ~0ull;
                if (Cache) {
                    const uint64_t zw = read_pair(extra, 3 * k);
                    if ((zw >> 32) == 1ull) {
                        Bq = double(qs.mc) + log2(double(__uint_as_float(uint32_t(zw))));
                        top_key = read_pair(extra, 3 * k + 1);
                    }
                }
                res.init(q.target(k), q.draft(k), c64, st[k], Bq, 1.0, a.V);
                res.top_key = top_key;
                res.log2C = log2(double(a.C));
            }
        }

        // Pass A: the tile sums (this workgroup's share when H > 1) and the
        // correction sums.
        double ps = 0.0, pgs = 0.0;
        if (a.H > 1) {
            // Helper j's share: its tiles' pairs and its correction sums.
            auto helper = [&](int j) {
                const int lo = int(int64_t(ntiles) * j / a.H);
                const int hi = int(int64_t(ntiles) * (j + 1) / a.H);
                double s0 = 0.0, s1 = 0.0;
                auto put = [&](int t, double tw, double tq) {
                    publish_pair(tiles + 4 * t, pack_f64(tw), ep);
                    publish_pair(tiles + 4 * t + 2, pack_f64(tq), ep);
                };
                if (resid) weight_tile_range<kBonusTiles>(res, lo, hi, put, s0, s1);
                else weight_tile_range<kBonusTiles>(tgt, lo, hi, put, s0, s1);
                if (resid) {
                    block_sum2(s0, s1);
                    if (threadIdx.x == 0) {
                        publish_pair(parts + 4 * j, pack_f64(s0), ep);
                        publish_pair(parts + 4 * j + 2, pack_f64(s1), ep);
                    }
                }
            };
            if (Finish) {
                for (int j = 0; j < a.H; ++j) helper(j);
            } else {
                helper(h);
            }
            // Each helper read the row values before publishing its tiles, so
            // once every tile pair is seen the row pairs may be zeroed.
            if (!last) return;
            __shared__ uint64_t s_parts[2 * kMaxBonusHelpers];
            const bool ok = wait_pairs(tiles, 2 * int64_t(ntiles), ep, ticks) &&
                            (!resid || gather_pairs(parts, 2 * a.H, ep, ticks, s_parts));
            if (!ok) {
                give_up();
                return;
            }
            if (resid) {  // the helpers' correction sums, in helper order
                for (int j = 0; j < a.H; ++j) {
                    ps += unpack_f64(s_parts[2 * j]);
                    pgs += unpack_f64(s_parts[2 * j + 1]);
                }
            }
            const double ca = resid ? correction_a(correction_kappa(ps, pgs)) : 0.0;
            for (int t = threadIdx.x; t < ntiles; t += kThreads)
                tl.w[t] = unpack_f64(read_pair(tiles, 2 * t)) + ca * unpack_f64(read_pair(tiles, 2 * t + 1));
            __syncthreads();
            zero_pairs(tiles, 2 * int64_t(ntiles));
            if (resid) zero_pairs(parts, 2 * int64_t(a.H));
            res.a = float(ca);
        } else {
            auto put = [&](int t, double tw, double tq) { tl.w[t] = tw; tl.q[t] = float(tq); };
            if (resid) weight_tile_range<kBonusTiles>(res, 0, ntiles, put, ps, pgs);
            else weight_tile_range<kBonusTiles>(tgt, 0, ntiles, put, ps, pgs);
            if (resid) block_sum2(ps, pgs);
            __syncthreads();
            const double ca = resid ? correction_a(correction_kappa(ps, pgs)) : 0.0;
            if (resid) {
                for (int t = threadIdx.x; t < ntiles; t += kThreads) tl.w[t] += ca * double(tl.q[t]);
            }
            res.a = float(ca);
        }
        const double total = tiles_total(tl.w, ntiles);

        int32_t bonus = -1;
        float mass = 0.0f;
        if (total > 0.0) {
            bonus = resid ? sample_from_tiles(res, a.V, v, tl.w, total) : sample_from_tiles(tgt, a.V, v, tl.w, total);
            mass = float(total);
        }
        if (bonus < 0) {  // a residual of zero mass (rounding only): p_t of row k
            TargetWeights<DT> pk;
            pk.init(q.target(k), c64, st[k], a.V);
            double x0 = 0.0, x1 = 0.0;
            weight_tile_range<kBonusTiles>(pk, 0, ntiles, [&](int t, double tw, double) { tl.w[t] = tw; }, x0, x1);
            const double W = tiles_total(tl.w, ntiles);
            bonus = sample_from_tiles(pk, a.V, v, tl.w, W);
            mass = 0.0f;
        }
        if (threadIdx.x == 0) { s_bonus = bonus; s_mass = mass; }
    }
    if (threadIdx.x == 0) s_cache_word = (Cache && a.out_hit) ? read_pair(extra, 3 * k + 2) : ~0ull;
    __syncthreads();
    zero_pairs(slots, nslots);   // consumed: back to the resting state
    __syncthreads();

    for (int j = threadIdx.x; j < q.out_len; j += kThreads) {
        int32_t t = -1;
        if (j < k) t = q.tokens[j];
        else if (j == k) t = s_bonus;
        q.out_tokens[j] = t;
    }
    if (threadIdx.x == 0) {
        a.out_nacc[b] = k;
        if (a.out_mass) a.out_mass[b] = s_mass;
        if (Cache && !NoDraft && a.out_hit) {  // (k, bonus) is in the cache iff the bonus is a candidate at k
            const uint64_t cw = s_cache_word;
            const int32_t bonus = s_bonus;
            const int32_t xk = k < gamma ? q.tokens[k] : -1;
            bool hit = false;
            if (cw != ~0ull && bonus >= 0 && bonus < a.V && bonus != xk)
                hit = full_key(load_elem<DT>(q.draft(k), bonus), bonus) >= cw;
            a.out_hit[b] = hit ? 1 : 0;
        }
    }
}

}  // namespace specv
