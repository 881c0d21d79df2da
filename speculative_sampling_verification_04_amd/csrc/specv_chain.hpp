// Chain verification pieces shared by the verify kernel and the fused
// verify + top-F kernel [Lecture 5: Speculative Decoding and SpecInfer, sec.
// 2.2, 2.7, 3.1; Speculative Decoding (dl-note), sec. 2.2-2.3 and Appendix
// "Implementation Details"].
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
#pragma once

#include "specv_launch.hpp"
#include "specv_sample.hpp"

namespace specv {

// Tiles in flight per wave in the bonus pass: the pass is spread over H
// workgroups, and it shares the kernel's register allocation with the
// streaming code, so one tile per wave keeps the streaming occupancy.
constexpr int kBonusTiles = 1;

__device__ __forceinline__ const void* row_ptr(const RowView& v, int esz, int64_t b, int64_t r) {
    return static_cast<const char*>(v.data) + (b * v.stride_seq + r * v.stride_row) * esz;
}

__device__ __forceinline__ float log2e_over(float T) { return float(1.4426950408889634 / double(T)); }

// Bonus workgroup h of sequence b. slots: the sequence's nslots row words
// (row r chunk j at r * S + j: target row r for r <= gamma, draft row
// r - gamma - 1 after that). tiles: its ntiles tile words (used when H > 1).
template <int DT>
__device__ __forceinline__ void chain_resolve(const ChainArgs& a, int b, float T, uint64_t* slots, int64_t nslots,
                                              uint64_t* tiles, int h) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int gamma = a.gamma;
    const int R = 2 * gamma + 1;
    const bool greedy = !(T > 0.0f);
    const bool last = h == a.H - 1;
    const float c = greedy ? 0.0f : log2e_over(T);
    const uint64_t* extra = slots + 2 * gamma + 2;  // the cache words, when a.cache_words

    if (greedy && !last) return;  // the greedy bonus is an argmax: nothing to share

    __shared__ RowStats st[2 * 64 + 1];
    __shared__ int32_t s_k;
    __shared__ int32_t s_bonus;
    __shared__ float s_mass;
    __shared__ uint64_t s_cache_word;
    __shared__ float tile_sum[kMaxTiles];

    if (!wait_slots(slots, nslots)) {  // never expected: see wait_slots
        if (last) {
            if (threadIdx.x == 0) a.out_nacc[b] = -1;
            zero_slots(slots, nslots);
        }
        return;
    }
    for (int r = threadIdx.x; r < R; r += kThreads) {
        const bool draft_row = r > gamma;
        st[r] = (greedy && draft_row) ? RowStats{-INFINITY, -INFINITY, -1, 0.0}
                                      : merge_slots(slots + int64_t(r) * a.S, a.S, greedy, c);
    }
    __syncthreads();

    // Accept tests: lane i of wave 0 takes position i.
    if (wave_id() == 0) {
        const int i = lane_id();
        bool reject = false;
        if (i < gamma) {
            const int32_t x = a.tokens[int64_t(b) * gamma + i];
            const bool in_range = x >= 0 && x < a.V;
            float pt_out = 0.0f, pd_out = 1.0f;
            if (greedy) {
                const bool acc = in_range && x == st[i].idx;
                pt_out = acc ? 1.0f : 0.0f;
                reject = !acc;
            } else {
                double pt = 0.0, pd = 0.0;
                if (in_range) {
                    const float zd = load_elem<DT>(row_ptr(a.draft, esz, b, i), x);
                    pt = prob_of(load_elem<DT>(row_ptr(a.target, esz, b, i), x), c, st[i]);
                    RowStats qs = st[gamma + 1 + i];
                    double scale = 1.0;
                    if (a.cache_words) {  // Saguaro sampling: q = sigma_{F_i,C}(draft_i / T)
                        const uint64_t zw = peek(extra + 3 * i);
                        if ((zw >> 32) == 1ull) {
                            qs.Z = double(__uint_as_float(uint32_t(zw)));
                            if (full_key(zd, x) + 1ull >= peek(extra + 3 * i + 1)) scale = double(a.C);
                        }
                    }
                    pd = scale * prob_of(zd, c, qs);
                }
                const float u = stream_uniform(a.seed, a.offset, uint32_t(b), 0u, uint32_t(i));
                reject = !(pd > 0.0 && double(u) <= pt / (double(a.lenience) * pd));
                pt_out = float(pt);
                pd_out = float(pd);
            }
            if (last && a.out_probs) {
                a.out_probs[(int64_t(b) * gamma + i) * 2 + 0] = pt_out;
                a.out_probs[(int64_t(b) * gamma + i) * 2 + 1] = pd_out;
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
        const int ntiles = int((int64_t(a.V) + kTileElems - 1) / kTileElems);
        const float v = stream_uniform(a.seed, a.offset, uint32_t(b), 0u, uint32_t(gamma));
        const void* trow = row_ptr(a.target, esz, b, k);
        ResidualWeights<DT> res;
        TargetWeights<DT> tgt;
        res.p.init(trow, c, st[k]);
        res.coef = 1.0f;
        res.V = a.V;
        tgt.p = res.p;
        tgt.V = a.V;
        if (k < gamma) {
            RowStats qs = st[gamma + 1 + k];
            uint64_t top_word = 0ull;
            if (a.cache_words) {
                const uint64_t zw = peek(extra + 3 * k);
                if ((zw >> 32) == 1ull) {
                    qs.Z = double(__uint_as_float(uint32_t(zw)));
                    top_word = peek(extra + 3 * k + 1);
                }
            }
            res.q.init(row_ptr(a.draft, esz, b, k), c, qs);
            res.q.scale = a.C;
            res.q.top_word = top_word;
        }

        // Tile sums of the bonus weights: residual of row k, or p_t of row gamma.
        if (a.H > 1) {
            const int lo = int(int64_t(ntiles) * h / a.H);
            const int hi = int(int64_t(ntiles) * (h + 1) / a.H);
            auto put = [&](int t, float ts) { publish(tiles + t, pack_tile(ts)); };
            if (k < gamma) weight_tile_range<kBonusTiles>(res, lo, hi, put);
            else weight_tile_range<kBonusTiles>(tgt, lo, hi, put);
            // Each helper read the row words before publishing its tiles, so
            // once every tile word is seen the row words may be zeroed.
            if (!last) return;
            if (!wait_slots(tiles, ntiles)) {
                if (threadIdx.x == 0) a.out_nacc[b] = -1;
                zero_slots(tiles, ntiles);
                zero_slots(slots, nslots);
                return;
            }
            for (int t = threadIdx.x; t < ntiles; t += kThreads) tile_sum[t] = tile_of(peek(tiles + t));
            zero_slots(tiles, ntiles);
        } else {
            auto put = [&](int t, float ts) { tile_sum[t] = ts; };
            if (k < gamma) weight_tile_range<kBonusTiles>(res, 0, ntiles, put);
            else weight_tile_range<kBonusTiles>(tgt, 0, ntiles, put);
        }
        const double total = tiles_total(tile_sum, ntiles);

        int32_t bonus = -1;
        float mass = 0.0f;
        if (total > 0.0) {
            bonus = k < gamma ? sample_from_tiles(res, a.V, v, tile_sum) : sample_from_tiles(tgt, a.V, v, tile_sum);
            mass = float(total);
        } else {  // a residual of zero mass (rounding only): p_t of row k
            weight_tiles<kBonusTiles>(tgt, a.V, tile_sum);
            bonus = sample_from_tiles(tgt, a.V, v, tile_sum);
        }
        if (threadIdx.x == 0) { s_bonus = bonus; s_mass = mass; }
    }
    if (threadIdx.x == 0) s_cache_word = (a.out_hit && a.cache_words) ? peek(extra + 3 * k + 2) : ~0ull;
    __syncthreads();
    zero_slots(slots, nslots);   // consumed: back to the resting state
    __syncthreads();

    for (int j = threadIdx.x; j <= gamma; j += kThreads) {
        int32_t t = -1;
        if (j < k) t = a.tokens[int64_t(b) * gamma + j];
        else if (j == k) t = s_bonus;
        a.out_tokens[int64_t(b) * (gamma + 1) + j] = t;
    }
    if (threadIdx.x == 0) {
        a.out_nacc[b] = k;
        if (a.out_mass) a.out_mass[b] = s_mass;
        if (a.out_hit) {  // (k, bonus) is in the cache iff the bonus is a candidate at k
            const uint64_t cw = s_cache_word;
            const int32_t bonus = s_bonus;
            const int32_t xk = k < gamma ? a.tokens[int64_t(b) * gamma + k] : -1;
            bool hit = false;
            if (cw != ~0ull && bonus >= 0 && bonus < a.V && bonus != xk)
                hit = full_key(load_elem<DT>(row_ptr(a.draft, esz, b, k), bonus), bonus) + 1ull >= cw;
            a.out_hit[b] = hit ? 1 : 0;
        }
    }
}

}  // namespace specv
