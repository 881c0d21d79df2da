// Chain verification pieces shared by the verify kernel and the fused
// verify + top-F kernel [Lecture 5: Speculative Decoding and SpecInfer, sec.
// 2.2, 2.7, 3.1; Speculative Decoding (dl-note), sec. 2.2-2.3 and Appendix
// "Implementation Details"].
#pragma once

#include "specv_launch.hpp"
#include "specv_sample.hpp"

namespace specv {

__device__ __forceinline__ const void* row_ptr(const RowView& v, int esz, int64_t b, int64_t r) {
    return static_cast<const char*>(v.data) + (b * v.stride_seq + r * v.stride_row) * esz;
}

__device__ __forceinline__ float log2e_over(float T) { return float(1.4426950408889634 / double(T)); }

// Resolves sequence b from its published row statistics: slots[r * S + chunk]
// holds target row r (r <= gamma) and draft row r - gamma - 1 (after that);
// nslots = all slots of the sequence (waited for, then zeroed).
template <int DT>
__device__ __forceinline__ void chain_resolve(const ChainArgs& a, int b, float T, uint64_t* slots, int64_t nslots) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int gamma = a.gamma;
    const int R = 2 * gamma + 1;
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : log2e_over(T);

    __shared__ RowStats st[2 * 64 + 1];
    __shared__ int32_t s_k;
    __shared__ int32_t s_bonus;
    __shared__ float s_mass;
    __shared__ float tile_sum[kMaxTiles];

    if (!wait_slots(slots, nslots)) {  // never expected: see wait_slots
        if (threadIdx.x == 0) a.out_nacc[b] = -1;
        zero_slots(slots, nslots);
        return;
    }
    for (int r = threadIdx.x; r < R; r += kThreads) {
        const bool draft_row = r > gamma;
        st[r] = (greedy && draft_row) ? RowStats{-INFINITY, -INFINITY, -1, 0.0}
                                      : merge_slots(slots + int64_t(r) * a.S, a.S, greedy, c);
    }
    __syncthreads();
    zero_slots(slots, nslots);   // consumed: back to the resting state

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
                    pt = prob_of(load_elem<DT>(row_ptr(a.target, esz, b, i), x), c, st[i]);
                    pd = prob_of(load_elem<DT>(row_ptr(a.draft, esz, b, i), x), c, st[gamma + 1 + i]);
                }
                const float u = stream_uniform(a.seed, a.offset, uint32_t(b), 0u, uint32_t(i));
                reject = !(pd > 0.0 && double(u) <= pt / pd);
                pt_out = float(pt);
                pd_out = float(pd);
            }
            if (a.out_probs) {
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
        const float v = stream_uniform(a.seed, a.offset, uint32_t(b), 0u, uint32_t(gamma));
        const void* trow = row_ptr(a.target, esz, b, k);
        int32_t bonus = -1;
        float mass = 0.0f;
        if (k < gamma) {
            ResidualWeights<DT> f;
            f.p.init(trow, c, st[k]);
            f.q.init(row_ptr(a.draft, esz, b, k), c, st[gamma + 1 + k]);
            f.coef = 1.0f;
            f.V = a.V;
            const double total = weight_tiles(f, a.V, tile_sum);
            if (total > 0.0) {
                bonus = sample_from_tiles(f, a.V, v, tile_sum);
                mass = float(total);
            }
        }
        if (bonus < 0) {  // every draft accepted, or a residual of zero mass
            TargetWeights<DT> f;
            f.p.init(trow, c, st[k]);
            f.V = a.V;
            const double total = weight_tiles(f, a.V, tile_sum);
            bonus = sample_from_tiles(f, a.V, v, tile_sum);
            if (k == gamma) mass = float(total);
        }
        if (threadIdx.x == 0) { s_bonus = bonus; s_mass = mass; }
    }
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
    }
}

}  // namespace specv
