// Fused chain verification + SSD bonus-token candidates in one pass over the
// logits [Lecture 5: Speculative Decoding and SpecInfer, sec. 2.2, 3.1;
// Speculative Speculative Decoding, sec. 4.1.1].
//
// specv_verify reads draft rows 0..gamma-1 of the T > 0 sequences and
// specv_bonus_topk reads all draft rows 0..gamma; run separately, the shared
// rows cross HBM twice. Here each draft row is streamed once by one workgroup
// that feeds both the softmax statistics (T > 0, row < gamma) and the top-F
// selection, writes that row's candidates directly, and publishes its
// statistics; target rows are as in the verify kernel. Per sequence the
// slots are target rows 0..gamma, then draft rows 0..gamma; the sequence's H
// bonus workgroups come after its rows (decode_fused) and resolve it
// (chain_resolve).
//
// Small batches (small_split; never with the cache outputs) split every row
// into S chunks, one workgroup each: a draft-row chunk publishes its
// statistics word and its F_k + 1 largest keys, and bonus workgroup h first
// merges the keys of draft rows h, h + H, ... into their outputs
// (topf_merge_chunks; each of a row's F_k + 1 largest keys is among its
// chunk's), which are exactly those of the one-workgroup search.
#include "specv_chain.hpp"
#include "specv_topk.hpp"

namespace specv {

namespace {

// Streaming shapes (16-byte steps per lane per iteration; 0 = prefetch form):
// target rows carry only the softmax or argmax, draft rows also the top-K.
constexpr int kTargetU = 4, kTargetD = 0;
constexpr int kDraftU = 2, kDraftD = 0;

template <int DT, int K>
struct SoftmaxTopK {
    SoftmaxAcc sm;
    TopKAcc<DT, K> tk;
    __device__ explicit SoftmaxTopK(float c) : sm(c) {}
    template <int U>
    __device__ __forceinline__ void block(const float (&v)[U][kLaneElems], const int64_t* base, const bool* valid) {
        sm.template block<U>(v, base, valid);
        tk.template block<U>(v, base, valid);
    }
    __device__ __forceinline__ void one(float z, int64_t j, bool ok) {
        sm.one(z, j, ok);
        tk.one(z, j, ok);
    }
};

// LDS of a workgroup: a bonus workgroup's (its top-F merges, then its
// resolve), or a draft row's top-K lists and final pick (a workgroup is one
// or the other).
template <int K>
union FusedLds {
    ResolveLds resolve;
    uint64_t merge[kMaxTopfChunks * kTopfKeyWords];
    struct {
        int32_t cand[kWaves][kCandCap];
        uint64_t cand_key[kWaves][kCandCap];
        uint64_t keys[topf_keys<K>()];
    } rows;
};

// The sigma_{F,C} normaliser value of a draft row: its softmax sum Z (relative
// to the reference m*c) loses (1 - C) of its F largest terms; 2 << 32 (no
// scaling) if nothing would be left.
__device__ __forceinline__ uint64_t sigma_word(const uint64_t* pick, int F, float c, float mc, double Z, float C) {
    double top = 0.0;
    for (int r = 0; r < F; ++r)
        if (pick[r] != 0ull) top += exp2(double(key_logit(uint32_t(pick[r] >> 32))) * double(c) - double(mc));
    const double zs = Z - (1.0 - double(C)) * top;
    return zs > 0.0 ? (1ull << 32) | uint64_t(__float_as_uint(float(zs))) : 2ull << 32;
}

template <int DT, int K, bool Cache>
__global__ __launch_bounds__(kThreads) void verify_topf_kernel(ChainArgs a) {
    __shared__ FusedLds<K> lds;
    constexpr int esz = ElemT<DT>::kBytes;
    const int R1 = 2 * a.gamma + 2;
    const int S = a.S;                       // chunks per row: S > 1 only for small batches
    const int half = (a.gamma + 1) * S;      // target-row tasks of a sequence (as many draft-row tasks)
    const Placement pl = place(a.temperature, a.B, [&](int nS, int& sidx, int64_t& w) {
        decode_fused(blockIdx.x, a.B, nS, half, a.H, a.D, sidx, w);
    });
    const int sidx = pl.sidx;
    const int slot = int(pl.w);              // row task: row slot * S + chunk, then the bonus workgroups
    const int b = pl.b;
    const float T = a.temperature[b];
    const bool greedy = !(T > 0.0f);
    const int64_t words = int64_t(R1) * S + (Cache ? 3 * (a.gamma + 1) : 0);  // pairs per sequence
    uint64_t* slots = a.slots + 2 * int64_t(sidx) * words;
    if (slot >= 2 * half) {  // bonus workgroup: dispatched after every row of the sequence
        const int h = slot - 2 * half;
        if (S > 1) {
            // Top-F of the draft rows searched in chunks: bonus workgroup h
            // merges rows h, h + H, ... (all of a sequence's chunks came
            // before it) and writes their outputs; with the cache outputs it
            // also publishes each row's three cache words, which the
            // sequence's resolve waits for with the row words.
            for (int row = h; row <= a.gamma; row += a.H) {
                const int Fk = a.Fk[row];
                const int F1 = Fk + 1;
                uint64_t* kw = a.topf_keys + 2 * (int64_t(b) * (a.gamma + 1) + row) * S * kTopfKeyWords;
                const uint64_t* pick = topf_merge_chunks<kTopfKeyWords>(kw, S * F1, F1, lds.merge, a.epoch,
                                                                        a.wait_ticks);
                const int32_t excl = row < a.gamma ? a.tokens[int64_t(b) * a.gamma + row] : -1;
                if (threadIdx.x == 0) {
                    const int64_t out = (int64_t(b) * (a.gamma + 1) + row) * a.F;
                    topf_write(pick, F1, Fk, a.F, excl, a.out_topk + out,
                               a.out_topk_logits ? a.out_topk_logits + out : nullptr);
                }
                if (Cache) {
                    const bool scaled = !greedy && row < a.gamma && a.C < 1.0f && Fk > 0;
                    const uint64_t* rw = slots + 2 * int64_t(a.gamma + 1 + row) * S;   // the row's chunk pairs
                    __shared__ uint64_t s_zword;
                    if (threadIdx.x == 0) s_zword = 2ull << 32;
                    if (scaled && wait_pairs(rw, S, a.epoch, a.wait_ticks) && wave_id() == 0) {
                        const RowStats st = merge_chunk_words(lane_id() < S ? read_pair(rw, lane_id()) : 0ull, S,
                                                              false, log2e_over(T));
                        if (lane_id() == 0) s_zword = sigma_word(pick, Fk, log2e_over(T), st.mc, st.Z, a.C);
                    }
                    __syncthreads();
                    if (threadIdx.x == 0) {
                        uint64_t* extra = slots + 2 * (int64_t(R1) * S + 3 * row);
                        publish_pair(extra + 0, s_zword, a.epoch);
                        publish_pair(extra + 2, topf_sigma_key(pick, Fk), a.epoch);
                        publish_pair(extra + 4, topf_cache_key(pick, Fk, excl), a.epoch);
                    }
                }
                zero_pairs(kw, S * F1);
                __syncthreads();
            }
        }
        chain_resolve<DT, false, Cache>(a, dense_seq<DT>(a, b), T, slots, words,
                                        a.tiles ? a.tiles + 4 * int64_t(sidx) * a.ntiles : nullptr,
                                        a.parts ? a.parts + 4 * int64_t(sidx) * a.H : nullptr, h, lds.resolve);
        return;
    }
    const int task = slot / S;               // row slot: target rows 0..gamma, then draft rows
    const int chunk = slot - task * S;
    const bool draft_row = task > a.gamma;
    const int row = draft_row ? task - (a.gamma + 1) : task;
    const int64_t V = a.V;
    const int64_t lo = int64_t(chunk) * a.chunk;
    const int64_t hi = min(V, lo + a.chunk);

    uint64_t word = pack_skipped();
    if (!draft_row) {
        const void* rp = row_ptr(a.target, esz, b, row);
        if (greedy) {
            ArgmaxAcc acc;
            stream_chunk<DT, kTargetU, kTargetD>(rp, lo, hi, acc);
            block_merge_argmax(acc.best, acc.idx);
            word = pack_argmax(acc.best, acc.idx);
        } else {
            SoftmaxAcc acc(log2e_over(T));
            stream_chunk_as<DT, kTargetU, kTargetD>(row < a.cache_rows, rp, lo, hi, acc);
            block_merge_softmax(acc.m, acc.mc, acc.s);
            word = pack_softmax(acc.m, acc.s);
        }
    } else {
        auto& cand = lds.rows.cand;
        auto& cand_key = lds.rows.cand_key;
        const void* rp = row_ptr(a.draft, esz, b, row);
        const int32_t excl = row < a.gamma ? a.tokens[int64_t(b) * a.gamma + row] : -1;
        const int Fk = a.Fk[row];
        int32_t* ids = a.out_topk + (int64_t(b) * (a.gamma + 1) + row) * a.F;
        float* vals = a.out_topk_logits ? a.out_topk_logits + (int64_t(b) * (a.gamma + 1) + row) * a.F : nullptr;
        uint64_t zword = 2ull << 32;  // sigma normaliser word: softmax (no Saguaro scaling on this row)
        const uint64_t* pick;
        if (!greedy && row < a.gamma) {
            SoftmaxTopK<DT, K> acc(log2e_over(T));
            acc.tk.init(cand[wave_id()], cand_key[wave_id()]);
            stream_chunk_as<DT, kDraftU, kDraftD>(row < a.cache_rows, rp, lo, hi, acc);
            block_merge_softmax(acc.sm.m, acc.sm.mc, acc.sm.s);
            word = pack_softmax(acc.sm.m, acc.sm.s);
            pick = S > 1 ? topf_pick<DT, K>(acc.tk, rp, V, Fk + 1, lds.rows.keys)
                         : topf_finish<DT, K>(acc.tk, rp, V, Fk, a.F, excl, ids, vals, lds.rows.keys);
            if (Cache && S == 1 && a.C < 1.0f && Fk > 0 && threadIdx.x == 0)
                zword = sigma_word(pick, Fk, log2e_over(T), acc.sm.mc, acc.sm.s, a.C);
        } else {
            TopKAcc<DT, K> acc;
            acc.init(cand[wave_id()], cand_key[wave_id()]);
            stream_chunk<DT, kDraftU, kDraftD>(rp, lo, hi, acc);
            pick = S > 1 ? topf_pick<DT, K>(acc, rp, V, Fk + 1, lds.rows.keys)
                         : topf_finish<DT, K>(acc, rp, V, Fk, a.F, excl, ids, vals, lds.rows.keys);
        }
        if (S > 1 && threadIdx.x <= Fk) {  // this chunk's Fk + 1 largest keys, for the merge
            uint64_t* kw = a.topf_keys + 2 * ((int64_t(b) * (a.gamma + 1) + row) * S * kTopfKeyWords + chunk * (Fk + 1));
            publish_pair(kw + 2 * threadIdx.x, pick[threadIdx.x], a.epoch);
        }
        if (Cache && S == 1 && threadIdx.x == 0) {
            uint64_t* extra = slots + 2 * (R1 + 3 * row);
            publish_pair(extra + 0, zword, a.epoch);
            publish_pair(extra + 2, topf_sigma_key(pick, Fk), a.epoch);
            publish_pair(extra + 4, topf_cache_key(pick, Fk, excl), a.epoch);
        }
    }
    if (threadIdx.x == 0) publish_pair(slots + 2 * slot, word, a.epoch);
}

template <int DT, bool Cache>
hipError_t launch_dt(const ChainArgs& a, hipStream_t stream) {
    if (a.S > 1 && (a.S > kMaxTopfChunks || a.F + 1 > kTopfKeyWords || a.topf_keys == nullptr))
        return hipErrorInvalidValue;   // the merge's LDS and key area
    const dim3 grid(unsigned(int64_t(a.B) * ((2 * a.gamma + 2) * int64_t(a.S) + a.H)));
    const int K = a.F + 1;
    const size_t lds = tile_lds_bytes(a.ntiles);
    if (K <= 2) hipLaunchKernelGGL((verify_topf_kernel<DT, 2, Cache>), grid, dim3(kThreads), lds, stream, a);
    else if (K <= 4) hipLaunchKernelGGL((verify_topf_kernel<DT, 4, Cache>), grid, dim3(kThreads), lds, stream, a);
    else if (K <= 8) hipLaunchKernelGGL((verify_topf_kernel<DT, 8, Cache>), grid, dim3(kThreads), lds, stream, a);
    else if (K <= 16) hipLaunchKernelGGL((verify_topf_kernel<DT, 16, Cache>), grid, dim3(kThreads), lds, stream, a);
    else hipLaunchKernelGGL((verify_topf_kernel<DT, 32, Cache>), grid, dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_topf(const ChainArgs& a, int dtype, hipStream_t stream) {
    if (a.cache_words)
        return dtype == DT_BF16 ? launch_dt<DT_BF16, true>(a, stream) : launch_dt<DT_F32, true>(a, stream);
    return dtype == DT_BF16 ? launch_dt<DT_BF16, false>(a, stream) : launch_dt<DT_F32, false>(a, stream);
}

}  // namespace specv
