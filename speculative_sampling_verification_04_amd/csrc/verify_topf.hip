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
// bonus tasks come after its rows (decode_fused) and resolve it
// (chain_resolve). Workgroup g runs task g; what a task leaves when it gives
// up waiting (a sequence's resolve, a draft row's merge) is done by the
// finisher launch (topf_finish_kernel).
//
// Small batches (small_split) split every row into S chunks, one task each:
// a draft-row chunk publishes its statistics and its F_k + 1 largest keys,
// and the row's last chunk task merges the row's keys into its outputs
// (topf_merge_chunks; each of a row's F_k + 1 largest keys is among its
// chunk's), which are exactly those of the one-workgroup search.
#include "specv_chain.hpp"
#include "specv_topk.hpp"

namespace specv {

namespace {

// Streaming shapes (16-byte steps per lane per iteration; 0 = prefetch form):
// target rows carry only the softmax or argmax, draft rows also the top-K.
constexpr int kTargetU = 4, kTargetD = 0;
constexpr int kDraftU = 4, kDraftD = 0;

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

// Rows searched in chunks (S > 1): the last chunk task of a draft row
// merges the row's chunk keys (every chunk task of the row has a smaller
// index), writes the row's top-F outputs and, with the cache outputs,
// publishes its three cache pairs, which the sequence's resolve waits for
// with the row statistics. If its waits run out it marks the merge deferred
// (mark: the sequence's merge mark) and the finisher (Finish) merges again,
// when every chunk's keys are published.
template <int DT, int K, bool Cache, bool Finish = false>
__device__ __forceinline__ void merge_draft_row(const ChainArgs& a, FusedLds<K>& lds, uint64_t* slots, uint64_t* mark,
                                                int b, int row, bool greedy, float T) {
    const int S = a.S;
    const int R1 = 2 * a.gamma + 2;
    const int Fk = a.Fk[row];
    const int F1 = Fk + 1;
    const uint64_t ticks = Finish ? kMaxWaitTicks : a.wait_ticks;
    uint64_t* kw = a.topf_keys + 2 * (int64_t(b) * (a.gamma + 1) + row) * S * kTopfKeyWords;
    const uint64_t* rw = slots + 2 * int64_t(a.gamma + 1 + row) * S;   // the row's chunk pairs
    const bool scaled = Cache && !greedy && row < a.gamma && a.C < 1.0f && Fk > 0;
    const bool ok = wait_pairs(kw, int64_t(S) * F1, a.epoch, ticks) && (!scaled || wait_pairs(rw, S, a.epoch, ticks));
    if (!ok && !Finish) {
        if (threadIdx.x == 0) publish_pair(mark, 1ull, a.epoch);
        return;
    }
    const uint64_t* pick = topf_merge_chunks<kTopfKeyWords>(kw, S * F1, F1, lds.merge, ok);
    const int32_t excl = row < a.gamma ? a.tokens[int64_t(b) * a.gamma + row] : -1;
    if (threadIdx.x == 0) {
        const int64_t out = (int64_t(b) * (a.gamma + 1) + row) * a.F;
        topf_write(pick, F1, Fk, a.F, excl, a.out_topk + out, a.out_topk_logits ? a.out_topk_logits + out : nullptr);
    }
    if (Cache) {
        __shared__ uint64_t s_zword;
        if (threadIdx.x == 0) s_zword = 2ull << 32;
        if (scaled && ok && wave_id() == 0) {
            const RowStats st = merge_chunk_words(lane_id() < S ? read_pair(rw, lane_id()) : 0ull, S, false,
                                                  log2e_over(T));
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
}

template <int DT, int K, bool Cache>
__global__ __launch_bounds__(kThreads) void verify_topf_kernel(ChainArgs a) {
    __shared__ FusedLds<K> lds;
    __shared__ SeqOrder ord;
    constexpr int esz = ElemT<DT>::kBytes;
    const int R1 = 2 * a.gamma + 2;
    const int S = a.S;                       // chunks per row: S > 1 only for small batches
    const int half = (a.gamma + 1) * S;      // target-row tasks of a sequence (as many draft-row tasks)
    ord.init(a.temperature, a.B);
    const Placement pl = place_task(ord, [&](int nS, int& sidx, int64_t& w) {
        decode_fused(blockIdx.x, a.B, nS, half, a.H, a.D, sidx, w);
    });
    const int sidx = pl.sidx;
    const int b = pl.b;
    const float T = ord.temperature_of(a.temperature, b);
    const bool greedy = !(T > 0.0f);
    const int64_t words = int64_t(R1) * S + (Cache ? 3 * (a.gamma + 1) : 0);  // pairs per sequence
    uint64_t* slots = a.slots + 2 * int64_t(sidx) * words;

    // Row chunk task `slot` (row slot * S + chunk: target rows 0..gamma, then
    // draft rows): publishes pair `slot`; a draft-row chunk also its top-F
    // (S = 1: the row's outputs and, with the cache outputs, its cache pairs;
    // S > 1: its chunk keys for merge_draft_row).
    auto row_task = [&](int slot) {
        const int task = slot / S;
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
    };

    const int slot = int(pl.w);              // row task: row slot * S + chunk, then the bonus tasks
    uint64_t* mark = a.marks + 4 * int64_t(sidx);
    if (slot >= 2 * half) {  // bonus task: after every row task of the sequence
        chain_resolve<DT, false, Cache>(a, dense_seq<DT>(a, b), T, slots, words,
                                        a.tiles ? a.tiles + 4 * int64_t(sidx) * a.ntiles : nullptr,
                                        a.parts ? a.parts + 4 * int64_t(sidx) * a.H : nullptr, mark, slot - 2 * half,
                                        lds.resolve);
        return;
    }
    row_task(slot);
    const int task = slot / S;
    if (task > a.gamma && S > 1 && slot - task * S == S - 1)
        merge_draft_row<DT, K, Cache>(a, lds, slots, mark + 2, b, task - (a.gamma + 1), greedy, T);
}

// Finisher: workgroup s completes the sequence in slot s if one of its tasks
// gave up waiting: first the draft-row merges still pending (their keys are
// still published: a merge that completed zeroed them), then the resolve.
// Every word it reads was published by the main launch.
template <int DT, int K, bool Cache>
__global__ __launch_bounds__(kThreads) void topf_finish_kernel(ChainArgs a) {
    __shared__ FusedLds<K> lds;
    __shared__ SeqOrder ord;
    const int sidx = int(blockIdx.x);
    uint64_t* mark = a.marks + 4 * int64_t(sidx);
    const bool resolve = pair_ok(peek(mark), peek(mark + 1), a.epoch);
    const bool merge = pair_ok(peek(mark + 2), peek(mark + 3), a.epoch);
    if (!resolve && !merge) return;
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.deferred, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ord.init(a.temperature, a.B);
    const int b = uniform_i64(ord.seq_wave(sidx));
    const float T = ord.temperature_of(a.temperature, b);
    const bool greedy = !(T > 0.0f);
    const int S = a.S;
    const int64_t words = int64_t(2 * a.gamma + 2) * S + (Cache ? 3 * (a.gamma + 1) : 0);
    uint64_t* slots = a.slots + 2 * int64_t(sidx) * words;
    if (merge && S > 1) {   // only chunked rows merge (and have a key area)
        for (int row = 0; row <= a.gamma; ++row) {
            const uint64_t* kw = a.topf_keys + 2 * (int64_t(b) * (a.gamma + 1) + row) * S * kTopfKeyWords;
            if (pair_ok(peek(kw), peek(kw + 1), a.epoch))
                merge_draft_row<DT, K, Cache, true>(a, lds, slots, mark + 2, b, row, greedy, T);
            __syncthreads();
        }
    }
    if (merge) zero_pairs(mark + 2, 1);
    if (resolve) {
        chain_resolve<DT, false, Cache, true>(a, dense_seq<DT>(a, b), T, slots, words,
                                              a.tiles ? a.tiles + 4 * int64_t(sidx) * a.ntiles : nullptr,
                                              a.parts ? a.parts + 4 * int64_t(sidx) * a.H : nullptr, mark, a.H - 1,
                                              lds.resolve);
        zero_pairs(mark, 1);
    }
}

template <int DT, bool Cache>
hipError_t launch_dt(const ChainArgs& a, hipStream_t stream) {
    if (a.S > 1 && (a.S > kMaxTopfChunks || a.F + 1 > kTopfKeyWords || a.topf_keys == nullptr))
        return hipErrorInvalidValue;   // the merge's LDS and key area
    const int64_t tasks = int64_t(a.B) * ((2 * a.gamma + 2) * int64_t(a.S) + a.H);
    const int K = a.F + 1;
    const size_t lds = tile_lds_bytes(a.ntiles);
    auto launch = [&](auto kernel, auto finish) {
        hipLaunchKernelGGL(kernel, dim3(unsigned(tasks)), dim3(kThreads), lds, stream, a);
        hipLaunchKernelGGL(finish, dim3(unsigned(a.B)), dim3(kThreads), lds, stream, a);
    };
    if (K <= 2) launch(verify_topf_kernel<DT, 2, Cache>, topf_finish_kernel<DT, 2, Cache>);
    else if (K <= 4) launch(verify_topf_kernel<DT, 4, Cache>, topf_finish_kernel<DT, 4, Cache>);
    else if (K <= 8) launch(verify_topf_kernel<DT, 8, Cache>, topf_finish_kernel<DT, 8, Cache>);
    else if (K <= 16) launch(verify_topf_kernel<DT, 16, Cache>, topf_finish_kernel<DT, 16, Cache>);
    else launch(verify_topf_kernel<DT, 32, Cache>, topf_finish_kernel<DT, 32, Cache>);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_topf(const ChainArgs& a, int dtype, hipStream_t stream) {
    if (a.cache_words)
        return dtype == DT_BF16 ? launch_dt<DT_BF16, true>(a, stream) : launch_dt<DT_F32, true>(a, stream);
    return dtype == DT_BF16 ? launch_dt<DT_BF16, false>(a, stream) : launch_dt<DT_F32, false>(a, stream);
}

}  // namespace specv
