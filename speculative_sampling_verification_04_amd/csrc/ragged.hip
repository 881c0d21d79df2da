// Chain verification of a ragged batch [Lecture 5: Speculative Decoding and
// SpecInfer, sec. 2.2, 2.7, 3.1; Speculative Decoding (dl-note), sec. 2.2-2.3
// and Appendix "Implementation Details"]: sequence b drafts gamma_b =
// offsets[b+1] - offsets[b] tokens (0 <= gamma_b <= G), its draft rows are
// packed rows offsets[b] .. offsets[b+1]-1 and its gamma_b + 1 target rows are
// packed rows offsets[b] + b .. offsets[b+1] + b. A draft without
// probabilities (an n-gram or prompt-lookup proposer) makes q the point mass
// at the drafted token: x is accepted iff u <= p_t(x), and the residual is
// p_t with x removed.
//
// The tasks have the shape of the dense verify kernel at gamma = G: per
// sequence G + 1 target-row tasks (and G draft-row tasks unless NoDraft), each
// in S chunks, then the H bonus tasks; tasks past gamma_b publish a skipped
// value without reading anything. Workgroup g runs task g of decode_chain; a
// sequence whose bonus task gave up waiting is resolved by the finisher
// launch (ragged_finish_kernel). Offsets that break the contract
// (decreasing, past num_draft, or more than G tokens) are caught here: the
// sequence reports out_num_accepted = -2 and reads no row.
#include "specv_chain.hpp"

namespace specv {

namespace {

constexpr int kU = 4;  // 16-byte steps per lane per iteration
constexpr int kD = 0;  // prefetch form (see stream_chunk)

// The resolve's view of sequence b (its gamma_b = gb tokens from offset o0).
template <int DT, bool NoDraft>
__device__ __forceinline__ SeqView ragged_seq(const ChainArgs& a, int b, int32_t o0, int gb) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int G = a.gamma;
    SeqView q;
    q.b = b;
    q.gamma = gb;
    q.G = G;
    q.tokens = a.tokens + o0;
    q.trow = static_cast<const char*>(row_ptr(a.target, esz, 0, int64_t(o0) + b));
    q.tstride = a.target.stride_row * esz;
    q.drow = NoDraft ? nullptr : static_cast<const char*>(row_ptr(a.draft, esz, 0, o0));
    q.dstride = NoDraft ? 0 : a.draft.stride_row * esz;
    q.out_tokens = a.out_tokens + int64_t(b) * (G + 1);
    q.out_len = G + 1;
    q.out_probs = a.out_probs ? a.out_probs + int64_t(o0) * 2 : nullptr;
    return q;
}

template <int DT, bool NoDraft>
__global__ __launch_bounds__(kThreads) void ragged_verify_kernel(ChainArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int G = a.gamma;
    const int R = NoDraft ? G + 1 : 2 * G + 1;
    const int64_t RS = int64_t(R) * a.S;
    __shared__ SeqOrder ord;
    __shared__ ResolveLds lds;
    // Up to kKeptTemps sequences the offsets are read with the temperatures,
    // in the same round trip, so the task needs no second one to find its
    // rows.
    __shared__ int32_t s_offs[SeqOrder::kKeptTemps + 1];
    const bool offs_kept = a.B <= SeqOrder::kKeptTemps;
    ord.init(a.temperature, a.B, [&] {
        if (!offs_kept) return;
        constexpr int kChunks = SeqOrder::kKeptTemps / kWaveSize;
        int32_t o[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {   // unconditional loads, clamped index
            const int i = c * kWaveSize + lane_id();
            o[c] = a.offsets[i <= a.B ? i : a.B];
        }
        const int32_t ob = a.offsets[a.B];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int i = c * kWaveSize + lane_id();
            if (i <= a.B) s_offs[i] = o[c];
        }
        if (lane_id() == 0) s_offs[a.B] = ob;
    });
    const Placement pl = place_task(ord, [&](int, int& s, int64_t& w) {
        decode_chain(blockIdx.x, a.B, ord.nS, RS, a.H, a.D, s, w);
    });
    const int sidx = pl.sidx;   // dispatch slot of the sequence
    const int b = pl.b;
    const float T = ord.temperature_of(a.temperature, b);
    const bool greedy = !(T > 0.0f);
    const int32_t o0 = offs_kept ? __builtin_amdgcn_readfirstlane(s_offs[b]) : a.offsets[b];
    const int32_t o1 = offs_kept ? __builtin_amdgcn_readfirstlane(s_offs[b + 1]) : a.offsets[b + 1];
    const bool valid = o0 >= 0 && o0 <= o1 && o1 <= a.num_draft && o1 - o0 <= G;
    const int gb = valid ? o1 - o0 : 0;
    uint64_t* slots = a.slots + 2 * int64_t(sidx) * RS;

    // Row task w of the sequence: chunk w % S of row slot w / S, published
    // as pair w (skipped past gamma_b, and for an invalid sequence).
    auto row_task = [&](int64_t w) {
        const int chunk = int(w % a.S);
        const int slot = int(w / a.S);
        const bool draft_row = slot > G;
        const int row = draft_row ? slot - (G + 1) : slot;
        const int64_t lo = int64_t(chunk) * a.chunk;
        const int64_t hi = min(int64_t(a.V), lo + a.chunk);
        const bool needed = valid && lo < hi && (draft_row ? (!greedy && row < gb) : row <= gb);
        uint64_t word = pack_skipped();
        if (needed) {
            const void* rp = draft_row ? row_ptr(a.draft, esz, 0, int64_t(o0) + row)
                                       : row_ptr(a.target, esz, 0, int64_t(o0) + b + row);
            if (greedy) {
                ArgmaxAcc acc;
                stream_chunk<DT, kU, kD>(rp, lo, hi, acc);
                block_merge_argmax(acc.best, acc.idx);
                word = pack_argmax(acc.best, acc.idx);
            } else {
                SoftmaxAcc acc(log2e_over(T));
                stream_chunk_as<DT, kU, kD>(row < a.cache_rows, rp, lo, hi, acc);
                block_merge_softmax(acc.m, acc.mc, acc.s);
                word = pack_softmax(acc.m, acc.s);
            }
        }
        if (threadIdx.x == 0) publish_pair(slots + 2 * w, word, a.epoch);
    };

    if (pl.w >= RS) {  // bonus workgroup
        const int h = int(pl.w - RS);
        if (!valid) {
            if (h == a.H - 1) {
                // Its rows publish skipped values; the finisher zeroes them
                // if they are not all seen in time.
                if (wait_pairs(slots, RS, a.epoch, a.wait_ticks)) zero_pairs(slots, RS);
                else if (threadIdx.x == 0) publish_pair(a.marks + 4 * int64_t(sidx), 1ull, a.epoch);
                for (int j = threadIdx.x; j <= G; j += kThreads) a.out_tokens[int64_t(b) * (G + 1) + j] = -1;
                if (threadIdx.x == 0) a.out_nacc[b] = -2;
            }
            return;
        }
        chain_resolve<DT, NoDraft>(a, ragged_seq<DT, NoDraft>(a, b, o0, gb), T, slots, RS,
                                   a.tiles ? a.tiles + 4 * int64_t(sidx) * a.ntiles : nullptr,
                                   a.parts ? a.parts + 4 * int64_t(sidx) * a.H : nullptr, a.marks + 4 * int64_t(sidx),
                                   h, lds);
        return;
    }
    row_task(pl.w);
}

// Finisher: workgroup s resolves the sequence in slot s if its bonus task
// gave up waiting (or, for a sequence with invalid offsets, zeroes its rows).
template <int DT, bool NoDraft>
__global__ __launch_bounds__(kThreads) void ragged_finish_kernel(ChainArgs a) {
    __shared__ SeqOrder ord;
    __shared__ ResolveLds lds;
    const int sidx = int(blockIdx.x);
    uint64_t* mark = a.marks + 4 * int64_t(sidx);
    if (!pair_ok(peek(mark), peek(mark + 1), a.epoch)) return;
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.deferred, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ord.init(a.temperature, a.B);
    const int b = uniform_i64(ord.seq_wave(sidx));
    const int G = a.gamma;
    const int64_t RS = int64_t(NoDraft ? G + 1 : 2 * G + 1) * a.S;
    uint64_t* slots = a.slots + 2 * int64_t(sidx) * RS;
    const int32_t o0 = a.offsets[b], o1 = a.offsets[b + 1];
    const bool valid = o0 >= 0 && o0 <= o1 && o1 <= a.num_draft && o1 - o0 <= G;
    if (valid) {
        chain_resolve<DT, NoDraft, false, true>(a, ragged_seq<DT, NoDraft>(a, b, o0, o1 - o0), ord.temperature_of(a.temperature, b), slots,
                                                RS, a.tiles ? a.tiles + 4 * int64_t(sidx) * a.ntiles : nullptr,
                                                a.parts ? a.parts + 4 * int64_t(sidx) * a.H : nullptr, mark, a.H - 1,
                                                lds);
    } else {
        zero_pairs(slots, RS);
    }
    zero_pairs(mark, 2);
}

template <int DT, bool NoDraft>
hipError_t launch_dt(const ChainArgs& a, hipStream_t stream) {
    const int64_t R = NoDraft ? a.gamma + 1 : 2 * a.gamma + 1;
    const int64_t tasks = int64_t(a.B) * (R * a.S + a.H);
    const size_t lds = tile_lds_bytes(a.ntiles);
    hipLaunchKernelGGL((ragged_verify_kernel<DT, NoDraft>), dim3(unsigned(tasks)), dim3(kThreads), lds, stream, a);
    hipLaunchKernelGGL((ragged_finish_kernel<DT, NoDraft>), dim3(unsigned(a.B)), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ragged(const ChainArgs& a, int dtype, bool no_draft, hipStream_t stream) {
    if (no_draft) return dtype == DT_BF16 ? launch_dt<DT_BF16, true>(a, stream) : launch_dt<DT_F32, true>(a, stream);
    return dtype == DT_BF16 ? launch_dt<DT_BF16, false>(a, stream) : launch_dt<DT_F32, false>(a, stream);
}

}  // namespace specv
