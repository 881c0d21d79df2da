// Chain verification kernel [Lecture 5: Speculative Decoding and SpecInfer,
// sec. 2.2, 2.7, 3.1; Speculative Decoding (dl-note), sec. 2.2-2.3 and
// Appendix "Implementation Details"].
//
// One launch: workgroup g runs task g of decode_chain. Sequences are taken
// T > 0 first (SeqOrder). Per sequence, row tasks stream one chunk of one
// row each: target rows 0..gamma and (for T > 0) draft rows 0..gamma-1, each
// read once from HBM with 16-byte loads, and publish the chunk's statistics
// (online max and sum of 2^(z*c - mc), or the greedy argmax) as one tagged
// pair of words. Then the sequence's H bonus tasks wait for those pairs and
// resolve the sequence (chain_resolve):
//   accept tests u_i <= p_t(x_i)/p_d(x_i) in fp64 (one lane per position),
//   k = first rejection by wave ballot,
//   bonus by inverse CDF over max(p_t - p_d, 0) of row k, or p_t of row gamma,
// then the last one writes the outcome and zeroes the words for the next call.
// A sequence whose bonus task gave up waiting is resolved by the finisher
// launch (chain_finish_kernel, one workgroup per sequence slot). The bonus
// pass's tile sums live in dynamic LDS (tile_lds_bytes).
#include "specv_chain.hpp"

namespace specv {

namespace {

constexpr int kU = 4;  // 16-byte steps per lane per iteration
constexpr int kD = 0;  // prefetch form (see stream_chunk)

template <int DT>
__global__ __launch_bounds__(kThreads) void chain_verify_kernel(ChainArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    __shared__ SeqOrder ord;
    __shared__ ResolveLds lds;
    const int R = 2 * a.gamma + 1;
    const int64_t RS = int64_t(R) * a.S;                 // row tasks per sequence
    ord.init(a.temperature, a.B);
    const Placement pl = place_task(ord, [&](int, int& s, int64_t& w) {
        decode_chain(blockIdx.x, a.B, ord.nS, RS, a.H, a.D, s, w);
    });
    const int sidx = pl.sidx;   // dispatch slot of the sequence
    const int b = pl.b;
    const float T = ord.temperature_of(a.temperature, b);
    const bool greedy = !(T > 0.0f);
    uint64_t* slots = a.slots + 2 * int64_t(sidx) * RS;
    // Row task w of the sequence: chunk w % S of row slot w / S, published
    // as pair w.
    auto row_task = [&](int64_t w) {
        const int chunk = int(w % a.S);
        const int slot = int(w / a.S);
        const bool draft_row = slot > a.gamma;
        const int row = draft_row ? slot - (a.gamma + 1) : slot;
        const int64_t lo = int64_t(chunk) * a.chunk;
        const int64_t hi = min(int64_t(a.V), lo + a.chunk);
        uint64_t word = pack_skipped();
        if (!(greedy && draft_row) && lo < hi) {
            const void* rp = row_ptr(draft_row ? a.draft : a.target, esz, b, row);
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
    if (pl.w >= RS) {  // bonus task: after every row task of the sequence
        chain_resolve<DT>(a, dense_seq<DT>(a, b), T, slots, RS,
                          a.tiles ? a.tiles + 4 * int64_t(sidx) * a.ntiles : nullptr,
                          a.parts ? a.parts + 4 * int64_t(sidx) * a.H : nullptr, a.marks + 4 * int64_t(sidx),
                          int(pl.w - RS), lds);
        return;
    }
    row_task(pl.w);
}

// Finisher: workgroup s resolves the sequence in slot s if its bonus task
// gave up waiting (every word it needs was published by the main launch).
template <int DT>
__global__ __launch_bounds__(kThreads) void chain_finish_kernel(ChainArgs a) {
    __shared__ SeqOrder ord;
    __shared__ ResolveLds lds;
    const int sidx = int(blockIdx.x);
    uint64_t* mark = a.marks + 4 * int64_t(sidx);
    if (!pair_ok(peek(mark), peek(mark + 1), a.epoch)) return;
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.deferred, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ord.init(a.temperature, a.B);
    const int b = uniform_i64(ord.seq_wave(sidx));
    const int64_t RS = int64_t(2 * a.gamma + 1) * a.S;
    chain_resolve<DT, false, false, true>(a, dense_seq<DT>(a, b), ord.temperature_of(a.temperature, b), a.slots + 2 * int64_t(sidx) * RS,
                                          RS, a.tiles ? a.tiles + 4 * int64_t(sidx) * a.ntiles : nullptr,
                                          a.parts ? a.parts + 4 * int64_t(sidx) * a.H : nullptr, mark, a.H - 1, lds);
    zero_pairs(mark, 2);
}

}  // namespace

hipError_t launch_chain(const ChainArgs& a, int dtype, hipStream_t stream) {
    const int64_t tasks = int64_t(a.B) * ((2 * a.gamma + 1) * int64_t(a.S) + a.H);
    const size_t lds = tile_lds_bytes(a.ntiles);
    if (dtype == DT_BF16) {
        hipLaunchKernelGGL(chain_verify_kernel<DT_BF16>, dim3(unsigned(tasks)), dim3(kThreads), lds, stream, a);
        hipLaunchKernelGGL(chain_finish_kernel<DT_BF16>, dim3(unsigned(a.B)), dim3(kThreads), lds, stream, a);
    } else {
        hipLaunchKernelGGL(chain_verify_kernel<DT_F32>, dim3(unsigned(tasks)), dim3(kThreads), lds, stream, a);
        hipLaunchKernelGGL(chain_finish_kernel<DT_F32>, dim3(unsigned(a.B)), dim3(kThreads), lds, stream, a);
    }
    return hipGetLastError();
}

}  // namespace specv
