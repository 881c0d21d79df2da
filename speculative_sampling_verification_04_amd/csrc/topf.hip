// SSD/Saguaro bonus-token candidates [Speculative Speculative Decoding, sec.
// 4.1.1 and Appendix A.3, Theorem 19]: for every sequence and lookahead
// position, the F draft tokens with the largest logits, excluding the token
// that was sampled at that position (nothing is excluded at position gamma).
//
// One workgroup per draft row, streaming it once (TopKAcc: lane maxima, a
// wave threshold and an LDS list of candidate 8-element groups); for small
// batches with a workspace, several per row and one more that merges them
// (topf_chunked_kernel). At the end of a stream every wave compacts its list to at most K groups, the workgroup keeps the
// keys that reach the largest wave threshold, and wave 0 pops the F + 1
// largest; the excluded token is dropped and the first F remain. Keeping
// F + 1 and dropping afterwards gives the same set as excluding first.
#include "specv_launch.hpp"
#include "specv_topk.hpp"

namespace specv {

namespace {

constexpr int kU = 2;  // 16-byte steps per lane per iteration
constexpr int kD = 2;  // ring of two buffers (see stream_chunk)

template <int DT, int K>
__global__ __launch_bounds__(kThreads) void topf_kernel(TopFArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int rows = a.gamma + 1;
    const int b = int(blockIdx.x / rows);
    const int k = int(blockIdx.x % rows);
    const void* rp = static_cast<const char*>(a.draft.data) +
                     (int64_t(b) * a.draft.stride_seq + int64_t(k) * a.draft.stride_row) * esz;

    __shared__ int32_t cand[kWaves][kCandCap];
    __shared__ uint64_t cand_key[kWaves][kCandCap];
    TopKAcc<DT, K> acc;
    acc.init(cand[wave_id()], cand_key[wave_id()]);
    stream_chunk<DT, kU, kD>(rp, 0, a.V, acc);
    const int32_t excl = (a.tokens != nullptr && k < a.gamma) ? a.tokens[int64_t(b) * a.gamma + k] : -1;
    const int64_t out = (int64_t(b) * rows + k) * a.F;
    __shared__ uint64_t keys[topf_keys<K>()];
    topf_finish<DT, K>(acc, rp, a.V, a.F, a.F, excl, a.out_topk + out, a.out_logits ? a.out_logits + out : nullptr, keys);
}

// Small batches: each row in S chunks, so that the batch still fills the
// GPU. Workgroups g < rows * S take chunk g % S of row g / S and publish the
// chunk's F + 1 largest keys (key + 1, or 1 for none; 0 = not yet written).
// Then one workgroup per row, dispatched after every chunk, waits for its
// row's S * (F + 1) words, pops the F + 1 largest (the row's own F + 1
// largest, since each is among its chunk's), writes the outputs exactly as
// the one-workgroup path does and returns the words to zero.
template <int DT, int K>
__global__ __launch_bounds__(kThreads) void topf_chunked_kernel(TopFArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int rows = a.gamma + 1;
    const int64_t nrows = int64_t(a.B) * rows;
    const int F1 = a.F + 1;
    const int64_t g = blockIdx.x;
    if (g < nrows * a.S) {
        const int64_t row = g / a.S;
        const int chunk = int(g % a.S);
        const int b = int(row / rows), k = int(row % rows);
        const void* rp = static_cast<const char*>(a.draft.data) +
                         (int64_t(b) * a.draft.stride_seq + int64_t(k) * a.draft.stride_row) * esz;
        const int64_t lo = int64_t(chunk) * a.chunk;
        const int64_t hi = min(int64_t(a.V), lo + a.chunk);
        __shared__ int32_t cand[kWaves][kCandCap];
        __shared__ uint64_t cand_key[kWaves][kCandCap];
        __shared__ uint64_t keys[topf_keys<K>()];
        TopKAcc<DT, K> acc;
        acc.init(cand[wave_id()], cand_key[wave_id()]);
        stream_chunk<DT, kU, kD>(rp, lo, hi, acc);
        const uint64_t* pick = topf_pick<DT, K>(acc, rp, a.V, F1, keys);
        uint64_t* kw = a.keys + row * a.S * kTopfKeyWords + chunk * F1;
        if (threadIdx.x < F1) publish(kw + threadIdx.x, pick[threadIdx.x] + 1ull);
        return;
    }
    // A row's area holds S * kTopfKeyWords words; its chunks use the first
    // S * (F + 1), chunk c's at c * (F + 1).
    const int64_t row = g - nrows * a.S;
    const int b = int(row / rows), k = int(row % rows);
    uint64_t* kw = a.keys + row * a.S * kTopfKeyWords;
    const int n = a.S * F1;
    __shared__ uint64_t mk[kMaxTopfChunks * kTopfKeyWords];
    const bool ok = wait_slots(kw, n);
    for (int i = threadIdx.x; i < n; i += kThreads) mk[i] = ok ? peek(kw + i) - 1ull : 0ull;
    __syncthreads();
    __shared__ uint64_t s_pick[kTopfKeyWords];
    if (wave_id() == 0) {
        for (int r = 0; r < F1; ++r) {
            uint64_t l = 0;
            for (int i = lane_id(); i < n; i += kWaveSize) l = umax64(l, mk[i]);
            const uint64_t w = wave_max_u64(l);
            for (int i = lane_id(); i < n; i += kWaveSize)
                if (w != 0 && mk[i] == w) mk[i] = 0;   // keys are unique: one owner
            if (lane_id() == 0) s_pick[r] = w;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int32_t excl = (a.tokens != nullptr && k < a.gamma) ? a.tokens[int64_t(b) * a.gamma + k] : -1;
        const int64_t out = (int64_t(b) * rows + k) * a.F;
        // (a wait that ran out leaves every key 0: the row reports -1s)
        topf_write(s_pick, F1, a.F, a.F, excl, a.out_topk + out, a.out_logits ? a.out_logits + out : nullptr);
    }
    zero_slots(kw, n);
}

template <int DT, int K>
void launch_topf_k(const TopFArgs& a, hipStream_t stream) {
    const int64_t rows = int64_t(a.B) * (a.gamma + 1);
    if (a.S > 1 && a.keys != nullptr)
        hipLaunchKernelGGL((topf_chunked_kernel<DT, K>), dim3(unsigned(rows * a.S + rows)), dim3(kThreads), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((topf_kernel<DT, K>), dim3(unsigned(rows)), dim3(kThreads), 0, stream, a);
}

template <int DT>
hipError_t launch_topf_dt(const TopFArgs& a, hipStream_t stream) {
    if (a.S > kMaxTopfChunks || a.F + 1 > kTopfKeyWords) return hipErrorInvalidValue;  // the merge's LDS
    const int K = a.F + 1;
    if (K <= 2) launch_topf_k<DT, 2>(a, stream);
    else if (K <= 4) launch_topf_k<DT, 4>(a, stream);
    else if (K <= 8) launch_topf_k<DT, 8>(a, stream);
    else if (K <= 16) launch_topf_k<DT, 16>(a, stream);
    else launch_topf_k<DT, 32>(a, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topf(const TopFArgs& a, int dtype, hipStream_t stream) {
    return dtype == DT_BF16 ? launch_topf_dt<DT_BF16>(a, stream) : launch_topf_dt<DT_F32>(a, stream);
}

}  // namespace specv
