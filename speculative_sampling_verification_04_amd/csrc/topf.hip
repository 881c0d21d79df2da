// SSD/Saguaro bonus-token candidates [Speculative Speculative Decoding, sec.
// 4.1.1 and Appendix A.3, Theorem 19]: for every sequence and lookahead
// position, the F draft tokens with the largest logits, excluding the token
// that was sampled at that position (nothing is excluded at position gamma).
//
// One workgroup per draft row, streaming it once (TopKAcc: lane maxima, a
// wave threshold and an LDS list of candidate 8-element groups). At the end
// every wave compacts its list to at most K groups, the workgroup keeps the
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

template <int DT>
hipError_t launch_topf_dt(const TopFArgs& a, hipStream_t stream) {
    const dim3 grid(unsigned(int64_t(a.B) * (a.gamma + 1)));
    const int K = a.F + 1;
    if (K <= 2) hipLaunchKernelGGL((topf_kernel<DT, 2>), grid, dim3(kThreads), 0, stream, a);
    else if (K <= 4) hipLaunchKernelGGL((topf_kernel<DT, 4>), grid, dim3(kThreads), 0, stream, a);
    else if (K <= 8) hipLaunchKernelGGL((topf_kernel<DT, 8>), grid, dim3(kThreads), 0, stream, a);
    else if (K <= 16) hipLaunchKernelGGL((topf_kernel<DT, 16>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((topf_kernel<DT, 32>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topf(const TopFArgs& a, int dtype, hipStream_t stream) {
    return dtype == DT_BF16 ? launch_topf_dt<DT_BF16>(a, stream) : launch_topf_dt<DT_F32>(a, stream);
}

}  // namespace specv
