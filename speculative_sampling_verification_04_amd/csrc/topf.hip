// SSD/Saguaro bonus-token candidates [Speculative Speculative Decoding, sec.
// 4.1.1 and Appendix A.3, Theorem 19]: for every sequence and lookahead
// position, the F draft tokens with the largest logits, excluding the token
// that was sampled at that position (nothing is excluded at position gamma).
//
// One workgroup per draft row. Every lane keeps its K = F + 1 largest keys
// (logit key << 32 | ~index) in registers; a wave-wide threshold (the largest
// K-th key over the wave's lanes) lets almost every 8-element step be rejected
// with one max and one compare. The workgroup then pops the K largest keys in
// K rounds of a block-wide maximum, drops the excluded token and keeps F.
// Keeping F + 1 and dropping afterwards gives the same set as excluding first.
#include "specv_launch.hpp"
#include "specv_sample.hpp"

namespace specv {

namespace {

constexpr int kUnroll = 4;

template <int DT, int K>
__global__ __launch_bounds__(kThreads) void topf_kernel(TopFArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int rows = a.gamma + 1;
    const int b = int(blockIdx.x / rows);
    const int k = int(blockIdx.x % rows);
    const void* rp = static_cast<const char*>(a.draft.data) +
                     (int64_t(b) * a.draft.stride_seq + int64_t(k) * a.draft.stride_row) * esz;

    TopKAcc<K> acc;
    stream_chunk<DT, kUnroll>(rp, 0, a.V, acc);

    __shared__ uint64_t s_wmax[kWaves];
    __shared__ uint64_t s_pick[K];
    for (int r = 0; r < K; ++r) {
        const uint64_t wm = wave_max_u64(acc.a[0]);
        if (lane_id() == 0) s_wmax[wave_id()] = wm;
        __syncthreads();
        uint64_t gm = s_wmax[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) gm = s_wmax[w] > gm ? s_wmax[w] : gm;
        if (gm != 0 && acc.a[0] == gm) {  // keys are unique: exactly one lane pops
#pragma unroll
            for (int i = 0; i < K - 1; ++i) acc.a[i] = acc.a[i + 1];
            acc.a[K - 1] = 0;
        }
        if (threadIdx.x == 0) s_pick[r] = gm;
        __syncthreads();
    }

    if (threadIdx.x == 0) {
        const int32_t excl = (a.tokens != nullptr && k < a.gamma) ? a.tokens[int64_t(b) * a.gamma + k] : -1;
        const int64_t out = (int64_t(b) * rows + k) * a.F;
        int n = 0;
        for (int r = 0; r < K && n < a.F; ++r) {
            const uint64_t key = s_pick[r];
            if (key == 0) break;
            const int32_t idx = int32_t(~uint32_t(key));
            if (idx == excl) continue;
            a.out_topk[out + n] = idx;
            if (a.out_logits) a.out_logits[out + n] = key_logit(uint32_t(key >> 32));
            ++n;
        }
        for (; n < a.F; ++n) {  // fewer candidates than F (only when vocab <= F)
            a.out_topk[out + n] = -1;
            if (a.out_logits) a.out_logits[out + n] = -INFINITY;
        }
    }
}

template <int DT>
hipError_t launch_topf_dt(const TopFArgs& a, hipStream_t stream) {
    const dim3 grid(unsigned(int64_t(a.B) * (a.gamma + 1)));
    const int K = a.F + 1;
    if (K <= 4) hipLaunchKernelGGL((topf_kernel<DT, 4>), grid, dim3(kThreads), 0, stream, a);
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
