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

constexpr int kUnroll = 2;

template <int DT, int K>
__global__ __launch_bounds__(kThreads) void topf_kernel(TopFArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int rows = a.gamma + 1;
    const int b = int(blockIdx.x / rows);
    const int k = int(blockIdx.x % rows);
    const void* rp = static_cast<const char*>(a.draft.data) +
                     (int64_t(b) * a.draft.stride_seq + int64_t(k) * a.draft.stride_row) * esz;

    __shared__ int32_t cand[kWaves][kCandCap];
    __shared__ uint64_t keys[kWaves * kLaneElems * K];
    __shared__ uint64_t s_theta[kWaves];
    __shared__ uint64_t s_pick[K];
    __shared__ int s_nkeys;

    TopKAcc<DT, K> acc;
    acc.init(rp, a.V, cand[wave_id()]);
    stream_chunk<DT, kUnroll>(rp, 0, a.V, acc);
    acc.compact();
    if (lane_id() == 0) s_theta[wave_id()] = acc.theta;
    if (threadIdx.x == 0) s_nkeys = 0;
    __syncthreads();
    uint64_t th = s_theta[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) th = umax64(th, s_theta[w]);

    // Keys that reach the workgroup threshold: at most 8 per kept group.
    for (int e = lane_id(); e < acc.count; e += kWaveSize) {
        const int32_t ent = acc.buf[e];
        const int64_t j0 = ent & ~kSingle;
        const int n = (ent & kSingle) ? 1 : kLaneElems;
        for (int q = 0; q < n; ++q) {
            if (j0 + q >= a.V) break;
            const uint64_t key = full_key(load_elem<DT>(rp, j0 + q), j0 + q);
            if (key >= th) keys[atomicAdd(&s_nkeys, 1)] = key;
        }
    }
    __syncthreads();

    const int need = a.F + 1;
    if (wave_id() == 0) {
        const int n = s_nkeys;
        for (int r = 0; r < need; ++r) {
            uint64_t l = 0;
            for (int i = lane_id(); i < n; i += kWaveSize) l = umax64(l, keys[i]);
            const uint64_t w = wave_max_u64(l);
            for (int i = lane_id(); i < n; i += kWaveSize)
                if (keys[i] == w) keys[i] = 0;   // keys are unique: one owner
            if (lane_id() == 0) s_pick[r] = w;
        }
    }
    __syncthreads();

    if (threadIdx.x == 0) {
        const int32_t excl = (a.tokens != nullptr && k < a.gamma) ? a.tokens[int64_t(b) * a.gamma + k] : -1;
        const int64_t out = (int64_t(b) * rows + k) * a.F;
        int n = 0;
        for (int r = 0; r < need && n < a.F; ++r) {
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
