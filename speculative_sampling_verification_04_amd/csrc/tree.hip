// Token-tree verification [Lecture 5: Speculative Decoding and SpecInfer,
// sec. 6.2 and 6.4]: VerifyGreedy for T = 0, multi-step speculative sampling
// (MSS) for T > 0.
//
// One launch. Pass 1 is the row-statistics stream of the chain kernel over
// every node's target row and over the draft rows of nodes that have children
// (the distribution their children were drawn from); every workgroup
// publishes one 64-bit word. The tree's highest-numbered workgroup waits for
// the others' words and walks the tree from the root.
//
// MSS bookkeeping: after j rejections at a node the residual is
//   r_j = max(0, p - c_j q) / M_j,  c_1 = 0, M_1 = 1,
//   c_{j+1} = c_j + M_j,  M_{j+1} = sum_x max(0, p - c_{j+1} q),
// which is r <- norm(max(0, r - q)) applied j times (if max(0, r_j - q) is
// positive only where p > c_j q + M_j q, and there it equals
// (p - (c_j + M_j) q) / M_j). So every rejection costs one pass over the
// node's target and draft rows, whose tile sums also serve the final
// inverse-CDF draw if every child is rejected. The accept test for a child
// with token t uses the gathered logits in fp64: u <= r_j(t) / q(t).
#include "specv_launch.hpp"
#include "specv_sample.hpp"

namespace specv {

namespace {

constexpr int kU = 4;  // 16-byte steps per lane per iteration
constexpr int kD = 1;  // ring of one buffer (see stream_chunk)

__device__ __forceinline__ const void* row_ptr(const RowView& v, int esz, int64_t b, int64_t r) {
    return static_cast<const char*>(v.data) + (b * v.stride_seq + r * v.stride_row) * esz;
}

__device__ __forceinline__ float log2e_over(float T) { return float(1.4426950408889634 / double(T)); }

// Smallest c > after (and > node) with parent[c] == node, or -1; wave 0 only.
__device__ int next_child(const int32_t* par, int N, int node, int after) {
    for (int base = max(after, node) + 1; base < N; base += kWaveSize) {
        const int c = base + lane_id();
        const uint64_t m = __ballot(c < N && par[c] == node);
        if (m) return base + __builtin_ctzll(m);
    }
    return -1;
}

// Lowest-id child of `node` carrying token g, or -1; wave 0 only.
__device__ int child_with_token(const int32_t* par, const int32_t* tok, int N, int node, int32_t g) {
    for (int base = node + 1; base < N; base += kWaveSize) {
        const int c = base + lane_id();
        const uint64_t m = __ballot(c < N && par[c] == node && tok[c] == g);
        if (m) return base + __builtin_ctzll(m);
    }
    return -1;
}

template <int DT>
__device__ __forceinline__ void tree_resolve(const TreeArgs& a, int b, float T, uint64_t* slots) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int N = a.N;
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : log2e_over(T);
    const int32_t* par = a.parent + int64_t(b) * N;
    const int32_t* tok = a.tokens + int64_t(b) * N;
    const float v = greedy ? 0.0f : stream_uniform(a.seed, a.offset, uint32_t(b), 1u, uint32_t(N));

    __shared__ float tile_sum[kMaxTiles];
    __shared__ RowStats s_tp, s_dp;
    __shared__ int s_node, s_nacc, s_child, s_bonus, s_accept;

    if (!wait_slots(slots, int64_t(2) * N * a.S)) {  // never expected: see wait_slots
        if (threadIdx.x == 0) { a.out_nacc[b] = -1; a.out_bonus[b] = -1; }
        zero_slots(slots, int64_t(2) * N * a.S);
        return;
    }
    if (threadIdx.x == 0) { s_node = 0; s_nacc = 0; s_bonus = -1; }
    __syncthreads();

    while (true) {
        const int node = s_node;
        if (threadIdx.x == 0) {
            s_tp = merge_slots(slots + int64_t(node) * a.S, a.S, greedy, c);
            if (!greedy) s_dp = merge_slots(slots + int64_t(N + node) * a.S, a.S, false, c);
        }
        __syncthreads();

        if (greedy) {  // VerifyGreedy
            if (wave_id() == 0) {
                const int32_t g = s_tp.idx;
                const int ch = child_with_token(par, tok, N, node, g);
                if (lane_id() == 0) {
                    if (ch >= 0) {
                        a.out_path[int64_t(b) * N + s_nacc] = ch;
                        s_nacc = s_nacc + 1;
                        s_node = ch;
                    } else {
                        s_bonus = g;
                    }
                }
            }
            __syncthreads();
            if (s_bonus >= 0 || s_node == node) break;
            continue;
        }

        const void* prow = row_ptr(a.target, esz, b, node);
        const void* qrow = row_ptr(a.draft, esz, b, node);
        if (wave_id() == 0) {
            const int ch = next_child(par, N, node, -1);
            if (lane_id() == 0) s_child = ch;
        }
        __syncthreads();

        if (s_child < 0) {  // leaf: the bonus is drawn from p of the leaf
            TargetWeights<DT> f;
            f.p.init(prow, c, s_tp);
            f.V = a.V;
            weight_tiles(f, a.V, tile_sum);
            const int32_t bonus = sample_from_tiles(f, a.V, v, tile_sum);
            if (threadIdx.x == 0) s_bonus = bonus;
            __syncthreads();
            break;
        }

        double cj = 0.0, Mj = 1.0;   // r = max(0, p - cj q) / Mj; identical in every thread
        bool tiles_valid = false;    // tile_sum holds the weights of the current r
        bool accepted = false;
        while (true) {
            const int child = s_child;
            if (threadIdx.x == 0) {
                const int32_t t = tok[child];
                bool acc = false;
                if (t >= 0 && t < a.V) {
                    const double pt = prob_of(load_elem<DT>(prow, t), c, s_tp);
                    const double qt = prob_of(load_elem<DT>(qrow, t), c, s_dp);
                    const double rt = fmax(pt - cj * qt, 0.0) / Mj;
                    const float u = stream_uniform(a.seed, a.offset, uint32_t(b), 1u, uint32_t(child));
                    acc = qt > 0.0 && double(u) <= rt / qt;
                }
                s_accept = acc;
                if (acc) {
                    a.out_path[int64_t(b) * N + s_nacc] = child;
                    s_nacc = s_nacc + 1;
                    s_node = child;
                }
            }
            __syncthreads();
            if (s_accept) { accepted = true; break; }

            // Rejected: r <- norm(max(0, r - q)).
            ResidualWeights<DT> f;
            f.p.init(prow, c, s_tp);
            f.q.init(qrow, c, s_dp);
            f.coef = float(cj + Mj);
            f.V = a.V;
            const double M = weight_tiles(f, a.V, tile_sum);
            if (M > 0.0) { cj = cj + Mj; Mj = M; tiles_valid = true; }
            else tiles_valid = false;

            if (wave_id() == 0) {
                const int ch = next_child(par, N, node, child);
                if (lane_id() == 0) s_child = ch;
            }
            __syncthreads();
            if (s_child < 0) break;
        }
        if (accepted) continue;

        // Every child rejected: draw the bonus from the last residual.
        int32_t bonus;
        if (cj == 0.0) {  // no residual of positive mass was formed: r = p
            TargetWeights<DT> f;
            f.p.init(prow, c, s_tp);
            f.V = a.V;
            weight_tiles(f, a.V, tile_sum);
            bonus = sample_from_tiles(f, a.V, v, tile_sum);
        } else {
            ResidualWeights<DT> f;
            f.p.init(prow, c, s_tp);
            f.q.init(qrow, c, s_dp);
            f.coef = float(cj);
            f.V = a.V;
            if (!tiles_valid) weight_tiles(f, a.V, tile_sum);
            bonus = sample_from_tiles(f, a.V, v, tile_sum);
        }
        if (threadIdx.x == 0) s_bonus = bonus;
        __syncthreads();
        break;
    }

    const int nacc = s_nacc;
    for (int j = nacc + threadIdx.x; j < N; j += kThreads) a.out_path[int64_t(b) * N + j] = -1;
    __syncthreads();
    zero_slots(slots, int64_t(2) * N * a.S);   // consumed: back to the resting state
    if (threadIdx.x == 0) {
        a.out_nacc[b] = nacc;
        a.out_bonus[b] = s_bonus;
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_verify_kernel(TreeArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int N = a.N;
    const int64_t g = blockIdx.x;
    const int chunk = int(g % a.S);
    const int64_t task = g / a.S;
    const int slot = int(task % (2 * N));
    const int tidx = int(task / (2 * N));                 // dispatch slot of the tree
    const int b = sequence_for_slot(a.temperature, a.B, tidx);
    const float T = a.temperature[b];
    const bool greedy = !(T > 0.0f);
    const bool draft_row = slot >= N;
    const int node = draft_row ? slot - N : slot;
    const int64_t lo = int64_t(chunk) * a.chunk;
    const int64_t hi = min(int64_t(a.V), lo + a.chunk);

    bool needed = lo < hi && !(greedy && draft_row);
    if (needed && draft_row) {  // a draft row is read only if the node has children
        const int32_t* par = a.parent + int64_t(b) * N;
        int has = 0;
        for (int c2 = node + 1 + threadIdx.x; c2 < N; c2 += kThreads) has |= (par[c2] == node);
        needed = __syncthreads_or(has) != 0;
    }

    uint64_t word = pack_skipped();
    if (needed) {
        const void* rp = row_ptr(draft_row ? a.draft : a.target, esz, b, node);
        if (greedy) {
            ArgmaxAcc acc;
            stream_chunk<DT, kU, kD>(rp, lo, hi, acc);
            block_merge_argmax(acc.best, acc.idx);
            word = pack_argmax(acc.best, acc.idx);
        } else {
            SoftmaxAcc acc(log2e_over(T));
            stream_chunk<DT, kU, kD>(rp, lo, hi, acc);
            block_merge_softmax(acc.m, acc.mc, acc.s);
            word = pack_softmax(acc.m, acc.s);
        }
    }
    if (threadIdx.x == 0) publish(a.slots + g, word);
    // The tree's last workgroup walks it.
    if (slot == 2 * N - 1 && chunk == a.S - 1) tree_resolve<DT>(a, b, T, a.slots + int64_t(tidx) * 2 * N * a.S);
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, int dtype, hipStream_t stream) {
    const int64_t grid = int64_t(a.B) * 2 * a.N * a.S;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(tree_verify_kernel<DT_BF16>, dim3(unsigned(grid)), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(tree_verify_kernel<DT_F32>, dim3(unsigned(grid)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace specv
