// Token-tree verification [Lecture 5: Speculative Decoding and SpecInfer,
// sec. 6.2 and 6.4]: VerifyGreedy for T = 0, multi-step speculative sampling
// (MSS) for T > 0.
//
// Two launches on the caller's stream.
//
// 1. tree_stats_kernel: the row-statistics stream of the chain kernel over
//    every node's target row and over the draft rows of nodes that have
//    children (the distribution their children were drawn from); every
//    workgroup publishes one 64-bit word.
//
// 2. tree_walk_kernel: H workgroups ("walkers") per tree, all resident at
//    once (a cooperative launch when H > 1). Walker 0 walks the tree from the
//    root; every full pass over a node's rows that the walk needs is shared by
//    all H walkers: walker 0 posts the pass as two command words tagged with
//    the pass number, each walker sums its share of the 512-element tiles and
//    publishes every tile sum as a word tagged with the same number, and
//    walker 0 collects them. A pass therefore costs a couple of memory round
//    trips instead of a single workgroup's walk over two rows.
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

constexpr int kU = 4;          // 16-byte steps per lane per iteration
constexpr int kD = 0;          // prefetch form (see stream_chunk)
constexpr int kWalkTiles = 8;  // tiles in flight per wave in a walk pass

// Pass kinds posted by walker 0.
constexpr uint32_t kPassTarget = 0;    // weights p of the node
constexpr uint32_t kPassResidual = 1;  // weights max(0, p - coef * q)
constexpr uint32_t kPassDone = 2;      // no more passes: acknowledge and exit

__device__ __forceinline__ const void* row_ptr(const RowView& v, int esz, int64_t b, int64_t r) {
    return static_cast<const char*>(v.data) + (b * v.stride_seq + r * v.stride_row) * esz;
}

__device__ __forceinline__ float log2e_over(float T) { return float(1.4426950408889634 / double(T)); }

// ------------------------------------------------------------------ pass 1

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_stats_kernel(TreeArgs a) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int N = a.N;
    const int64_t g = blockIdx.x;
    const int chunk = int(g % a.S);
    const int64_t task = g / a.S;
    const int slot = int(task % (2 * N));
    const int b = int(task / (2 * N));
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
}

// ------------------------------------------------------------------ walk

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

__device__ __forceinline__ uint32_t word_hi(uint64_t w) { return uint32_t(w >> 32); }

// Waits until every one of the n words carries tag `p` in its high half
// (wave 0 polls; bounded like wait_slots). Whole workgroup.
__device__ bool wait_tagged(const uint64_t* w, int n, uint32_t p) {
    __shared__ int s_ok;
    if (wave_id() == 0) {
        int ok = 0;
        for (int spin = 0; spin < kMaxSpin; ++spin) {
            bool mine = true;
            for (int i = lane_id(); i < n; i += kWaveSize) mine = mine && word_hi(peek(w + i)) == p;
            if (__all(mine)) { ok = 1; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane_id() == 0) s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

struct Walk {
    uint64_t* cmd;    // [0]: tag | kind << 16 | node, [1]: tag | bits(coef)
    uint64_t* ack;    // one per walker
    uint64_t* tiles;  // ntiles tile words: tag | bits(tile sum)
};

__device__ __forceinline__ Walk walk_of(const TreeArgs& a, int b) {
    uint64_t* w = a.walk + int64_t(b) * (kWalkHeader + a.ntiles);
    return Walk{w, w + 2, w + kWalkHeader};
}

// Walker h's share of pass p: the tile sums of the pass's weights over tiles
// [ntiles*h/H, ntiles*(h+1)/H), each published as tag p | bits(sum).
template <int DT>
__device__ __forceinline__ void share_pass(const TreeArgs& a, int b, float c, int node, uint32_t kind, float coef,
                                           uint32_t p, int h, const Walk& w) {
    constexpr int esz = ElemT<DT>::kBytes;
    __shared__ RowStats s_st[2];
    const uint64_t* slots = a.slots + int64_t(b) * 2 * a.N * a.S;
    if (threadIdx.x == 0) {
        s_st[0] = merge_slots(slots + int64_t(node) * a.S, a.S, false, c);
        s_st[1] = merge_slots(slots + int64_t(a.N + node) * a.S, a.S, false, c);
    }
    __syncthreads();
    const int lo = int(int64_t(a.ntiles) * h / a.H);
    const int hi = int(int64_t(a.ntiles) * (h + 1) / a.H);
    auto put = [&](int t, float ts) { publish(w.tiles + t, (uint64_t(p) << 32) | __float_as_uint(ts)); };
    if (kind == kPassTarget) {
        TargetWeights<DT> f;
        f.p.init(row_ptr(a.target, esz, b, node), c, s_st[0]);
        f.V = a.V;
        weight_tile_range<kWalkTiles>(f, lo, hi, put);
    } else {
        ResidualWeights<DT> f;
        f.p.init(row_ptr(a.target, esz, b, node), c, s_st[0]);
        f.q.init(row_ptr(a.draft, esz, b, node), c, s_st[1]);
        f.coef = coef;
        f.V = a.V;
        weight_tile_range<kWalkTiles>(f, lo, hi, put);
    }
    __syncthreads();
}

// Walkers 1 .. H-1: serve passes until walker 0 posts kPassDone.
template <int DT>
__device__ __forceinline__ void walk_helper(const TreeArgs& a, int b, int h) {
    const float T = a.temperature[b];
    const float c = T > 0.0f ? log2e_over(T) : 0.0f;
    const Walk w = walk_of(a, b);
    for (uint32_t p = 1;; ++p) {
        if (!wait_tagged(w.cmd, 2, p)) return;  // walker 0 reports the failure
        const uint64_t c0 = peek(w.cmd), c1 = peek(w.cmd + 1);
        const uint32_t kind = (uint32_t(c0) >> 16) & 3u;
        if (kind == kPassDone) {
            if (threadIdx.x == 0) publish(w.ack + h, 1ull);
            return;
        }
        share_pass<DT>(a, b, c, int(uint32_t(c0) & 0xffffu), kind, __uint_as_float(uint32_t(c1)), p, h, w);
    }
}

// Walker 0: the walk itself.
template <int DT>
__device__ __forceinline__ void walk_tree(const TreeArgs& a, int b) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int N = a.N;
    const float T = a.temperature[b];
    const bool greedy = !(T > 0.0f);
    const float c = greedy ? 0.0f : log2e_over(T);
    const int32_t* par = a.parent + int64_t(b) * N;
    const int32_t* tok = a.tokens + int64_t(b) * N;
    const float v = greedy ? 0.0f : stream_uniform(a.seed, a.offset, uint32_t(b), 1u, uint32_t(N));
    uint64_t* slots = a.slots + int64_t(b) * 2 * N * a.S;
    const Walk w = walk_of(a, b);

    __shared__ float tile_sum[kMaxTiles];
    __shared__ RowStats s_tp, s_dp;
    __shared__ int s_node, s_nacc, s_child, s_bonus, s_accept, s_fail;

    uint32_t pass = 0;
    // One shared pass: post it, do walker 0's share, collect every tile sum
    // into LDS. Returns the total weight (fp64), or -1 if a wait ran out.
    auto run_pass = [&](int node, uint32_t kind, float coef) -> double {
        ++pass;
        if (threadIdx.x == 0) {
            publish(w.cmd + 1, (uint64_t(pass) << 32) | __float_as_uint(coef));
            publish(w.cmd, (uint64_t(pass) << 32) | (kind << 16) | uint32_t(node));
        }
        share_pass<DT>(a, b, c, node, kind, coef, pass, 0, w);
        if (!wait_tagged(w.tiles, a.ntiles, pass)) {
            if (threadIdx.x == 0) s_fail = 1;
            __syncthreads();
            return -1.0;
        }
        for (int t = threadIdx.x; t < a.ntiles; t += kThreads) tile_sum[t] = __uint_as_float(uint32_t(peek(w.tiles + t)));
        return tiles_total(tile_sum, a.ntiles);
    };

    if (threadIdx.x == 0) { s_node = 0; s_nacc = 0; s_bonus = -1; s_fail = 0; }
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
            if (run_pass(node, kPassTarget, 0.0f) < 0.0) break;
            TargetWeights<DT> f;
            f.p.init(prow, c, s_tp);
            f.V = a.V;
            const int32_t bonus = sample_from_tiles(f, a.V, v, tile_sum);
            if (threadIdx.x == 0) s_bonus = bonus;
            __syncthreads();
            break;
        }

        double cj = 0.0, Mj = 1.0;   // r = max(0, p - cj q) / Mj; identical in every thread
        bool tiles_valid = false;    // tile_sum holds the weights of the current r
        bool accepted = false;
        bool failed = false;
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
            const double M = run_pass(node, kPassResidual, float(cj + Mj));
            if (M < 0.0) { failed = true; break; }
            if (M > 0.0) { cj = cj + Mj; Mj = M; tiles_valid = true; }
            else tiles_valid = false;

            if (wave_id() == 0) {
                const int ch = next_child(par, N, node, child);
                if (lane_id() == 0) s_child = ch;
            }
            __syncthreads();
            if (s_child < 0) break;
        }
        if (failed) break;
        if (accepted) continue;

        // Every child rejected: draw the bonus from the last residual.
        int32_t bonus = -1;
        if (cj == 0.0) {  // no residual of positive mass was formed: r = p
            if (run_pass(node, kPassTarget, 0.0f) >= 0.0) {
                TargetWeights<DT> f;
                f.p.init(prow, c, s_tp);
                f.V = a.V;
                bonus = sample_from_tiles(f, a.V, v, tile_sum);
            }
        } else {
            ResidualWeights<DT> f;
            f.p.init(prow, c, s_tp);
            f.q.init(qrow, c, s_dp);
            f.coef = float(cj);
            f.V = a.V;
            if (tiles_valid || run_pass(node, kPassResidual, float(cj)) >= 0.0)
                bonus = sample_from_tiles(f, a.V, v, tile_sum);
        }
        if (threadIdx.x == 0) s_bonus = bonus;
        __syncthreads();
        break;
    }

    // Release the other walkers, wait until they are gone, then return every
    // word this tree used to zero.
    ++pass;
    if (threadIdx.x == 0) {
        publish(w.cmd + 1, uint64_t(pass) << 32);
        publish(w.cmd, (uint64_t(pass) << 32) | (kPassDone << 16));
    }
    if (a.H > 1) {
        __shared__ int s_acked;
        if (wave_id() == 0) {
            int ok = 0;
            for (int spin = 0; spin < kMaxSpin; ++spin) {
                const bool mine = lane_id() == 0 || lane_id() >= a.H || peek(w.ack + lane_id()) != 0ull;
                if (__all(mine)) { ok = 1; break; }
                __builtin_amdgcn_s_sleep(2);
            }
            if (lane_id() == 0) s_acked = ok;
        }
        __syncthreads();
        if (!s_acked && threadIdx.x == 0) s_fail = 1;
    }
    __syncthreads();
    const int nacc = s_nacc;
    for (int j = nacc + threadIdx.x; j < N; j += kThreads) a.out_path[int64_t(b) * N + j] = -1;
    zero_slots(slots, int64_t(2) * N * a.S);
    zero_slots(w.cmd, kWalkHeader + a.ntiles);
    __syncthreads();
    if (threadIdx.x == 0) {
        a.out_nacc[b] = s_fail ? -1 : nacc;
        a.out_bonus[b] = s_fail ? -1 : s_bonus;
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_walk_kernel(TreeArgs a) {
    const int b = int(blockIdx.x / a.H);
    const int h = int(blockIdx.x % a.H);
    if (h == 0) walk_tree<DT>(a, b);
    else walk_helper<DT>(a, b, h);
}

template <int DT>
hipError_t launch_tree_dt(TreeArgs a, hipStream_t stream) {
    const int64_t grid = int64_t(a.B) * 2 * a.N * a.S;
    hipLaunchKernelGGL(tree_stats_kernel<DT>, dim3(unsigned(grid)), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // Every walker of every tree must be resident at once (walkers wait on
    // each other), so H is capped by what the device holds.
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(tree_walk_kernel<DT>),
                                                          kThreads, 0)) != hipSuccess)
        return e;
    const int64_t resident = int64_t(cus) * per_cu;
    int64_t H = a.H;
    if (int64_t(a.B) * H > resident) H = resident / a.B > 1 ? resident / a.B : 1;
    a.H = int32_t(H);
    const dim3 walk_grid(unsigned(int64_t(a.B) * a.H));
    if (a.H > 1) {
        void* args[] = {&a};
        e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(tree_walk_kernel<DT>), walk_grid, dim3(kThreads),
                                       args, 0, stream);
    } else {
        hipLaunchKernelGGL(tree_walk_kernel<DT>, walk_grid, dim3(kThreads), 0, stream, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, int dtype, hipStream_t stream) {
    return dtype == DT_BF16 ? launch_tree_dt<DT_BF16>(a, stream) : launch_tree_dt<DT_F32>(a, stream);
}

}  // namespace specv
