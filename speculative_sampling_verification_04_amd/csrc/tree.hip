// Token-tree verification [Lecture 5: Speculative Decoding and SpecInfer,
// sec. 6.2 and 6.4]: VerifyGreedy for T = 0, multi-step speculative sampling
// (MSS) for T > 0.
//
// Two kinds of workgroup, in one launch for trees of up to kFusedTreeNodes
// nodes (tree_fused_kernel: each tree's walkers follow the rows of a later
// tree in dispatch order, so walks overlap the stream) and in two launches
// beyond (tree_stats_kernel, then tree_walk_kernel).
//
// 1. Rows (tree_row): the row-statistics stream of the chain kernel over
//    every node's target row and over the draft rows of nodes that have
//    children (the distribution their children were drawn from); every
//    workgroup publishes one tagged pair.
//
// 2. Walkers (tree_walk): H workgroups per tree (launch_tree_dt says why
//    they are all resident together). Every walker of a tree runs
//    the same walk on the same data and takes the same decisions; each full pass
//    over a node's rows that the walk needs is split between them: walker h
//    sums the weights over its share of the 512-element tiles, keeps its tile
//    sums in LDS and publishes its share's totals tagged with the pass
//    number, and every walker then adds the H totals in walker order. A
//    pass therefore costs one exchange of H messages, with no command round trip;
//    the accept tests of a node's children are prepared in parallel when the
//    walk reaches the node. The final draw is made by the walker whose share
//    holds the inverse-CDF point.
//
// MSS bookkeeping: after j rejections at a node the residual is
//   r_j = max(0, p - c_j q) / M_j,  c_1 = 0, M_1 = 1,
//   c_{j+1} = c_j + M_j,  M_{j+1} = sum_x max(0, p - c_{j+1} q),
// which is r <- norm(max(0, r - q)) applied j times (if max(0, r_j - q) is
// positive only where p > c_j q + M_j q, and there it equals
// (p - (c_j + M_j) q) / M_j). So every rejection costs one pass over the
// node's target and draft rows, whose tile sums also serve the final
// inverse-CDF draw if every child is rejected. The accept test for a child
// with token t uses the gathered logits in fp64: u <= r_j(t) / q(t), with
// r_j(t) / q(t) = max(0, p(t)/q(t) - c_j) / M_j and p(t)/q(t) formed from the
// two logits (never as a difference of probabilities).
//
// Accuracy (see specv_sample.hpp): the node's first residual pass measures
// the correction kappa of the two rows' normaliser ratio and sum p~ = A; its
// tile sums are corrected once kappa is known, later passes at the node fold
// kappa into their exponent, and masses are taken in probability units
// (sums / A), so c_j and M_j carry only the weights' own rounding.
#include "specv_launch.hpp"
#include "specv_sample.hpp"

namespace specv {

namespace {

// Row streaming (16-byte steps per lane per iteration, prefetch form; see
// stream_chunk): the stats launch streams 4 steps deep at full occupancy;
// the one-launch form, whose walker holds three workgroups per CU (its
// registers), streams 8 deep, so each row workgroup keeps twice the bytes in
// flight in registers it has anyway.
constexpr int kU = 4;
constexpr int kFusedU = 8;
constexpr int kD = 0;
constexpr int kWalkTiles = 8;       // tiles in flight per wave in a walk pass (walk launch)
constexpr int kFusedWalkTiles = 2;  // the same in the one-launch form (its registers set the rows' occupancy)

__device__ __forceinline__ const void* row_ptr(const RowView& v, int esz, int64_t b, int64_t r) {
    return static_cast<const char*>(v.data) + (b * v.stride_seq + r * v.stride_row) * esz;
}

__device__ __forceinline__ float log2e_over(float T) { return float(1.4426950408889634 / double(T)); }

// ------------------------------------------------------------------ rows

// Row task w of tree b (w = task * S + chunk; task < N: target row of node
// task, else draft row of node task - N) -> its statistics word.
template <int DT, int U>
__device__ __forceinline__ void tree_row(const TreeArgs& a, int b, int64_t w) {
    constexpr int esz = ElemT<DT>::kBytes;
    const int N = a.N;
    const int chunk = int(w % a.S);
    const int task = int(w / a.S);
    const float T = a.temperature[b];
    const bool greedy = !(T > 0.0f);
    const bool draft_row = task >= N;
    const int node = draft_row ? task - N : task;
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
            stream_chunk<DT, U, kD>(rp, lo, hi, acc);
            block_merge_argmax(acc.best, acc.idx);
            word = pack_argmax(acc.best, acc.idx);
        } else {
            SoftmaxAcc acc(log2e_over(T));
            stream_chunk_as<DT, U, kD>(node < a.cache_nodes, rp, lo, hi, acc);
            block_merge_softmax(acc.m, acc.mc, acc.s);
            word = pack_softmax(acc.m, acc.s);
        }
    }
    if (threadIdx.x == 0) publish_pair(a.slots + 2 * (int64_t(b) * 2 * N * a.S + w), word, a.epoch);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_stats_kernel(TreeArgs a) {
    const int64_t RS = int64_t(2) * a.N * a.S;
    tree_row<DT, kU>(a, int(blockIdx.x / RS), blockIdx.x % RS);   // rows never wait: hardware order is fine
}

// ------------------------------------------------------------------ walk

// Walk words of one tree (a.walk + b * kWalkWords, zero at rest), all as
// tagged pairs: the walkers' pass messages, double-buffered by pass parity
// (four fp64 values per walker: the sums of w~ and q~ over its share, and of
// p and p (2^h - 1) when the pass measures the correction; tag = epoch and
// pass number), one acknowledgement per walker and the drawn token (tag =
// the epoch).
constexpr int kPassValues = 4;
static_assert(kMaxWalkers * kPassValues <= kWaveSize, "one pair per lane in the pass exchange's gather");
struct WalkWords {
    uint64_t* part;   // [2][kMaxWalkers][kPassValues] pairs
    uint64_t* ack;    // [kMaxWalkers] pairs
    uint64_t* bonus;  // [1] pair
};
static_assert(kWalkWords == 2 * (2 * kMaxWalkers * kPassValues + kMaxWalkers + 1), "walk words of one tree");

__device__ __forceinline__ WalkWords walk_of(const TreeArgs& a, int b) {
    uint64_t* w = a.walk + int64_t(b) * kWalkWords;
    uint64_t* ack = w + 2 * (2 * kMaxWalkers * kPassValues);
    return WalkWords{w, ack, ack + 2 * kMaxWalkers};
}

// Tag of the pass messages: the epoch's low 16 bits (never 0) and the pass
// number (1 .. < 2^16), so neither a zero word, a message of the pass before
// last in the same buffer nor one of another call reads as this pass's.
__device__ __forceinline__ uint32_t pass_tag(uint32_t epoch, uint32_t pass) {
    return ((epoch & 0xffffu) << 16) | (pass & 0xffffu);
}

// Waits until the words of node `node`'s target row (and, with `draft`, its
// draft row) are published (wave 0 polls), and leaves their values in out
// (LDS): chunk j of the target row at out[j], of the draft row at out[S + j]
// (S <= kWaveSize). Whole workgroup; false if the bound was reached.
__device__ bool wait_node(const uint64_t* slots, int N, int S, int node, bool draft, uint32_t ep, uint64_t ticks,
                          uint64_t* out) {
    __shared__ int s_ok;
    if (wave_id() == 0) {
        int ok = 0;
        const int n = draft ? 2 * S : S;
        for (const WaitBound t(ticks); !t.expired();) {
            bool mine = true;
            for (int i = lane_id(); i < n; i += kWaveSize) {
                const int64_t k = i < S ? int64_t(node) * S + i : int64_t(N + node) * S + (i - S);
                const uint64_t hi = peek(slots + 2 * k), lo = peek(slots + 2 * k + 1);
                mine &= pair_ok(hi, lo, ep);
                out[i] = pair_value(hi, lo);   // the last poll's values stay
            }
            if (__all(mine)) { ok = 1; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane_id() == 0) s_ok = ok;
    }
    __syncthreads();
    return s_ok != 0;
}

// Per-walker state of one walk (LDS of the walker), for trees of up to NM
// nodes.
template <int NM>
struct WalkLds {
    RowStats sp, sq;              // statistics of the current node's target and draft rows
    int32_t kid[kThreads];        // a batch of the current node's children, ascending
    double pc[kThreads], qc[kThreads];  // p(t), q(t) of each child's token t (streaming statistics)
    float zp[kThreads], zq[kThreads];   // the two logits at each child's token
    float u[kThreads];            // each child's uniform
    uint64_t msg[kMaxWalkers * kPassValues];  // the walkers' pass messages, as gathered
    uint64_t nodew[2 * kWaveSize];  // the current node's row words, as the wait for them found them
    double part[kMaxWalkers];     // the walkers' totals of the last pass (corrected)
    double tile[kMaxWalkTiles];   // this walker's tile sums of the last pass (corrected)
    float tile_q[kMaxWalkTiles];  // their q~ sums (a pass that measures the correction)
    int32_t par[NM];              // the tree's parents and tokens
    int32_t tok[NM];
    int nk, from;                 // batch size; next position of the child scan
    int ok;
};

// The weights of one pass over the current node's rows.
enum PassKind { kPassTarget = 0, kPassFirst = 1, kPassResid = 2 };

// TIF: tiles in flight per wave in a pass. kStreaming: the tree's rows may
// still be streaming, so a node's words are awaited before they are read.
template <int DT, int NM, int TIF, bool kStreaming>
struct Walker {
    const TreeArgs& a;
    int b, h, N, lo, hi;
    float c, v;
    double c64;                   // exponent scale of the pass weights and p/q ratios (fp64 log2(e)/T)
    WalkWords w;
    WalkLds<NM>& s;
    const void* prow;
    const void* qrow;
    uint32_t pass = 0;
    // The node's correction (measured by its first residual pass): kappa,
    // and the sum of p~ over the row (masses in probability units = sums of
    // weights / A).
    double kappa = 0.0, A = 1.0;

    // One shared pass over the current node's weights: p (kPassTarget); the
    // first residual max(0, p - q), which also measures the node's
    // correction (kPassFirst); or max(0, p - coef q) with the correction
    // known (kPassResid). Sets *total to the fp64 sum of the H walker
    // totals (corrected; every walker computes the same totals in the same
    // order); false if a wait ran out.
    __device__ __forceinline__ bool run_pass(PassKind kind, double coef, double* total) {
        ++pass;
        double ps = 0.0, pgs = 0.0;
        auto put = [&](int t, double tw, double tq) { s.tile[t - lo] = tw; s.tile_q[t - lo] = float(tq); };
        if (kind == kPassTarget) {
            TargetWeights<DT> f;
            f.init(prow, c64, s.sp, a.V);
            weight_tile_range<TIF>(f, lo, hi, put, ps, pgs);
        } else if (kind == kPassResid) {   // the correction is known: w~ alone
            ResidualWeights<DT, false, false> f;
            f.init(prow, qrow, c64, s.sp, log2_norm(s.sq), coef, a.V);
            f.Hk += kappa;
            weight_tile_range<TIF>(f, lo, hi, put, ps, pgs);
        } else {
            ResidualWeights<DT> f;
            f.init(prow, qrow, c64, s.sp, log2_norm(s.sq), coef, a.V);
            weight_tile_range<TIF>(f, lo, hi, put, ps, pgs);
        }
        const int nt = hi - lo;
        double mw = 0.0, mq = 0.0;
        __shared__ double s_mw, s_mq;
        __syncthreads();
        if (wave_id() == 0) {
            double x = 0.0, y = 0.0;
            for (int t = lane_id(); t < nt; t += kWaveSize) { x += s.tile[t]; y += double(s.tile_q[t]); }
            x = wave_sum(x);
            y = wave_sum(y);
            if (lane_id() == 0) { s_mw = x; s_mq = y; }
        }
        if (kind == kPassFirst) block_sum2(ps, pgs);
        __syncthreads();
        mw = s_mw;
        mq = s_mq;
        const uint32_t tag = pass_tag(a.epoch, pass);
        uint64_t* part = w.part + 2 * (int64_t(pass & 1u) * kMaxWalkers * kPassValues);
        if (threadIdx.x == 0) {
            uint64_t* mine = part + 2 * kPassValues * h;
            publish_pair(mine + 0, pack_f64(mw), tag);
            publish_pair(mine + 2, pack_f64(mq), tag);
            publish_pair(mine + 4, pack_f64(ps), tag);
            publish_pair(mine + 6, pack_f64(pgs), tag);
        }
        if (!gather_pairs(part, a.H * kPassValues, tag, a.wait_ticks, s.msg)) return false;
        __shared__ double s_kappa, s_A;
        if (threadIdx.x == 0) {
            double P = 0.0, PG = 0.0;
            if (kind == kPassFirst) {
                for (int k = 0; k < a.H; ++k) {
                    P += unpack_f64(s.msg[kPassValues * k + 2]);
                    PG += unpack_f64(s.msg[kPassValues * k + 3]);
                }
            }
            const double kap = kind == kPassFirst ? correction_kappa(P, PG) : kappa;
            const double ca = kind == kPassFirst ? correction_a(kap) : 0.0;
            for (int k = 0; k < a.H; ++k)
                s.part[k] = unpack_f64(s.msg[kPassValues * k]) + ca * unpack_f64(s.msg[kPassValues * k + 1]);
            s_kappa = kap;
            s_A = kind == kPassFirst ? P : A;
        }
        __syncthreads();
        if (kind == kPassFirst) {
            kappa = s_kappa;
            A = s_A > 0.0 ? s_A : 1.0;
            const double ca = correction_a(kappa);
            for (int t = threadIdx.x; t < nt; t += kThreads) s.tile[t] += ca * double(s.tile_q[t]);
            __syncthreads();
        }
        double t = 0.0;
        for (int k = 0; k < a.H; ++k) t += s.part[k];
        *total = t;
        return true;
    }

    // The next batch of the node's children (ascending ids; the first batch
    // of a node starts after the node and also brings the node's statistics)
    // and their accept-test inputs. The children's logits are loaded while
    // the node's words are awaited (the wait leaves them in LDS), so the two
    // take one round trip. Whole workgroup; false if a wait for the node's
    // words ran out.
    __device__ __forceinline__ bool next_batch(int node, bool first) {
        const uint64_t* slots = a.slots + 2 * int64_t(b) * 2 * N * a.S;
        if (wave_id() == 0) {
            int n = 0, base = first ? node + 1 : s.from;
            for (; base < N && n <= kThreads - kWaveSize; base += kWaveSize) {
                const int ch = base + lane_id();
                const bool is = ch < N && s.par[ch] == node;
                const uint64_t m = __ballot(is);
                if (is) s.kid[n + lanes_below(m)] = ch;
                n += __popcll(m);
            }
            if (lane_id() == 0) { s.nk = n; s.from = base; }
        }
        __syncthreads();
        // The children's logits are inputs: their loads are in flight while
        // the node's words are awaited.
        const bool mine = threadIdx.x < s.nk;
        const int ch = mine ? s.kid[threadIdx.x] : 0;
        const int32_t t = mine ? s.tok[ch] : -1;
        const bool in_range = t >= 0 && t < a.V;
        const float zp = in_range ? load_elem<DT>(prow, t) : -INFINITY;
        const float zq = in_range ? load_elem<DT>(qrow, t) : -INFINITY;
        if (first) {
            if (kStreaming && !wait_node(slots, N, a.S, node, true, a.epoch, a.wait_ticks, s.nodew)) return false;
            if (wave_id() == 1) {  // the node's statistics
                const bool lane_ok = lane_id() < a.S;
                uint64_t wp = 0ull, wq = 0ull;
                if (lane_ok) {
                    wp = kStreaming ? s.nodew[lane_id()] : read_pair(slots, int64_t(node) * a.S + lane_id());
                    wq = kStreaming ? s.nodew[a.S + lane_id()]
                                    : read_pair(slots, int64_t(N + node) * a.S + lane_id());
                }
                const RowStats sp = merge_chunk_words(wp, a.S, false, c);
                const RowStats sq = merge_chunk_words(wq, a.S, false, c);
                if (lane_id() == 0) { s.sp = sp; s.sq = sq; }
            }
        }
        __syncthreads();
        if (mine) {
            s.pc[threadIdx.x] = in_range ? prob_of(zp, c, s.sp) : 0.0;
            s.qc[threadIdx.x] = in_range ? prob_of(zq, c, s.sq) : 0.0;
            s.zp[threadIdx.x] = zp;
            s.zq[threadIdx.x] = zq;
            s.u[threadIdx.x] = stream_uniform(a.seed, a.offset, uint32_t(b), 1u, uint32_t(ch));
        }
        __syncthreads();
        return true;
    }

    // p(t) / q(t) at child k of the batch once the node's correction is
    // known: 2^(kappa - h), h = (zq - zp) c - (B_q - B_p), in fp64 (no
    // difference of probabilities).
    __device__ __forceinline__ double p_over_q(int k) const {
        const double hk = fma(double(s.zq[k]) - double(s.zp[k]), c64, -(log2_norm(s.sq) - log2_norm(s.sp)));
        return exp2(kappa - hk);
    }

    // Final draw from the weights of the last pass (the walkers' totals in
    // s.part, total W): the walker whose share holds v * W finds the tile and
    // the token and publishes it. Returns whether a draw was made.
    __device__ __forceinline__ bool draw(PassKind kind, double coef, double W) {
        if (!(W > 0.0)) return false;
        const double want = double(v) * W;
        int owner = -1;
        double base = 0.0, acc = 0.0;
        for (int k = 0; k < a.H; ++k) {  // same in every thread of every walker
            const double P = s.part[k];
            if (P > 0.0) {
                owner = k;
                base = acc;
                if (acc + P >= want) break;
            }
            acc += P;
        }
        if (h == owner) {
            double tin = 0.0;
            const int t = find_tile(s.tile, hi - lo, base, want, &tin);
            int32_t bonus = -1;
            if (t >= 0) {
                if (kind == kPassTarget) {
                    TargetWeights<DT> f;
                    f.init(prow, c64, s.sp, a.V);
                    bonus = sample_in_tile(f, lo + t, tin);
                } else {
                    ResidualWeights<DT> f;
                    f.init(prow, qrow, c64, s.sp, log2_norm(s.sq), coef, a.V);
                    if (kind == kPassResid) f.Hk += kappa;
                    else f.a = float(correction_a(kappa));
                    bonus = sample_in_tile(f, lo + t, tin);
                }
            }
            if (threadIdx.x == 0) publish_pair(w.bonus, uint64_t(uint32_t(bonus)), a.epoch);
        }
        return owner >= 0;
    }
};

// Walker h of tree b (N <= NM). kStreaming: the tree's rows may still be
// streaming (one-launch form): the walk waits for each node's words when it
// reaches the node (rows are dispatched in node order, so the walk follows
// the stream of its tree), and walker 0 waits for every word of the tree
// before returning them to zero. The words are written once, so all walkers
// see the same statistics and take the same walk.
template <int DT, int NM, int TIF, bool kStreaming>
__device__ __forceinline__ void tree_walk(const TreeArgs& a, int b, int h) {
    constexpr int esz = ElemT<DT>::kBytes;
    __shared__ WalkLds<NM> s;
    __shared__ int s_nacc, s_fail;
    const int N = a.N;
    const float T = a.temperature[b];
    const bool greedy = !(T > 0.0f);
    const WalkWords w = walk_of(a, b);
    uint64_t* slots = a.slots + 2 * int64_t(b) * 2 * N * a.S;

    if (greedy && h != 0) {  // VerifyGreedy is one walker's argmax walk
        if (threadIdx.x == 0) publish_pair(w.ack + 2 * h, 1ull, a.epoch);
        return;
    }
    if (threadIdx.x == 0) { s_nacc = 0; s_fail = 0; }
    for (int i = threadIdx.x; i < N; i += kThreads) {
        s.par[i] = a.parent[int64_t(b) * N + i];
        s.tok[i] = a.tokens[int64_t(b) * N + i];
    }
    __syncthreads();

    int32_t bonus = -1;
    bool drew = false;
    if (greedy) {  // VerifyGreedy
        int node = 0;
        while (true) {
            if (kStreaming && !wait_node(slots, N, a.S, node, false, a.epoch, a.wait_ticks, s.nodew)) {
                if (threadIdx.x == 0) s_fail = 1;
                break;
            }
            if (wave_id() == 0) {
                uint64_t wg = 0ull;
                if (lane_id() < a.S) wg = kStreaming ? s.nodew[lane_id()] : read_pair(slots, int64_t(node) * a.S + lane_id());
                const RowStats sg = merge_chunk_words(wg, a.S, true, 0.0f);
                if (lane_id() == 0) s.sp = sg;
            }
            __syncthreads();
            const int32_t g = s.sp.idx;
            if (wave_id() == 0) {
                int ch = -1;
                for (int base = node + 1; base < N && ch < 0; base += kWaveSize) {
                    const int c2 = base + lane_id();
                    const uint64_t m = __ballot(c2 < N && s.par[c2] == node && s.tok[c2] == g);
                    if (m) ch = base + __builtin_ctzll(m);
                }
                if (lane_id() == 0) {
                    if (ch >= 0) a.out_path[int64_t(b) * N + s_nacc] = ch;
                    s.ok = ch;
                    if (ch >= 0) s_nacc = s_nacc + 1;
                }
            }
            __syncthreads();
            if (s.ok < 0) { bonus = g; break; }
            node = s.ok;
        }
    } else {  // MSS
        Walker<DT, NM, TIF, kStreaming> wk{a, b, h, N, int(int64_t(a.ntiles) * h / a.H), int(int64_t(a.ntiles) * (h + 1) / a.H),
                      log2e_over(T), stream_uniform(a.seed, a.offset, uint32_t(b), 1u, uint32_t(N)),
                      1.4426950408889634 / double(T), w, s, nullptr, nullptr};
        int node = 0;
        bool failed = false;
        while (!failed) {
            wk.prow = row_ptr(a.target, esz, b, node);
            wk.qrow = row_ptr(a.draft, esz, b, node);
            if (!wk.next_batch(node, true)) { failed = true; break; }
            // r = max(0, p - cj q) / Mj (probability units); identical in every
            // walker. The node's first rejection measures its correction.
            double cj = 0.0, Mj = 1.0;
            bool measured = false;
            bool tiles_valid = false;    // the last pass's tiles hold the weights of the current r
            PassKind last_kind = kPassTarget;
            bool any_child = false, accepted = false;
            int k = 0;
            while (true) {
                if (k == s.nk) {
                    if (s.from >= N) break;
                    __syncthreads();   // every thread is done with the previous batch
                    wk.next_batch(node, false);   // no wait: the node's words were read already
                    k = 0;
                    continue;
                }
                any_child = true;
                double ratio;        // r(t) / q(t)
                if (!measured) {     // r = p: the streaming statistics suffice
                    const double pt = s.pc[k], qt = s.qc[k];
                    ratio = qt > 0.0 ? pt / qt : -1.0;
                } else {
                    ratio = s.qc[k] > 0.0 ? fmax(wk.p_over_q(k) - cj, 0.0) / Mj : -1.0;
                }
                if (ratio >= 0.0 && double(s.u[k]) <= ratio) {
                    const int ch = s.kid[k];
                    if (threadIdx.x == 0) {
                        if (h == 0) a.out_path[int64_t(b) * N + s_nacc] = ch;
                        s_nacc = s_nacc + 1;
                    }
                    node = ch;
                    accepted = true;
                    break;
                }
                // Rejected: r <- norm(max(0, r - q)).
                const PassKind kind = measured ? kPassResid : kPassFirst;
                const double coef = cj + Mj;
                double Wsum = 0.0;
                if (!wk.run_pass(kind, coef, &Wsum)) { failed = true; break; }
                measured = true;
                const double M = Wsum / wk.A;
                if (M > 0.0) { cj = coef; Mj = M; tiles_valid = true; last_kind = kind; }
                else tiles_valid = false;
                ++k;
            }
            if (failed) break;
            if (accepted) { __syncthreads(); continue; }

            // Every child rejected (or a leaf): draw the bonus from the last
            // residual, or from p when no residual of positive mass was formed.
            const bool from_p = !any_child || cj == 0.0;
            double W = Mj * wk.A;
            PassKind kind = last_kind;
            bool ok = true;
            if (from_p) { kind = kPassTarget; ok = wk.run_pass(kPassTarget, 0.0, &W); }
            else if (!tiles_valid) { kind = kPassResid; ok = wk.run_pass(kPassResid, cj, &W); }
            if (!ok) { failed = true; break; }
            drew = wk.draw(kind, kind == kPassTarget ? 0.0 : cj, W);
            break;
        }
        if (failed && threadIdx.x == 0) s_fail = 1;
    }
    __syncthreads();

    if (h != 0) {  // done with every word of the tree: acknowledge and leave
        if (threadIdx.x == 0) publish_pair(w.ack + 2 * h, 1ull, a.epoch);
        return;
    }
    // Walker 0: wait for the other walkers (and the drawn token), write the
    // outcome, return every word of the tree to zero.
    __shared__ int s_done;
    if (wave_id() == 0) {
        int ok = 0;
        for (const WaitBound t(a.wait_ticks); !t.expired();) {
            bool mine = lane_id() == 0 || lane_id() >= a.H ||
                        pair_ok(peek(w.ack + 2 * lane_id()), peek(w.ack + 2 * lane_id() + 1), a.epoch);
            if (lane_id() == 0 && drew) mine = pair_ok(peek(w.bonus), peek(w.bonus + 1), a.epoch);
            if (__all(mine)) { ok = 1; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane_id() == 0) s_done = ok;
    }
    __syncthreads();
    if (drew && threadIdx.x == 0) bonus = s_done ? int32_t(uint32_t(read_pair(w.bonus, 0))) : -1;
    // No row of the tree may publish after its words are returned to zero.
    const bool rows_done = !kStreaming || wait_pairs(slots, int64_t(2) * N * a.S, a.epoch, a.wait_ticks);
    const bool fail = s_fail || !s_done || !rows_done;
    const int nacc = s_nacc;
    for (int j = nacc + threadIdx.x; j < N; j += kThreads) a.out_path[int64_t(b) * N + j] = -1;
    zero_pairs(slots, int64_t(2) * N * a.S);
    for (int i = threadIdx.x; i < kWalkWords; i += kThreads) clear_word(w.part + i);
    if (threadIdx.x == 0) {
        a.out_nacc[b] = fail ? -1 : nacc;
        a.out_bonus[b] = fail ? -1 : bonus;
    }
}

// Walkers of a tree wait for each other: each workgroup takes its walker's
// number from the ticket counter (claim_one), so a tree's walkers are always
// claimed by running workgroups or by the next ones to start.
template <int DT>
__global__ __launch_bounds__(kThreads) void tree_walk_kernel(TreeArgs a) {
    const int64_t g = claim_one(a.queue, int64_t(a.B) * a.H);
    tree_walk<DT, kMaxTreeNodes, kWalkTiles, false>(a, int(g / a.H), int(g % a.H));
}

// Trees of up to kFusedTreeNodes nodes: rows and walkers in one launch, in the
// dispatch order of the chain launches (decode_chain): the H walkers of tree b
// follow the rows of tree b + D (D = 2), so that each walk overlaps the rows
// of later trees instead of waiting for the end of the whole stream. The walker's LDS
// is sized for the small trees and its passes keep fewer tiles in flight, so
// that the row workgroups keep their residency.
// The walker's registers (about 168 with two tiles in flight per wave, a few
// bytes spilled) set the whole launch's allocation; the bound keeps it at
// three workgroups per CU for the row workgroups.
template <int DT>
__global__ __launch_bounds__(kThreads, 3) void tree_fused_kernel(TreeArgs a) {
    const int64_t RS = int64_t(2) * a.N * a.S;
    const int64_t g = claim_one(a.queue, int64_t(a.B) * (RS + a.H));   // the one-launch grid (tree_grid)
    int b;
    int64_t w;
    decode_chain(g, a.B, a.B, RS, a.H, a.D, b, w);
    if (w >= RS) tree_walk<DT, kFusedTreeNodes, kFusedWalkTiles, true>(a, b, int(w - RS));
    else tree_row<DT, kFusedU>(a, b, w);
}

template <int DT>
hipError_t launch_tree_dt(const TreeArgs& a, hipStream_t stream) {
    if (tree_fused(a.N)) {
        // One launch, one task per workgroup in ticket order (claim_one).
        // Rows never wait; a walker waits for its tree's rows (smaller
        // numbers) and for its tree's other walkers (neighbouring numbers).
        // Every task a waiter depends on is claimed by a running workgroup or
        // by the next workgroup to start, and rows always finish, so the
        // launch drains whatever order the hardware starts workgroups in.
        hipLaunchKernelGGL(tree_fused_kernel<DT>, dim3(unsigned(tree_grid(a.B, a.N, a.S, a.H))), dim3(kThreads), 0,
                           stream, a);
        return hipGetLastError();
    }
    const int64_t grid = int64_t(a.B) * 2 * a.N * a.S;
    hipLaunchKernelGGL(tree_stats_kernel<DT>, dim3(unsigned(grid)), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // The walkers of a tree wait only for each other (tickets, claim_one); a
    // cooperative launch is not needed (it cost ~10-20 us here).
    hipLaunchKernelGGL(tree_walk_kernel<DT>, dim3(unsigned(int64_t(a.B) * a.H)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, int dtype, hipStream_t stream) {
    return dtype == DT_BF16 ? launch_tree_dt<DT_BF16>(a, stream) : launch_tree_dt<DT_F32>(a, stream);
}

}  // namespace specv
