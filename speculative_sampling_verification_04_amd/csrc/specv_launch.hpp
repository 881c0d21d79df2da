// Kernel argument blocks and launchers (library-private; the public interface
// is include/specv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "specv_device.hpp"
#include "specv_dispatch.hpp"

namespace specv {

constexpr int kMaxPositions = 65;  // gamma + 1 <= SPECV_MAX_GAMMA + 1

struct RowView {
    const void* data;
    int64_t stride_seq;
    int64_t stride_row;
};

// Chain verification. Per sequence there are R = 2*gamma + 1 row tasks
// (target rows 0..gamma, then draft rows 0..gamma-1), each split into S
// chunks of `chunk` elements, then H bonus workgroups; row chunk j of the
// sequence in dispatch slot s publishes its statistics as pair s * R * S + j
// of `slots` (two 64-bit words per pair, tagged with the call's epoch).
struct ChainArgs {
    RowView target, draft;
    const int32_t* tokens;
    const float* temperature;
    int32_t B, gamma, V, S;
    int64_t chunk;
    uint64_t seed, offset;
    int32_t* out_tokens;
    int32_t* out_nacc;
    float* out_probs;
    float* out_mass;
    uint64_t* slots;
    // Bonus draw of T > 0 sequences: H workgroups per sequence (dispatched
    // after its rows) share the tile sums of the weights; the last of them
    // resolves. With H > 1 they meet in `tiles` (ntiles words per sequence).
    int32_t H, ntiles;
    uint64_t* tiles;         // two pairs per tile per sequence slot (4 * ntiles words)
    uint64_t* parts;         // two pairs per bonus workgroup per sequence slot (4 * H words)
    int32_t D;               // bonus workgroups trail their rows by D sequences (see decode_chain)
    int32_t cache_rows;      // rows 0 .. cache_rows-1 of T > 0 sequences: cacheable loads (cached_positions)
    // Fused top-F (verify_topf_kernel only): F_k candidates at position k
    // (Fk[k] <= F), written with row stride F.
    int32_t F;
    int32_t* out_topk;
    float* out_topk_logits;
    int32_t Fk[kMaxPositions];
    // With S > 1 (small batches, no cache outputs): every draft-row chunk's
    // Fk + 1 largest keys, kTopfKeyWords words per chunk, merged by the
    // sequence's bonus workgroups; zero at rest.
    uint64_t* topf_keys;
    // SSD cache extensions (verify_topf_kernel only; off when cache_words = 0):
    // draft distribution sigma_{F_k,C} (C = 1: softmax), lenience l, and the
    // hit flag. With cache_words, every draft row also publishes three words
    // (after the 2*gamma + 2 row words of its sequence): the sigma
    // normaliser, the sigma threshold key and the cache threshold key.
    int32_t cache_words;
    float C;
    float lenience;
    int32_t* out_hit;
    // Ragged batches (ragged_verify_kernel only): sequence b's draft tokens are
    // tokens[offsets[b] .. offsets[b+1]); gamma is the largest allowed count.
    const int32_t* offsets;
    int32_t num_draft;
    uint64_t wait_ticks;     // bound on a bonus task's wait for other tasks' words; past it the sequence is deferred
    uint32_t epoch;          // this call's tag on every published pair (nonzero)
    // Deferral marks, two pairs per sequence slot (zero at rest): the
    // resolve, and (fused kernel) a draft row's top-F merge, left to the
    // finisher launch.
    uint64_t* marks;
    uint64_t* deferred;      // count of the sequences the finisher completed (a statistic; only grows)
};

// Tree verification. Per tree there are 2N row tasks (target rows of every
// node, then draft rows of every node), each split into S chunks, one pair
// per chunk (pair (b * 2N + task) * S + chunk of `slots`), and H walkers that
// meet in `walk` (kWalkWords words per tree: the walkers' pass messages for
// two pass parities, one acknowledgement per walker, the drawn token).
constexpr int kMaxWalkers = 16;   // their pass messages (4 pairs each) are gathered by one wave
constexpr int kMaxTreeNodes = 4096;  // SPECV_MAX_TREE_NODES
// Tiles of one walker's share: ceil(tiles / H) with H = tree_walkers(V) is at
// most 24 while tiles <= 384, and at most kMaxTiles / kMaxWalkers beyond.
constexpr int kMaxWalkTiles = kMaxTiles / kMaxWalkers;
constexpr int kWalkWords = 2 * (2 * kMaxWalkers * 4 + kMaxWalkers + 1);

struct TreeArgs {
    RowView target, draft;
    const int32_t* parent;
    const int32_t* tokens;
    const float* temperature;
    int32_t B, N, V, S;
    int64_t chunk;
    uint64_t seed, offset;
    int32_t* out_path;
    int32_t* out_nacc;
    int32_t* out_bonus;
    uint64_t* slots;
    int32_t H, ntiles;
    uint64_t* walk;
    // Nodes 0 .. cache_nodes-1 of T > 0 trees are streamed with ordinary
    // (cacheable) loads: the walk's passes re-read the rows of the nodes it
    // visits, shallow ones first (cached_positions with D = the batch).
    int32_t cache_nodes;
    // One-launch form (tree_fused): the walkers of tree b follow the rows of
    // tree b + D in dispatch order.
    int32_t D;
    uint64_t wait_ticks;     // bound on every wait for another workgroup's word (WaitBound)
    uint32_t epoch;          // this call's tag on every published pair (nonzero, low 16 bits too)
    uint64_t* queue;         // the launch's ticket counter (TaskQueue; zero at rest)
};

// Trees of up to this many nodes are verified in one launch.
constexpr int kFusedTreeNodes = 256;
inline bool tree_fused(int64_t N) { return N <= kFusedTreeNodes; }

// Workgroups of the tree launch that streams the rows: 2N row tasks of S
// chunks per tree, and in the one-launch form the H walkers.
inline int64_t tree_grid(int64_t B, int64_t N, int64_t S, int64_t H) {
    return B * (2 * N * S + (tree_fused(N) ? H : 0));
}

struct TopFArgs {
    RowView draft;
    const int32_t* tokens;   // may be null
    int32_t B, gamma, V, F;
    int32_t* out_topk;
    float* out_logits;       // may be null
};

// Workgroups that share the bonus draw of one T > 0 sequence: about 32 tiles
// (16K elements of the row pair) each, at most kMaxBonusHelpers (their two
// correction sums each are gathered by one wave). Batches of up to 64
// sequences leave most of the GPU idle while the draws run, so there each
// takes about 16 tiles (a shorter draw; at larger batches the extra
// workgroups cost more slots than they save).
constexpr int kMaxBonusHelpers = 16;
static_assert(2 * kMaxBonusHelpers <= kWaveSize, "one pair per lane in the resolve's gather");
inline int32_t bonus_helpers(int64_t V, int64_t B) {
    const int64_t ntiles = (V + kTileElems - 1) / kTileElems;
    const int64_t per = B <= 64 ? 16 : 32;
    const int64_t h = (ntiles + per - 1) / per;
    return int32_t(h < 1 ? 1 : h > kMaxBonusHelpers ? kMaxBonusHelpers : h);
}

// Positions whose rows a T > 0 sequence streams with ordinary (cacheable)
// loads: its bonus draw re-reads the rows of the first rejected position k,
// about D sequences (the bonus delay) after its rows were read, and low
// positions are the likely k's. The rows at those positions of D sequences
// must fit a share (kCacheBudget) of the device's last-level cache (256 MB of
// Infinity Cache on MI355X) for the re-read to hit there instead of HBM.
constexpr int64_t kCacheBudget = int64_t(160) << 20;
inline int32_t cached_positions(int64_t D, int64_t row_bytes, int64_t positions) {
    const int64_t per = 2 * D * row_bytes;   // one position's target and draft row over D sequences
    const int64_t p = per > 0 ? kCacheBudget / per : 0;
    return int32_t(p < positions ? p : positions);
}

// Walkers per tree for a vocabulary of V: about 24 tiles each, at most
// kMaxWalkers (measured on 32 trees of 64 nodes over V = 152064: 230 us at 24
// tiles per walker, 233 at 32, 238 at 16, 247 at 48; more walkers shorten
// each pass but hold more of the slots the rows stream in).
inline int32_t tree_walkers(int64_t V) {
    const int64_t ntiles = (V + kTileElems - 1) / kTileElems;
    const int64_t h = (ntiles + 23) / 24;
    return int32_t(h < 1 ? 1 : h > kMaxWalkers ? kMaxWalkers : h);
}

hipError_t launch_chain(const ChainArgs& a, int dtype, hipStream_t stream);
hipError_t launch_verify_topf(const ChainArgs& a, int dtype, hipStream_t stream);
hipError_t launch_ragged(const ChainArgs& a, int dtype, bool no_draft, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, int dtype, hipStream_t stream);
hipError_t launch_topf(const TopFArgs& a, int dtype, hipStream_t stream);
hipError_t launch_uniforms(uint64_t seed, uint64_t offset, int32_t tag, int32_t B,
                           int32_t J, float* out, hipStream_t stream);

}  // namespace specv
