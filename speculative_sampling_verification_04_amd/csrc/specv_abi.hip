// C ABI of libspecv.so (declared in include/specv.h): argument validation,
// workspace sizing and kernel launches. Nothing here allocates device memory
// or synchronises; a non-OK status means nothing was launched (except
// SPECV_ERR_HIP, a failed launch).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>
#include <string>

#include "specv.h"
#include "specv_device.hpp"
#include "specv_launch.hpp"

namespace specv {

namespace {

thread_local std::string g_error;

specv_status fail(specv_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

specv_status ok() {
    g_error.clear();
    return SPECV_OK;
}

// Bound on the kernels' waits for each other's words (WaitBound ticks); only
// tests change it (specv_debug_set_wait_bound). A chain bonus task waits at
// most kRescueTicks before it defers its sequence to the finisher launch; a
// tree task's wait that reaches the bound makes its tree report -1.
std::atomic<uint64_t> g_wait_ticks{kMaxWaitTicks};
uint64_t wait_ticks() { return g_wait_ticks.load(std::memory_order_relaxed); }
uint64_t chain_wait_ticks() {
    const uint64_t t = wait_ticks();
    return t < kRescueTicks ? t : kRescueTicks;
}

// Every call tags the values its workgroups publish with a new epoch, so a
// word left in a workspace by an earlier call (a writer that published after
// its reader's bounded wait gave up) never reads as published. Epochs skip
// values whose low 16 bits are 0 (the tree's pass tags keep those bits).
std::atomic<uint32_t> g_epoch{0};
uint32_t next_epoch() {
    uint32_t e;
    do {
        e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    } while ((e & 0xffffu) == 0);
    return e;
}

int elem_size(int32_t dtype) { return dtype == SPECV_BF16 ? 2 : 4; }


constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

static_assert(kMaxTreeNodes == SPECV_MAX_TREE_NODES, "the walk keeps a whole tree in LDS");
static_assert(kMaxPositions == SPECV_MAX_GAMMA + 1, "per-position fan-out table");
static_assert(kTopfKeyWords == SPECV_MAX_TOPF + 1, "F + 1 chunk keys per top-F chunk");

// Largest grid the launches accept (grid.x * 256 threads must fit 32 bits).
constexpr int64_t kMaxGrid = (int64_t(1) << 32) / kThreads - 1;

specv_status check_logits(const char* name, const specv_logits& l) {
    if (l.data == nullptr) return fail(SPECV_ERR_INVALID_ARG, "%s.data is NULL", name);
    if (l.dtype != SPECV_F32 && l.dtype != SPECV_BF16)
        return fail(SPECV_ERR_UNSUPPORTED, "%s.dtype %d is not SPECV_F32 or SPECV_BF16", name, l.dtype);
    if (reinterpret_cast<uintptr_t>(l.data) % elem_size(l.dtype) != 0)
        return fail(SPECV_ERR_INVALID_ARG, "%s.data is not aligned to its element size", name);
    if (l.stride_seq < 0 || l.stride_row < 0)
        return fail(SPECV_ERR_INVALID_ARG, "%s strides must be >= 0", name);
    return SPECV_OK;
}

specv_status check_workspace(void* ws, size_t have, size_t need) {
    if (need > 0 && ws == nullptr) return fail(SPECV_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
        return fail(SPECV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (have < need)
        return fail(SPECV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    return SPECV_OK;
}

RowView view(const specv_logits& l) { return RowView{l.data, l.stride_seq, l.stride_row}; }

// Workspace: a 256-byte header (word 0: a tree launch's ticket counter,
// TaskQueue, zero at rest; word 1: the number of sequences that chain
// launches left to their finisher, a statistic that only grows), then every value a tagged pair of 64-bit words (kPair
// bytes): one pair per row chunk (its statistics); then, when the bonus draw
// is shared by H > 1 workgroups, two pairs per residual tile of every
// sequence (the tile's sums of w~ and q~) and two per bonus workgroup (its
// correction sums); the fused kernel's top-F chunk keys; last, two deferral
// pairs per sequence (chain launches; the finisher's).
constexpr size_t kPair = 2 * sizeof(uint64_t);
constexpr size_t kHeader = 256;
struct Layout {
    int32_t S;
    int64_t chunk;
    int32_t H;
    int32_t ntiles;
    size_t slot_bytes;
    size_t tile_bytes;
    size_t part_bytes;
    size_t key_bytes = 0;    // fused kernel with S > 1: the draft-row chunks' top-F keys
    size_t mark_bytes;       // chain launches: two deferral pairs per sequence (the finisher's)
    size_t mark_offset() const { return kHeader + slot_bytes + tile_bytes + part_bytes + key_bytes; }
    size_t total() const { return mark_offset() + mark_bytes; }
};

Layout layout_for(int64_t batch, int64_t row_tasks_per_seq, int64_t vocab) {
    Layout L;
    choose_split(batch * row_tasks_per_seq, vocab, &L.S, &L.chunk);
    L.H = bonus_helpers(vocab, batch);
    L.ntiles = int32_t((vocab + kTileElems - 1) / kTileElems);
    L.slot_bytes = round_up(size_t(batch) * row_tasks_per_seq * L.S * kPair);
    L.tile_bytes = L.H > 1 ? round_up(size_t(batch) * L.ntiles * 2 * kPair) : 0;
    L.part_bytes = L.H > 1 ? round_up(size_t(batch) * L.H * 2 * kPair) : 0;
    L.mark_bytes = round_up(size_t(batch) * 2 * kPair);
    return L;
}

// Layout of the fused kernel: 2*gamma + 2 rows per sequence in S chunks
// (small_split) and, with the cache outputs, three cache words per draft row;
// then the tile words; then, with S > 1, the draft-row chunks' top-F keys.
Layout fused_layout(int64_t batch, int64_t gamma, int64_t vocab, bool cache_words = false) {
    Layout L = layout_for(batch, 2 * gamma + 2, vocab);
    small_split(batch * (2 * gamma + 2), vocab, &L.S, &L.chunk);
    const int64_t pairs = (2 * gamma + 2) * L.S + (cache_words ? 3 * (gamma + 1) : 0);
    L.slot_bytes = round_up(size_t(batch) * pairs * kPair);
    L.key_bytes = L.S > 1 ? round_up(size_t(batch) * (gamma + 1) * L.S * kTopfKeyWords * kPair) : 0;
    return L;
}

// Plain chain verification: softmax drafts, exact rule, no cache outputs.
void set_plain(ChainArgs& a, int32_t F) {
    a.F = F;
    for (int k = 0; k < kMaxPositions; ++k) a.Fk[k] = F;
    a.cache_words = 0;
    a.C = 1.0f;
    a.lenience = 1.0f;
    a.out_hit = nullptr;
}

void set_bonus(ChainArgs& a, const Layout& L, int64_t row_words, void* workspace, int esz) {
    a.D = bonus_delay(a.B, row_words);
    a.cache_rows = cached_positions(a.D, int64_t(a.V) * esz, int64_t(a.gamma) + 1);
    a.S = L.S;
    a.chunk = L.chunk;
    a.H = L.H;
    a.ntiles = L.ntiles;
    a.marks = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + L.mark_offset());
    a.deferred = static_cast<uint64_t*>(workspace) + 1;
    char* ws = static_cast<char*>(workspace) + kHeader;
    a.slots = reinterpret_cast<uint64_t*>(ws);
    a.tiles = L.H > 1 ? reinterpret_cast<uint64_t*>(ws + L.slot_bytes) : nullptr;
    a.parts = L.H > 1 ? reinterpret_cast<uint64_t*>(ws + L.slot_bytes + L.tile_bytes) : nullptr;
    a.epoch = next_epoch();
}

specv_status check_chain_sizes(int32_t batch, int32_t gamma, int32_t vocab) {
    if (batch < 1) return fail(SPECV_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (gamma < 1 || gamma > SPECV_MAX_GAMMA)
        return fail(SPECV_ERR_INVALID_ARG, "gamma must be in [1, %d] (got %d)", SPECV_MAX_GAMMA, gamma);
    if (vocab < 1 || vocab > SPECV_MAX_VOCAB)
        return fail(SPECV_ERR_INVALID_ARG, "vocab must be in [1, %d] (got %d)", SPECV_MAX_VOCAB, vocab);
    return SPECV_OK;
}

size_t verify_topk_bytes(int64_t batch, int64_t gamma, int64_t vocab) {
    return fused_layout(batch, gamma, vocab).total();
}

// Tree workspace: the header (ticket counter), the row pairs, then per tree
// the walk words (the walkers' pass messages, acknowledgements, the drawn
// token).
size_t tree_walk_offset(int64_t batch, int64_t nodes, int64_t vocab) {
    return kHeader + layout_for(batch, 2 * nodes, vocab).slot_bytes;
}
size_t tree_bytes(int64_t batch, int64_t nodes, int64_t vocab) {
    return tree_walk_offset(batch, nodes, vocab) + round_up(size_t(batch) * kWalkWords * sizeof(uint64_t));
}

specv_status check_tree_sizes(int32_t batch, int32_t nodes, int32_t vocab) {
    if (batch < 1) return fail(SPECV_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (nodes < 1 || nodes > SPECV_MAX_TREE_NODES)
        return fail(SPECV_ERR_INVALID_ARG, "nodes must be in [1, %d] (got %d)", SPECV_MAX_TREE_NODES, nodes);
    if (vocab < 1 || vocab > SPECV_MAX_VOCAB)
        return fail(SPECV_ERR_INVALID_ARG, "vocab must be in [1, %d] (got %d)", SPECV_MAX_VOCAB, vocab);
    return SPECV_OK;
}

specv_status check_ragged_sizes(int32_t batch, int32_t max_gamma, int32_t vocab) {
    if (batch < 1) return fail(SPECV_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (max_gamma < 0 || max_gamma > SPECV_MAX_GAMMA)
        return fail(SPECV_ERR_INVALID_ARG, "max_gamma must be in [0, %d] (got %d)", SPECV_MAX_GAMMA, max_gamma);
    if (vocab < 1 || vocab > SPECV_MAX_VOCAB)
        return fail(SPECV_ERR_INVALID_ARG, "vocab must be in [1, %d] (got %d)", SPECV_MAX_VOCAB, vocab);
    return SPECV_OK;
}

int64_t ragged_rows(int32_t max_gamma, bool has_draft) { return has_draft ? 2 * int64_t(max_gamma) + 1 : max_gamma + 1; }

}  // namespace

__global__ void uniforms_kernel(uint64_t seed, uint64_t offset, uint32_t tag, int32_t B, int32_t J, float* out) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < int64_t(B) * J)
        out[i] = stream_uniform(seed, offset, uint32_t(i / J), tag, uint32_t(i % J));
}

hipError_t launch_uniforms(uint64_t seed, uint64_t offset, int32_t tag, int32_t B, int32_t J, float* out,
                           hipStream_t stream) {
    const int64_t n = int64_t(B) * J;
    const unsigned blocks = unsigned((n + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(uniforms_kernel, dim3(blocks), dim3(kThreads), 0, stream, seed, offset, uint32_t(tag), B,
                       J, out);
    return hipGetLastError();
}

// The workspace of specv_verify_topk_noalloc: one array per GPU, held until
// the process ends. Host code never uses the name `scratch` as an address
// (on the host it stands for the symbol, not device memory): it asks each
// device for the array's address once (noalloc_scratch) and passes that.
constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

__global__ void zero_words_kernel(uint64_t* p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0;
}

namespace {
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // the array's address on each device, once set up
}  // namespace

// The array's address on the current device. The first call on a device
// looks it up (with that device current, as the lookup needs) and enqueues
// a clear of the whole array on `stream` (a kernel: no memset node, so the
// call can be captured in a graph). Allocates nothing.
specv_status noalloc_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SPECV_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
                                                  kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(SPECV_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
        hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(kThreads), 0, stream, static_cast<uint64_t*>(p),
                           int64_t(kScratchBytes / sizeof(uint64_t)));
        e = hipGetLastError();
        if (e != hipSuccess) return fail(SPECV_ERR_HIP, "clearing the scratch array failed: %s", hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SPECV_OK;
}

}  // namespace specv

using namespace specv;

extern "C" {

uint64_t specv_debug_set_wait_bound(uint64_t ticks) {
    return g_wait_ticks.exchange(ticks == 0 ? kMaxWaitTicks : ticks);
}

const char* specv_last_error(void) { return g_error.c_str(); }

const char* specv_version(void) { return "specv 0.1 (gfx950)"; }

specv_status specv_verify_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, size_t* bytes) {
    if (bytes == nullptr) return fail(SPECV_ERR_INVALID_ARG, "bytes is NULL");
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    *bytes = layout_for(batch, 2 * int64_t(gamma) + 1, vocab).total();
    return ok();
}

specv_status specv_verify_topk_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, size_t* bytes) {
    if (bytes == nullptr) return fail(SPECV_ERR_INVALID_ARG, "bytes is NULL");
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    *bytes = verify_topk_bytes(batch, gamma, vocab);
    return ok();
}

specv_status specv_tree_verify_workspace_size(int32_t batch, int32_t nodes, int32_t vocab, size_t* bytes) {
    if (bytes == nullptr) return fail(SPECV_ERR_INVALID_ARG, "bytes is NULL");
    specv_status st = check_tree_sizes(batch, nodes, vocab);
    if (st != SPECV_OK) return st;
    *bytes = tree_bytes(batch, nodes, vocab);
    return ok();
}

specv_status specv_verify(specv_logits target, specv_logits draft, const int32_t* draft_tokens,
                          const float* temperature, int32_t batch, int32_t gamma, int32_t vocab, uint64_t seed,
                          uint64_t offset, int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                          float* out_bonus_mass, void* workspace, size_t workspace_bytes, void* stream) {
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    if ((st = check_logits("target", target)) != SPECV_OK) return st;
    if ((st = check_logits("draft", draft)) != SPECV_OK) return st;
    if (target.dtype != draft.dtype)
        return fail(SPECV_ERR_UNSUPPORTED, "target and draft must have the same dtype");
    if (!draft_tokens || !temperature || !out_tokens || !out_num_accepted)
        return fail(SPECV_ERR_INVALID_ARG, "draft_tokens, temperature, out_tokens and out_num_accepted are required");
    const Layout L = layout_for(batch, 2 * int64_t(gamma) + 1, vocab);
    const int64_t grid = int64_t(batch) * ((2 * gamma + 1) * int64_t(L.S) + L.H);
    if (grid > kMaxGrid) return fail(SPECV_ERR_INVALID_ARG, "batch too large for one launch (%lld workgroups)", (long long)grid);
    if ((st = check_workspace(workspace, workspace_bytes, L.total())) != SPECV_OK) return st;

    ChainArgs a{};
    a.wait_ticks = chain_wait_ticks();
    a.target = view(target);
    a.draft = view(draft);
    a.tokens = draft_tokens;
    a.temperature = temperature;
    a.B = batch;
    a.gamma = gamma;
    a.V = vocab;
    set_bonus(a, L, (2 * int64_t(gamma) + 1) * L.S, workspace, elem_size(target.dtype));
    set_plain(a, 0);
    a.seed = seed;
    a.offset = offset;
    a.out_tokens = out_tokens;
    a.out_nacc = out_num_accepted;
    a.out_probs = out_probs;
    a.out_mass = out_bonus_mass;
    const hipError_t e = launch_chain(a, target.dtype == SPECV_BF16 ? DT_BF16 : DT_F32,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "specv_verify launch failed: %s", hipGetErrorString(e));
    return ok();
}

specv_status specv_verify_topk(specv_logits target, specv_logits draft, const int32_t* draft_tokens,
                               const float* temperature, int32_t batch, int32_t gamma, int32_t vocab, int32_t F,
                               uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_num_accepted,
                               float* out_probs, float* out_bonus_mass, int32_t* out_topk, float* out_topk_logits,
                               void* workspace, size_t workspace_bytes, void* stream) {
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    if ((st = check_logits("target", target)) != SPECV_OK) return st;
    if ((st = check_logits("draft", draft)) != SPECV_OK) return st;
    if (target.dtype != draft.dtype)
        return fail(SPECV_ERR_UNSUPPORTED, "target and draft must have the same dtype");
    if (F < 1 || F > SPECV_MAX_TOPF || F > vocab - 1)
        return fail(SPECV_ERR_INVALID_ARG, "F must be in [1, min(%d, vocab - 1)] (got %d, vocab %d)", SPECV_MAX_TOPF,
                    F, vocab);
    if (!draft_tokens || !temperature || !out_tokens || !out_num_accepted || !out_topk)
        return fail(SPECV_ERR_INVALID_ARG,
                    "draft_tokens, temperature, out_tokens, out_num_accepted and out_topk are required");
    const Layout L = fused_layout(batch, gamma, vocab);
    const int64_t grid = int64_t(batch) * ((2 * gamma + 2) * int64_t(L.S) + L.H);
    if (grid > kMaxGrid) return fail(SPECV_ERR_INVALID_ARG, "batch too large for one launch");
    if ((st = check_workspace(workspace, workspace_bytes, verify_topk_bytes(batch, gamma, vocab))) != SPECV_OK)
        return st;

    ChainArgs a{};
    a.wait_ticks = chain_wait_ticks();
    a.target = view(target);
    a.draft = view(draft);
    a.tokens = draft_tokens;
    a.temperature = temperature;
    a.B = batch;
    a.gamma = gamma;
    a.V = vocab;
    set_bonus(a, L, (2 * int64_t(gamma) + 2) * L.S, workspace, elem_size(target.dtype));
    if (L.S > 1)
        a.topf_keys = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kHeader + L.slot_bytes +
                                                  L.tile_bytes + L.part_bytes);
    a.seed = seed;
    a.offset = offset;
    a.out_tokens = out_tokens;
    a.out_nacc = out_num_accepted;
    a.out_probs = out_probs;
    a.out_mass = out_bonus_mass;
    set_plain(a, F);
    a.out_topk = out_topk;
    a.out_topk_logits = out_topk_logits;
    const hipError_t e = launch_verify_topf(a, target.dtype == SPECV_BF16 ? DT_BF16 : DT_F32,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "specv_verify_topk launch failed: %s", hipGetErrorString(e));
    return ok();
}

specv_status specv_verify_topk_noalloc(specv_logits target, specv_logits draft, const int32_t* draft_tokens,
                                       const float* temperature, int32_t batch, int32_t gamma, int32_t vocab,
                                       int32_t F, uint64_t seed, uint64_t offset, int32_t* out_tokens,
                                       int32_t* out_num_accepted, float* out_probs, float* out_bonus_mass,
                                       int32_t* out_topk, float* out_topk_logits, void* stream) {
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    const size_t need = verify_topk_bytes(batch, gamma, vocab);
    if (need > kScratchBytes)
        return fail(SPECV_ERR_WORKSPACE,
                    "specv_verify_topk_noalloc: batch %d, gamma %d, vocab %d need %zu workspace bytes, more than "
                    "its static %zu; use specv_verify_topk with a workspace",
                    batch, gamma, vocab, need, kScratchBytes);
    void* ws = nullptr;
    if ((st = noalloc_scratch(static_cast<hipStream_t>(stream), &ws)) != SPECV_OK) return st;
    return specv_verify_topk(target, draft, draft_tokens, temperature, batch, gamma, vocab, F, seed, offset,
                             out_tokens, out_num_accepted, out_probs, out_bonus_mass, out_topk, out_topk_logits, ws,
                             kScratchBytes, stream);
}

specv_status specv_verify_cache_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, size_t* bytes) {
    if (bytes == nullptr) return fail(SPECV_ERR_INVALID_ARG, "bytes is NULL");
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    *bytes = fused_layout(batch, gamma, vocab, true).total();
    return ok();
}

specv_status specv_verify_cache(specv_logits target, specv_logits draft, const int32_t* draft_tokens,
                                const float* temperature, int32_t batch, int32_t gamma, int32_t vocab,
                                const int32_t* fanout, float saguaro_C, float lenience, uint64_t seed,
                                uint64_t offset, int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                float* out_bonus_mass, int32_t* out_topk, float* out_topk_logits, int32_t* out_hit,
                                void* workspace, size_t workspace_bytes, void* stream) {
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    if ((st = check_logits("target", target)) != SPECV_OK) return st;
    if ((st = check_logits("draft", draft)) != SPECV_OK) return st;
    if (target.dtype != draft.dtype)
        return fail(SPECV_ERR_UNSUPPORTED, "target and draft must have the same dtype");
    if (fanout == nullptr) return fail(SPECV_ERR_INVALID_ARG, "fanout is NULL");
    int32_t fmax = 0;
    for (int k = 0; k <= gamma; ++k) {
        if (fanout[k] < 0 || fanout[k] > SPECV_MAX_TOPF || fanout[k] > vocab - 1)
            return fail(SPECV_ERR_INVALID_ARG, "fanout[%d] = %d must be in [0, min(%d, vocab - 1)]", k, fanout[k],
                        SPECV_MAX_TOPF);
        fmax = fanout[k] > fmax ? fanout[k] : fmax;
    }
    if (fmax < 1) return fail(SPECV_ERR_INVALID_ARG, "at least one fanout entry must be >= 1");
    if (!(saguaro_C >= 0.0f && saguaro_C <= 1.0f))
        return fail(SPECV_ERR_INVALID_ARG, "saguaro_C must be in [0, 1] (got %g)", double(saguaro_C));
    if (!(lenience > 0.0f && lenience <= 1.0f))
        return fail(SPECV_ERR_INVALID_ARG, "lenience must be in (0, 1] (got %g)", double(lenience));
    if (!draft_tokens || !temperature || !out_tokens || !out_num_accepted || !out_topk)
        return fail(SPECV_ERR_INVALID_ARG,
                    "draft_tokens, temperature, out_tokens, out_num_accepted and out_topk are required");
    const Layout L = fused_layout(batch, gamma, vocab, true);
    const int64_t grid = int64_t(batch) * ((2 * gamma + 2) * int64_t(L.S) + L.H);
    if (grid > kMaxGrid) return fail(SPECV_ERR_INVALID_ARG, "batch too large for one launch");
    if ((st = check_workspace(workspace, workspace_bytes, L.total())) != SPECV_OK) return st;

    ChainArgs a{};
    a.wait_ticks = chain_wait_ticks();
    a.target = view(target);
    a.draft = view(draft);
    a.tokens = draft_tokens;
    a.temperature = temperature;
    a.B = batch;
    a.gamma = gamma;
    a.V = vocab;
    set_bonus(a, L, (2 * int64_t(gamma) + 2) * L.S, workspace, elem_size(target.dtype));
    if (L.S > 1)
        a.topf_keys = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kHeader + L.slot_bytes +
                                                  L.tile_bytes + L.part_bytes);
    a.seed = seed;
    a.offset = offset;
    a.out_tokens = out_tokens;
    a.out_nacc = out_num_accepted;
    a.out_probs = out_probs;
    a.out_mass = out_bonus_mass;
    a.F = fmax;
    for (int k = 0; k < kMaxPositions; ++k) a.Fk[k] = k <= gamma ? fanout[k] : 0;
    a.out_topk = out_topk;
    a.out_topk_logits = out_topk_logits;
    a.cache_words = 1;
    a.C = saguaro_C;
    a.lenience = lenience;
    a.out_hit = out_hit;
    const hipError_t e = launch_verify_topf(a, target.dtype == SPECV_BF16 ? DT_BF16 : DT_F32,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "specv_verify_cache launch failed: %s", hipGetErrorString(e));
    return ok();
}

specv_status specv_verify_ragged_workspace_size(int32_t batch, int32_t max_gamma, int32_t vocab, int32_t has_draft,
                                                size_t* bytes) {
    if (bytes == nullptr) return fail(SPECV_ERR_INVALID_ARG, "bytes is NULL");
    specv_status st = check_ragged_sizes(batch, max_gamma, vocab);
    if (st != SPECV_OK) return st;
    *bytes = layout_for(batch, ragged_rows(max_gamma, has_draft != 0), vocab).total();
    return ok();
}

specv_status specv_verify_ragged(specv_logits target, specv_logits draft, const int32_t* draft_offsets,
                                 const int32_t* draft_tokens, const float* temperature, int32_t batch,
                                 int32_t max_gamma, int32_t num_draft, int32_t vocab, uint64_t seed, uint64_t offset,
                                 int32_t* out_tokens, int32_t* out_num_accepted, float* out_probs,
                                 float* out_bonus_mass, void* workspace, size_t workspace_bytes, void* stream) {
    specv_status st = check_ragged_sizes(batch, max_gamma, vocab);
    if (st != SPECV_OK) return st;
    const bool has_draft = draft.data != nullptr;
    if ((st = check_logits("target", target)) != SPECV_OK) return st;
    if (has_draft) {
        if ((st = check_logits("draft", draft)) != SPECV_OK) return st;
        if (target.dtype != draft.dtype)
            return fail(SPECV_ERR_UNSUPPORTED, "target and draft must have the same dtype");
    }
    if (num_draft < 0) return fail(SPECV_ERR_INVALID_ARG, "num_draft must be >= 0");
    if (!draft_offsets || !temperature || !out_tokens || !out_num_accepted || (num_draft > 0 && !draft_tokens))
        return fail(SPECV_ERR_INVALID_ARG,
                    "draft_offsets, draft_tokens, temperature, out_tokens and out_num_accepted are required");
    const Layout L = layout_for(batch, ragged_rows(max_gamma, has_draft), vocab);
    const int64_t grid = int64_t(batch) * (ragged_rows(max_gamma, has_draft) * L.S + L.H);
    if (grid > kMaxGrid) return fail(SPECV_ERR_INVALID_ARG, "batch too large for one launch");
    if ((st = check_workspace(workspace, workspace_bytes, L.total())) != SPECV_OK) return st;

    ChainArgs a{};
    a.wait_ticks = chain_wait_ticks();
    a.target = view(target);
    a.draft = view(draft);
    a.tokens = draft_tokens;
    a.temperature = temperature;
    a.B = batch;
    a.gamma = max_gamma;
    a.V = vocab;
    set_bonus(a, L, ragged_rows(max_gamma, has_draft) * L.S, workspace, elem_size(target.dtype));
    set_plain(a, 0);
    a.seed = seed;
    a.offset = offset;
    a.out_tokens = out_tokens;
    a.out_nacc = out_num_accepted;
    a.out_probs = out_probs;
    a.out_mass = out_bonus_mass;
    a.offsets = draft_offsets;
    a.num_draft = num_draft;
    const hipError_t e = launch_ragged(a, target.dtype == SPECV_BF16 ? DT_BF16 : DT_F32, !has_draft,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "specv_verify_ragged launch failed: %s", hipGetErrorString(e));
    return ok();
}

specv_status specv_geometric_fanout(int32_t K, double accept_rate, double r, int32_t budget, int32_t* out) {
    if (out == nullptr) return fail(SPECV_ERR_INVALID_ARG, "out is NULL");
    if (K < 0 || K > SPECV_MAX_GAMMA) return fail(SPECV_ERR_INVALID_ARG, "K must be in [0, %d]", SPECV_MAX_GAMMA);
    if (!(accept_rate > 0.0 && accept_rate < 1.0))
        return fail(SPECV_ERR_INVALID_ARG, "accept_rate must be in (0, 1) (got %g)", accept_rate);
    if (!(r > 0.0 && r < 1e6)) return fail(SPECV_ERR_INVALID_ARG, "r must be > 0 (got %g)", r);
    if (budget < 0) return fail(SPECV_ERR_INVALID_ARG, "budget must be >= 0");
    // Theorem 12: F_k = F0 a^(k/(1+r)) (k < K), F_K = F0 a^(K/(1+r)) (1-a)^(-1/(1+r)),
    // F0 from the budget.
    const double e = 1.0 / (1.0 + r);
    const double g = pow(accept_rate, e);
    const double tail = pow(accept_rate, K * e) * pow(1.0 - accept_rate, -e);
    const double F0 = double(budget) / (tail + (1.0 - pow(g, K)) / (1.0 - g));
    double F[SPECV_MAX_GAMMA + 1];
    for (int k = 0; k < K; ++k) F[k] = F0 * pow(accept_rate, k * e);
    F[K] = F0 * tail;
    // Largest remainder: floors, then +1 to the largest fractional parts
    // (lower k first among equal parts) until the budget is met.
    int64_t used = 0;
    for (int k = 0; k <= K; ++k) {
        out[k] = int32_t(floor(F[k]));
        used += out[k];
    }
    bool taken[SPECV_MAX_GAMMA + 1] = {};
    for (int64_t left = budget - used; left > 0; --left) {
        int best = -1;
        for (int k = 0; k <= K; ++k)
            if (!taken[k] && (best < 0 || F[k] - floor(F[k]) > F[best] - floor(F[best]))) best = k;
        if (best < 0) break;
        taken[best] = true;
        ++out[best];
    }
    return ok();
}

specv_status specv_bonus_topk(specv_logits draft, const int32_t* draft_tokens, int32_t batch, int32_t gamma,
                              int32_t vocab, int32_t F, int32_t* out_topk, float* out_topk_logits, void* stream) {
    specv_status st = check_chain_sizes(batch, gamma, vocab);
    if (st != SPECV_OK) return st;
    if ((st = check_logits("draft", draft)) != SPECV_OK) return st;
    if (F < 1 || F > SPECV_MAX_TOPF || F > vocab - 1)
        return fail(SPECV_ERR_INVALID_ARG, "F must be in [1, min(%d, vocab - 1)] (got %d, vocab %d)", SPECV_MAX_TOPF,
                    F, vocab);
    if (!out_topk) return fail(SPECV_ERR_INVALID_ARG, "out_topk is required");
    const int64_t grid = int64_t(batch) * (gamma + 1);
    if (grid > kMaxGrid) return fail(SPECV_ERR_INVALID_ARG, "batch too large for one launch");
    TopFArgs a;
    a.draft = view(draft);
    a.tokens = draft_tokens;
    a.B = batch;
    a.gamma = gamma;
    a.V = vocab;
    a.F = F;
    a.out_topk = out_topk;
    a.out_logits = out_topk_logits;
    const hipError_t e = launch_topf(a, draft.dtype == SPECV_BF16 ? DT_BF16 : DT_F32, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "specv_bonus_topk launch failed: %s", hipGetErrorString(e));
    return ok();
}

specv_status specv_tree_verify(specv_logits target, specv_logits draft, const int32_t* parent, const int32_t* tokens,
                               const float* temperature, int32_t batch, int32_t nodes, int32_t vocab, uint64_t seed,
                               uint64_t offset, int32_t* out_path, int32_t* out_num_accepted, int32_t* out_bonus,
                               void* workspace, size_t workspace_bytes, void* stream) {
    specv_status st = check_tree_sizes(batch, nodes, vocab);
    if (st != SPECV_OK) return st;
    if ((st = check_logits("target", target)) != SPECV_OK) return st;
    if ((st = check_logits("draft", draft)) != SPECV_OK) return st;
    if (target.dtype != draft.dtype)
        return fail(SPECV_ERR_UNSUPPORTED, "target and draft must have the same dtype");
    if (!parent || !tokens || !temperature || !out_path || !out_num_accepted || !out_bonus)
        return fail(SPECV_ERR_INVALID_ARG, "parent, tokens, temperature and the outputs are required");
    const Layout L = layout_for(batch, 2 * int64_t(nodes), vocab);
    const int32_t H = tree_walkers(vocab);
    if (tree_grid(batch, nodes, L.S, H) > kMaxGrid) return fail(SPECV_ERR_INVALID_ARG, "batch too large for one launch");
    if ((st = check_workspace(workspace, workspace_bytes, tree_bytes(batch, nodes, vocab))) != SPECV_OK) return st;

    TreeArgs a;
    a.wait_ticks = wait_ticks();
    a.target = view(target);
    a.draft = view(draft);
    a.parent = parent;
    a.tokens = tokens;
    a.temperature = temperature;
    a.B = batch;
    a.N = nodes;
    a.V = vocab;
    a.S = L.S;
    a.chunk = L.chunk;
    a.seed = seed;
    a.offset = offset;
    a.out_path = out_path;
    a.out_nacc = out_num_accepted;
    a.out_bonus = out_bonus;
    a.queue = static_cast<uint64_t*>(workspace);
    a.slots = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kHeader);
    a.H = H;
    a.ntiles = int32_t((int64_t(vocab) + kTileElems - 1) / kTileElems);
    // The walkers of tree b follow the rows of tree b + 2: a walk lasts
    // longer than its tree's rows take to stream (its passes are serial), so
    // it starts as soon as they are under way and follows them node by node
    // (measured: 245-250 us at 0-4 trees of delay, 263 us at ~one GPU-full,
    // 298 us at 24, for 32 trees of 64 nodes over V = 152064).
    a.D = tree_fused(nodes) ? (batch < 2 ? batch : 2) : 0;
    a.cache_nodes = cached_positions(batch, int64_t(vocab) * elem_size(target.dtype), nodes);
    a.walk = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + tree_walk_offset(batch, nodes, vocab));
    a.epoch = next_epoch();
    const hipError_t e = launch_tree(a, target.dtype == SPECV_BF16 ? DT_BF16 : DT_F32,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "specv_tree_verify launch failed: %s", hipGetErrorString(e));
    return ok();
}

specv_status specv_uniforms(uint64_t seed, uint64_t offset, int32_t tag, int32_t batch, int32_t count, float* out,
                            void* stream) {
    if (batch < 1 || count < 1) return fail(SPECV_ERR_INVALID_ARG, "batch and count must be >= 1");
    if (tag < 0 || tag > 255) return fail(SPECV_ERR_INVALID_ARG, "tag must be in [0, 255]");
    if (count > (1 << 26)) return fail(SPECV_ERR_INVALID_ARG, "count must be <= 2^26");
    if (int64_t(batch) * count > (int64_t(1) << 31)) return fail(SPECV_ERR_INVALID_ARG, "batch * count too large");
    if (!out) return fail(SPECV_ERR_INVALID_ARG, "out is NULL");
    const hipError_t e = launch_uniforms(seed, offset, tag, batch, count, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SPECV_ERR_HIP, "specv_uniforms launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
