// Kernel argument blocks and launchers (library-private; the public interface
// is include/specv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specv {

struct RowView {
    const void* data;
    int64_t stride_seq;
    int64_t stride_row;
};

// Chain verification. Per sequence there are R = 2*gamma + 1 row tasks
// (target rows 0..gamma, then draft rows 0..gamma-1), each split into S
// chunks of `chunk` elements; workgroup g publishes its chunk's statistics in
// slots[g] (one 64-bit word).
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
    // Fused top-F (verify_topf_kernel only).
    int32_t F;
    int32_t* out_topk;
    float* out_topk_logits;
};

// Tree verification. Per tree there are 2N row tasks (target rows of every
// node, then draft rows of every node), each split into S chunks, one slot
// per chunk.
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
};

struct TopFArgs {
    RowView draft;
    const int32_t* tokens;   // may be null
    int32_t B, gamma, V, F;
    int32_t* out_topk;
    float* out_logits;       // may be null
};

// Split of a row into chunks so that small batches still fill the GPU:
// aim for ~2048 workgroups, never chunks shorter than 4096 elements.
inline void choose_split(int64_t row_tasks, int64_t V, int32_t* S, int64_t* chunk) {
    int64_t s = (2048 + row_tasks - 1) / row_tasks;
    const int64_t by_len = V / 4096 > 0 ? V / 4096 : 1;
    if (s > by_len) s = by_len;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    int64_t c = (V + s - 1) / s;
    c = (c + 7) / 8 * 8;
    s = (V + c - 1) / c;
    *S = int32_t(s);
    *chunk = c;
}

hipError_t launch_chain(const ChainArgs& a, int dtype, hipStream_t stream);
hipError_t launch_verify_topf(const ChainArgs& a, int dtype, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, int dtype, hipStream_t stream);
hipError_t launch_topf(const TopFArgs& a, int dtype, hipStream_t stream);
hipError_t launch_uniforms(uint64_t seed, uint64_t offset, int32_t tag, int32_t B,
                           int32_t J, float* out, hipStream_t stream);

}  // namespace specv
